"""GPU parity of the int8-MFMA GEMM (Q4_K weights x Q8_K activations).

The product of page 'The GGML ecosystem, and where synapse fits', section 5
('Products: weights against quantized activations'), on matrix cores: every
output must satisfy |y - y_ref| <= 1e-5 * T against the CPU oracle, for
ragged M and N (partial tiles in both directions), both workgroup tile
widths, grids with K split between two wave groups (at most 256 tiles and an
even count of super-blocks) and without, and any N through algo=2; results
are deterministic and nothing is written past y."""
import numpy as np
import pytest
import torch

import block_quantized_amd as Q
import oracle as O
import synth
from gpu_util import assert_within_tolerance, run_product, tile_rows, to_cpu, to_gpu

pytestmark = pytest.mark.gpu


def run(W, xq, M, N, K, algo=2):
    return run_product(Q.QMM_Q4_K, W, xq, M, N, K, algo=algo)


@pytest.mark.parametrize("M,N,K", [(32, 32, 256), (1, 9, 256), (31, 33, 512), (130, 100, 768), (300, 129, 1024),
                                   (128, 512, 4096), (4113, 64, 2048), (77, 1, 256), (64, 8, 512), (2000, 200, 256),
                                   (16384, 65, 512), (16400, 65, 512)])
def test_gemm_q4k_shapes(M, N, K):
    g = np.random.default_rng(M * 7 + N * 13 + K)
    W = synth.q4_k_random(g, M, K)
    x = g.standard_normal((N, K), dtype=np.float32)
    xq = O.quantize(O.Q8_K, x)
    print("gemm", M, N, K, flush=True)
    y = run(W, xq, M, N, K)
    y_ref, T = O.mul_mat(O.Q4_K, W, xq, M, N, K)
    assert_within_tolerance(y, y_ref, T, what=f"GEMM {M}x{K} N={N}")


def test_gemm_matches_gemv_within_tolerance():
    g = np.random.default_rng(5)
    M, N, K = 256, 24, 4096
    W = synth.q4_k_random(g, M, K)
    xq = O.quantize(O.Q8_K, g.standard_normal((N, K), dtype=np.float32))
    y_gemm = run(W, xq, M, N, K, algo=2)
    y_gemv = run(W, xq, M, N, K, algo=1)
    y_ref, T = O.mul_mat(O.Q4_K, W, xq, M, N, K)
    assert_within_tolerance(y_gemm, y_ref, T, what="gemm")
    assert_within_tolerance(y_gemv, y_ref, T, what="gemv")
    assert np.all(np.abs(y_gemm.astype(np.float64) - y_gemv) <= 2e-5 * T)


def test_gemm_extreme_scales_and_zero_rows():
    # scales and mins at their 6-bit maxima, all nibbles 15: the largest
    # integer sums the kernel can see; plus an all-zero activation row
    g = np.random.default_rng(9)
    M, N, K = 64, 40, 1024
    W = synth.q4_k_random(g, M, K).reshape(M, K // 256, 144)
    W[:8, :, 4:16] = 0xFF
    W[:8, :, 16:] = 0xFF
    W = W.reshape(M, -1)
    x = g.standard_normal((N, K), dtype=np.float32)
    x[3] = 0
    x[5] = np.sign(x[5]) * 50.0
    xq = O.quantize(O.Q8_K, x)
    y = run(W, xq, M, N, K)
    y_ref, T = O.mul_mat(O.Q4_K, W, xq, M, N, K)
    assert_within_tolerance(y, y_ref, T, what="extremes")
    assert np.all(y[3] == 0)


def test_gemm_deterministic_and_in_bounds():
    g = np.random.default_rng(11)
    M, N, K = 1000, 150, 2048
    W = to_gpu(synth.q4_k_random(g, M, K))
    xq = to_gpu(O.quantize(O.Q8_K, g.standard_normal((N, K), dtype=np.float32)))
    outs = []
    for _ in range(3):
        buf = torch.full((N * M + 512,), float("nan"), dtype=torch.float32, device=W.device)
        assert Q.qmm_mul_mat_algo(Q.QMM_Q4_K, W, xq, buf, M, N, K, 2) == Q.QMM_OK
        b = to_cpu(buf)
        assert np.all(np.isnan(b[N * M:])), "wrote past the end of y"
        assert not np.any(np.isnan(b[:N * M]))
        outs.append(b[:N * M].view(np.uint32).copy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("M,N,K", [(33, 1, 2816), (100, 7, 2304), (4096, 32, 4096), (17, 31, 14336),
                                   (64, 2, 256), (4131, 16, 2048), (8192, 16, 4096), (4096, 12, 14336),
                                   (9000, 5, 1024)])
def test_gemm_q4k_narrow(M, N, K):
    # N <= 32 runs the narrow kernels: the super-blocks are split over the
    # waves of a workgroup (K/256 = 11, 9, 16, 56, 1, 8, 16, 56, 4 super-blocks:
    # some waves get none) and the partial tiles are summed in LDS; N <= 16
    # with M <= 8192 takes 16-row tiles (8 or 4 waves), the rest 32-row tiles
    g = np.random.default_rng(M * 3 + N * 5 + K)
    W = synth.q4_k_random(g, M, K)
    xq = O.quantize(O.Q8_K, g.standard_normal((N, K), dtype=np.float32))
    print("narrow", M, N, K, flush=True)
    y = run(W, xq, M, N, K)
    y_ref, T = O.mul_mat(O.Q4_K, W, xq, M, N, K)
    assert_within_tolerance(y, y_ref, T, what=f"narrow {M}x{K} N={N}")


@pytest.mark.parametrize("M,N,K", [(1000, 20, 3328), (1000, 13, 3328)])
def test_gemm_q4k_narrow_deterministic_and_in_bounds(M, N, K):
    g = np.random.default_rng(12 + N)
    W = to_gpu(synth.q4_k_random(g, M, K))
    xq = to_gpu(O.quantize(O.Q8_K, g.standard_normal((N, K), dtype=np.float32)))
    outs = []
    for _ in range(3):
        buf = torch.full((N * M + 512,), float("nan"), dtype=torch.float32, device=W.device)
        assert Q.qmm_mul_mat_algo(Q.QMM_Q4_K, W, xq, buf, M, N, K, 2) == Q.QMM_OK
        b = to_cpu(buf)
        assert np.all(np.isnan(b[N * M:])), "wrote past the end of y"
        assert not np.any(np.isnan(b[:N * M]))
        outs.append(b[:N * M].view(np.uint32).copy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


# ------------------------------------------------------------------ Q6_K

def run_q6k(W, xq, M, N, K, algo=2):
    return run_product(Q.QMM_Q6_K, W, xq, M, N, K, algo=algo)


@pytest.mark.parametrize("M,N,K", [(32, 32, 256), (1, 9, 256), (31, 33, 512), (130, 100, 768), (300, 32, 2048),
                                   (129, 65, 256), (77, 1, 256), (4100, 32, 4096), (64, 8, 1280),
                                   # N <= 32 with 11 / 9 / 4 super-blocks per row and ragged M
                                   (33, 5, 2816), (9000, 17, 2304), (8200, 31, 1024),
                                   # N > 32: K in two parts (ragged M and N, and a grid of more
                                   # than 256 tiles), and an odd super-block count that keeps K whole
                                   (200, 70, 2048), (33000, 40, 512), (1000, 40, 768)])
def test_gemm_q6k_shapes(M, N, K):
    g = np.random.default_rng(M * 5 + N * 17 + K)
    W = synth.q6_k_random(g, M, K)
    x = g.standard_normal((N, K), dtype=np.float32)
    xq = O.quantize(O.Q8_K, x)
    print("gemm q6_k", M, N, K, flush=True)
    y = run_q6k(W, xq, M, N, K)
    y_ref, T = O.mul_mat(O.Q6_K, W, xq, M, N, K)
    assert_within_tolerance(y, y_ref, T, what=f"Q6_K GEMM {M}x{K} N={N}")


def test_gemm_q6k_extreme_scales():
    # int8 scale extremes (-128, 127), all-ones and all-zero 6-bit codes, a
    # large activation row and a zero row
    g = np.random.default_rng(21)
    M, N, K = 96, 40, 1024
    W = synth.q6_k_random(g, M, K).reshape(M, K // 256, 210)
    W[:16, :, 192:208] = np.array([0x80, 0x7F] * 8, dtype=np.uint8)
    W[:8, :, :192] = 0xFF      # q = 63
    W[8:16, :, :192] = 0x00    # q = 0
    W = W.reshape(M, -1)
    x = g.standard_normal((N, K), dtype=np.float32)
    x[3] = 0
    x[5] = np.sign(x[5]) * 50.0
    xq = O.quantize(O.Q8_K, x)
    y = run_q6k(W, xq, M, N, K)
    y_ref, T = O.mul_mat(O.Q6_K, W, xq, M, N, K)
    assert_within_tolerance(y, y_ref, T, what="Q6_K extremes")
    assert np.all(y[3] == 0)


def test_gemm_q6k_head_sampled():
    # the 128256 x 4096 output head at batch 32, as the automatic choice runs
    # it: every output written, one row of every 32-row tile against the oracle
    g = np.random.default_rng(0)
    M, K = 128256, 4096
    N = 32
    W = synth.q6_k_random(g, M, K)
    xq = O.quantize(O.Q8_K, g.standard_normal((N, K), dtype=np.float32))
    y = run_product(Q.QMM_Q6_K, W, xq, M, N, K)
    rows = np.unique(np.concatenate([np.arange(8), M - 1 - np.arange(8), tile_rows(M, seed=1)]))
    y_ref, T = O.mul_mat(O.Q6_K, np.ascontiguousarray(W[rows]), xq, len(rows), N, K)
    assert_within_tolerance(y[:, rows], y_ref, T, what="Q6_K head N=32 (one row per 32-row tile)")


def test_gemm_q6k_ffn_down_batch512():
    # the 8B ffn_down (4096 x 14336, kept at Q6_K by Q4_K_M) at batch 512, as
    # the benchmark runs it: every output written, one row of every 32-row
    # tile against the oracle
    g = np.random.default_rng(3)
    M, K, N = 4096, 14336, 512
    W = synth.q6_k_random(g, M, K)
    xq = O.quantize(O.Q8_K, g.standard_normal((N, K), dtype=np.float32))
    print("gemm q6_k ffn_down b512", flush=True)
    y = run_product(Q.QMM_Q6_K, W, xq, M, N, K)
    rows = tile_rows(M, seed=3)
    y_ref, T = O.mul_mat(O.Q6_K, np.ascontiguousarray(W[rows]), xq, len(rows), N, K)
    assert_within_tolerance(y[:, rows], y_ref, T, what="Q6_K 4096x14336 N=512 (one row per 32-row tile)")


def test_gemm_q6k_deterministic_in_bounds_and_matches_gemv():
    g = np.random.default_rng(23)
    M, N, K = 700, 50, 2048
    W = to_gpu(synth.q6_k_random(g, M, K))
    xq = to_gpu(O.quantize(O.Q8_K, g.standard_normal((N, K), dtype=np.float32)))
    outs = []
    for _ in range(2):
        buf = torch.full((N * M + 512,), float("nan"), dtype=torch.float32, device=W.device)
        assert Q.qmm_mul_mat_algo(Q.QMM_Q6_K, W, xq, buf, M, N, K, 2) == Q.QMM_OK
        b = to_cpu(buf)
        assert np.all(np.isnan(b[N * M:])), "wrote past the end of y"
        outs.append(b[:N * M])
    assert np.array_equal(outs[0], outs[1])
    y_gemv = to_cpu(Q.mul_mat(Q.QMM_Q6_K, W, xq, M, N, K, algo=1)).reshape(-1)
    y_ref, T = O.mul_mat(O.Q6_K, to_cpu(W), to_cpu(xq), M, N, K)
    assert np.all(np.abs(outs[0].astype(np.float64) - y_gemv) <= 2e-5 * T.reshape(-1))


# ----------------------------------------------- Q4_0, Q5_0, Q8_0 (Q8_0 x)

def _q32_weights(g, wtype, M, K):
    if wtype == Q.QMM_Q5_0:
        return synth.q5_0_random(g, M, K)
    return O.quantize({Q.QMM_Q4_0: O.Q4_0, Q.QMM_Q8_0: O.Q8_0}[wtype], synth.normal_f32(g, (M, K), 0.02))


@pytest.mark.parametrize("wtype", [Q.QMM_Q4_0, Q.QMM_Q5_0, Q.QMM_Q8_0])
@pytest.mark.parametrize("M,N,K", [(32, 64, 128), (1, 9, 32), (31, 65, 96), (130, 100, 896), (300, 129, 1024),
                                   (128, 512, 2048), (77, 1, 160), (16384, 65, 512), (16400, 65, 512),
                                   # 258 and 512 tiles: K in two parts
                                   (16400, 100, 512), (8192, 512, 256),
                                   # chunks not a multiple of the parts: K in four
                                   # parts of 1, 2, 2, 2 and 9, 10, 9, 10 chunks,
                                   # in two parts of 1 and 2
                                   (896, 24, 896), (4864, 100, 896), (300, 70, 4864), (500, 40, 384)])
def test_gemm_q32_shapes(wtype, M, N, K):
    g = np.random.default_rng(M * 11 + N * 3 + K + wtype)
    W = _q32_weights(g, wtype, M, K)
    xq = O.quantize(O.Q8_0, g.standard_normal((N, K), dtype=np.float32))
    print("gemm q32", wtype, M, N, K, flush=True)
    y = run_product(wtype, W, xq, M, N, K, algo=2)
    ow = {Q.QMM_Q4_0: O.Q4_0, Q.QMM_Q5_0: O.Q5_0, Q.QMM_Q8_0: O.Q8_0}[wtype]
    y_ref, T = O.mul_mat(ow, W, xq, M, N, K)
    assert_within_tolerance(y, y_ref, T, what=f"GEMM type {wtype} {M}x{K} N={N}")


@pytest.mark.parametrize("wtype", [Q.QMM_Q4_0, Q.QMM_Q5_0, Q.QMM_Q8_0])
def test_gemm_q32_extremes_and_determinism(wtype):
    # codes at their extremes, a zero activation row, a large one; two runs
    # bit-identical and nothing written past y
    g = np.random.default_rng(50 + wtype)
    M, N, K = 96, 40, 512
    W = _q32_weights(g, wtype, M, K)
    S = {Q.QMM_Q4_0: 18, Q.QMM_Q5_0: 22, Q.QMM_Q8_0: 34}[wtype]
    bl = W.reshape(M, K // 32, S)
    bl[:8, :, 2:] = 0xFF
    bl[8:16, :, 2:] = 0x00 if wtype != Q.QMM_Q8_0 else 0x80
    x = g.standard_normal((N, K), dtype=np.float32)
    x[3] = 0
    x[5] = np.sign(x[5]) * 50.0
    xq = O.quantize(O.Q8_0, x)
    Wg, Xg = to_gpu(W), to_gpu(xq)
    outs = []
    for _ in range(2):
        buf = torch.full((N * M + 256,), float("nan"), dtype=torch.float32, device=Wg.device)
        assert Q.qmm_mul_mat_algo(wtype, Wg, Xg, buf, M, N, K, 2) == Q.QMM_OK
        b = to_cpu(buf)
        assert np.all(np.isnan(b[N * M:])), "wrote past the end of y"
        outs.append(b[:N * M].reshape(N, M))
    assert np.array_equal(outs[0], outs[1])
    ow = {Q.QMM_Q4_0: O.Q4_0, Q.QMM_Q5_0: O.Q5_0, Q.QMM_Q8_0: O.Q8_0}[wtype]
    y_ref, T = O.mul_mat(ow, W, xq, M, N, K)
    assert_within_tolerance(outs[0], y_ref, T, what="q32 extremes")
    assert np.all(outs[0][3] == 0)


@pytest.mark.parametrize("wtype", [Q.QMM_Q4_0, Q.QMM_Q5_0, Q.QMM_Q8_0])
@pytest.mark.parametrize("M,N,K", [(96, 40, 1024), (200, 70, 384), (70, 40, 128), (40, 33, 96)])
def test_gemm_q32_scale_extremes(wtype, M, N, K):
    # fp16 block scales at the ends of their range, on both sides: the
    # smallest and largest subnormals, the smallest normal, the largest finite
    # value and -0 for the weights; subnormal and large activation scales.  The
    # GEMM forms d_x d_w on the matrix core from fp16 operands, so subnormal
    # inputs must not be flushed.  Shapes: K split in four parts, in two
    # uneven parts, whole chunks without the split, a partial chunk.
    g = np.random.default_rng(70 + wtype + K)
    W = _q32_weights(g, wtype, M, K)
    S = {Q.QMM_Q4_0: 18, Q.QMM_Q5_0: 22, Q.QMM_Q8_0: 34}[wtype]
    bl = W.reshape(M, K // 32, S)
    for r0, bits in ((0, 0x0001), (8, 0x03FF), (16, 0x0400), (24, 0x7BFF), (32, 0x8000)):
        bl[r0:r0 + 8, :, 0] = bits & 0xFF
        bl[r0:r0 + 8, :, 1] = bits >> 8
    xq = O.quantize(O.Q8_0, g.standard_normal((N, K), dtype=np.float32))
    xb = xq.reshape(N, K // 32, 34)
    for r0, bits in ((0, 0x0001), (4, 0x0155), (8, 0x7BFF)):
        xb[r0:r0 + 4, :, 0] = bits & 0xFF
        xb[r0:r0 + 4, :, 1] = bits >> 8
    print("gemm q32 scale extremes", wtype, M, N, K, flush=True)
    ow = {Q.QMM_Q4_0: O.Q4_0, Q.QMM_Q5_0: O.Q5_0, Q.QMM_Q8_0: O.Q8_0}[wtype]
    y_ref, T = O.mul_mat(ow, W, xq, M, N, K)
    for algo in (2, 1):
        y = run_product(wtype, W, xq, M, N, K, algo=algo)
        assert np.all(np.isfinite(y))
        assert_within_tolerance(y, y_ref, T, what=f"q32 scale extremes algo {algo}")
    # products of two subnormal scales are far below the others but not zero
    assert np.all(y_ref[0:4, 0:8] != 0)


@pytest.mark.parametrize("wtype", [Q.QMM_Q4_0, Q.QMM_Q5_0, Q.QMM_Q8_0])
def test_gemm_q32_bench_size_sampled(wtype):
    # the 4096 x 4096, N = 512 product the benchmark times (automatic choice):
    # every output written, one row of every 32-row tile against the oracle
    M, N, K = 4096, 512, 4096
    g = synth.rng(0)
    W = _q32_weights(g, wtype, M, K)
    xq = O.quantize(O.Q8_0, synth.normal_f32(g, (N, K), 1.0))
    print("gemm q32 bench size", wtype, flush=True)
    y = run_product(wtype, W, xq, M, N, K)
    rows = tile_rows(M, seed=2)
    ow = {Q.QMM_Q4_0: O.Q4_0, Q.QMM_Q5_0: O.Q5_0, Q.QMM_Q8_0: O.Q8_0}[wtype]
    y_ref, T = O.mul_mat(ow, np.ascontiguousarray(W[rows]), xq, len(rows), N, K)
    assert_within_tolerance(y[:, rows], y_ref, T, what=f"GEMM type {wtype} 4096x4096 N=512")
