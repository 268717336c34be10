"""GPU parity of the product through the C ABI.

y[n][m] = sum_k w[m][k] x[n][k] (page 'ggml', examples/simple: ggml_mul_mat(A,
B^T) = C^T), computed per block as an integer dot scaled by the block scales
(page 'The GGML ecosystem, and where synapse fits', section 5, 'Products:
weights against quantized activations').  The GPU result must satisfy
|y - y_ref| <= 1e-5 * T per output, with y_ref and T from the CPU oracle
(T = sum of |terms|; for Q4_K the scale and min parts are counted apart).
Full workload sizes are checked on one row of every 32-row tile (all columns),
which the oracle computes one by one, and every output must have been written.
"""
import sys

import numpy as np
import pytest
import torch

import block_quantized_amd as Q
import oracle as O
import synth
from gpu_util import assert_within_tolerance, run_product, tile_rows, to_cpu, to_gpu

pytestmark = pytest.mark.gpu

WTYPES = [Q.QMM_Q4_0, Q.QMM_Q8_0, Q.QMM_Q4_K, Q.QMM_Q6_K]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_weights(g, wt, M, K):
    if wt == Q.QMM_Q4_K:
        return synth.q4_k_random(g, M, K)
    if wt == Q.QMM_Q6_K:
        return synth.q6_k_random(g, M, K)
    if wt == Q.QMM_Q5_0:
        return synth.q5_0_random(g, M, K)
    return O.quantize(O.Q8_0 if wt == Q.QMM_Q8_0 else O.Q4_0, synth.normal_f32(g, (M, K), 0.02))


def check(wt, W, x, M, N, K, rows=None, algo=0, what=""):
    """Run the GPU product on the full matrix; compare all rows or `rows`
    (all N columns of each)."""
    xt = O.VEC_DOT_TYPE[wt]
    xq = O.quantize(xt, x)
    y = run_product(wt, W, xq, M, N, K, algo=algo)  # every output written, nothing past y
    if rows is None:
        y_ref, T = O.mul_mat(wt, W, xq, M, N, K)
        assert_within_tolerance(y, y_ref, T, what=what)
    else:
        Ws = np.ascontiguousarray(W[rows])
        y_ref, T = O.mul_mat(wt, Ws, xq, len(rows), N, K)
        assert_within_tolerance(y[:, rows], y_ref, T, what=what)
    return y


# ----------------------------------------------------- the five workloads

def test_config_q8_0_gemv_2048():
    g = synth.rng(0)
    Wf = synth.normal_f32(g, (2048, 2048), 0.02)
    x = synth.normal_f32(g, (1, 2048), 1.0)
    say("Q8_0 2048x2048 N=1")
    check(Q.QMM_Q8_0, O.quantize(O.Q8_0, Wf), x, 2048, 1, 2048, what="Q8_0 GEMV")


@pytest.mark.parametrize("M,K", [(2048, 2048), (512, 2048), (8192, 2048), (2048, 8192)])
def test_config_q4_0_gemv_1b_shapes(M, K):
    g = synth.rng(0)
    W = O.quantize(O.Q4_0, synth.normal_f32(g, (M, K), 0.02))
    x = synth.normal_f32(g, (1, K), 1.0)
    say("Q4_0", M, K)
    check(Q.QMM_Q4_0, W, x, M, 1, K, what=f"Q4_0 {M}x{K}")


@pytest.mark.parametrize("M,K", [(4096, 4096), (14336, 4096), (4096, 14336)])
def test_config_q4_k_gemv_8b_shapes(M, K):
    g = synth.rng(0)
    W = synth.q4_k_random(g, M, K)
    for N in (1, 4, 8):
        x = synth.normal_f32(g, (N, K), 1.0)
        say("Q4_K", M, K, N)
        check(Q.QMM_Q4_K, W, x, M, N, K, what=f"Q4_K {M}x{K} N={N}")


@pytest.mark.parametrize("M", [4096, 14336])
def test_config_q4_k_prefill_512(M):
    g = synth.rng(0)
    W = synth.q4_k_random(g, M, 4096)
    x = synth.normal_f32(g, (512, 4096), 1.0)
    say("Q4_K prefill", M)
    check(Q.QMM_Q4_K, W, x, M, 512, 4096, rows=tile_rows(M), what=f"Q4_K {M}x4096 N=512")


@pytest.mark.parametrize("N", [1, 32])
def test_config_q6_k_head(N):
    g = synth.rng(0)
    M, K = 128256, 4096
    W = synth.q6_k_random(g, M, K)
    x = synth.normal_f32(g, (N, K), 1.0)
    say("Q6_K head N", N)
    check(Q.QMM_Q6_K, W, x, M, N, K, rows=None if N == 1 else tile_rows(M),
          what=f"Q6_K head N={N}")


# ---------------------------------------------- shapes, tails, edge cases

@pytest.mark.parametrize("wt", WTYPES)
def test_small_and_ragged_shapes(wt):
    g = np.random.default_rng(50 + wt)
    shapes = [(1, 1, 256), (7, 3, 256), (33, 8, 512), (100, 2, 1024), (257, 5, 768),
              (65, 1, 16384), (9, 2, 16640), (3, 1, 33024), (130, 4, 2304),
              (65, 3, 6144), (300, 1, 4096), (4, 8, 14336)]
    if wt in (Q.QMM_Q4_0, Q.QMM_Q8_0):
        shapes += [(5, 2, 32), (17, 1, 96), (64, 3, 288), (3, 8, 2080)]
    for M, N, K in shapes:
        W = make_weights(g, wt, M, K)
        x = g.standard_normal((N, K), dtype=np.float32)
        say("shape", wt, M, N, K)
        check(wt, W, x, M, N, K, what=f"type {wt} {M}x{K} N={N}")


@pytest.mark.parametrize("wt", [Q.QMM_Q4_0, Q.QMM_Q5_0, Q.QMM_Q8_0])
def test_auto_choice_wide_matrix_mid_batch(wt):
    # M > 8192 moves the GEMV/GEMM switch of these types down to N > 12 (Q8_0: 10)
    g = np.random.default_rng(90 + wt)
    M, N, K = 8200, 25, 512
    W = make_weights(g, wt, M, K)
    x = g.standard_normal((N, K), dtype=np.float32)
    check(wt, W, x, M, N, K, algo=0, what=f"auto {M}x{K} N={N}")


@pytest.mark.parametrize("wt", WTYPES)
def test_batch_above_8_column_groups(wt):
    g = np.random.default_rng(70 + wt)
    M, K = 200, 1024
    W = make_weights(g, wt, M, K)
    for N in (9, 17):
        x = g.standard_normal((N, K), dtype=np.float32)
        check(wt, W, x, M, N, K, algo=1, what=f"gemv N={N}")
        check(wt, W, x, M, N, K, algo=0, what=f"auto N={N}")


@pytest.mark.parametrize("wt", WTYPES)
def test_zero_activations_and_scales(wt):
    g = np.random.default_rng(80 + wt)
    M, N, K = 64, 2, 512
    W = make_weights(g, wt, M, K)
    x = np.zeros((N, K), np.float32)
    y = check(wt, W, x, M, N, K, what="zero x")
    assert np.all(y == 0)


@pytest.mark.parametrize("wt", WTYPES)
def test_deterministic_and_in_bounds(wt):
    g = np.random.default_rng(90 + wt)
    M, N, K = 1000, 3, 4096
    W = to_gpu(make_weights(g, wt, M, K))
    xq = to_gpu(O.quantize(O.VEC_DOT_TYPE[wt], g.standard_normal((N, K), dtype=np.float32)))
    outs = []
    for _ in range(3):
        buf = torch.full((N * M + 256,), float("nan"), dtype=torch.float32, device=W.device)
        assert Q.qmm_mul_mat(wt, W, xq, buf, M, N, K) == Q.QMM_OK
        b = to_cpu(buf)
        assert np.all(np.isnan(b[N * M:])), "wrote past the end of y"
        assert not np.any(np.isnan(b[:N * M]))
        outs.append(b[:N * M].view(np.uint32).copy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_error_leaves_output_untouched():
    W = torch.zeros(18 * 4, dtype=torch.uint8, device="cuda")
    xq = torch.zeros(34, dtype=torch.uint8, device="cuda")
    y = torch.full((4,), 7.0, device="cuda")
    assert Q.qmm_mul_mat(Q.QMM_Q4_0, W, xq, y, 4, 1, 48) == Q.QMM_ERR_SHAPE
    assert torch.all(y == 7.0).item()


@pytest.mark.parametrize("wt", [Q.QMM_Q4_0, Q.QMM_Q5_0, Q.QMM_Q8_0, Q.QMM_Q4_K, Q.QMM_Q6_K])
@pytest.mark.parametrize("M", [1000, 4096, 8200])
def test_automatic_choice_at_its_switch(wt, M):
    # qmm_mul_mat on both sides of the GEMV / GEMM switch it reports; all
    # outputs written, sampled rows (one per 32-row tile) compared
    g = np.random.default_rng(100 + wt + M)
    K = 512
    W = make_weights(g, wt, M, K)
    ch = [Q.qmm_mul_mat_choice(wt, M, n, K) for n in range(1, 65)]
    assert ch[0] == 1 and set(ch) == {1, 2}
    t = ch.index(2)  # the first N (minus one) that takes the GEMM
    assert all(c == 1 for c in ch[:t]) and all(c == 2 for c in ch[t:])
    for N in (t, t + 1):
        x = g.standard_normal((N, K), dtype=np.float32)
        say("auto switch", wt, M, N, "gemv" if ch[N - 1] == 1 else "gemm")
        check(wt, W, x, M, N, K, rows=tile_rows(M), algo=0, what=f"type {wt} M={M} N={N}")


@pytest.mark.parametrize("wt", [Q.QMM_Q4_0, Q.QMM_Q5_0, Q.QMM_Q8_0, Q.QMM_Q4_K, Q.QMM_Q6_K])
def test_seeded_random_shapes_every_kernel_family(wt):
    # 12 seeded random shapes per type (ragged M and N, K any multiple of the
    # block, up to 4096), each through the automatic choice and both kernel
    # families; sampled rows (one per 32-row tile) against the oracle
    g = np.random.default_rng(1000 + wt)
    B = 256 if wt in (Q.QMM_Q4_K, Q.QMM_Q6_K) else 32
    for case in range(12):
        M = int(g.integers(1, 3000))
        N = int(g.integers(1, 80))
        K = B * int(g.integers(1, 4096 // B + 1))
        W = make_weights(g, wt, M, K)
        x = g.standard_normal((N, K), dtype=np.float32) * np.float32(10.0 ** g.uniform(-3, 3))
        for algo in (0, 1, 2):
            say("random shape", wt, case, M, N, K, "algo", algo)
            check(wt, W, x, M, N, K, rows=tile_rows(M, seed=case), algo=algo,
                  what=f"type {wt} case {case} {M}x{K} N={N} algo {algo}")
