"""GPU parity of the codecs through the C ABI: activation quantization (Q8_0,
Q8_K), the Q4_0 weight encoder and the dequantizers must equal the CPU oracle
bit for bit, on the workloads' tensors and on edge cases, and be identical
run to run.  Formats: the format table of page 'The GGML ecosystem, and where
synapse fits', section 5."""
import sys

import numpy as np
import pytest

import block_quantized_amd as Q
import oracle as O
import synth
from gpu_util import assert_bytes_equal, assert_f32_bits_equal, to_cpu, to_gpu

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_quantize(t, x, act=True):
    xt = to_gpu(x)
    out = (Q.quantize_act if act else Q.quantize)(t, xt)
    return to_cpu(out)


def edge_rows(K):
    g = np.random.default_rng(5)
    rows = [np.zeros(K, np.float32),
            g.standard_normal(K, dtype=np.float32) * np.float32(1e-30),
            g.standard_normal(K, dtype=np.float32) * np.float32(3e4),
            np.full(K, 1.5, np.float32), np.full(K, -2.5, np.float32)]
    tie = np.zeros(K, np.float32)
    tie[:8] = [127, -127, 62.5, 0.5, -0.5, -62.5, 1.5, 2.5]
    rows.append(tie)
    tiny = np.zeros(K, np.float32)
    tiny[0], tiny[1] = 2e-37, -1e-38    # 1/d overflows: codes saturate, zeros stay 0
    rows.append(tiny)
    tiny2 = np.zeros(K, np.float32)
    tiny2[0] = 1e-44                     # d rounds to 0
    rows.append(tiny2)
    rows.append(((np.arange(K) % 256 - 128) / 64).astype(np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("t", [Q.QMM_Q8_0, Q.QMM_Q8_K])
def test_quantize_act_workload_tensors(t):
    g = synth.rng(0)
    cases = []
    if t == Q.QMM_Q8_0:
        cases.append(("W 2048x2048 N(0,0.02)", synth.normal_f32(g, (2048, 2048), 0.02)))
        cases.append(("x 1x2048", synth.normal_f32(g, (1, 2048), 1.0)))
        cases.append(("x 1x8192", synth.normal_f32(g, (1, 8192), 1.0)))
    else:
        for N in (1, 4, 8):
            for K in (4096, 14336):
                cases.append((f"x {N}x{K}", synth.normal_f32(g, (N, K), 1.0)))
        cases.append(("x 512x4096", synth.normal_f32(g, (512, 4096), 1.0)))
        cases.append(("x 32x4096", synth.normal_f32(g, (32, 4096), 1.0)))
    for name, x in cases:
        say("quantize", t, name)
        assert_bytes_equal(gpu_quantize(t, x), O.quantize(t, x), name)


@pytest.mark.parametrize("t", [Q.QMM_Q8_0, Q.QMM_Q8_K])
def test_quantize_act_edges_and_ragged(t):
    B = 32 if t == Q.QMM_Q8_0 else 256
    x = edge_rows(4 * B)
    assert_bytes_equal(gpu_quantize(t, x), O.quantize(t, x), "edges")
    g = np.random.default_rng(9)
    for rows, nb in ((1, 1), (3, 5), (7, 33), (1, 129), (65, 3)):
        xx = g.standard_normal((rows, nb * B), dtype=np.float32) * np.float32(g.uniform(1e-3, 10))
        assert_bytes_equal(gpu_quantize(t, xx), O.quantize(t, xx), f"{rows}x{nb * B}")


def test_quantize_q4_0_weights():
    g = synth.rng(0)
    for rows, K in ((2048, 2048), (512, 2048), (2048, 8192), (5, 96)):
        say("q4_0", rows, K)
        W = synth.normal_f32(g, (rows, K), 0.02)
        assert_bytes_equal(gpu_quantize(Q.QMM_Q4_0, W, act=False), O.quantize(O.Q4_0, W), f"{rows}x{K}")
    e = edge_rows(128)
    e[1, 0], e[1, 1] = -3.0, 3.0   # equal magnitudes: the first wins
    e[2, 5] = -0.0
    assert_bytes_equal(gpu_quantize(Q.QMM_Q4_0, e, act=False), O.quantize(O.Q4_0, e), "edges")
    z = np.zeros((1, 32), np.float32)
    z[0, 0] = -0.0
    assert_bytes_equal(gpu_quantize(Q.QMM_Q4_0, z, act=False), O.quantize(O.Q4_0, z), "signed zero")


def test_quantize_q4_0_nan_is_never_the_maximum():
    # NaN at the first element of a lane's four (elements 0, 4k) and elsewhere;
    # the magnitude search skips NaN, as the oracle's strict '>' does
    g = np.random.default_rng(13)
    x = g.standard_normal((6, 64), dtype=np.float32)
    x[0, 0] = np.nan
    x[1, 4] = np.nan
    x[2, 28] = np.nan
    x[3, 0:32] = np.nan              # a block of NaN only: m = 0, every code 8
    x[4, 32] = np.nan
    x[4, 33] = -np.inf
    x[5, 16] = np.nan
    x[5, 0] = 1e-40
    assert_bytes_equal(gpu_quantize(Q.QMM_Q4_0, x, act=False), O.quantize(O.Q4_0, x), "NaN inputs")


def test_quantize_q4_0_hand_block(golden):
    h = golden("hand_blocks.json")["q4_0_encoder_ties"]
    b = gpu_quantize(Q.QMM_Q4_0, np.array(h["x"], np.float32)[None, :], act=False).reshape(-1)
    assert int(b[0]) | (int(b[1]) << 8) == h["d_fp16_bits"]
    assert b[2:18].tolist() == h["qs_bytes"]


def random_blocks(t, rows, K, g):
    """Random block bytes with finite scales (NaN/Inf scales are no parity case)."""
    nb = K // O.BLOCK_SIZE[t]
    S = O.BLOCK_BYTES[t]
    b = g.integers(0, 256, (rows, nb, S), dtype=np.uint8)
    if t in (O.Q4_0, O.Q8_0):
        b[:, :, 1] &= 0x7B
    elif t == O.Q4_K:
        b[:, :, 1] &= 0x7B
        b[:, :, 3] &= 0x7B
    elif t == O.Q6_K:
        b[:, :, 209] &= 0x7B
    else:
        b[:, :, 0:4] = (g.standard_normal((rows, nb), dtype=np.float32) * np.float32(1e-2)) \
            .view(np.uint8).reshape(rows, nb, 4)
    return b.reshape(rows, nb * S)


@pytest.mark.parametrize("t", [Q.QMM_Q4_0, Q.QMM_Q8_0, Q.QMM_Q4_K, Q.QMM_Q6_K, Q.QMM_Q8_K])
def test_dequantize_bit_exact(t):
    g = np.random.default_rng(100 + t)
    B = O.BLOCK_SIZE[t]
    for rows, nb in ((1, 1), (3, 7), (64, 16), (257, 2)):
        K = nb * B
        blocks = random_blocks(t, rows, K, g)
        say("dequant", t, rows, K)
        got = to_cpu(Q.dequantize(t, to_gpu(blocks), rows, K))
        assert_f32_bits_equal(got, O.dequantize(t, blocks, rows, K), f"type {t} {rows}x{K}")


def test_dequantize_workload_weights():
    g = synth.rng(0)
    W = synth.q4_k_random(g, 4096, 4096)
    say("dequant q4_k 4096x4096")
    assert_f32_bits_equal(to_cpu(Q.dequantize(Q.QMM_Q4_K, to_gpu(W), 4096, 4096)),
                          O.dequantize(O.Q4_K, W, 4096, 4096), "Q4_K 4096x4096")
    W = synth.q6_k_random(g, 2048, 4096)
    say("dequant q6_k 2048x4096")
    assert_f32_bits_equal(to_cpu(Q.dequantize(Q.QMM_Q6_K, to_gpu(W), 2048, 4096)),
                          O.dequantize(O.Q6_K, W, 2048, 4096), "Q6_K 2048x4096")


def test_codecs_deterministic():
    g = synth.rng(3)
    x = to_gpu(synth.normal_f32(g, (64, 4096), 1.0))
    a = [to_cpu(Q.quantize_act(Q.QMM_Q8_K, x)) for _ in range(3)]
    assert all(np.array_equal(a[0], b) for b in a[1:])
    W = to_gpu(synth.q6_k_random(g, 128, 4096))
    d = [to_cpu(Q.dequantize(Q.QMM_Q6_K, W, 128, 4096)) for _ in range(3)]
    assert all(np.array_equal(d[0].view(np.uint32), b.view(np.uint32)) for b in d[1:])


@pytest.mark.parametrize("t", [Q.QMM_Q4_K, Q.QMM_Q6_K])
def test_dequantize_bench_size(t):
    # the 14336 x 4096 dequantization the benchmark times, every value bit-exact
    g = synth.rng(0)
    W = (synth.q4_k_random if t == Q.QMM_Q4_K else synth.q6_k_random)(g, 14336, 4096)
    say("dequant bench size", t)
    ot = O.Q4_K if t == Q.QMM_Q4_K else O.Q6_K
    assert_f32_bits_equal(to_cpu(Q.dequantize(t, to_gpu(W), 14336, 4096)), O.dequantize(ot, W, 14336, 4096),
                          f"type {t} 14336x4096")
