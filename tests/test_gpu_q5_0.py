"""GPU parity for Q5_0 weights (format table of page 'The GGML ecosystem, and
where synapse fits', §5: fp16 d, a 32-bit word of fifth bits, 32 four-bit
low parts, w = d(q - 16)).  Q5_0 is what a K-quant mix gives rows whose
length is not a multiple of 256 (§3, fallback rule), so the Qwen2.5-0.5B
896-wide rows are the workload.  Dequantization is bit-exact; products are
within 1e-5 * sum|terms| on both GEMV paths (256-value lane units when K is a
multiple of 256, one wavefront per row otherwise), the fused-quantize form
equals the plain one bit for bit."""
import numpy as np
import pytest

import block_quantized_amd as Q
import oracle as O
import synth
from gpu_util import assert_f32_bits_equal, assert_within_tolerance, to_cpu, to_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,K", [(3, 32), (7, 896), (64, 4096), (33, 4864)])
def test_q5_0_dequantize_bit_exact(rows, K):
    g = np.random.default_rng(rows + K)
    W = synth.q5_0_random(g, rows, K)
    got = to_cpu(Q.dequantize(Q.QMM_Q5_0, to_gpu(W), rows, K))
    assert_f32_bits_equal(got, O.dequantize(O.Q5_0, W, rows, K), f"Q5_0 {rows}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (5, 3, 96), (896, 1, 896), (128, 4, 896), (4864, 1, 896),
                                   (300, 1, 1024), (65, 8, 2048), (200, 9, 512), (4, 2, 16384)])
def test_q5_0_mul_mat(M, N, K):
    g = np.random.default_rng(M * 3 + N * 7 + K)
    W = synth.q5_0_random(g, M, K)
    xq = O.quantize(O.Q8_0, g.standard_normal((N, K), dtype=np.float32))
    print("q5_0", M, N, K, flush=True)
    y = to_cpu(Q.mul_mat(Q.QMM_Q5_0, to_gpu(W), to_gpu(xq), M, N, K))
    y_ref, T = O.mul_mat(O.Q5_0, W, xq, M, N, K)
    assert_within_tolerance(y, y_ref, T, what=f"Q5_0 {M}x{K} N={N}")


def test_q5_0_qwen_layer_shapes():
    # every 896-wide matrix of a Qwen2.5-0.5B layer, batch 1
    g = synth.rng(0)
    x = synth.normal_f32(g, (1, 896), 1.0)
    xq = O.quantize(O.Q8_0, x)
    for name, M, K in synth.QWEN_0_5B_Q5_0:
        W = synth.q5_0_random(g, M, K)
        y = to_cpu(Q.mul_mat(Q.QMM_Q5_0, to_gpu(W), to_gpu(xq), M, 1, K))
        y_ref, T = O.mul_mat(O.Q5_0, W, xq, M, 1, K)
        assert_within_tolerance(y, y_ref, T, what=name)


def test_q5_0_fused_and_multi_equal_single():
    g = np.random.default_rng(77)
    K, N = 2048, 2
    Ms = (640, 256, 256)
    Ws = [synth.q5_0_random(g, M, K) for M in Ms]
    x = g.standard_normal((N, K), dtype=np.float32)
    xq = to_gpu(O.quantize(O.Q8_0, x))
    Wg = [to_gpu(w) for w in Ws]
    single = [to_cpu(Q.mul_mat(Q.QMM_Q5_0, w, xq, M, N, K)) for w, M in zip(Wg, Ms)]
    multi = [to_cpu(t) for t in Q.mul_mat_multi(Q.QMM_Q5_0, Wg, Ms, xq, N, K)]
    fused = [to_cpu(t) for t in Q.mul_mat_multi(Q.QMM_Q5_0, Wg, Ms, to_gpu(x), N, K, x_is_f32=True)]
    for a, b, c in zip(single, multi, fused):
        assert np.array_equal(a, b) and np.array_equal(a, c)
    for w, M, y in zip(Ws, Ms, single):
        y_ref, T = O.mul_mat(O.Q5_0, w, to_cpu(xq), M, N, K)
        assert_within_tolerance(y, y_ref, T, what="Q5_0 multi")
