"""GPU parity of qmm_mul_mat_multi: several matrices sharing the activation
rows in one launch, with either quantized activations or fp32 activations
that the launch quantizes itself.

The fused quantization must reproduce qmm_quantize_act exactly (the page 'The
GGML ecosystem, and where synapse fits', section 5: activations are quantized
once per row to the weight's vec_dot_type), so each output must equal, bit for
bit, the single-matrix product of the separately quantized rows; and every
output must meet the oracle's 1e-5 * T bound."""
import sys

import numpy as np
import pytest
import torch

import block_quantized_amd as Q
import oracle as O
import synth
from gpu_util import assert_within_tolerance, to_cpu, to_gpu

pytestmark = pytest.mark.gpu


def make_weights(g, wt, M, K):
    if wt == Q.QMM_Q4_K:
        return synth.q4_k_random(g, M, K)
    if wt == Q.QMM_Q6_K:
        return synth.q6_k_random(g, M, K)
    return O.quantize(O.Q8_0 if wt == Q.QMM_Q8_0 else O.Q4_0, synth.normal_f32(g, (M, K), 0.02))


# the first four are the launches of the 1B-Llama decode sweep (q|k|v, ffn_down, o, gate|up)
CASES = [(Q.QMM_Q4_0, 2048, (2048, 512, 512)), (Q.QMM_Q4_0, 8192, (2048,)), (Q.QMM_Q4_0, 2048, (2048,)),
         (Q.QMM_Q4_0, 2048, (8192, 8192)), (Q.QMM_Q8_0, 2048, (300, 2048)),
         (Q.QMM_Q4_K, 4096, (4096, 1024, 1024)), (Q.QMM_Q4_K, 14336, (4096,)), (Q.QMM_Q6_K, 4096, (1000, 77)),
         (Q.QMM_Q6_K, 768, (33, 64)), (Q.QMM_Q6_K, 18176, (70,)), (Q.QMM_Q4_0, 256, (5, 3, 1, 9))]


@pytest.mark.parametrize("wt,K,Ms", CASES)
@pytest.mark.parametrize("N", [1, 3, 8])
def test_multi_fused_matches_separate_and_oracle(wt, K, Ms, N):
    g = np.random.default_rng(1000 + wt * 7 + K + N)
    Ws = [make_weights(g, wt, M, K) for M in Ms]
    x = g.standard_normal((N, K), dtype=np.float32)
    x[0, :64] *= 1e-3
    xt = O.VEC_DOT_TYPE[wt]
    xg = to_gpu(x)
    Wg = [to_gpu(W) for W in Ws]
    xq_gpu = Q.quantize_act(xt, xg)
    print("multi", wt, K, Ms, N, flush=True)
    fused = [to_cpu(y) for y in Q.mul_mat_multi(wt, Wg, Ms, xg, N, K, x_is_f32=True)]
    multi_q = [to_cpu(y) for y in Q.mul_mat_multi(wt, Wg, Ms, xq_gpu, N, K, x_is_f32=False)]
    xq = O.quantize(xt, x)
    for i, (W, M) in enumerate(zip(Ws, Ms)):
        # the multi launch runs the GEMV kernels: compare with the same kernels
        # run one matrix at a time (algo 1), bit for bit
        single = to_cpu(Q.mul_mat(wt, Wg[i], xq_gpu, M, N, K, algo=1))
        assert np.array_equal(fused[i].view(np.uint32), single.view(np.uint32)), f"fused != single (matrix {i})"
        assert np.array_equal(multi_q[i].view(np.uint32), single.view(np.uint32)), f"multi != single (matrix {i})"
        y_ref, T = O.mul_mat(wt, W, xq, M, N, K)
        assert_within_tolerance(fused[i], y_ref, T, what=f"matrix {i}")


def test_multi_errors():
    W = torch.zeros(18 * 64, dtype=torch.uint8, device="cuda")
    x = torch.zeros((9, 2048), dtype=torch.float32, device="cuda")
    y = torch.zeros(64 * 9, dtype=torch.float32, device="cuda")
    mm = Q.qmm_mul_mat_multi
    assert mm(Q.QMM_Q4_0, 1, [W], [y], [1], x, True, 9, 2048) == Q.QMM_ERR_UNSUPPORTED  # fp32 needs N <= 8
    assert mm(Q.QMM_Q4_0, 1, [W], [y], [1], x, True, 1, 96) == Q.QMM_ERR_UNSUPPORTED   # K % 256 != 0
    assert torch.all(y == 0).item()
    # any whole number of Q6_K super-blocks is supported (zero weights: zero output)
    assert mm(Q.QMM_Q6_K, 1, [W], [y], [1], x, True, 1, 256) == Q.QMM_OK
    torch.cuda.synchronize()
    assert torch.all(y == 0).item()
