"""Q8_0 KV-cache quantization on the GPU: K and V rows of the 8B GQA model
(8 KV heads x 128 = 1024 values per token and layer) quantized to Q8_0 as
llama.cpp's --cache-type-k/v q8_0 stores them (page "llama.cpp and GGUF",
context and cache options; KV memory per token 2 x L x n_kv x d_h values).
Codes must equal the oracle's bit for bit, whether a prefill slab is
quantized at once or decode tokens are appended one row at a time into a
preallocated cache, and the cache must dequantize bit-exactly."""
import numpy as np
import pytest
import torch

import block_quantized_amd as Q
import oracle as O
import synth
from gpu_util import assert_bytes_equal, assert_f32_bits_equal, to_cpu, to_gpu

pytestmark = pytest.mark.gpu

ROW = synth.LLAMA_8B_KV_ROW
ROWB = (ROW // 32) * 34


def test_kv_prefill_slab_bit_exact():
    g = synth.rng(0)
    x = synth.normal_f32(g, (512, ROW), 1.0)   # one layer's K for a 512-token prompt
    got = to_cpu(Q.quantize_act(Q.QMM_Q8_0, to_gpu(x)))
    assert_bytes_equal(got, O.quantize(O.Q8_0, x), "K slab 512 x 1024")


def test_kv_decode_append_into_cache():
    # a cache of T_max token rows; a prompt of 37 tokens, then 11 decode steps
    # each appending one row at its offset; rows never written stay untouched
    g = synth.rng(1)
    T_max, prompt, steps = 64, 37, 11
    toks = synth.normal_f32(g, (prompt + steps, ROW), 1.0)
    cache = torch.full((T_max, ROWB), 0xA5, dtype=torch.uint8, device=Q_dev())
    xg = to_gpu(toks)
    rc = Q.qmm_quantize_act(Q.QMM_Q8_0, xg, cache, prompt, ROW)
    assert rc == Q.QMM_OK
    for t in range(prompt, prompt + steps):
        rc = Q.qmm_quantize_act(Q.QMM_Q8_0, xg.data_ptr() + 4 * ROW * t, cache.data_ptr() + ROWB * t, 1, ROW)
        assert rc == Q.QMM_OK
    c = to_cpu(cache)
    assert_bytes_equal(c[:prompt + steps], O.quantize(O.Q8_0, toks), "appended cache")
    assert np.all(c[prompt + steps:] == 0xA5), "rows past the last token were written"
    # reading the cache back (what attention would consume) is exact too
    deq = to_cpu(Q.dequantize(Q.QMM_Q8_0, cache[:prompt + steps], prompt + steps, ROW))
    assert_f32_bits_equal(deq, O.dequantize(O.Q8_0, c[:prompt + steps], prompt + steps, ROW), "cache read back")


def test_kv_round_trip_bound():
    # per element |x - fp16(d) q| <= d/2 + |q| |d - fp16(d)| (the Q8_0 pin)
    g = synth.rng(2)
    x = synth.normal_f32(g, (96, ROW), 1.0) * np.float32(3.0)
    blocks = to_cpu(Q.quantize_act(Q.QMM_Q8_0, to_gpu(x)))
    deq = to_cpu(Q.dequantize(Q.QMM_Q8_0, to_gpu(blocks), 96, ROW)).astype(np.float64)
    xb = x.reshape(96, -1, 32).astype(np.float64)
    d = np.abs(xb).max(axis=2, keepdims=True) / 127.0
    d16 = blocks.reshape(96, -1, 34)[:, :, :2].copy().view(np.float16).astype(np.float64)
    q = blocks.reshape(96, -1, 34)[:, :, 2:].view(np.int8).astype(np.float64)
    bound = d / 2 + np.abs(q) * np.abs(d - d16) + 1e-12
    assert np.all(np.abs(xb - deq.reshape(xb.shape)) <= bound)


def Q_dev():
    return torch.device("cuda:0")
