"""Seeded synthetic inputs for the block-quantized matrix product.

This module only draws random numbers and places random fields at their byte
offsets inside blocks.  It holds none of the product's arithmetic (no
quantizer, no decoder, no dot product), so both the oracle side and the GPU
side may take their inputs from it.

Distributions follow the workloads the pages' decode discussion is built on
(Llama-family shapes; page "llama.cpp and GGUF", "Worked example" of the
decode ceiling for an 8B Q4_K_M model, and the 1B-class widths 2048/512/8192):

- fp32 weights ~ N(0, 0.02) and fp32 activations ~ N(0, 1);
- random raw Q4_K super-blocks: every byte uniform, then d and dmin
  overwritten by fp16(|N(0, 1e-3)|);
- random raw Q6_K super-blocks: every byte uniform, then the 16 int8
  sub-block scales overwritten by U[-32, 31] and d by fp16(|N(0, 1e-3)|).

All draws use ``numpy.random.default_rng(seed)`` (PCG64); weights are drawn
before activations.  Byte offsets of the overwritten fields: Q4_K d at 0, dmin
at 2; Q6_K scales at 192..207 and d at 208 (GGUF field order).
"""
from __future__ import annotations

import numpy as np

Q4_K_BYTES = 144
Q6_K_BYTES = 210


def rng(seed: int = 0) -> np.random.Generator:
    return np.random.default_rng(seed)


def normal_f32(g: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    """float32 draws ~ N(0, sigma^2)."""
    return g.standard_normal(shape, dtype=np.float32) * np.float32(sigma)


def _abs_normal_fp16_bytes(g: np.random.Generator, shape, sigma: float) -> np.ndarray:
    v = np.abs(normal_f32(g, shape, sigma)).astype(np.float16)
    return v.view(np.uint8).reshape(*shape, 2)


def q4_k_random(g: np.random.Generator, rows: int, K: int) -> np.ndarray:
    """(rows, K/256*144) uint8 of random raw Q4_K super-blocks."""
    assert K % 256 == 0
    nb = K // 256
    blk = g.integers(0, 256, size=(rows, nb, Q4_K_BYTES), dtype=np.uint8)
    blk[:, :, 0:2] = _abs_normal_fp16_bytes(g, (rows, nb), 1e-3)
    blk[:, :, 2:4] = _abs_normal_fp16_bytes(g, (rows, nb), 1e-3)
    return blk.reshape(rows, nb * Q4_K_BYTES)


def q6_k_random(g: np.random.Generator, rows: int, K: int) -> np.ndarray:
    """(rows, K/256*210) uint8 of random raw Q6_K super-blocks."""
    assert K % 256 == 0
    nb = K // 256
    blk = g.integers(0, 256, size=(rows, nb, Q6_K_BYTES), dtype=np.uint8)
    sc = g.integers(-32, 32, size=(rows, nb, 16), dtype=np.int8)
    blk[:, :, 192:208] = sc.view(np.uint8)
    blk[:, :, 208:210] = _abs_normal_fp16_bytes(g, (rows, nb), 1e-3)
    return blk.reshape(rows, nb * Q6_K_BYTES)


def q5_0_random(g: np.random.Generator, rows: int, K: int) -> np.ndarray:
    """(rows, K/32*22) uint8 of random raw Q5_0 blocks: uniform fifth-bit
    words and nibbles, d = fp16(|N(0, 1e-3)|) as for the K-quant workloads."""
    assert K % 32 == 0
    nb = K // 32
    blk = g.integers(0, 256, size=(rows, nb, 22), dtype=np.uint8)
    blk[:, :, 0:2] = _abs_normal_fp16_bytes(g, (rows, nb), 1e-3)
    return blk.reshape(rows, nb * 22)


# Qwen2.5-0.5B-shaped layer: 896-wide rows are not a multiple of 256, so a
# K-quant mix stores them as Q5_0 (page "The GGML ecosystem, and where synapse
# fits", §3, the fallback rule); ffn_down's 4864-wide rows are.
QWEN_0_5B_Q5_0 = (("attn_q", 896, 896), ("attn_k", 128, 896), ("attn_v", 128, 896),
                  ("attn_output", 896, 896), ("ffn_gate", 4864, 896), ("ffn_up", 4864, 896))


def uniform_bytes(g: np.random.Generator, shape) -> np.ndarray:
    return g.integers(0, 256, size=shape, dtype=np.uint8)


# Workload shapes (rows M x inputs K, batch N).  The 1B-class layer: q and o
# are 2048x2048, k and v 512x2048, gate and up 8192x2048, down 2048x8192.
# The 8B-class layer: 4096x4096, 14336x4096 (gate/up), 4096x14336 (down);
# the 128256-row output head at K = 4096.
LLAMA_1B_LAYER = (
    ("attn_q", 2048, 2048), ("attn_k", 512, 2048), ("attn_v", 512, 2048),
    ("attn_output", 2048, 2048), ("ffn_gate", 8192, 2048), ("ffn_up", 8192, 2048),
    ("ffn_down", 2048, 8192),
)
LLAMA_1B_LAYERS = 16
LLAMA_8B_SHAPES = ((4096, 4096), (14336, 4096), (4096, 14336))
LLAMA_8B_HEAD = (128256, 4096)

# KV cache of the 8B GQA model ("llama.cpp and GGUF", KV memory: 2 x L x n_kv x
# d_h values per token): 32 layers, 8 KV heads of 128 -> one K row and one V
# row of 1024 values per token and layer.
LLAMA_8B_KV = {"layers": 32, "kv_heads": 8, "head_dim": 128}
LLAMA_8B_KV_ROW = LLAMA_8B_KV["kv_heads"] * LLAMA_8B_KV["head_dim"]
