"""CPU oracle for the GGUF block-quantized matrix product.

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; nothing on the
product path does.  It shares no code with the GPU library: the arithmetic
lives in ``qmm_oracle.c`` (plain C, fp64 accumulation, built with
``-ffp-contract=off``), and this module only marshals numpy arrays.

Sources: the page "The GGML ecosystem, and where synapse fits", §5
"Quantization" (format table; "Products: weights against quantized
activations"), and the page "ggml", examples/simple, for the orientation
``y[n][m] = sum_k W[m][k] * x[n][k]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmm_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

# Oracle type codes (its own).
Q4_0, Q8_0, Q4_K, Q6_K, Q8_K, Q5_0 = 1, 2, 3, 4, 5, 6
TYPE_NAMES = {Q4_0: "Q4_0", Q8_0: "Q8_0", Q4_K: "Q4_K", Q6_K: "Q6_K", Q8_K: "Q8_K", Q5_0: "Q5_0"}
BLOCK_SIZE = {Q4_0: 32, Q8_0: 32, Q4_K: 256, Q6_K: 256, Q8_K: 256, Q5_0: 32}
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34, Q4_K: 144, Q6_K: 210, Q8_K: 292, Q5_0: 22}
VEC_DOT_TYPE = {Q4_0: Q8_0, Q8_0: Q8_0, Q4_K: Q8_K, Q6_K: Q8_K, Q5_0: Q8_0}

CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
          "-Wall", "-Wextra", "-shared", "-fPIC"]


def build() -> str:
    """Compile liboracle.so from qmm_oracle.c (always recompiles)."""
    tmp = LIB_PATH + ".tmp"
    subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_block_size.argtypes = [I]
        L.orc_block_size.restype = I
        L.orc_block_bytes.argtypes = [I]
        L.orc_block_bytes.restype = ctypes.c_size_t
        L.orc_fp16_to_f32_n.argtypes = [P, P, I64]
        L.orc_f32_to_fp16_n.argtypes = [P, P, I64]
        for f in (L.orc_quantize_q8_0, L.orc_quantize_q8_k, L.orc_quantize_q4_0):
            f.argtypes = [P, P, I64, I64]
            f.restype = I
        for f in (L.orc_dequantize_f32, L.orc_dequantize_f64):
            f.argtypes = [I, P, P, I64, I64]
            f.restype = I
        L.orc_mul_mat.argtypes = [I, P, P, P, P, I64, I64, I64]
        L.orc_mul_mat.restype = I
        L.orc_mul_mat_blockwise.argtypes = [I, P, P, P, I64, I64, I64]
        L.orc_mul_mat_blockwise.restype = I
        L.orc_q4k_scale_min.argtypes = [P, I, ctypes.POINTER(I), ctypes.POINTER(I)]
        L.orc_q6k_quant.argtypes = [P, I]
        L.orc_q6k_quant.restype = I
        L.orc_q4k_scale_min_n.argtypes = [P, I64, P, P]
        L.orc_q6k_quant_n.argtypes = [P, I64, P]
        L.orc_q5_0_quant_n.argtypes = [P, I64, P]
        L.orc_num_threads.restype = I
        L.orc_set_num_threads.argtypes = [I]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def row_bytes(t: int, K: int) -> int:
    assert K % BLOCK_SIZE[t] == 0
    return K // BLOCK_SIZE[t] * BLOCK_BYTES[t]


def fp16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_fp16_to_f32_n(_ptr(h), _ptr(out), h.size)
    return out


def f32_to_fp16(f) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().orc_f32_to_fp16_n(_ptr(f), _ptr(out), f.size)
    return out


def quantize(t: int, x: np.ndarray) -> np.ndarray:
    """Quantize a (rows, K) fp32 array to `t` blocks -> (rows, row_bytes) uint8.
    t is Q8_0 or Q8_K (activation quantizers) or Q4_0 (weight encoder)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    rows, K = x.shape
    out = np.zeros((rows, row_bytes(t, K)), np.uint8)
    fn = {Q8_0: lib().orc_quantize_q8_0, Q8_K: lib().orc_quantize_q8_k,
          Q4_0: lib().orc_quantize_q4_0}[t]
    rc = fn(_ptr(x), _ptr(out), rows, K)
    assert rc == 0, rc
    return out


def dequantize(t: int, blocks: np.ndarray, rows: int, K: int, f64: bool = False) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    assert blocks.size == rows * row_bytes(t, K)
    out = np.empty((rows, K), np.float64 if f64 else np.float32)
    fn = lib().orc_dequantize_f64 if f64 else lib().orc_dequantize_f32
    rc = fn(t, _ptr(blocks), _ptr(out), rows, K)
    assert rc == 0, rc
    return out


def mul_mat(wtype: int, W: np.ndarray, xq: np.ndarray, M: int, N: int, K: int,
            with_T: bool = True):
    """y[n][m] = sum_k w[m][k] x[n][k] in fp64 (plain definition), and the
    per-output magnitude sum T.  Returns (y, T) as (N, M) float64 arrays."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    assert W.size == M * row_bytes(wtype, K)
    assert xq.size == N * row_bytes(VEC_DOT_TYPE[wtype], K)
    y = np.empty((N, M), np.float64)
    T = np.empty((N, M), np.float64) if with_T else None
    rc = lib().orc_mul_mat(wtype, _ptr(W), _ptr(xq), _ptr(y),
                           _ptr(T) if with_T else None, M, N, K)
    assert rc == 0, rc
    return y, T


def mul_mat_blockwise(wtype: int, W: np.ndarray, xq: np.ndarray, M: int, N: int, K: int):
    W = np.ascontiguousarray(W, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    y = np.empty((N, M), np.float64)
    rc = lib().orc_mul_mat_blockwise(wtype, _ptr(W), _ptr(xq), _ptr(y), M, N, K)
    assert rc == 0, rc
    return y


def q4k_scale_min(scales12, j: int):
    s = np.ascontiguousarray(scales12, dtype=np.uint8)
    assert s.size == 12
    sc, m = ctypes.c_int(), ctypes.c_int()
    lib().orc_q4k_scale_min(_ptr(s), j, ctypes.byref(sc), ctypes.byref(m))
    return sc.value, m.value


def q6k_quant(block210, e: int) -> int:
    b = np.ascontiguousarray(block210, dtype=np.uint8)
    assert b.size == 210
    return lib().orc_q6k_quant(_ptr(b), e)


def q4k_scale_min_n(scales: np.ndarray):
    """(n, 12) uint8 -> (sc, m), each (n, 8) int32."""
    s = np.ascontiguousarray(scales, dtype=np.uint8).reshape(-1, 12)
    sc = np.empty((s.shape[0], 8), np.int32)
    m = np.empty((s.shape[0], 8), np.int32)
    lib().orc_q4k_scale_min_n(_ptr(s), s.shape[0], _ptr(sc), _ptr(m))
    return sc, m


def q6k_quant_n(blocks: np.ndarray) -> np.ndarray:
    """(n, 210) uint8 -> (n, 256) unsigned 6-bit quants."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1, 210)
    q = np.empty((b.shape[0], 256), np.uint8)
    lib().orc_q6k_quant_n(_ptr(b), b.shape[0], _ptr(q))
    return q


def q5_0_quant_n(blocks: np.ndarray) -> np.ndarray:
    """Unsigned 5-bit quants of n Q5_0 blocks -> (n, 32) uint8."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1, 22)
    q = np.empty((b.shape[0], 32), np.uint8)
    lib().orc_q5_0_quant_n(_ptr(b), b.shape[0], _ptr(q))
    return q


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads for the oracle's parallel loops (timing only; results do not depend on it)."""
    lib().orc_set_num_threads(n)
