"""Python binding of libqmm, the gfx950 GGUF block-quantized matrix product.

Argument marshalling only: every function named ``qmm_*`` forwards to the C
function of the same name in ``libqmm.so`` (declared in ``include/qmm.h`` and
``include/qmm_probe.h``).
Device buffers may be passed as torch tensors (their ``data_ptr()`` is used)
or as integer device addresses; ``stream`` defaults to torch's current
stream.  The ``qmm_*`` functions return the C status code.  The helpers
below them (``quantize_act``, ``dequantize``, ``mul_mat`` ...) allocate their
outputs with torch and raise :class:`QmmError` on a non-zero status.

There is no fallback: if ``libqmm.so`` is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqmm.so")

QMM_Q4_0, QMM_Q8_0, QMM_Q4_K, QMM_Q6_K, QMM_Q8_K, QMM_Q5_0 = 1, 2, 3, 4, 5, 6
QMM_OK, QMM_ERR_TYPE, QMM_ERR_SHAPE, QMM_ERR_NULL = 0, -1, -2, -3
QMM_ERR_ALIGN, QMM_ERR_UNSUPPORTED, QMM_ERR_HIP = -4, -5, -6

TYPES = {"Q4_0": QMM_Q4_0, "Q8_0": QMM_Q8_0, "Q4_K": QMM_Q4_K, "Q6_K": QMM_Q6_K, "Q8_K": QMM_Q8_K,
         "Q5_0": QMM_Q5_0}

_lib = None


class QmmError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {qmm_strerror(code)} ({code})")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libqmm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_quantized_amd.build` "
                               "(or __graft_entry__.build()); there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        I, I64, P, SZ = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        sig = {
            "qmm_block_size": (I, [I]),
            "qmm_block_bytes": (SZ, [I]),
            "qmm_row_bytes": (SZ, [I, I64]),
            "qmm_vec_dot_type": (I, [I]),
            "qmm_quantize_act": (I, [I, P, P, I64, I64, P]),
            "qmm_quantize": (I, [I, P, P, I64, I64, P]),
            "qmm_dequantize": (I, [I, P, P, I64, I64, P]),
            "qmm_mul_mat": (I, [I, P, P, P, I64, I64, I64, P]),
            "qmm_mul_mat_algo": (I, [I, P, P, P, I64, I64, I64, I, P]),
            "qmm_mul_mat_multi": (I, [I, I, P, P, P, P, I, I64, I64, P]),
            "qmm_mul_mat_choice": (I, [I, I64, I64, I64]),
            "qmm_strerror": (ctypes.c_char_p, [I]),
            "qmm_probe_read": (I, [P, I64, P, I, P]),
            "qmm_probe_mfma": (I, [I, I64, P, P]),
            "qmm_probe_mfma_ops": (I64, [I, I64]),
            "qmm_probe_mfma16": (I, [I, I64, P, P]),
            "qmm_probe_mfma16_ops": (I64, [I, I64]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


EXPORTED = ("qmm_block_size", "qmm_block_bytes", "qmm_row_bytes", "qmm_vec_dot_type", "qmm_quantize_act",
            "qmm_quantize", "qmm_dequantize", "qmm_mul_mat", "qmm_mul_mat_algo", "qmm_mul_mat_multi",
            "qmm_mul_mat_choice",
            "qmm_strerror", "qmm_probe_read", "qmm_probe_mfma", "qmm_probe_mfma_ops",
            "qmm_probe_mfma16", "qmm_probe_mfma16_ops")


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------ C-ABI names

def qmm_block_size(t: int) -> int:
    return lib().qmm_block_size(t)


def qmm_block_bytes(t: int) -> int:
    return lib().qmm_block_bytes(t)


def qmm_row_bytes(t: int, K: int) -> int:
    return lib().qmm_row_bytes(t, K)


def qmm_vec_dot_type(wtype: int) -> int:
    return lib().qmm_vec_dot_type(wtype)


def qmm_quantize_act(dst, x, xq, N, K, stream=None) -> int:
    return lib().qmm_quantize_act(dst, _ptr(x), _ptr(xq), N, K, _stream(stream))


def qmm_quantize(dst, x, out, rows, K, stream=None) -> int:
    return lib().qmm_quantize(dst, _ptr(x), _ptr(out), rows, K, _stream(stream))


def qmm_dequantize(t, blocks, out, rows, K, stream=None) -> int:
    return lib().qmm_dequantize(t, _ptr(blocks), _ptr(out), rows, K, _stream(stream))


def qmm_mul_mat(wtype, W, xq, y, M, N, K, stream=None) -> int:
    return lib().qmm_mul_mat(wtype, _ptr(W), _ptr(xq), _ptr(y), M, N, K, _stream(stream))


def qmm_mul_mat_algo(wtype, W, xq, y, M, N, K, algo, stream=None) -> int:
    return lib().qmm_mul_mat_algo(wtype, _ptr(W), _ptr(xq), _ptr(y), M, N, K, algo, _stream(stream))


def qmm_mul_mat_choice(wtype, M, N, K) -> int:
    return lib().qmm_mul_mat_choice(wtype, M, N, K)


def qmm_mul_mat_multi(wtype, count, W, y, M, x, x_is_f32, N, K, stream=None) -> int:
    """W, y: sequences of `count` device buffers (tensors or addresses); M: row counts."""
    Wa = (ctypes.c_void_p * max(count, 1))(*[_ptr(w) for w in W[:count]]) if W is not None else None
    ya = (ctypes.c_void_p * max(count, 1))(*[_ptr(t) for t in y[:count]]) if y is not None else None
    Ma = (ctypes.c_int64 * max(count, 1))(*M[:count]) if M is not None else None
    return lib().qmm_mul_mat_multi(wtype, count, Wa, ya, Ma, _ptr(x), int(bool(x_is_f32)), N, K, _stream(stream))


def qmm_probe_read(src, nbytes, sink, workgroups=0, stream=None) -> int:
    return lib().qmm_probe_read(_ptr(src), nbytes, _ptr(sink), workgroups, _stream(stream))


def qmm_probe_mfma(workgroups, iters, sink, stream=None) -> int:
    return lib().qmm_probe_mfma(workgroups, iters, _ptr(sink), _stream(stream))


def qmm_probe_mfma_ops(workgroups, iters) -> int:
    return lib().qmm_probe_mfma_ops(workgroups, iters)


def qmm_probe_mfma16(workgroups, iters, sink, stream=None) -> int:
    return lib().qmm_probe_mfma16(workgroups, iters, _ptr(sink), _stream(stream))


def qmm_probe_mfma16_ops(workgroups, iters) -> int:
    return lib().qmm_probe_mfma16_ops(workgroups, iters)


def qmm_strerror(code: int) -> str:
    return lib().qmm_strerror(code).decode()


# ------------------------------------------------------ allocating helpers

def _check(code: int, what: str):
    if code != QMM_OK:
        raise QmmError(code, what)


def quantize(dst: int, x, stream=None):
    """fp32 (rows, K) CUDA tensor -> (rows, row_bytes) uint8 tensor of dst blocks."""
    import torch
    rows, K = x.shape
    out = torch.empty((rows, qmm_row_bytes(dst, K)), dtype=torch.uint8, device=x.device)
    _check(qmm_quantize(dst, x, out, rows, K, stream), "qmm_quantize")
    return out


def quantize_act(dst: int, x, stream=None):
    import torch
    rows, K = x.shape
    out = torch.empty((rows, qmm_row_bytes(dst, K)), dtype=torch.uint8, device=x.device)
    _check(qmm_quantize_act(dst, x, out, rows, K, stream), "qmm_quantize_act")
    return out


def dequantize(t: int, blocks, rows: int, K: int, stream=None):
    import torch
    out = torch.empty((rows, K), dtype=torch.float32, device=blocks.device)
    _check(qmm_dequantize(t, blocks, out, rows, K, stream), "qmm_dequantize")
    return out


def mul_mat_multi(wtype: int, Ws, Ms, x, N: int, K: int, x_is_f32: bool = False, stream=None):
    """Several matrices sharing x in one launch -> list of (N, M_i) outputs."""
    import torch
    ys = [torch.empty((N, M), dtype=torch.float32, device=x.device) for M in Ms]
    _check(qmm_mul_mat_multi(wtype, len(Ws), Ws, ys, list(Ms), x, x_is_f32, N, K, stream), "qmm_mul_mat_multi")
    return ys


def mul_mat(wtype: int, W, xq, M: int, N: int, K: int, algo: int = 0, stream=None):
    import torch
    y = torch.empty((N, M), dtype=torch.float32, device=W.device)
    _check(qmm_mul_mat_algo(wtype, W, xq, y, M, N, K, algo, stream), "qmm_mul_mat")
    return y
