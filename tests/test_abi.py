"""The C-ABI library: it loads, exports every function include/*.h declares,
and rejects invalid arguments before launching anything.  None of these calls
reaches the GPU (validation returns first), so they run without one."""
import glob
import os
import re

import pytest

import block_quantized_amd as Q
from conftest import ROOT

HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(qmm_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    return Q.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(Q.EXPORTED)


def test_sizes(L):
    assert [Q.qmm_block_size(t) for t in range(1, 6)] == [32, 32, 256, 256, 256]
    assert [Q.qmm_block_bytes(t) for t in range(1, 6)] == [18, 34, 144, 210, 292]
    assert Q.qmm_block_size(0) == 0 and Q.qmm_block_bytes(9) == 0
    assert Q.qmm_row_bytes(Q.QMM_Q4_0, 2048) == 64 * 18
    assert Q.qmm_row_bytes(Q.QMM_Q6_K, 4096) == 16 * 210
    assert Q.qmm_row_bytes(Q.QMM_Q4_K, 300) == 0 and Q.qmm_row_bytes(Q.QMM_Q8_0, 0) == 0
    assert Q.qmm_vec_dot_type(Q.QMM_Q4_0) == Q.QMM_Q8_0
    assert Q.qmm_vec_dot_type(Q.QMM_Q8_0) == Q.QMM_Q8_0
    assert Q.qmm_vec_dot_type(Q.QMM_Q4_K) == Q.QMM_Q8_K
    assert Q.qmm_vec_dot_type(Q.QMM_Q6_K) == Q.QMM_Q8_K
    assert Q.qmm_vec_dot_type(Q.QMM_Q5_0) == Q.QMM_Q8_0
    assert Q.qmm_block_size(Q.QMM_Q5_0) == 32 and Q.qmm_block_bytes(Q.QMM_Q5_0) == 22
    assert Q.qmm_row_bytes(Q.QMM_Q5_0, 896) == 28 * 22 and Q.qmm_block_size(7) == 0
    assert Q.qmm_vec_dot_type(Q.QMM_Q8_K) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_vec_dot_type(42) == Q.QMM_ERR_TYPE
    for c in (0, -1, -2, -3, -4, -5, -6, -99):
        assert isinstance(Q.qmm_strerror(c), str) and Q.qmm_strerror(c)


# Fake, never dereferenced device addresses: validation fails before any use.
A = 0x7F0000000000  # 16-byte aligned
S = 0  # null stream


def test_quantize_errors(L):
    assert Q.qmm_quantize_act(99, A, A, 1, 32, S) == Q.QMM_ERR_TYPE
    assert Q.qmm_quantize_act(Q.QMM_Q4_0, A, A, 1, 32, S) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_quantize_act(Q.QMM_Q4_K, A, A, 1, 256, S) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_quantize(Q.QMM_Q6_K, A, A, 1, 256, S) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_quantize(Q.QMM_Q5_0, A, A, 1, 256, S) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_quantize_act(Q.QMM_Q5_0, A, A, 1, 256, S) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_quantize_act(Q.QMM_Q8_0, 0, A, 1, 32, S) == Q.QMM_ERR_NULL
    assert Q.qmm_quantize_act(Q.QMM_Q8_0, A, 0, 1, 32, S) == Q.QMM_ERR_NULL
    assert Q.qmm_quantize_act(Q.QMM_Q8_0, A + 4, A, 1, 32, S) == Q.QMM_ERR_ALIGN
    assert Q.qmm_quantize_act(Q.QMM_Q8_0, A, A + 2, 1, 32, S) == Q.QMM_ERR_ALIGN
    assert Q.qmm_quantize_act(Q.QMM_Q8_0, A, A, 0, 32, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_quantize_act(Q.QMM_Q8_0, A, A, 1, 48, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_quantize_act(Q.QMM_Q8_K, A, A, 1, 128, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_quantize_act(Q.QMM_Q8_K, A, A, -5, 256, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_quantize_act(Q.QMM_Q8_K, A, A, 2 ** 62, 256, S) == Q.QMM_ERR_SHAPE


def test_dequantize_errors(L):
    assert Q.qmm_dequantize(0, A, A, 1, 32, S) == Q.QMM_ERR_TYPE
    assert Q.qmm_dequantize(Q.QMM_Q4_K, A, A, 1, 32, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_dequantize(Q.QMM_Q4_0, 0, A, 1, 32, S) == Q.QMM_ERR_NULL
    assert Q.qmm_dequantize(Q.QMM_Q4_0, A, A + 8, 1, 32, S) == Q.QMM_ERR_ALIGN


def test_mul_mat_errors(L):
    mm = Q.qmm_mul_mat
    assert mm(77, A, A, A, 4, 1, 256, S) == Q.QMM_ERR_TYPE
    assert mm(Q.QMM_Q8_K, A, A, A, 4, 1, 256, S) == Q.QMM_ERR_UNSUPPORTED
    assert mm(Q.QMM_Q4_K, 0, A, A, 4, 1, 256, S) == Q.QMM_ERR_NULL
    assert mm(Q.QMM_Q4_K, A, 0, A, 4, 1, 256, S) == Q.QMM_ERR_NULL
    assert mm(Q.QMM_Q4_K, A, A, 0, 4, 1, 256, S) == Q.QMM_ERR_NULL
    assert mm(Q.QMM_Q4_K, A + 2, A, A, 4, 1, 256, S) == Q.QMM_ERR_ALIGN
    assert mm(Q.QMM_Q4_K, A, A, A + 4, 4, 1, 256, S) == Q.QMM_ERR_ALIGN
    assert mm(Q.QMM_Q4_K, A, A, A, 4, 1, 128, S) == Q.QMM_ERR_SHAPE   # K % 256
    assert mm(Q.QMM_Q4_0, A, A, A, 4, 1, 48, S) == Q.QMM_ERR_SHAPE    # K % 32
    assert mm(Q.QMM_Q5_0, A, A, A, 4, 1, 48, S) == Q.QMM_ERR_SHAPE
    assert mm(7, A, A, A, 4, 1, 32, S) == Q.QMM_ERR_TYPE
    assert mm(Q.QMM_Q4_0, A, A, A, 0, 1, 32, S) == Q.QMM_ERR_SHAPE
    assert mm(Q.QMM_Q4_0, A, A, A, 4, 0, 32, S) == Q.QMM_ERR_SHAPE
    assert mm(Q.QMM_Q4_0, A, A, A, 2 ** 31, 1, 32, S) == Q.QMM_ERR_SHAPE
    assert mm(Q.QMM_Q6_K, A, A, A, 4, 1, 65536 + 256, S) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_mul_mat_algo(Q.QMM_Q4_0, A, A, A, 4, 1, 32, 3, S) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_mul_mat_algo(Q.QMM_Q4_0, A, A, A, 4, 1, 32, -1, S) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_mul_mat_algo(Q.QMM_Q8_K, A, A, A, 4, 16, 256, 2, S) == Q.QMM_ERR_UNSUPPORTED  # Q8_K is never a weight


def test_binding_has_no_fallback(monkeypatch, tmp_path):
    # With the library path pointing nowhere, loading must raise, not degrade.
    monkeypatch.setattr(Q, "_lib", None)
    monkeypatch.setattr(Q, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        Q.lib()


def test_multi_errors_cpu(L):
    mm = Q.qmm_mul_mat_multi
    assert mm(99, 1, [A], [A], [4], A, 0, 1, 256, S) == Q.QMM_ERR_TYPE
    assert mm(Q.QMM_Q8_K, 1, [A], [A], [4], A, 0, 1, 256, S) == Q.QMM_ERR_UNSUPPORTED
    assert mm(Q.QMM_Q4_K, 0, [A], [A], [4], A, 0, 1, 256, S) == Q.QMM_ERR_SHAPE
    assert mm(Q.QMM_Q4_K, 5, [A] * 5, [A] * 5, [4] * 5, A, 0, 1, 256, S) == Q.QMM_ERR_SHAPE
    assert mm(Q.QMM_Q4_K, 1, None, [A], [4], A, 0, 1, 256, S) == Q.QMM_ERR_NULL
    assert mm(Q.QMM_Q4_K, 2, [A, 0], [A, A], [4, 4], A, 0, 1, 256, S) == Q.QMM_ERR_NULL
    assert mm(Q.QMM_Q4_K, 2, [A, A + 2], [A, A], [4, 4], A, 0, 1, 256, S) == Q.QMM_ERR_ALIGN
    assert mm(Q.QMM_Q4_K, 2, [A, A], [A, A], [4, 0], A, 0, 1, 256, S) == Q.QMM_ERR_SHAPE
    assert mm(Q.QMM_Q4_K, 1, [A], [A], [4], A, 0, 1, 384, S) == Q.QMM_ERR_SHAPE
    assert mm(Q.QMM_Q4_K, 1, [A], [A], [4], 0, 0, 1, 256, S) == Q.QMM_ERR_NULL
    assert mm(Q.QMM_Q4_K, 1, [A], [A], [4], A, 1, 9, 256, S) == Q.QMM_ERR_UNSUPPORTED
    assert mm(Q.QMM_Q4_0, 1, [A], [A], [4], A, 1, 1, 96, S) == Q.QMM_ERR_UNSUPPORTED


def test_mul_mat_choice_cpu(L):
    # the automatic GEMV / GEMM switch of qmm_mul_mat, at the crossovers
    # measured on MI355X (host logic: no GPU needed)
    ch = Q.qmm_mul_mat_choice
    assert [ch(Q.QMM_Q4_K, 14336, n, 4096) for n in (1, 2, 3, 8)] == [1, 1, 2, 2]
    assert [ch(Q.QMM_Q4_K, 4096, n, 4096) for n in (1, 2, 3, 32)] == [1, 1, 2, 2]
    assert [ch(Q.QMM_Q4_K, 1024, n, 4096) for n in (2, 3)] == [1, 2]
    assert [ch(Q.QMM_Q4_K, 1000, n, 4096) for n in (2, 3)] == [1, 2]
    assert [ch(Q.QMM_Q4_K, 256, n, 1536) for n in (2, 3)] == [1, 2]
    assert [ch(Q.QMM_Q4_K, 8960, n, 1536) for n in (4, 5)] == [1, 2]
    assert [ch(Q.QMM_Q4_K, 14336, n, 4096) for n in (2, 3)] == [1, 2]
    assert [ch(Q.QMM_Q6_K, 128256, n, 4096) for n in (4, 5, 32)] == [1, 2, 2]
    assert [ch(Q.QMM_Q6_K, 4096, n, 14336) for n in (30, 31)] == [1, 2]
    assert [ch(Q.QMM_Q6_K, 32000, n, 4096) for n in (4, 5)] == [1, 2]
    assert [ch(Q.QMM_Q6_K, 14336, n, 4096) for n in (6, 7)] == [1, 2]
    assert [ch(Q.QMM_Q6_K, 8960, n, 1536) for n in (6, 7)] == [1, 2]
    assert [ch(Q.QMM_Q6_K, 1536, n, 8960) for n in (54, 55)] == [1, 2]
    # Q4_0 / Q5_0 / Q8_0: by rows above 8192, else by K and M
    shapes = ((32000, 4096), (65536, 2048), (14336, 4096), (8960, 1536), (896, 896), (1536, 1536), (2048, 1024), (4864, 896),
              (8192, 2048), (4096, 4096), (1024, 4096), (896, 4864), (1536, 8960), (2048, 8192))
    for wt, t in ((Q.QMM_Q4_0, (8, 8, 12, 12, 21, 14, 14, 7, 17, 28, 23, 30, 30, 47)),
                  (Q.QMM_Q5_0, (8, 8, 12, 12, 23, 16, 16, 8, 19, 32, 26, 33, 33, 51)),
                  (Q.QMM_Q8_0, (7, 7, 10, 10, 26, 15, 15, 7, 17, 26, 26, 31, 31, 45))):
        for (M, K), tm in zip(shapes, t):
            assert [ch(wt, M, n, K) for n in (tm, tm + 1)] == [1, 2], (wt, M, K)
        assert ch(wt, 8193, 40, 32768) == 2 and ch(wt, 4096, 33, 512) == 2
    # what qmm_mul_mat rejects
    assert ch(Q.QMM_Q8_K, 4096, 1, 4096) == 0           # not a weight type
    assert ch(0, 4096, 1, 4096) == 0
    assert ch(Q.QMM_Q4_K, 4096, 1, 4000) == 0           # K % 256
    assert ch(Q.QMM_Q4_0, 0, 1, 4096) == 0
    assert ch(Q.QMM_Q4_0, 64, 0, 4096) == 0
    assert ch(Q.QMM_Q4_0, 64, 1, 65536 + 32) == 0       # K beyond the supported range


def test_probe_errors_cpu(L):
    assert Q.qmm_probe_read(0, 64, A, 0, S) == Q.QMM_ERR_NULL
    assert Q.qmm_probe_read(A, 64, 0, 0, S) == Q.QMM_ERR_NULL
    assert Q.qmm_probe_read(A + 4, 64, A, 0, S) == Q.QMM_ERR_ALIGN
    assert Q.qmm_probe_read(A, 0, A, 0, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_probe_read(A, 40, A, 0, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_probe_read(A, 64, A, -1, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_probe_read(A, 64, A, 65537, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_probe_mfma(512, 10, 0, S) == Q.QMM_ERR_NULL
    assert Q.qmm_probe_mfma(0, 10, A, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_probe_mfma(512, 0, A, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_probe_mfma(512, 2 ** 30 + 1, A, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_probe_mfma_ops(2, 3) == 2 * 4 * 4 * 3 * 2 * 32 * 32 * 32
    assert Q.qmm_probe_mfma_ops(0, 3) == 0
    assert Q.qmm_probe_mfma16(512, 10, 0, S) == Q.QMM_ERR_NULL
    assert Q.qmm_probe_mfma16(0, 10, A, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_probe_mfma16(65537, 10, A, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_probe_mfma16(512, 0, A, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_probe_mfma16(512, 2 ** 30 + 1, A, S) == Q.QMM_ERR_SHAPE
    assert Q.qmm_probe_mfma16_ops(2, 3) == 2 * 4 * 8 * 3 * 2 * 16 * 16 * 64
    assert Q.qmm_probe_mfma16_ops(2, 0) == 0


def test_launch_configuration_error_is_reported_cpu(L):
    # Arguments that pass validation (M <= INT_MAX, every size fits) but whose
    # GEMM grid would exceed 2^32 work-items: the launcher refuses before any
    # HIP call and the status is QMM_ERR_HIP (no GPU needed, nothing enqueued).
    assert Q.qmm_mul_mat_algo(Q.QMM_Q4_0, A, A, A, 2 ** 30, 512, 32, 2, S) == Q.QMM_ERR_HIP
    assert Q.qmm_mul_mat(Q.QMM_Q8_0, A, A, A, 2 ** 30, 512, 32, S) == Q.QMM_ERR_HIP
