"""Launch status on the GPU: a call reports the status of its own launches
only.  An error that an earlier, unrelated HIP call left as the thread's last
error is neither reported nor cleared by the library."""
import ctypes

import pytest
import torch

import block_quantized_amd as Q

pytestmark = pytest.mark.gpu

HIP_ERROR_INVALID_DEVICE = 101


def test_earlier_hip_error_is_neither_reported_nor_cleared():
    hip = ctypes.CDLL("libamdhip64.so")  # the runtime torch has loaded
    hip.hipGetLastError.restype = ctypes.c_int
    hip.hipSetDevice.restype = ctypes.c_int
    x = torch.randn(4, 64, device="cuda")
    xq = torch.empty(4 * Q.qmm_row_bytes(Q.QMM_Q8_0, 64), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    assert hip.hipGetLastError() == 0
    assert hip.hipSetDevice(9999) == HIP_ERROR_INVALID_DEVICE  # leaves a last error, changes nothing
    try:
        assert Q.qmm_quantize_act(Q.QMM_Q8_0, x, xq, 4, 64) == Q.QMM_OK
    finally:
        planted = hip.hipGetLastError()  # clears it for the tests that follow
    assert planted == HIP_ERROR_INVALID_DEVICE
    ref = Q.quantize_act(Q.QMM_Q8_0, x)
    assert torch.equal(ref.view(-1), xq)
