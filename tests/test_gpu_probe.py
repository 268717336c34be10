"""The measurement kernels of include/qmm_probe.h: the streaming read reads
every byte exactly once (the XOR of its per-workgroup words equals numpy's
XOR over the same buffer) and writes nothing past its workgroups' words; the
int8-MFMA loop is deterministic."""
import sys

import numpy as np
import pytest
import torch

import block_quantized_amd as Q
from gpu_util import to_cpu, to_gpu

pytestmark = pytest.mark.gpu

WORDS = 65536  # QMM_PROBE_SINK_WORDS


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("nbytes,groups", [(16, 0), (4096 + 48, 0), (1 << 20, 3), (10 * (1 << 20) + 16 * 7, 0),
                                           ((64 << 20) + 4096, 0), ((64 << 20) + 4096, 2048)])
def test_read_checksum(nbytes, groups):
    g = np.random.default_rng(nbytes + groups)
    buf = g.integers(0, 256, size=nbytes, dtype=np.uint8)
    say("probe read", nbytes, groups)
    src = to_gpu(buf)
    sink = torch.full((WORDS + 64,), -1, dtype=torch.int32, device="cuda")
    assert Q.qmm_probe_read(src, nbytes, sink, groups) == Q.QMM_OK
    got = to_cpu(sink).view(np.uint32)
    used = groups or min(2048, max(1, (nbytes // 16 + 255) // 256))
    want = np.bitwise_xor.reduce(buf.view(np.uint32))
    assert np.bitwise_xor.reduce(got[:used]) == want
    assert np.all(got[used:] == 0xFFFFFFFF), "wrote past its workgroups' words"


@pytest.mark.parametrize("form", ["32x32x32", "16x16x64"])
def test_mfma_deterministic(form):
    say("probe mfma", form)
    run = Q.qmm_probe_mfma if form == "32x32x32" else Q.qmm_probe_mfma16
    sinks = [torch.full((WORDS,), -1, dtype=torch.int32, device="cuda") for _ in range(2)]
    for s in sinks:
        assert run(64, 100, s) == Q.QMM_OK
    a, b = (to_cpu(s).view(np.uint32) for s in sinks)
    assert np.array_equal(a, b)
    assert np.all(a[64:] == 0xFFFFFFFF)
    assert np.any(a[:64] != 0)
