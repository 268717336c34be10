"""Pins the oracle's IEEE binary16 conversions against numpy's float16, an
independent implementation of the same IEEE 754 definition (round to nearest,
ties to even, with subnormals).  The fp16 block scales of every format on the
format table of page 'The GGML ecosystem, and where synapse fits' (section 5)
go through these conversions."""
import numpy as np

import oracle as O


def _same_f32(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    nan = np.isnan(a)
    assert np.array_equal(nan, np.isnan(b))
    assert np.array_equal(a[~nan].view(np.uint32), b[~nan].view(np.uint32))


def test_decode_all_65536_patterns():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    _same_f32(O.fp16_to_f32(h), h.view(np.float16).astype(np.float32))


def test_encode_edge_cases():
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.996, 65520.0, 65536.0, 1e9, -1e9,
            np.inf, -np.inf, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26,
            2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 2.0 ** -26, 5.960464477539063e-08,
            1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -11 + 2.0 ** -20,
            0.015748031437397003, 1e-3, 7.0e-5, 6.1e-5, 1e-40, -1e-45]
    f = np.array(vals, np.float32)
    got = O.f32_to_fp16(f)
    want = f.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want), (f, got, want)
    nan = O.f32_to_fp16(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0


def test_encode_every_halfway_point():
    # Midpoints between consecutive finite fp16 values are exact in fp32 and
    # are exactly where ties-to-even decides; check all of them, plus one fp32
    # ulp either side.
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    for v in (mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0))):
        for s in (v, -v):
            assert np.array_equal(O.f32_to_fp16(s), s.astype(np.float16).view(np.uint16))


def test_encode_random_sweep():
    g = np.random.default_rng(1234)
    # Random bit patterns concentrated on the exponents that fp16 can reach.
    bits = g.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    exp = g.integers(100, 146, size=bits.size).astype(np.uint32)
    bits = (bits & np.uint32(0x807FFFFF)) | (exp << np.uint32(23))
    f = bits.view(np.float32)
    assert np.array_equal(O.f32_to_fp16(f), f.astype(np.float16).view(np.uint16))
    f2 = g.standard_normal(2_000_000, dtype=np.float32) * np.float32(1e-3)
    assert np.array_equal(O.f32_to_fp16(f2), f2.astype(np.float16).view(np.uint16))
