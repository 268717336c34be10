"""Pins the oracle's round-to-nearest quantizers.

Source: page 'The GGML ecosystem, and where synapse fits', section 5
'Quantization' (Q8_0 = fp16 d + 32 int8, w = d q; Q8_K = float d, 256 int8,
sixteen int16 sums) and 'Products: weights against quantized activations'
(activations are converted to the weight's vec_dot_type once per row).  The
rounding steps are not printed; the reading is d = amax/127 (fp32),
id = 1/d, q = roundf(x*id) (ties away from zero).

Pins: hand-worked blocks (ties, ramps, sums), closed-form properties (the
amax element lands on +-127, error bound d/2, nearest integer with ties away
from zero, exact sums, zero block, sign and power-of-two symmetry).
"""
import numpy as np
import pytest
from hypothesis import example, given, settings, strategies as st
from hypothesis.extra.numpy import arrays

import oracle as O


def split_q8_0(b):
    b = b.reshape(-1, 34)
    d16 = b[:, 0:2].copy().view(np.uint16)[:, 0]
    return d16, b[:, 2:].view(np.int8)


def split_q8_k(b):
    b = b.reshape(-1, 292)
    d = b[:, 0:4].copy().view(np.float32)[:, 0]
    q = b[:, 4:260].view(np.int8)
    s = b[:, 260:292].copy().view(np.int16)
    return d, q, s


# ---------------------------------------------------------- hand-worked

def test_hand_q8_0_ties(golden):
    h = golden("hand_blocks.json")["q8_0_ties"]
    b = O.quantize(O.Q8_0, np.array(h["x"], np.float32))
    d16, q = split_q8_0(b)
    assert d16[0] == h["d_fp16_bits"]
    assert q[0].tolist() == h["q"]
    assert q[0, :8].tolist() != h["q_if_ties_to_even"]


def test_hand_q8_0_ramp(golden):
    h = golden("hand_blocks.json")["q8_0_ramp"]
    x = ((np.arange(32) - 16) / 8).astype(np.float32)
    b = O.quantize(O.Q8_0, x)
    d16, q = split_q8_0(b)
    assert d16[0] == h["d_fp16_bits"]
    assert q[0].tolist() == h["q"]
    w = O.dequantize(O.Q8_0, b, 1, 32)[0]
    assert np.abs(w - x).max() == h["max_abs_roundtrip_error"]


def test_hand_q8_k_ramp(golden):
    h = golden("hand_blocks.json")["q8_k_ramp"]
    x = ((np.arange(256) - 128) / 64).astype(np.float32)
    d, q, s = split_q8_k(O.quantize(O.Q8_K, x))
    assert float(d[0]) == h["d_f32"]
    assert q[0, :4].tolist() == h["q_first4"] and q[0, -4:].tolist() == h["q_last4"]
    assert s[0].tolist() == h["bsums"]


# ---------------------------------------------------------- properties

def _check_rtn(x, d, q, B):
    """x (rows, K) fp32; d fp32 per block; q int8.  Closed-form checks."""
    xb = x.reshape(-1, B).astype(np.float64)
    qb = q.reshape(-1, B).astype(np.int64)
    d = d.astype(np.float64)
    amax = np.abs(xb).max(axis=1)
    nz = d > 0
    # the element of largest magnitude lands on +-127
    i = np.abs(xb).argmax(axis=1)
    assert np.all(np.abs(qb[np.arange(len(i)), i][nz]) == 127)
    # Blocks whose 1/d overflows fp32 (amax below about 127 / FLT_MAX): every
    # x * id is +-Inf, so each nonzero value saturates to +-127 and zeros stay 0
    # (0 * Inf is NaN, read as 0).
    with np.errstate(divide="ignore", over="ignore"):
        ovf = nz & ~np.isfinite(np.float32(1) / d.astype(np.float32))
    assert np.array_equal(qb[ovf], (127 * np.sign(xb[ovf])).astype(np.int64))
    # Elsewhere |x - d q| <= d/2, up to the rounding of d and of x*id (a few
    # fp32 ulps).  Where d is subnormal its own rounding (half the 2^-149
    # quantum, times up to 127 steps) adds to the bound.
    err = np.abs(xb - d[:, None] * qb)
    slack = np.where(d < 2.0 ** -126, 127 * 2.0 ** -150, 0.0)
    assert np.all((err <= d[:, None] * (0.5 + 1e-5) + slack[:, None] + 1e-45)[~ovf])
    # zero blocks: d = 0 and q = 0
    assert np.all(qb[amax == 0] == 0) and np.all(d[amax == 0] == 0)
    assert np.all(np.abs(qb) <= 127)


def _nearest_ties_away(x, d, q, B):
    """q is the integer nearest to t = x*id (fp32 product), ties away."""
    xb = x.reshape(-1, B)
    d32 = d.astype(np.float32)
    with np.errstate(divide="ignore"):
        id32 = np.where(d32 != 0, np.float32(1) / d32, np.float32(0)).astype(np.float32)
    with np.errstate(invalid="ignore"):
        t = (xb * id32[:, None]).astype(np.float64)
    qb = q.reshape(-1, B).astype(np.float64)
    # where 1/d overflowed, t is +-Inf or NaN and q saturates (tested apart)
    fin = np.isfinite(t)
    t, qb = t[fin], qb[fin]
    dist = np.abs(qb - t)
    assert np.all(dist <= 0.5)
    tie = dist == 0.5
    assert np.all(np.abs(qb[tie]) > np.abs(t[tie]))


@pytest.mark.parametrize("sigma", [1.0, 0.02, 1e-3, 3e4])
def test_q8_0_properties(sigma):
    g = np.random.default_rng(17)
    x = g.standard_normal((64, 1024), dtype=np.float32) * np.float32(sigma)
    x[3, 64:96] = 0.0
    b = O.quantize(O.Q8_0, x)
    d16, q = split_q8_0(b)
    d16f = d16.view(np.float16).astype(np.float32)
    # recover the fp32 d from the definition's inputs and check fp16 storage
    amax = np.abs(x.reshape(-1, 32)).max(axis=1)
    d32 = amax / np.float32(127)
    assert np.array_equal(d32.astype(np.float16).view(np.uint16), d16)
    _check_rtn(x, d32, q, 32)
    _nearest_ties_away(x, d32, q, 32)
    # round-trip through the stored fp16 scale: d/2 + |q| |d - fp16(d)|
    w = O.dequantize(O.Q8_0, b, 64, 1024).reshape(-1, 32).astype(np.float64)
    bound = d32[:, None] / 2 + np.abs(q) * np.abs(d32 - d16f)[:, None] + 1e-6 * d32[:, None]
    assert np.all(np.abs(w - x.reshape(-1, 32)) <= bound)


def test_q8_k_properties():
    g = np.random.default_rng(19)
    x = g.standard_normal((32, 4096), dtype=np.float32)
    x[1, :256] = 0
    x[2, :] *= np.float32(1e-30)
    d, q, s = split_q8_k(O.quantize(O.Q8_K, x))
    _check_rtn(x, d, q, 256)
    _nearest_ties_away(x, d, q, 256)
    assert np.array_equal(s, q.reshape(-1, 16, 16).astype(np.int64).sum(axis=2))
    w = O.dequantize(O.Q8_K, O.quantize(O.Q8_K, x), 32, 4096).reshape(-1, 256)
    assert np.all(np.abs(w - x.reshape(-1, 256)) <= d[:, None] * (0.5 + 1e-5))


@settings(max_examples=200, deadline=None)
@given(arrays(np.float32, 256, elements=st.floats(-1e6, 1e6, width=32, allow_subnormal=True)))
def test_q8_k_hypothesis(x):
    d, q, s = split_q8_k(O.quantize(O.Q8_K, x))
    _check_rtn(x[None], d, q, 256)
    _nearest_ties_away(x[None], d, q, 256)
    assert np.array_equal(s, q.reshape(-1, 16, 16).astype(np.int64).sum(axis=2))


@settings(max_examples=200, deadline=None)
@given(arrays(np.float32, 32, elements=st.floats(-6e4, 6e4, width=32)))
@example(np.array([2.0 ** -126] + [2.0 ** -149] * 31, np.float32))  # 1/d overflows
def test_q8_0_hypothesis(x):
    b = O.quantize(O.Q8_0, x)
    amax = np.abs(x).max()
    d32 = np.array([amax / np.float32(127)], np.float32)
    _, q = split_q8_0(b)
    _check_rtn(x[None], d32, q, 32)
    _nearest_ties_away(x[None], d32, q, 32)


def test_sign_and_power_of_two_symmetry():
    g = np.random.default_rng(23)
    x = g.standard_normal((8, 512), dtype=np.float32)
    for t in (O.Q8_0, O.Q8_K):
        b0 = O.quantize(t, x)
        bn = O.quantize(t, -x)
        b2 = O.quantize(t, x * np.float32(4.0))
        if t == O.Q8_0:
            d0, q0 = split_q8_0(b0)
            dn, qn = split_q8_0(bn)
            d2, q2 = split_q8_0(b2)
            assert np.array_equal(d0, dn)
            assert np.array_equal(d2.view(np.float16), (d0.view(np.float16) * 4))
        else:
            d0, q0, _ = split_q8_k(b0)
            dn, qn, _ = split_q8_k(bn)
            d2, q2, _ = split_q8_k(b2)
            assert np.array_equal(d0, dn) and np.array_equal(d2, d0 * 4)
        assert np.array_equal(qn, -q0)
        assert np.array_equal(q2, q0)


def test_tiny_values_do_not_produce_nan_codes():
    # amax so small that d = amax/127 is subnormal and 1/d overflows to Inf:
    # the zero elements' product is NaN and encodes as 0; nonzero elements
    # saturate at +-127.
    x = np.zeros((1, 256), np.float32)
    x[0, 0] = np.float32(2e-37)
    x[0, 1] = np.float32(-1e-38)
    d, q, s = split_q8_k(O.quantize(O.Q8_K, x))
    assert 0 < d[0] < 2.0 ** -126 and np.isinf(np.float32(1) / d[0])
    assert q[0, 0] == 127 and q[0, 1] == -127 and np.all(q[0, 2:] == 0)
    assert s[0, 0] == 0
    b = O.quantize(O.Q8_0, x[:, :32])
    d16, q = split_q8_0(b)
    assert d16[0] == 0
    assert q[0, 0] == 127 and q[0, 1] == -127 and np.all(q[0, 2:] == 0)
    # amax so small that d rounds to zero: the block is all zeros
    x[0, 0], x[0, 1] = np.float32(1e-44), np.float32(-1e-45)
    d, q, s = split_q8_k(O.quantize(O.Q8_K, x))
    assert d[0] == 0 and np.all(q == 0) and np.all(s == 0)


# --------------------------------------------------- Q4_0 weight encoder

def test_q4_0_encoder():
    g = np.random.default_rng(29)
    x = g.standard_normal((128, 2048), dtype=np.float32) * np.float32(0.02)
    x[5, :32] = 0
    b = O.quantize(O.Q4_0, x)
    bl = b.reshape(-1, 18)
    d16 = bl[:, 0:2].copy().view(np.float16)[:, 0].astype(np.float64)
    w = O.dequantize(O.Q4_0, b, 128, 2048).reshape(-1, 32).astype(np.float64)
    xb = x.reshape(-1, 32).astype(np.float64)
    i = np.abs(xb).argmax(axis=1)
    m = xb[np.arange(len(i)), i]
    # d = m / -8; the extreme element is stored at level 0 (value -8 d)
    assert np.array_equal(d16.astype(np.float16), (m.astype(np.float32) / np.float32(-8)).astype(np.float16))
    lo = np.where(i < 16, bl[np.arange(len(i)), 2 + (i % 16)] & 15, bl[np.arange(len(i)), 2 + (i % 16)] >> 4)
    assert np.all(lo[m != 0] == 0)
    # every element is within |d| of its value (half a step, or one step for
    # the level +8 that does not exist and clamps to +7), plus fp16 scale error
    dd = np.abs(m / 8)
    assert np.all(np.abs(w - xb) <= dd[:, None] * (1 + 1e-6) + 8 * np.abs(d16 + m / 8)[:, None])
    assert np.all(w[5 * 64] == 0)


def _q4_0_codes(b):
    bl = b.reshape(-1, 18)
    qs = bl[:, 2:]
    return bl[:, 0:2].copy().view(np.uint16)[:, 0], np.concatenate([qs & 15, qs >> 4], axis=1)


def test_hand_q4_0_encoder_ties(golden):
    h = golden("hand_blocks.json")["q4_0_encoder_ties"]
    b = O.quantize(O.Q4_0, np.array(h["x"], np.float32))
    d16, q = _q4_0_codes(b)
    assert d16[0] == h["d_fp16_bits"]
    assert q[0].tolist() == h["q"]
    assert b.reshape(-1)[2:18].tolist() == h["qs_bytes"]
    assert q[0].tolist() != h["q_if_ties_to_even"]


def test_hand_q4_0_encoder_nan(golden):
    h = golden("hand_blocks.json")["q4_0_encoder_nan"]
    x = np.array([np.nan if v == "nan" else v for v in h["x"]], np.float32)
    d16, q = _q4_0_codes(O.quantize(O.Q4_0, x))
    assert d16[0] == h["d_fp16_bits"]
    assert q[0].tolist() == h["q"]


def test_reciprocal_of_d_is_what_multiplies():
    # id is 1/d with d = amax/127 already rounded to fp32, not 127/amax.  Find
    # amax values where the two differ in fp32, and values x whose products
    # with each round to different integers; the quantizer must follow 1/d.
    g = np.random.default_rng(43)
    amax = (g.random(200_000, dtype=np.float32) + np.float32(0.5)).astype(np.float32)
    id_recip = np.float32(1) / (amax / np.float32(127))
    id_direct = np.float32(127) / amax
    found = 0
    for i in np.nonzero(id_recip != id_direct)[0][:2000]:
        for n in range(1, 127):
            x = np.float32((n + 0.5) / float(id_recip[i]))  # near a rounding boundary
            for xx in (x, np.nextafter(x, np.float32(0)), np.nextafter(x, np.float32(1e9))):
                if xx > amax[i]:
                    continue
                q1 = np.floor(np.float64(np.float32(xx * id_recip[i])) + 0.5)
                q2 = np.floor(np.float64(np.float32(xx * id_direct[i])) + 0.5)
                if q1 != q2:
                    blk = np.zeros(32, np.float32)
                    blk[0], blk[1] = amax[i], xx
                    _, q = split_q8_0(O.quantize(O.Q8_0, blk))
                    assert q[0, 1] == q1, (amax[i], xx, q1, q2)
                    found += 1
                    break
        if found >= 5:
            break
    assert found >= 5
