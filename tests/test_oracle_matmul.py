"""Pins the oracle's matrix product.

Sources:
- page 'ggml', examples/simple README ('Simple'): the printed example
  ggml_mul_mat(A, B^T) = C^T pins the orientation y[n][m] = sum_k W[m][k] x[n][k]
  (tests/golden/ggml_simple_mul_mat.json);
- page 'The GGML ecosystem, and where synapse fits', section 5: the element
  formulas of the format table, and 'Products: weights against quantized
  activations' (integer block dot, float block scales; equal to the plain
  product apart from float summation order).

Pins: the printed example for all four weight types; unit-scale and
integer-scale cases against numpy's int64 matmul (exact); the method's
block-formula product against the plain definition; numpy's fp64 matmul of
the dequantized arrays; exact linearity in the activation scale.

The blocks here are built by small encoders written in this file from the
same layout reading (the encoding direction), independent of the oracle's
decoders.
"""
import numpy as np
import pytest

import oracle as O
import synth

ONE = 0x3C00


def h16(bits, shape):
    return np.broadcast_to(np.array(bits, np.uint16), shape).copy().view(np.uint8).reshape(*shape, 2)


# ------------------------------------------------------------- encoders

def enc_q8_0(q, d_bits=ONE):
    M, K = q.shape
    b = np.zeros((M, K // 32, 34), np.uint8)
    b[:, :, 0:2] = h16(d_bits, (M, K // 32))
    b[:, :, 2:] = q.astype(np.int8).reshape(M, K // 32, 32).view(np.uint8)
    return b.reshape(M, -1)


def enc_q4_0(q, d_bits=ONE):
    M, K = q.shape
    q = q.reshape(M, K // 32, 32).astype(np.uint8)
    b = np.zeros((M, K // 32, 18), np.uint8)
    b[:, :, 0:2] = h16(d_bits, (M, K // 32))
    b[:, :, 2:] = q[:, :, :16] | (q[:, :, 16:] << 4)
    return b.reshape(M, -1)


def enc_q5_0(q, d_bits=ONE):
    """q: (M, K) in 0..31 -> Q5_0 blocks: low parts as Q4_0's nibbles, fifth
    bit of element e in bit e of the little-endian 32-bit qh."""
    M, K = q.shape
    q = q.reshape(M, K // 32, 32).astype(np.int64)
    b = np.zeros((M, K // 32, 22), np.uint8)
    b[:, :, 0:2] = h16(d_bits, (M, K // 32))
    qh = ((q >> 4) << np.arange(32)).sum(axis=2).astype("<u4")
    b[:, :, 2:6] = qh[..., None].view(np.uint8).reshape(M, K // 32, 4)
    lo = (q & 15).astype(np.uint8)
    b[:, :, 6:] = lo[:, :, :16] | (lo[:, :, 16:] << 4)
    return b.reshape(M, -1)


def enc_q4_k_scales(sc, m):
    """sc, m: (..., 8) in 0..63 -> (..., 12) bytes."""
    sc = sc.astype(np.uint8)
    m = m.astype(np.uint8)
    s = np.zeros(sc.shape[:-1] + (12,), np.uint8)
    s[..., 0:4] = sc[..., 0:4] | ((sc[..., 4:8] >> 4) << 6)
    s[..., 4:8] = m[..., 0:4] | ((m[..., 4:8] >> 4) << 6)
    s[..., 8:12] = (sc[..., 4:8] & 15) | ((m[..., 4:8] & 15) << 4)
    return s


def enc_q4_k(q, sc, m, d_bits=ONE, dmin_bits=ONE):
    M, K = q.shape
    nb = K // 256
    b = np.zeros((M, nb, 144), np.uint8)
    b[:, :, 0:2] = h16(d_bits, (M, nb))
    b[:, :, 2:4] = h16(dmin_bits, (M, nb))
    b[:, :, 4:16] = enc_q4_k_scales(sc, m)
    q = q.reshape(M, nb, 4, 2, 32).astype(np.uint8)  # (pair g, parity, l)
    b[:, :, 16:] = (q[:, :, :, 0, :] | (q[:, :, :, 1, :] << 4)).reshape(M, nb, 128)
    return b.reshape(M, -1)


def enc_q6_k(q, sc, d_bits=ONE):
    M, K = q.shape
    nb = K // 256
    q = q.reshape(M, nb, 2, 4, 32).astype(np.uint8)  # (half, quarter, l)
    b = np.zeros((M, nb, 210), np.uint8)
    lo, hi = q & 15, q >> 4
    ql = np.zeros((M, nb, 2, 64), np.uint8)
    ql[..., 0:32] = lo[:, :, :, 0] | (lo[:, :, :, 2] << 4)
    ql[..., 32:64] = lo[:, :, :, 1] | (lo[:, :, :, 3] << 4)
    qh = hi[:, :, :, 0] | (hi[:, :, :, 1] << 2) | (hi[:, :, :, 2] << 4) | (hi[:, :, :, 3] << 6)
    b[:, :, 0:128] = ql.reshape(M, nb, 128)
    b[:, :, 128:192] = qh.reshape(M, nb, 64)
    b[:, :, 192:208] = sc.astype(np.int8).view(np.uint8)
    b[:, :, 208:210] = h16(d_bits, (M, nb))
    return b.reshape(M, -1)


def enc_q8_k(q, d=1.0):
    N, K = q.shape
    nb = K // 256
    b = np.zeros((N, nb, 292), np.uint8)
    b[:, :, 0:4] = np.full((N, nb), d, np.float32).view(np.uint8).reshape(N, nb, 4)
    b[:, :, 4:260] = q.astype(np.int8).reshape(N, nb, 256).view(np.uint8)
    b[:, :, 260:] = q.astype(np.int16).reshape(N, nb, 16, 16).sum(axis=3).astype(np.int16) \
        .view(np.uint8).reshape(N, nb, 32)
    return b.reshape(N, -1)


# ------------------------------------------------- printed worked example

@pytest.mark.parametrize("wtype", [O.Q8_0, O.Q4_0, O.Q4_K, O.Q6_K])
def test_ggml_simple_example(golden, wtype):
    g = golden("ggml_simple_mul_mat.json")
    A = np.array(g["A"])      # M x 2
    BT = np.array(g["B_T"])   # N x 2
    CT = np.array(g["C_T"])   # N x M
    M, N = A.shape[0], BT.shape[0]
    K = O.BLOCK_SIZE[wtype]
    Ap = np.zeros((M, K), np.int64)
    Ap[:, :2] = A
    Bp = np.zeros((N, K), np.int64)
    Bp[:, :2] = BT
    if wtype == O.Q8_0:
        W = enc_q8_0(Ap)
    elif wtype == O.Q4_0:
        W = enc_q4_0(8 - Ap, d_bits=0xBC00)  # w = -1 * (q - 8) = A
    elif wtype == O.Q4_K:
        nb = K // 256
        W = enc_q4_k(Ap, np.ones((M, nb, 8)), np.zeros((M, nb, 8)))
    else:
        nb = K // 256
        W = enc_q6_k(Ap + 32, np.ones((M, nb, 16)))
    X = enc_q8_0(Bp) if O.VEC_DOT_TYPE[wtype] == O.Q8_0 else enc_q8_k(Bp)
    y, T = O.mul_mat(wtype, W, X, M, N, K)
    assert np.array_equal(y, CT.astype(np.float64))
    assert np.array_equal(O.mul_mat_blockwise(wtype, W, X, M, N, K), CT.astype(np.float64))
    assert np.array_equal(T, np.abs(Bp) @ np.abs(Ap).T)


# ------------------------------------- integer cases vs numpy int64 matmul

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_integer_cases_match_int_matmul(seed):
    g = np.random.default_rng(100 + seed)
    M, N = 7, 5
    # Q8_0 x Q8_0, d = 1 on both sides
    K = 32 * int(g.integers(1, 17))
    qw = g.integers(-128, 128, (M, K))
    qx = g.integers(-127, 128, (N, K))
    y, T = O.mul_mat(O.Q8_0, enc_q8_0(qw), enc_q8_0(qx), M, N, K)
    assert np.array_equal(y, (qx @ qw.T).astype(np.float64))
    assert np.array_equal(T, (np.abs(qx) @ np.abs(qw).T).astype(np.float64))
    # Q4_0: w = q - 8
    qn = g.integers(0, 16, (M, K))
    y, T = O.mul_mat(O.Q4_0, enc_q4_0(qn), enc_q8_0(qx), M, N, K)
    assert np.array_equal(y, (qx @ (qn - 8).T).astype(np.float64))
    assert np.array_equal(T, (np.abs(qx) @ np.abs(qn - 8).T).astype(np.float64))
    # Q5_0: w = q - 16, q = low nibble | fifth bit << 4
    q5 = g.integers(0, 32, (M, K))
    y, _ = O.mul_mat(O.Q5_0, enc_q5_0(q5), enc_q8_0(qx), M, N, K)
    assert np.array_equal(y, (qx @ (q5 - 16).T).astype(np.float64))
    assert np.array_equal(O.q5_0_quant_n(enc_q5_0(q5)).reshape(M, K), q5)
    # Q4_K with d = dmin = 1 and random 6-bit scales and mins: w = sc q - m
    K = 256 * int(g.integers(1, 4))
    nb = K // 256
    q = g.integers(0, 16, (M, K))
    sc = g.integers(0, 64, (M, nb, 8))
    mn = g.integers(0, 64, (M, nb, 8))
    w = np.repeat(sc.reshape(M, -1), 32, axis=1) * q - np.repeat(mn.reshape(M, -1), 32, axis=1)
    qx = g.integers(-127, 128, (N, K))
    W = enc_q4_k(q, sc, mn)
    X = enc_q8_k(qx)
    y, T = O.mul_mat(O.Q4_K, W, X, M, N, K)
    assert np.array_equal(y, (qx @ w.T).astype(np.float64))
    # term sum: the scale part sc q and the min part m count separately
    t_w = np.repeat(sc.reshape(M, -1), 32, axis=1) * q + np.repeat(mn.reshape(M, -1), 32, axis=1)
    assert np.array_equal(T, (np.abs(qx) @ t_w.T).astype(np.float64))
    assert np.array_equal(O.mul_mat_blockwise(O.Q4_K, W, X, M, N, K), (qx @ w.T).astype(np.float64))
    assert np.array_equal(O.dequantize(O.Q4_K, W, M, K), w.astype(np.float32))
    # Q6_K with d = 1 and random int8 scales over the full range: w = sc (q - 32)
    q6 = g.integers(0, 64, (M, K))
    sc6 = g.integers(-128, 128, (M, nb, 16))
    w6 = np.repeat(sc6.reshape(M, -1), 16, axis=1) * (q6 - 32)
    W6 = enc_q6_k(q6, sc6)
    y, T = O.mul_mat(O.Q6_K, W6, X, M, N, K)
    assert np.array_equal(y, (qx @ w6.T).astype(np.float64))
    assert np.array_equal(T, (np.abs(qx) @ np.abs(w6).T).astype(np.float64))
    assert np.array_equal(O.mul_mat_blockwise(O.Q6_K, W6, X, M, N, K), (qx @ w6.T).astype(np.float64))
    assert np.array_equal(O.dequantize(O.Q6_K, W6, M, K), w6.astype(np.float32))


# ------------------------------- block formula vs plain definition (fp64)

def _random_case(g, wtype, M, N, K):
    if wtype == O.Q4_K:
        W = synth.q4_k_random(g, M, K)
    elif wtype == O.Q6_K:
        W = synth.q6_k_random(g, M, K)
    elif wtype == O.Q5_0:
        W = synth.q5_0_random(g, M, K)
    else:
        W = O.quantize(wtype, synth.normal_f32(g, (M, K), 0.02))
    X = O.quantize(O.VEC_DOT_TYPE[wtype], synth.normal_f32(g, (N, K), 1.0))
    return W, X


@pytest.mark.parametrize("wtype", [O.Q8_0, O.Q4_0, O.Q4_K, O.Q6_K, O.Q5_0])
def test_blockwise_matches_definition(wtype):
    g = np.random.default_rng(31)
    for M, N, K in ((33, 3, 256), (9, 8, 1024), (1, 1, 256), (64, 17, 512)):
        W, X = _random_case(g, wtype, M, N, K)
        y, T = O.mul_mat(wtype, W, X, M, N, K)
        yb = O.mul_mat_blockwise(wtype, W, X, M, N, K)
        assert np.all(np.abs(y - yb) <= 1e-12 * T)
        # numpy fp64 matmul on the exact dequantized values
        Wd = O.dequantize(wtype, W, M, K, f64=True)
        Xd = O.dequantize(O.VEC_DOT_TYPE[wtype], X, N, K, f64=True)
        assert np.all(np.abs(y - Xd @ Wd.T) <= 1e-12 * T)
        Tn = np.abs(Xd) @ np.abs(Wd).T
        if wtype == O.Q4_K:
            assert np.all(T >= Tn * (1 - 1e-12))   # |a - b| <= |a| + |b|
        else:
            assert np.allclose(T, Tn, rtol=1e-12, atol=0)
        assert np.all(np.abs(y) <= T * (1 + 1e-12))


@pytest.mark.parametrize("wtype", [O.Q8_0, O.Q4_0, O.Q4_K, O.Q6_K, O.Q5_0])
def test_linear_in_activation_scale(wtype):
    g = np.random.default_rng(37)
    M, N, K = 16, 2, 512
    W, X = _random_case(g, wtype, M, N, K)
    X2 = X.copy()
    if O.VEC_DOT_TYPE[wtype] == O.Q8_0:
        bl = X2.reshape(N, -1, 34)
        d = bl[:, :, 0:2].copy().view(np.float16) * np.float16(2)
        bl[:, :, 0:2] = d.view(np.uint8)
    else:
        bl = X2.reshape(N, -1, 292)
        d = bl[:, :, 0:4].copy().view(np.float32) * np.float32(2)
        bl[:, :, 0:4] = d.view(np.uint8)
    y1, _ = O.mul_mat(wtype, W, X, M, N, K)
    y2, _ = O.mul_mat(wtype, W, X2, M, N, K)
    assert np.array_equal(y2, 2 * y1)


def test_zero_activation_gives_zero_output():
    g = np.random.default_rng(41)
    W = synth.q4_k_random(g, 5, 512)
    X = O.quantize(O.Q8_K, np.zeros((2, 512), np.float32))
    y, T = O.mul_mat(O.Q4_K, W, X, 5, 2, 512)
    assert np.all(y == 0) and np.all(T == 0)


def test_thread_count_does_not_change_results():
    # the oracle parallelises over weight rows only: one thread and many give
    # the same bits (timing control, no arithmetic effect)
    g = np.random.default_rng(7)
    M, N, K = 37, 3, 512
    W = O.quantize(O.Q4_0, g.standard_normal((M, K), dtype=np.float32))
    xq = O.quantize(O.Q8_0, g.standard_normal((N, K), dtype=np.float32))
    n = O.num_threads()
    y1, T1 = O.mul_mat(O.Q4_0, W, xq, M, N, K)
    O.set_num_threads(1)
    try:
        y2, T2 = O.mul_mat(O.Q4_0, W, xq, M, N, K)
    finally:
        O.set_num_threads(n)
    assert O.num_threads() == n
    assert np.array_equal(y1.view(np.uint64), y2.view(np.uint64))
    assert np.array_equal(T1.view(np.uint64), T2.view(np.uint64))
