"""Helpers shared by the GPU parity tests (no product arithmetic here)."""
import numpy as np


def dev():
    import torch
    return torch.device("cuda:0")


def to_gpu(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_cpu(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_bytes_equal(got, want, what=""):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        diff = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
        raise AssertionError(f"{what}: {diff.size} bytes differ, first at {diff[:8]}")


def assert_f32_bits_equal(got, want, what=""):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), what
    g = got[~nan].view(np.uint32)
    w = want[~nan].view(np.uint32)
    if not np.array_equal(g, w):
        i = np.nonzero(g != w)[0]
        raise AssertionError(f"{what}: {i.size} values differ, first {got[~nan][i[:4]]} vs {want[~nan][i[:4]]}")


def assert_within_tolerance(y, y_ref, T, rel=1e-5, what=""):
    """|y - y_ref| <= rel * T per output; where T == 0 the output must be 0."""
    y = np.asarray(y, np.float64)
    err = np.abs(y - y_ref)
    bad = err > rel * T
    if bad.any():
        i = np.argwhere(bad)[:4]
        raise AssertionError(f"{what}: {bad.sum()} outputs out of tolerance; e.g. at {i.tolist()}: "
                             f"got {y[tuple(i.T)]}, want {y_ref[tuple(i.T)]}, T {T[tuple(i.T)]}")


def tile_rows(M, tile=32, seed=0):
    """One row from every `tile`-row block of the M weight rows (a random
    offset inside each block), plus the first and last rows: every row tile
    of every product kernel (16, 32, 64 or 128 rows) contributes a row."""
    g = np.random.default_rng(seed)
    starts = np.arange(0, M, tile)
    span = np.minimum(tile, M - starts)
    r = starts + (g.random(starts.size) * span).astype(np.int64)
    return np.unique(np.concatenate([[0, M - 1], r]))


def run_product(wt, W, xq, M, N, K, algo=0):
    """y = W x^T on the GPU through the C ABI, into an output that starts as
    NaN with a NaN canary behind it: every output must have been written
    (finite) and nothing past y.  Returns y (N, M) on the host."""
    import torch
    import block_quantized_amd as Q
    Wg = W if isinstance(W, torch.Tensor) else to_gpu(W)
    xg = xq if isinstance(xq, torch.Tensor) else to_gpu(xq)
    buf = torch.full((N * M + 256,), float("nan"), dtype=torch.float32, device=dev())
    rc = Q.qmm_mul_mat_algo(wt, Wg, xg, buf, M, N, K, algo)
    assert rc == Q.QMM_OK, Q.qmm_strerror(rc)
    b = to_cpu(buf)
    assert np.all(np.isnan(b[N * M:])), "wrote past the end of y"
    y = b[:N * M].reshape(N, M)
    bad = ~np.isfinite(y)
    if bad.any():
        i = np.argwhere(bad)[:4]
        raise AssertionError(f"{bad.sum()} outputs not written (or not finite), e.g. (n, m) = {i.tolist()}")
    return y
