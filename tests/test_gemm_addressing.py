"""Host-side check of the Q4_K GEMM's operand staging (gemm_q4k_kernel in
block_quantized_amd/csrc/gemm.hip): every byte a buffer read takes from
global memory lies inside an activation (or weight) row that exists, rows
past N (or M) read as zeros (the buffer descriptor's range check, which
covers the lane offset only), and the LDS stores of those reads fill the
tiles exactly as the operand reads expect.

The kernel's workgroup holds KS groups of W waves over a tile of BN = 32 TN
activation rows; per super-block each wave reads (and stores to LDS)
  - codes: instructions i = w + W k (k < 8 TN / W), each one 16-byte-per-lane
    copy of tile rows 4 i + lane/16 (row 4 (i%4) + lane/16 of 16-row group
    i/4), position lane%16 of the row, which receives chunk
    (lane%16) ^ (row & 15) of the row's 256 codes;
  - sums: 32-row group g2 = (w + W k) % TN for k < max(1, TN/W): lane l
    copies 16 bytes (half l%2) of row 32 g2 + l/2's sixteen int16 sums;
  - scales: 64-row group g4 = (w + W k) % (TN/2) for k < max(1, TN/2/W):
    lane l copies row 64 g4 + l's d.
One descriptor starts at the tile's first row n0 and holds min(BN, N - n0)
rows; each copy's lane offset holds its row, the super-block and the bytes
within the record (the scalar offset is 0).  This restates those formulas in plain Python, so that a change to
either that breaks a bound fails here, on the CPU, rather than on the GPU.
"""
import pytest

Q8K = 292
CONFIGS = [(4, 8, 1), (2, 4, 2), (2, 4, 1), (4, 4, 1), (4, 2, 2), (2, 8, 1), (4, 1, 1)]  # (TN, W, KS) the launcher uses


def copies(TN, W, N, K, n0, wave, sb):
    """(kind, lds_row, lds_pos, global_row or None, byte offset within the row, size, what) per lane."""
    rowsB = K // 256 * Q8K
    BN = 32 * TN
    so = sb * Q8K
    nrec = min(BN, N - n0) * rowsB  # one descriptor for the tile's rows, based at row n0

    def lane_copy(kind, lds_row, pos, vo, size, what):
        # vo is the whole offset from the descriptor base (row, super-block,
        # bytes); the range check covers it
        if vo + size <= nrec:
            return (kind, lds_row, pos, n0 + vo // rowsB, vo % rowsB, size, what)
        return (kind, lds_row, pos, None, None, size, what)

    out = []
    for k in range(8 * TN // W):
        i = wave + W * k
        for lane in range(64):
            row = 4 * i + lane // 16
            pos = lane % 16
            chunk = pos ^ (row & 15)
            out.append(lane_copy("codes", row, pos, row * rowsB + 4 + 16 * chunk + so, 16, chunk))
    for k in range(max(1, TN // W)):
        g2 = (wave + W * k) % TN
        for lane in range(64):
            row, half = lane // 2, lane % 2
            out.append(lane_copy("sums", 32 * g2 + row, half, (32 * g2 + row) * rowsB + 260 + 16 * half + so, 16, half))
    for k in range(max(1, TN // 2 // W)):
        g4 = (wave + W * k) % (TN // 2)
        for lane in range(64):
            out.append(lane_copy("dx", 64 * g4 + lane, 0, (64 * g4 + lane) * rowsB + so, 4, 0))
    return out


@pytest.mark.parametrize("TN,W,KS", CONFIGS)
@pytest.mark.parametrize("N,K", [(512, 4096), (33, 256), (65, 512), (129, 768), (200, 1024), (100, 2304), (1, 256)])
def test_copies_stay_in_rows_and_fill_the_tile(TN, W, KS, N, K):
    if (K // 256) % KS:
        pytest.skip("the launcher splits K only when the super-blocks divide evenly")
    BN = 32 * TN
    rowsB = K // 256 * Q8K
    SB = K // 256
    for cb in range((N + BN - 1) // BN):
        n0 = cb * BN
        for kp in range(KS):
            for sb in (kp * (SB // KS), (kp + 1) * (SB // KS) - 1):
                got = {}
                for wave in range(W):
                    for kind, lrow, pos, grow, off, size, what in copies(TN, W, N, K, n0, wave, sb):
                        assert 0 <= lrow < BN, (kind, lrow)
                        if grow is None:
                            assert n0 + lrow >= N, f"{kind}: existing row {n0 + lrow} read as zero"
                            val = None
                        else:
                            assert grow == n0 + lrow and grow < N, (kind, grow, N)
                            # inside the row's bytes, and inside super-block sb
                            assert sb * Q8K <= off and off + size <= (sb + 1) * Q8K <= rowsB, (kind, off)
                            val = (grow, off)
                        key = (kind, lrow, pos)
                        # a slot written twice must receive the same bytes
                        assert got.setdefault(key, val) == val, key
                        if kind == "codes":
                            assert val is None or off - sb * Q8K == 4 + 16 * what
                # every LDS slot of the tile is written: codes, sums, scales
                for r in range(BN):
                    for p in range(16):
                        assert ("codes", r, p) in got
                    assert ("sums", r, 0) in got and ("sums", r, 1) in got
                    assert ("dx", r, 0) in got


Q4K = 144
WAVE_REGION = 5 * 64 * 16


def weight_copies(M, K, m0, sb):
    """(lds offset in the wave's region, global byte offset or None) per lane
    of the 5 weight-copy instructions of the wave whose rows start at m0."""
    wrowB = K // 256 * Q4K
    rows = max(0, min(32, M - m0))
    nrec = rows * wrowB  # descriptor based at row min(m0, M - 1)
    base_row = min(m0, M - 1)
    out = []
    for k in range(5):
        for lane in range(64):
            ch = (64 * k + lane) % 288
            vo = (ch // 9) * wrowB + 16 * (ch % 9) + sb * Q4K
            lds = 1024 * k + 16 * lane
            g = (base_row * wrowB + vo) if vo + 16 <= nrec else None
            out.append((lds, ch, g))
    return out


@pytest.mark.parametrize("M,K", [(14336, 4096), (4096, 4096), (33, 256), (100, 2304), (1, 256), (300, 768)])
def test_weight_copies_stay_in_rows_and_fill_the_region(M, K):
    wrowB = K // 256 * Q4K
    for m0 in range(0, M + 64, 32):
        if m0 >= M + 32:
            break
        for sb in {0, K // 256 - 1}:
            seen = {}
            for lds, ch, g in weight_copies(M, K, m0, sb):
                assert 0 <= lds and lds + 16 <= WAVE_REGION
                row, part = ch // 9, ch % 9
                if lds < 32 * Q4K:
                    # bytes the kernel reads: chunk (row, part) of super-block sb
                    assert lds == row * Q4K + 16 * part
                if g is None:
                    assert m0 + row >= M, "an existing weight row read as zero"
                else:
                    assert m0 + row < M and g == (m0 + row) * wrowB + sb * Q4K + 16 * part
                    assert g + 16 <= M * wrowB
                assert seen.setdefault(lds, g) == g
            for r in range(32):
                for part in range(9):
                    assert r * Q4K + 16 * part in seen
