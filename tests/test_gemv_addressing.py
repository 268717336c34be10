"""Host-side check of the decode GEMV's weight addressing: every byte that
gemv_kernel (block_quantized_amd/csrc/gemv.hip) loads lies inside the
weight matrix of its segment.

The kernel gives each lane one unit of 256 weights; lanes without a unit
re-read their work item's first unit.  Q6_K units (210 bytes, 2-byte
aligned) are read as 14 pieces of 16 bytes from the 4-byte boundary at or
below the unit, which reach up to 14 bytes into the next unit; the work item
that holds a matrix's last unit reads each unit's own last 16 bytes as the
14th piece instead.  This test restates that work split and those byte
ranges in plain Python and checks them against the matrix extent for a
spread of shapes, so that a change to either that breaks the bound fails
here, on the CPU, rather than as a fault on the GPU."""
import pytest

# unit bytes and 16-byte loads per unit, per weight type
UNITS = {"q4_0": (144, 9), "q8_0": (272, 17), "q5_0": (176, 11), "q4_k": (144, 9), "q6_k": (210, 14)}


def split(K):
    GU = K // 256
    Pl = min(GU, 64)
    logP = 0
    while (1 << logP) < Pl:
        logP += 1
    P = 1 << logP
    return GU, P, 64 >> logP, (GU + P - 1) // P


def ranges_read(kind, M, K):
    """Yield (lo, hi) byte ranges, relative to the matrix base, that some lane loads."""
    UB, NV = UNITS[kind]
    GU, P, RW, NKC = split(K)
    rowB = GU * UB
    items = (M + RW - 1) // RW
    for wi in range(items):
        row0 = wi * RW
        for kc in range(NKC):
            tail = row0 + RW >= M and kc == NKC - 1
            for lane in range(64):
                lr, lg = lane // P, lane % P
                gu, row = kc * P + lg, row0 + lr
                valid = gu < GU and lr < RW and row < M
                p = row * rowB + gu * UB if valid else row0 * rowB + kc * P * UB
                if kind == "q6_k":
                    a = p - (p % 4)
                    yield a, a + 16 * (NV - 1)
                    yield (p + UB - 16, p + UB) if tail else (a + 16 * (NV - 1), a + 16 * NV)
                else:
                    yield p, p + 16 * NV


SHAPES = [(1, 256), (2, 256), (3, 768), (7, 256), (33, 512), (257, 768), (65, 16384), (9, 16640),
          (3, 33024), (130, 2304), (300, 4096), (4, 14336), (5, 18176), (1000, 3328)]


@pytest.mark.parametrize("kind", sorted(UNITS))
@pytest.mark.parametrize("M,K", SHAPES)
def test_every_load_stays_inside_the_matrix(kind, M, K):
    UB, _ = UNITS[kind]
    size = M * (K // 256) * UB
    lo = min(r[0] for r in ranges_read(kind, M, K))
    hi = max(r[1] for r in ranges_read(kind, M, K))
    assert lo >= 0
    assert hi <= size, f"{kind} {M}x{K}: reads up to byte {hi} of {size}"


def test_q6_k_pieces_cover_each_unit():
    # the bytes a lane reads cover its whole unit (both skews, tail or not)
    UB, NV = UNITS["q6_k"]
    for p in (0, 210, 420, 630, 3360 - 210):
        a = p - p % 4
        for tail in (False, True):
            got = set(range(a, a + 16 * (NV - 1)))
            got |= set(range(p + UB - 16, p + UB)) if tail else set(range(a + 16 * (NV - 1), a + 16 * NV))
            assert set(range(p, p + UB)) <= got
