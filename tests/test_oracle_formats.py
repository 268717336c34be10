"""Pins the oracle's block decoders.

Sources: page 'The GGML ecosystem, and where synapse fits', section 5
'Quantization' (format table).  The pages give each format's fields, byte
count and (for Q4_0, Q8_0, Q4_K) element formula; they do not print the bit
arrangement inside a block.  The arrangement used is GGUF's on-disk one (the
reading recorded in the oracle's header), and these tests pin the decoders to
it three independent ways:
  1. sizes and bits per weight printed on the pages;
  2. hand-worked blocks (tests/golden/hand_blocks.json);
  3. structural invariants: every stored bit feeds exactly one field bit
     (single-bit flips), each field's source bits follow a bit-position
     table, swept exhaustively over every byte pair that feeds a field.
"""
import numpy as np
import pytest

import oracle as O

NAMES = {"Q4_0": O.Q4_0, "Q8_0": O.Q8_0, "Q4_K": O.Q4_K, "Q6_K": O.Q6_K, "Q8_K": O.Q8_K, "Q5_0": O.Q5_0}


def fp16_bytes(bits):
    return np.array([bits], np.uint16).view(np.uint8)


# --------------------------------------------------------------- sizes, bpw

def test_format_table_sizes(golden):
    g = golden("format_table.json")
    for name, f in g["formats"].items():
        t = NAMES[name]
        assert O.lib().orc_block_size(t) == f["block_size"]
        assert O.lib().orc_block_bytes(t) == f["block_bytes"]
        assert O.BLOCK_SIZE[t] == f["block_size"] and O.BLOCK_BYTES[t] == f["block_bytes"]
    # bits per weight printed on the pages
    bpw = {n: 8 * f["block_bytes"] / f["block_size"] for n, f in g["formats"].items()}
    assert bpw["Q4_K"] == g["bits_per_weight"]["Q4_K"]
    assert bpw["Q4_0"] == 4.5
    assert bpw["Q5_0"] == 5.5   # 2 + 4 + 16 bytes per 32
    assert abs(bpw["Q8_0"] - g["bits_per_weight"]["Q8_0"]) < 1e-12
    lo, hi = g["k_quant_bpw_range"]
    assert lo <= bpw["Q6_K"] <= hi and lo <= bpw["Q4_K"] <= hi
    # field sums: Q4_0 2+16, Q8_0 2+32, Q4_K 2+2+12+128, Q6_K 128+64+16+2, Q8_K 4+256+32
    assert (2 + 32 // 2, 2 + 32, 4 + 12 + 256 // 2, 256 // 2 + 256 // 4 + 16 + 2, 4 + 256 + 2 * 16) == \
        (18, 34, 144, 210, 292)


# ------------------------------------------------------- hand-worked blocks

def test_hand_q4_0(golden):
    h = golden("hand_blocks.json")["q4_0"]
    blk = np.zeros(18, np.uint8)
    blk[0:2] = fp16_bytes(h["d_fp16_bits"])
    blk[2:18] = 0x80 | np.arange(16)
    w = O.dequantize(O.Q4_0, blk, 1, 32)[0]
    assert w.tolist() == h["w"]
    x = np.zeros(34, np.uint8)
    x[0:2] = fp16_bytes(0x3C00)
    x[2:] = 1
    y, T = O.mul_mat(O.Q4_0, blk, x, 1, 1, 32)
    assert y[0, 0] == h["dot_with_q8_0_d1_all_ones"]
    assert O.mul_mat_blockwise(O.Q4_0, blk, x, 1, 1, 32)[0, 0] == h["dot_with_q8_0_d1_all_ones"]
    assert T[0, 0] == sum(abs(v) for v in h["w"])


@pytest.mark.parametrize("which", ["a", "b"])
def test_hand_q5_0(golden, which):
    h = golden("hand_blocks.json")["q5_0"][which]
    blk = np.zeros(22, np.uint8)
    blk[0:2] = fp16_bytes(h["d_fp16_bits"])
    blk[2:6] = np.array([h["qh"]], "<u4").view(np.uint8)
    if h["qs_rule"] == "qs[j] = 0x80 | j":
        blk[6:22] = 0x80 | np.arange(16)
    w = O.dequantize(O.Q5_0, blk, 1, 32)[0]
    assert w.tolist() == h["w"]
    x = np.zeros(34, np.uint8)
    x[0:2] = fp16_bytes(0x3C00)
    x[2:] = 1
    y, T = O.mul_mat(O.Q5_0, blk, x, 1, 1, 32)
    assert y[0, 0] == h["dot_with_q8_0_d1_all_ones"]
    assert O.mul_mat_blockwise(O.Q5_0, blk, x, 1, 1, 32)[0, 0] == h["dot_with_q8_0_d1_all_ones"]
    assert T[0, 0] == sum(abs(v) for v in h["w"])


def q4k_block(h):
    blk = np.zeros(144, np.uint8)
    blk[0:2] = fp16_bytes(h["d_fp16_bits"])
    blk[2:4] = fp16_bytes(h["dmin_fp16_bits"])
    blk[4:16] = h["scales"]
    blk[16:] = h["qs_byte"]
    return blk


def test_hand_q4_k(golden):
    h = golden("hand_blocks.json")["q4_k"]
    blk = q4k_block(h)
    for j, (sc, m) in enumerate(h["sc_m"]):
        assert O.q4k_scale_min(blk[4:16], j) == (sc, m)
    w = O.dequantize(O.Q4_K, blk, 1, 256)[0]
    assert np.array_equal(w, np.repeat(np.array(h["w_per_subblock"], np.float32), 32))
    x = np.zeros(292, np.uint8)
    x[0:4] = np.array([1.0], np.float32).view(np.uint8)
    x[4:260] = 1
    x[260:] = np.full(16, 16, np.int16).view(np.uint8)
    y, T = O.mul_mat(O.Q4_K, blk, x, 1, 1, 256)
    assert y[0, 0] == h["dot_with_q8_k_d1_all_ones"]
    # the tolerance's term sum counts the scale part and the min part apart
    assert T[0, 0] == h["term_sum_with_q8_k_d1_all_ones"]
    assert O.mul_mat_blockwise(O.Q4_K, blk, x, 1, 1, 256)[0, 0] == h["dot_with_q8_k_d1_all_ones"]
    hb = h["high_bits_case"]
    blk[4 + 0] = hb["scales_0"]
    blk[4 + 4] = hb["scales_4"]
    assert O.q4k_scale_min(blk[4:16], 4) == tuple(hb["sc_m_4"])
    assert O.q4k_scale_min(blk[4:16], 0) == tuple(h["sc_m"][0])


def test_hand_q6_k(golden):
    h = golden("hand_blocks.json")["q6_k"]
    blk = np.zeros(210, np.uint8)
    blk[0:128] = h["ql_byte"]
    blk[128:192] = h["qh_byte"]
    blk[192:208] = np.array(h["scales"], np.int8).view(np.uint8)
    blk[208:210] = fp16_bytes(h["d_fp16_bits"])
    q = O.q6k_quant_n(blk)[0].astype(int) - 32
    quarters = np.array(h["q_minus_32_per_quarter"])
    assert np.array_equal(q, np.tile(np.repeat(quarters, 32), 2))
    w = O.dequantize(O.Q6_K, blk, 1, 256)[0]
    for e, v in h["w_at"].items():
        assert w[int(e)] == v
    assert w.astype(np.float64).sum() == h["sum_w"]


# ------------------------------------------------- bit-position invariants

def _flip_test(decode, nbytes, field_of_bit):
    """For random base blocks, flip every bit in turn; exactly one decoded
    field must change, by +-2^k, and it must be the one the table names."""
    g = np.random.default_rng(7)
    for _ in range(4):
        base = g.integers(0, 256, nbytes, dtype=np.uint8)
        f0 = decode(base[None])[0].astype(np.int64)
        flips = np.repeat(base[None], nbytes * 8, axis=0)
        for bit in range(nbytes * 8):
            flips[bit, bit // 8] ^= np.uint8(1 << (bit % 8))
        f1 = decode(flips).astype(np.int64)
        for bit in range(nbytes * 8):
            diff = np.nonzero(f1[bit] != f0)[0]
            want = field_of_bit(bit)
            if want is None:
                assert diff.size == 0, bit
                continue
            field, k = want
            assert diff.tolist() == [field], (bit, diff, want)
            assert abs(f1[bit, field] - f0[field]) == 1 << k, (bit, want)


def q4k_scale_source_table():
    """(byte, bit) -> (field index, field bit) for the 12 scale bytes.
    Fields 0..7 are sc_0..sc_7, fields 8..15 are m_0..m_7."""
    t = {}
    for j in range(4):
        for k in range(6):
            t[(j, k)] = (j, k)              # sc_j low six bits of byte j
            t[(j + 4, k)] = (8 + j, k)      # m_j  low six bits of byte j+4
    for j in range(4, 8):
        for k in range(4):
            t[(j + 4, k)] = (j, k)          # sc_j bits 0-3: low nibble of byte j+4
            t[(j + 4, 4 + k)] = (8 + j, k)  # m_j  bits 0-3: high nibble of byte j+4
        for k in range(2):
            t[(j - 4, 6 + k)] = (j, 4 + k)  # sc_j bits 4-5: top bits of byte j-4
            t[(j, 6 + k)] = (8 + j, 4 + k)  # m_j  bits 4-5: top bits of byte j
    return t


def test_q4k_scale_bits_bijective_and_placed():
    t = q4k_scale_source_table()
    assert len(t) == 96 and len(set(t.values())) == 96  # table is a bijection

    def decode(s):
        sc, m = O.q4k_scale_min_n(s)
        return np.concatenate([sc, m], axis=1)

    _flip_test(decode, 12, lambda bit: t[(bit // 8, bit % 8)])


def _q4k_fields_from_table(s):
    t = q4k_scale_source_table()
    out = np.zeros((s.shape[0], 16), np.int64)
    for (byte, bit), (field, k) in t.items():
        out[:, field] |= ((s[:, byte].astype(np.int64) >> bit) & 1) << k
    return out


def test_q4k_scale_exhaustive_byte_pairs():
    # Every field reads at most two bytes; sweep all 65536 values of each such
    # pair with the other ten bytes random.
    g = np.random.default_rng(11)
    pairs = [(j, j + 4) for j in range(4)] + [(j + 4, j - 4) for j in range(4, 8)] + \
            [(j + 4, j) for j in range(4, 8)]
    a, b = np.meshgrid(np.arange(256), np.arange(256), indexing="ij")
    for p, q in pairs:
        s = g.integers(0, 256, (65536, 12), dtype=np.uint8)
        s[:, p] = a.ravel()
        s[:, q] = b.ravel()
        sc, m = O.q4k_scale_min_n(s)
        assert np.array_equal(np.concatenate([sc, m], axis=1), _q4k_fields_from_table(s))


def q4k_qs_source(bit):
    """bit of the 128 qs bytes -> (element, bit of its 4-bit quant)."""
    byte, k = bit // 8, bit % 8
    g, l = byte // 32, byte % 32
    j = 2 * g + (1 if k >= 4 else 0)
    return 32 * j + l, k % 4


def test_q4k_quant_bits():
    def decode(qs):
        n = qs.shape[0]
        blk = np.zeros((n, 144), np.uint8)
        blk[:, 0:2] = fp16_bytes(0x3C00)  # d = 1
        blk[:, 4:8] = 1                   # sc_0..3 = 1, m_0..3 = 0
        blk[:, 12:16] = 1                 # sc_4..7 = 1, m_4..7 = 0
        blk[:, 16:] = qs
        return O.dequantize(O.Q4_K, blk, n, 256).astype(np.int64)

    _flip_test(decode, 128, q4k_qs_source)


def q6k_source(bit):
    """bit of ql (bytes 0-127) or qh (bytes 128-191) -> (element, q bit)."""
    byte, k = bit // 8, bit % 8
    if byte < 128:
        h, r = byte // 64, byte % 64
        c = (r // 32) + (2 if k >= 4 else 0)
        return 128 * h + 32 * c + r % 32, k % 4
    if byte < 192:
        h, l = (byte - 128) // 32, (byte - 128) % 32
        c = k // 2
        return 128 * h + 32 * c + l, 4 + k % 2
    return None


def test_q6k_quant_bits():
    seen = {q6k_source(b) for b in range(192 * 8)}
    assert len(seen) == 256 * 6  # every (element, bit) fed exactly once
    _flip_test(lambda b: O.q6k_quant_n(np.pad(b, ((0, 0), (0, 210 - b.shape[1])))), 192, q6k_source)


def test_q6k_exhaustive_byte_pairs():
    # All ql bytes = a and all qh bytes = b, for all 65536 (a, b): every
    # element's quant is then the nibble and bit pair its class selects.
    a, b = np.meshgrid(np.arange(256, dtype=np.uint8), np.arange(256, dtype=np.uint8), indexing="ij")
    blk = np.zeros((65536, 210), np.uint8)
    blk[:, :128] = a.ravel()[:, None]
    blk[:, 128:192] = b.ravel()[:, None]
    q = O.q6k_quant_n(blk).astype(np.int64)
    A = a.ravel().astype(np.int64)[:, None]
    B = b.ravel().astype(np.int64)[:, None]
    e = np.arange(256)[None, :]
    c = (e % 128) // 32
    want = np.where(c < 2, A & 15, A >> 4) | (((B >> (2 * c)) & 3) << 4)
    assert np.array_equal(q, want)


def test_q4_0_bits():
    def decode(qs):
        n = qs.shape[0]
        blk = np.zeros((n, 18), np.uint8)
        blk[:, 0:2] = fp16_bytes(0x3C00)
        blk[:, 2:] = qs
        return O.dequantize(O.Q4_0, blk, n, 32).astype(np.int64)

    _flip_test(decode, 16, lambda bit: ((bit // 8) + (16 if bit % 8 >= 4 else 0), bit % 4))


def test_q5_0_bits():
    # qh bit e moves element e by 16; qs bit b of byte j moves element j
    # (b < 4) or j + 16 (b >= 4) by 2^(b % 4); the scale bytes are left alone
    def decode(raw):
        n = raw.shape[0]
        blk = np.zeros((n, 22), np.uint8)
        blk[:, 0:2] = fp16_bytes(0x3C00)
        blk[:, 2:] = raw
        return O.dequantize(O.Q5_0, blk, n, 32).astype(np.int64)

    def field(bit):
        byte, b = bit // 8, bit % 8
        if byte < 4:
            return (8 * byte + b, 4)
        j = byte - 4
        return (j + (16 if b >= 4 else 0), b % 4)

    _flip_test(decode, 20, field)


# ------------------------------------- fp32 dequantizer = exact value rounded

@pytest.mark.parametrize("t", [O.Q4_0, O.Q8_0, O.Q4_K, O.Q6_K, O.Q8_K, O.Q5_0])
def test_f32_dequant_is_correctly_rounded_exact_value(t):
    # Each fp32 element has at most one rounding from exact operands, so it
    # must equal the exact (fp64) value rounded once to fp32.  Q4_0, Q8_0 and
    # Q6_K elements are exact in fp32 outright.
    g = np.random.default_rng(3)
    rows, K = 64, 512
    blocks = g.integers(0, 256, (rows, O.row_bytes(t, K)), dtype=np.uint8)
    nb = K // O.BLOCK_SIZE[t]
    S = O.BLOCK_BYTES[t]
    bl = blocks.reshape(rows, nb, S)
    # keep scales finite (NaN/Inf scales are not a parity case)
    if t in (O.Q4_0, O.Q8_0, O.Q4_K, O.Q5_0):
        bl[:, :, 1] &= 0x7B
        if t == O.Q4_K:
            bl[:, :, 3] &= 0x7B
    elif t == O.Q6_K:
        bl[:, :, 209] &= 0x7B
    else:
        bl[:, :, 0:4] = (g.standard_normal((rows, nb), dtype=np.float32) * 1e-2).view(np.uint8).reshape(rows, nb, 4)
    f32 = O.dequantize(t, blocks, rows, K)
    f64 = O.dequantize(t, blocks, rows, K, f64=True)
    assert np.array_equal(f32, f64.astype(np.float32))
    if t in (O.Q4_0, O.Q8_0, O.Q6_K, O.Q5_0):
        assert np.array_equal(f32.astype(np.float64), f64)


def test_unit_scale_dequant_equals_integers():
    g = np.random.default_rng(5)
    # Q8_0 with d = 1: w = q
    q = g.integers(-128, 128, (4, 64)).astype(np.int8)
    blk = np.zeros((4, 2, 34), np.uint8)
    blk[:, :, 0:2] = fp16_bytes(0x3C00)
    blk[:, :, 2:] = q.reshape(4, 2, 32).view(np.uint8)
    assert np.array_equal(O.dequantize(O.Q8_0, blk, 4, 64), q.astype(np.float32))
    # Q8_K with d = 1: w = q
    q = g.integers(-127, 128, (2, 256)).astype(np.int8)
    blk = np.zeros((2, 292), np.uint8)
    blk[:, 0:4] = np.array([1.0], np.float32).view(np.uint8)
    blk[:, 4:260] = q.view(np.uint8)
    assert np.array_equal(O.dequantize(O.Q8_K, blk, 2, 256), q.astype(np.float32))
