"""Test-side block ENCODERS: integer fields -> block bytes, in the GGUF layouts.

These go the opposite way from the oracle's decoders and share nothing with them, so a probe
built here pins where each field lands.  Layouts (GGUF block definitions; the MMQ page gives the
Q4_K size (144 B per 256 values), the half2 (d, dmin), the low/high nibble split per pair of
sub-blocks, and the Q6_K ql/qh bit composition):

  q4_K: d f16 @0, dmin f16 @2, 12 bytes of packed 6-bit (sc, m) @4, qs[128] @16
  q5_K: the q4_K header @0..15, qh[32] @16 (bit j of qh[l] = fifth bit of value 32j + l),
        qs[128] @48 laid out as q4_K's (the pages give Q5_K the Q4_K scale packing)
  q6_K: ql[128] @0, qh[64] @128, int8 scales[16] @192, d f16 @208
  q8_0: d f16 @0, int8 qs[32] @2
  q4_0: d f16 @0, qs[16] @2 (low nibble of qs[i] = value i, high nibble = value i + 16; code q - 8)
  q3_K, iq4_xs: below, beside their encoders (the GP100 patch page names both types, Q3_K's -4
  code offset and IQ4_XS's codebook; the layouts are GGUF's)
"""
import numpy as np


def f16_bits(x):
    return int(np.array([x], dtype=np.float32).astype(np.float16).view(np.uint16)[0])


def _put16(buf, off, bits):
    buf[off] = bits & 0xFF
    buf[off + 1] = (bits >> 8) & 0xFF


def pack_q4_K(d, dmin, sc, m, q):
    """sc, m: 8 ints in [0,63]; q: 256 ints in [0,15] (value index order).  Returns 144 bytes."""
    sc = [int(v) for v in sc]
    m = [int(v) for v in m]
    q = [int(v) for v in q]
    assert len(sc) == 8 and len(m) == 8 and len(q) == 256
    assert all(0 <= v < 64 for v in sc + m) and all(0 <= v < 16 for v in q)
    b = np.zeros(144, dtype=np.uint8)
    _put16(b, 0, f16_bits(d))
    _put16(b, 2, f16_bits(dmin))
    s = [0] * 12
    for j in range(4):
        # sub-blocks 0..3 keep their low 6 bits in bytes 0..3 (scale) and 4..7 (min)
        s[j] |= sc[j] & 63
        s[j + 4] |= m[j] & 63
    for j in range(4, 8):
        # sub-blocks 4..7: low 4 bits in bytes 8..11 (scale low nibble, min high nibble),
        # top 2 bits in the spare top bits of bytes j-4 (scale) and j (min)
        s[j + 4] |= (sc[j] & 15) | ((m[j] & 15) << 4)
        s[j - 4] |= (sc[j] >> 4) << 6
        s[j] |= (m[j] >> 4) << 6
    b[4:16] = s
    for chunk in range(4):                      # 64 values per 32 bytes
        for l in range(32):
            lo = q[64 * chunk + l]              # first sub-block of the pair -> low nibble
            hi = q[64 * chunk + 32 + l]         # second sub-block -> high nibble
            b[16 + 32 * chunk + l] = lo | (hi << 4)
    return b


def pack_q5_K(d, dmin, sc, m, q):
    """sc, m: 8 ints in [0,63]; q: 256 ints in [0,31] (value index order).  Returns 176 bytes."""
    q = [int(v) for v in q]
    assert len(q) == 256 and all(0 <= v < 32 for v in q)
    low = pack_q4_K(d, dmin, sc, m, [v & 15 for v in q])
    b = np.zeros(176, dtype=np.uint8)
    b[0:16] = low[0:16]
    b[48:176] = low[16:144]
    for v in range(256):
        if q[v] >> 4:
            b[16 + v % 32] |= 1 << (v // 32)
    return b


def pack_q6_K(d, sc, q):
    """sc: 16 ints in [-128,127]; q: 256 ints in [0,63] (stored 6-bit values, value index order)."""
    q = [int(v) for v in q]
    assert len(q) == 256 and all(0 <= v < 64 for v in q)
    b = np.zeros(210, dtype=np.uint8)
    for half in range(2):                       # 128 values per half
        for l in range(32):
            v0 = q[128 * half + l]
            v1 = q[128 * half + 32 + l]
            v2 = q[128 * half + 64 + l]
            v3 = q[128 * half + 96 + l]
            b[64 * half + l] = (v0 & 15) | ((v2 & 15) << 4)
            b[64 * half + 32 + l] = (v1 & 15) | ((v3 & 15) << 4)
            b[128 + 32 * half + l] = (v0 >> 4) | ((v1 >> 4) << 2) | ((v2 >> 4) << 4) | ((v3 >> 4) << 6)
    b[192:208] = np.array(sc, dtype=np.int8).view(np.uint8)
    _put16(b, 208, f16_bits(d))
    return b


def pack_q8_0(d, q):
    b = np.zeros(34, dtype=np.uint8)
    _put16(b, 0, f16_bits(d))
    b[2:34] = np.array(q, dtype=np.int8).view(np.uint8)
    return b


def pack_q4_0(d, q):
    """q: 32 ints in [0,15] (stored nibbles, value order).  Returns 18 bytes."""
    q = [int(v) for v in q]
    assert len(q) == 32 and all(0 <= v < 16 for v in q)
    b = np.zeros(18, dtype=np.uint8)
    _put16(b, 0, f16_bits(d))
    for i in range(16):
        b[2 + i] = q[i] | (q[i + 16] << 4)
    return b


def random_q4_0_row(rng, k):
    blocks, fields = [], []
    for _ in range(k // 32):
        d = f16_value(rng.uniform(0.001, 0.02))
        q = rng.integers(0, 16, 32)
        blocks.append(pack_q4_0(d, q))
        fields.append((d, q))
    return np.concatenate(blocks), fields


def f16_value(x):
    return float(np.float32(x).astype(np.float16))


def random_q4_K_row(rng, k):
    """Returns (bytes, fields) for one row of k values."""
    blocks, fields = [], []
    for _ in range(k // 256):
        d = f16_value(rng.uniform(0.001, 0.02))
        dmin = f16_value(rng.uniform(0.001, 0.02))
        sc = rng.integers(0, 64, 8)
        m = rng.integers(0, 64, 8)
        q = rng.integers(0, 16, 256)
        blocks.append(pack_q4_K(d, dmin, sc, m, q))
        fields.append((d, dmin, sc, m, q))
    return np.concatenate(blocks), fields


def random_q5_K_row(rng, k):
    blocks, fields = [], []
    for _ in range(k // 256):
        d = f16_value(rng.uniform(0.001, 0.02))
        dmin = f16_value(rng.uniform(0.001, 0.02))
        sc = rng.integers(0, 64, 8)
        m = rng.integers(0, 64, 8)
        q = rng.integers(0, 32, 256)
        blocks.append(pack_q5_K(d, dmin, sc, m, q))
        fields.append((d, dmin, sc, m, q))
    return np.concatenate(blocks), fields


def random_q6_K_row(rng, k):
    blocks, fields = [], []
    for _ in range(k // 256):
        d = f16_value(rng.uniform(0.001, 0.02))
        sc = rng.integers(-32, 32, 16)
        q = rng.integers(0, 64, 256)
        blocks.append(pack_q6_K(d, sc, q))
        fields.append((d, sc, q))
    return np.concatenate(blocks), fields


def random_q8_0_row(rng, k):
    blocks, fields = [], []
    for _ in range(k // 32):
        d = f16_value(rng.uniform(0.001, 0.02))
        q = rng.integers(-127, 128, 32)
        blocks.append(pack_q8_0(d, q))
        fields.append((d, q))
    return np.concatenate(blocks), fields


def weight_codes(qtype, fields):
    """Integer weight codes per value (Q4_K: [0,15]; Q5_K: [0,31]; Q6_K: q-32; Q8_0: int8) for one row."""
    if qtype in (12, 13):
        return np.concatenate([f[4] for f in fields]).astype(np.int64)
    if qtype == 2:
        return np.concatenate([f[1] for f in fields]).astype(np.int64) - 8
    if qtype == 14:
        return np.concatenate([f[2] for f in fields]).astype(np.int64) - 32
    if qtype == 11:
        return np.concatenate([f[2] for f in fields]).astype(np.int64) - 4
    if qtype == 23:
        return np.array(IQ4_CODEBOOK, dtype=np.int64)[np.concatenate([f[2] for f in fields])]
    return np.concatenate([f[1] for f in fields]).astype(np.int64)


def q8_1_codes(xq_row):
    """int8 codes of one canonical q8_1 row (36-byte blocks: d, s, 32 codes)."""
    blk = np.asarray(xq_row, dtype=np.uint8).reshape(-1, 36)
    return blk[:, 4:36].view(np.int8).reshape(-1).astype(np.int64)


def q8_1_scales(xq_row):
    blk = np.ascontiguousarray(np.asarray(xq_row, dtype=np.uint8).reshape(-1, 36))
    d = blk[:, 0:2].copy().view(np.float16).reshape(-1).astype(np.float64)
    s = blk[:, 2:4].copy().view(np.float16).reshape(-1).astype(np.float64)
    return d, s


# q3_K: hmask[32] @0, qs[64] @32, 12 bytes of packed 6-bit scales @96, d f16 @108.  Value v sits in
# half h = v // 128, shift group j = (v % 128) // 32, lane l = v % 32: its low two bits are bits
# 2j, 2j+1 of qs[32h + l] and its third bit is bit 4h + j of hmask[l].  Scale t (values 16t..):
# its low nibble in byte t % 8 (t < 8: low nibble; t >= 8: high nibble; bytes 0-3 for t % 8 < 4,
# 4-7 otherwise), its top two bits in byte 8 + t % 4 at bit 2 * (t // 4).
def pack_q3_K(d, sc6, q):
    """sc6: 16 ints in [0,63] (stored scales, value = sc6 - 32); q: 256 ints in [0,7] (stored
    3-bit codes, value = q - 4).  Returns 110 bytes."""
    sc6 = [int(v) for v in sc6]
    q = [int(v) for v in q]
    assert len(sc6) == 16 and len(q) == 256
    assert all(0 <= v < 64 for v in sc6) and all(0 <= v < 8 for v in q)
    b = np.zeros(110, dtype=np.uint8)
    for v in range(256):
        h, j, l = v // 128, (v % 128) // 32, v % 32
        b[32 + 32 * h + l] |= (q[v] & 3) << (2 * j)
        b[l] |= (q[v] >> 2) << (4 * h + j)
    for t in range(16):
        low, top = sc6[t] & 15, sc6[t] >> 4
        byte = t % 8
        b[96 + byte] |= low if t < 8 else low << 4
        b[96 + 8 + t % 4] |= top << (2 * (t // 4))
    _put16(b, 108, f16_bits(d))
    return b


# iq4_xs: d f16 @0, scales_h u16 @2 (bits 2b, 2b+1: top bits of sub-block b's scale), scales_l[4]
# @4 (sub-block b's low nibble in byte b // 2, low nibble for even b), qs[128] @8 (sub-block b:
# bytes 16b..16b+15, low nibble of byte i = index of value i, high nibble = value 16 + i).
def pack_iq4_xs(d, ls, idx):
    """ls: 8 ints in [0,63] (stored scales, value = ls - 32); idx: 256 codebook indices in [0,15]."""
    ls = [int(v) for v in ls]
    idx = [int(v) for v in idx]
    assert len(ls) == 8 and len(idx) == 256
    assert all(0 <= v < 64 for v in ls) and all(0 <= v < 16 for v in idx)
    b = np.zeros(136, dtype=np.uint8)
    _put16(b, 0, f16_bits(d))
    sh = 0
    for sb in range(8):
        sh |= (ls[sb] >> 4) << (2 * sb)
        b[4 + sb // 2] |= (ls[sb] & 15) << (4 * (sb % 2))
        for i in range(16):
            b[8 + 16 * sb + i] = idx[32 * sb + i] | (idx[32 * sb + 16 + i] << 4)
    _put16(b, 2, sh)
    return b


# The IQ4_XS codebook (the format's fixed 16-entry table; no page prints its values).
IQ4_CODEBOOK = [-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113]


def random_q3_K_row(rng, k):
    blocks, fields = [], []
    for _ in range(k // 256):
        d = f16_value(rng.uniform(0.001, 0.02))
        sc6 = rng.integers(0, 64, 16)
        q = rng.integers(0, 8, 256)
        blocks.append(pack_q3_K(d, sc6, q))
        fields.append((d, sc6, q))
    return np.concatenate(blocks), fields


def random_iq4_xs_row(rng, k):
    blocks, fields = [], []
    for _ in range(k // 256):
        d = f16_value(rng.uniform(0.001, 0.02))
        ls = rng.integers(0, 64, 8)
        idx = rng.integers(0, 16, 256)
        blocks.append(pack_iq4_xs(d, ls, idx))
        fields.append((d, ls, idx))
    return np.concatenate(blocks), fields
