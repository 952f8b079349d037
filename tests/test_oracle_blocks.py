"""Pins for the oracle's weight-block decoders (CPU only).

Probes are built by the test-side encoder in blockpack.py (the inverse direction, written from the
GGUF layouts) and by hand-written golden blocks in tests/golden/, derived from the MMQ page's
statements on Q4_K (144 B / 256 values, value = d*sc*q - dmin*m, low nibble = first sub-block of a
pair) and Q6_K (6-bit value from ql's 4 low bits and qh's 2 high bits, minus 32, int8 scale per
16 values).  Byte-for-byte parity with real GGUF files stays unpinned: no such file is available.
"""
import os

import numpy as np
import pytest

import oracle
from blockpack import pack_q4_0, pack_q4_K, pack_q5_K, pack_q6_K, pack_q8_0, f16_value

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_kv(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(":", 1)
                out.append((k.strip(), v.strip()))
    return out


def _golden_q4_K_block(kv):
    b = np.zeros(144, dtype=np.uint8)
    for k, v in kv:
        if k == "d_bits":
            bits = int(v, 16); b[0], b[1] = bits & 255, bits >> 8
        elif k == "dmin_bits":
            bits = int(v, 16); b[2], b[3] = bits & 255, bits >> 8
        elif k == "scales":
            b[4:16] = [int(t, 16) for t in v.split()]
        elif k == "qs":
            for item in v.split():
                off, val = item.split(":")
                b[16 + int(off)] = int(val, 16)
        elif k == "qs_fill":
            b[16:144] = int(v, 16)
    return b


def test_q4_K_golden_nibble_probe():
    kv = _read_kv("q4_K_nibble_probe.txt")
    blk = _golden_q4_K_block(kv)
    w = oracle.dequantize(oracle.Q4_K, blk, 1, 256)[0]
    bg = [float(t) for k, v in kv if k == "background" for t in v.split()]
    expect = np.repeat(np.array(bg), 32)
    for k, v in kv:
        if k == "value":
            pos, val = v.split()
            expect[int(pos)] = float(val)
    assert np.array_equal(w, expect), np.nonzero(w != expect)


def test_q4_K_golden_scale_topbits_probe():
    kv = _read_kv("q4_K_scale_topbits_probe.txt")
    blk = _golden_q4_K_block(kv)
    w = oracle.dequantize(oracle.Q4_K, blk, 1, 256)[0]
    sb = [float(t) for k, v in kv if k == "subblock_values" for t in v.split()]
    assert np.array_equal(w, np.repeat(np.array(sb), 32))


def test_q4_K_encoder_roundtrip_random():
    rng = np.random.default_rng(10)
    for _ in range(50):
        d, dmin = f16_value(rng.uniform(-2, 2)), f16_value(rng.uniform(-2, 2))
        sc, m, q = rng.integers(0, 64, 8), rng.integers(0, 64, 8), rng.integers(0, 16, 256)
        w = oracle.dequantize(oracle.Q4_K, pack_q4_K(d, dmin, sc, m, q), 1, 256)[0]
        expect = d * np.repeat(sc, 32) * q - dmin * np.repeat(m, 32)
        assert np.array_equal(w, expect)


@pytest.mark.parametrize("v", list(range(0, 256, 7)) + [31, 32, 63, 64, 255])
def test_q4_K_one_hot_position(v):
    q = np.zeros(256, dtype=int); q[v] = 9
    sc = np.ones(8, dtype=int)
    w = oracle.dequantize(oracle.Q4_K, pack_q4_K(1.0, 0.0, sc, np.zeros(8, int), q), 1, 256)[0]
    assert np.nonzero(w)[0].tolist() == [v] and w[v] == 9.0


@pytest.mark.parametrize("j", range(8))
def test_q4_K_single_scale(j):
    """All scales and mins zero except sub-block j: only its 32 values are nonzero."""
    sc = np.zeros(8, dtype=int); m = np.zeros(8, dtype=int)
    sc[j] = 63; m[j] = 33
    q = np.full(256, 15)
    w = oracle.dequantize(oracle.Q4_K, pack_q4_K(0.5, 0.25, sc, m, q), 1, 256)[0]
    expect = np.zeros(256); expect[32 * j:32 * j + 32] = 0.5 * 63 * 15 - 0.25 * 33
    assert np.array_equal(w, expect)


def test_q5_K_encoder_roundtrip_random():
    rng = np.random.default_rng(12)
    for _ in range(50):
        d, dmin = f16_value(rng.uniform(-2, 2)), f16_value(rng.uniform(-2, 2))
        sc, m, q = rng.integers(0, 64, 8), rng.integers(0, 64, 8), rng.integers(0, 32, 256)
        w = oracle.dequantize(oracle.Q5_K, pack_q5_K(d, dmin, sc, m, q), 1, 256)[0]
        expect = d * np.repeat(sc, 32) * q - dmin * np.repeat(m, 32)
        assert np.array_equal(w, expect)


@pytest.mark.parametrize("v", list(range(0, 256, 7)) + [31, 32, 63, 64, 95, 255])
@pytest.mark.parametrize("code", [9, 16, 25])
def test_q5_K_one_hot_position(v, code):
    """A single nonzero code (low nibble only, fifth bit only, both) lands at its own value."""
    q = np.zeros(256, dtype=int); q[v] = code
    w = oracle.dequantize(oracle.Q5_K, pack_q5_K(1.0, 0.0, np.ones(8, int), np.zeros(8, int), q), 1, 256)[0]
    assert np.nonzero(w)[0].tolist() == [v] and w[v] == float(code)


def test_q5_K_fifth_bits_are_bit_j_of_qh_l():
    """Stated from the layout directly: setting bit j of qh byte l (and nothing else, scale 1)
    gives the value 16 at position 32*j + l."""
    for j in range(8):
        for l in (0, 5, 31):
            blk = pack_q5_K(1.0, 0.0, np.ones(8, int), np.zeros(8, int), np.zeros(256, int))
            blk[16 + l] |= 1 << j
            w = oracle.dequantize(oracle.Q5_K, blk, 1, 256)[0]
            assert np.nonzero(w)[0].tolist() == [32 * j + l] and w[32 * j + l] == 16.0


def test_q5_K_without_fifth_bits_is_q4_K():
    rng = np.random.default_rng(13)
    d, dmin = f16_value(0.37), f16_value(0.11)
    sc, m, q = rng.integers(0, 64, 8), rng.integers(0, 64, 8), rng.integers(0, 16, 256)
    w5 = oracle.dequantize(oracle.Q5_K, pack_q5_K(d, dmin, sc, m, q), 1, 256)[0]
    w4 = oracle.dequantize(oracle.Q4_K, pack_q4_K(d, dmin, sc, m, q), 1, 256)[0]
    assert np.array_equal(w5, w4)


def test_q4_0_encoder_roundtrip_and_one_hot():
    rng = np.random.default_rng(14)
    for _ in range(50):
        d = f16_value(rng.uniform(-2, 2))
        q = rng.integers(0, 16, 32)
        w = oracle.dequantize(oracle.Q4_0, pack_q4_0(d, q), 1, 32)[0]
        assert np.array_equal(w, d * (q - 8.0))
    for v in range(32):
        q = np.full(32, 8); q[v] = 13          # code 8 is the zero point
        w = oracle.dequantize(oracle.Q4_0, pack_q4_0(1.0, q), 1, 32)[0]
        assert np.nonzero(w)[0].tolist() == [v] and w[v] == 5.0
    w = oracle.dequantize(oracle.Q4_0, pack_q4_0(0.5, np.zeros(32, int)), 1, 32)[0]
    assert np.all(w == -4.0)                 # nibble 0 is -8 * d


def test_q6_K_encoder_roundtrip_random():
    rng = np.random.default_rng(11)
    for _ in range(50):
        d = f16_value(rng.uniform(-2, 2))
        sc = rng.integers(-128, 128, 16)
        q = rng.integers(0, 64, 256)
        w = oracle.dequantize(oracle.Q6_K, pack_q6_K(d, sc, q), 1, 256)[0]
        assert np.array_equal(w, d * np.repeat(sc, 16) * (q - 32))


@pytest.mark.parametrize("v", list(range(0, 256, 5)) + [15, 16, 127, 128, 255])
def test_q6_K_one_hot_position(v):
    q = np.full(256, 32); q[v] = 32 + 27          # code 27 at v, zero everywhere else
    w = oracle.dequantize(oracle.Q6_K, pack_q6_K(1.0, np.ones(16, int), q), 1, 256)[0]
    assert np.nonzero(w)[0].tolist() == [v] and w[v] == 27.0


@pytest.mark.parametrize("txi", range(32))
def test_q6_K_ql_qh_pairing_from_page(txi):
    """MMQ page, "Q6_K load" section: 32-bit word txi of ql (8 values) is combined with qh word
    8*(txi/16) + txi%8, shifted right by (txi & 8) >> 2; the low nibbles take qh bits
    [shift, shift+1] and the high nibbles bits [shift+4, shift+5] (moved to bits 4-5), then 32 is
    subtracted.  Build one byte of each word that way and check the decoded 6-bit codes (the page
    does not print where each code lands, so only the set of codes is compared)."""
    for byte in range(4):
        blk = np.zeros(210, dtype=np.uint8)
        blk[192:208] = 1                                          # scales = 1
        blk[208], blk[209] = 0x00, 0x3c                           # d = 1.0
        blk[128:192] = 0x00
        # every other value's stored 6-bit code must be 32 (code 0): low nibbles 0 and qh bits
        # 10b for every 2-bit field -> 0b10 << 4 = 32
        blk[128:192] = 0b10101010
        ql_off = 4 * txi + byte
        qh_off = 128 + 4 * (8 * (txi // 16) + txi % 8) + byte
        shift = (txi & 8) >> 2
        lo_nib, hi_nib, lo_top, hi_top = 5, 11, 3, 1
        blk[ql_off] = lo_nib | (hi_nib << 4)
        qh = int(blk[qh_off])
        qh &= ~((3 << shift) | (3 << (shift + 4))) & 0xFF
        qh |= (lo_top << shift) | (hi_top << (shift + 4))
        blk[qh_off] = qh
        w = oracle.dequantize(oracle.Q6_K, blk, 1, 256)[0]
        nz = sorted(w[w != 0].tolist())
        expect = sorted([(lo_nib | (lo_top << 4)) - 32, (hi_nib | (hi_top << 4)) - 32])
        assert nz == expect, (txi, byte, nz)


def test_q8_0_roundtrip_and_one_hot():
    rng = np.random.default_rng(12)
    for _ in range(20):
        d = f16_value(rng.uniform(-2, 2))
        q = rng.integers(-128, 128, 32)
        w = oracle.dequantize(oracle.Q8_0, pack_q8_0(d, q), 1, 32)[0]
        assert np.array_equal(w, d * q)
    for v in range(32):
        q = np.zeros(32, dtype=int); q[v] = -77
        w = oracle.dequantize(oracle.Q8_0, pack_q8_0(0.5, q), 1, 32)[0]
        assert np.nonzero(w)[0].tolist() == [v] and w[v] == -38.5


def test_row_major_block_order():
    """A row is its blocks back to back; rows follow each other (weights stored [rows][k])."""
    blocks = [pack_q8_0(1.0, np.full(32, i + 1)) for i in range(6)]
    w = oracle.dequantize(oracle.Q8_0, np.concatenate(blocks).reshape(2, 3 * 34), 2, 96)
    assert np.array_equal(w[0], np.repeat([1.0, 2.0, 3.0], 32))
    assert np.array_equal(w[1], np.repeat([4.0, 5.0, 6.0], 32))


def test_bad_arguments_rejected():
    with pytest.raises(ValueError):
        oracle.dequantize(oracle.Q4_K, np.zeros(144, np.uint8), 1, 100)
    with pytest.raises(ValueError):
        oracle.dequantize(99, np.zeros(144, np.uint8), 1, 256)


# ---------------------------------------------------------------------------------------------
# Q3_K (GP100 patch page, "How" step 3: the type's codes carry a -4 offset; layout GGUF's)
# ---------------------------------------------------------------------------------------------
from blockpack import IQ4_CODEBOOK, pack_iq4_xs, pack_q3_K  # noqa: E402


def test_q3_K_encoder_roundtrip_random():
    rng = np.random.default_rng(31)
    for _ in range(50):
        d = f16_value(rng.uniform(-2, 2))
        sc6 = rng.integers(0, 64, 16)
        q = rng.integers(0, 8, 256)
        w = oracle.dequantize(oracle.Q3_K, pack_q3_K(d, sc6, q), 1, 256)[0]
        assert np.array_equal(w, d * np.repeat(sc6 - 32, 16) * (q - 4))


@pytest.mark.parametrize("v", list(range(0, 256, 7)) + [31, 32, 127, 128, 255])
def test_q3_K_one_hot_position(v):
    q = np.full(256, 4); q[v] = 7                 # code +3 at v, zero everywhere else
    w = oracle.dequantize(oracle.Q3_K, pack_q3_K(1.0, np.full(16, 33), q), 1, 256)[0]
    assert np.nonzero(w)[0].tolist() == [v] and w[v] == 3.0


@pytest.mark.parametrize("t", range(16))
def test_q3_K_single_scale(t):
    sc6 = np.full(16, 32); sc6[t] = 32 + 5        # scale 5 on sub-block t, 0 elsewhere
    w = oracle.dequantize(oracle.Q3_K, pack_q3_K(1.0, sc6, np.full(256, 5)), 1, 256)[0]
    assert np.nonzero(w)[0].tolist() == list(range(16 * t, 16 * t + 16))
    assert np.all(w[16 * t:16 * t + 16] == 5.0)


def test_q3_K_hand_placed_bits():
    """Bytes set by hand from the layout statement (not by the encoder): hmask[5] = 0x10 is the
    third bit of value 128 + 5 (h = 1, j = 0); qs[32 + 7] = 0x30 puts low bits 3 on value
    128 + 2*32 + 7 = 199 (h = 1, j = 2); scale bytes: s[2] = 0x0F and s[10] = 0x03 give scale 2 the
    stored value 63, s[8 + 1] = 0x40 puts top bits 01 on scale 13 (= 4 + 1 + 8), whose low nibble is the
    high nibble of s[5]; all other stored codes 0 (value -4) and scales 0 (value -32)."""
    b = np.zeros(110, dtype=np.uint8)
    b[5] = 0x10
    b[32 + 32 + 7] = 0x30
    b[96 + 2] = 0x0F
    b[96 + 10] = 0x03
    b[96 + 9] = 0x40
    b[96 + 5] = 0x20
    b[108], b[109] = 0x00, 0x3C                   # d = 1.0
    w = oracle.dequantize(oracle.Q3_K, b, 1, 256)[0]
    sc = np.full(16, -32); sc[2] = 63 - 32; sc[13] = (0x2 | (1 << 4)) - 32
    code = np.full(256, -4); code[133] = 4 - 4; code[199] = 3 - 4
    assert np.array_equal(w, np.repeat(sc, 16) * code)


# ---------------------------------------------------------------------------------------------
# IQ4_XS (GP100 patch page, "How" step 3: a non-linear 4-bit codebook; layout GGUF's).  The
# codebook's 16 values are the format's table: no page prints them, so they are unpinned beyond
# the properties below; the index and scale placement is pinned.
# ---------------------------------------------------------------------------------------------
def _iq4_code_of(idx):
    w = oracle.dequantize(oracle.IQ4_XS, pack_iq4_xs(1.0, np.full(8, 33), np.full(256, idx)), 1, 256)[0]
    assert np.all(w == w[0])
    return w[0]


def test_iq4_xs_codebook_properties():
    cb = [_iq4_code_of(i) for i in range(16)]
    assert cb == [float(v) for v in IQ4_CODEBOOK]
    assert all(a < b for a, b in zip(cb, cb[1:]))              # strictly increasing
    assert cb[0] == -127 and max(abs(v) for v in cb) == 127    # within int8, symmetric extreme


def test_iq4_xs_encoder_roundtrip_random():
    rng = np.random.default_rng(32)
    for _ in range(50):
        d = f16_value(rng.uniform(-2, 2))
        ls = rng.integers(0, 64, 8)
        idx = rng.integers(0, 16, 256)
        w = oracle.dequantize(oracle.IQ4_XS, pack_iq4_xs(d, ls, idx), 1, 256)[0]
        assert np.array_equal(w, d * np.repeat(ls - 32, 32) * np.array(IQ4_CODEBOOK)[idx])


@pytest.mark.parametrize("v", list(range(0, 256, 9)) + [15, 16, 31, 32, 255])
def test_iq4_xs_one_hot_position(v):
    idx = np.full(256, 8); idx[v] = 15            # codebook entry 8 (= 1) everywhere, entry 15 at v
    w = oracle.dequantize(oracle.IQ4_XS, pack_iq4_xs(1.0, np.full(8, 33), idx), 1, 256)[0]
    assert np.nonzero(w != 1.0)[0].tolist() == [v] and w[v] == IQ4_CODEBOOK[15]


def test_iq4_xs_hand_placed_bits():
    """Bytes set by hand: scales_h = 0x8000 gives sub-block 7 top scale bits 10; scales_l[3] =
    0x50 its low nibble 5 (odd sub-block: high nibble) -> stored 37, scale 5; every other
    sub-block stores 0 (scale -32).  qs[8 + 16*7 + 3] = 0xF0: value 32*7 + 16 + 3 = 243 takes
    index 15, every other index 0."""
    b = np.zeros(136, dtype=np.uint8)
    b[0], b[1] = 0x00, 0x3C                       # d = 1.0
    b[2], b[3] = 0x00, 0x80
    b[4 + 3] = 0x50
    b[8 + 16 * 7 + 3] = 0xF0
    w = oracle.dequantize(oracle.IQ4_XS, b, 1, 256)[0]
    sc = np.full(8, -32); sc[7] = 37 - 32
    code = np.full(256, IQ4_CODEBOOK[0]); code[243] = IQ4_CODEBOOK[15]
    assert np.array_equal(w, np.repeat(sc, 32) * code)
