/*
 * qmm_oracle.c -- plain, slow CPU oracle for block-quantized matmul with q8_1 activations.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference the HIP kernels are checked against.
 * Only the tests, the smoke check and the bench's CPU-baseline leg may load it; the product
 * library never links, calls or falls back to it, and it shares no code, header or table with
 * the HIP sources.
 *
 * What it computes (sources: the three web pages on the subject):
 *  - q8_1 activation blocks: 32 int8 values with an fp16 scale d and an fp16 sum term s = d * sum(q)
 *    ("llama.cpp MMQ" page, introduction and the "dp4a path Q4_K" section, where the
 *    activation half2 (d, s) and s = d*sum(q) are described).
 *  - Q4_K weights: value = d*sc*q - dmin*m over 32-value sub-blocks of a 144-byte super-block
 *    ("llama.cpp MMQ" page, "why not dequantize" and "Q4_K load" sections).
 *  - Q5_K weights: as Q4_K with a fifth code bit, value = d*sc*q - dmin*m with q in [0, 31]; the
 *    pages name Q5_K beside Q4_K and give the two the same 6-bit scale/min packing ("llama.cpp MMQ"
 *    page, "Q4_K load" section); the byte layout is GGUF's block_q5_K.
 *  - Q6_K weights: value = d*sc*(q - 32), 6-bit q built from 4 low bits (ql) and 2 high bits (qh),
 *    signed 8-bit scale per 16 values ("llama.cpp MMQ" page, "Q6_K load" and "Q6_K dot" sections).
 *  - Q8_0 weights: value = d*q, int8 q, fp16 d per 32 values (named on the GP100 patch page and the
 *    candle page; the byte layout follows the GGUF block_q8_0 definition).
 *  - Q4_0 weights: value = d*(q - 8), 4-bit q, fp16 d per 32 values (named with the other types on
 *    the MMQ page, whose tile-size table gives it only qs and one scale; the byte layout is GGUF's
 *    block_q4_0: low nibbles of qs[0..15] are values 0..15, high nibbles values 16..31).
 *  - Q3_K weights: value = d * (sc - 32) * (q - 4), a 3-bit code q and an unsigned 6-bit scale per
 *    16 values; the GP100 patch page ("How", step 3) names the type and its -4 code offset; the
 *    byte layout and the 6-bit scale packing are GGUF's block_q3_K.
 *  - IQ4_XS weights: value = d * (ls - 32) * cb[q], a 4-bit index q into a fixed 16-entry
 *    non-linear codebook cb and an unsigned 6-bit scale ls per 32 values; the GP100 page ("How",
 *    step 3) names the type and its codebook; the byte layout and the codebook are GGUF's
 *    block_iq4_xs and its 4-bit non-linear table.
 *  - fp16-activation mode ("GP100 MMVQ" page, "How" step 1 and the accuracy paragraph under the
 *    results table): per 32 values of a column a power-of-two prescale 2^e, e the largest integer
 *    with max|x| * 2^e < 2^15 (e = 0 for an all-zero block), the values rounded once to fp16, and
 *    the product taken with those fp16 values unscaled by 2^-e per block.  The page's fp16
 *    partial sums are an implementation of that product on its card; the oracle takes the plain
 *    definition (exact fp64 sums, one rounding to fp32).
 *  - The product: per 32-value activation block b, an exact integer dot D_b of weight codes and
 *    activation codes, then the scale fixups of the "dp4a path Q4_K" / "Q6_K dot" sections.
 *    This oracle combines every exact term in fp64 and rounds to fp32 once.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *  - q8_1: d32 = amax/127 in fp32; q = roundf(x / d32) (IEEE fp32 divide by the unrounded
 *    d32, round half away from zero); d = fp16_rne(d32); s = fp16_rne(d32 * (float)sum(q)).
 *    amax == 0 gives d = s = 0 and q = 0.
 *  - Block byte layouts follow GGUF: q4_K {d, dmin, scales[12], qs[128]} (144 B),
 *    q6_K {ql[128], qh[64], scales[16], d} (210 B), q8_0 {d, qs[32]} (34 B),
 *    q8_1 {d, s, qs[32]} (36 B); fp16 is little-endian IEEE binary16.  q5_K {d, dmin, scales[12],
 *    qh[32], qs[128]} (176 B): the low 4 bits of value v as in Q4_K, the fifth bit is bit v/32 of
 *    qh[v % 32].
 *  - q3_K {hmask[32], qs[64], scales[12], d} (110 B): value v, h = v/128, j = (v%128)/32,
 *    l = v%32: low 2 bits = bits 2j..2j+1 of qs[32h + l], third bit = bit 4h + j of hmask[l];
 *    16 6-bit scales from the 12 bytes s: scale i (i < 4) = (s[i] & 15) | ((s[8+i] & 3) << 4),
 *    4+i: (s[4+i] & 15) | (((s[8+i] >> 2) & 3) << 4), 8+i: (s[i] >> 4) | (((s[8+i] >> 4) & 3) << 4),
 *    12+i: (s[4+i] >> 4) | (((s[8+i] >> 6) & 3) << 4); scale t serves values 16t..16t+15.
 *  - iq4_xs {d, scales_h (u16), scales_l[4], qs[128]} (136 B): sub-block b (32 values) has
 *    ls = ((scales_l[b/2] >> 4(b%2)) & 15) | (((scales_h >> 2b) & 3) << 4); its values i < 16 take
 *    the low nibble of qs[16b + i], values 16 + i the high nibble; codebook -127 -104 -83 -65 -49
 *    -35 -22 -10 1 13 25 38 53 69 89 113 (the format's table: parity unpinned, no page prints it).
 *  - Q4_K 6-bit scale/min unpacking (the page's description is garbled) follows GGUF:
 *    j < 4: sc = s[j] & 63, m = s[j+4] & 63;
 *    j >= 4: sc = (s[j+4] & 15) | ((s[j-4] >> 6) << 4), m = (s[j+4] >> 4) | ((s[j] >> 6) << 4).
 *
 * Parity pins (tests/test_oracle_*.py): closed-form q8_1 blocks and rounding ties, fp16 conversion
 * against numpy, one-hot / single-scale weight probes built by an independent encoder, a golden
 * probe written from the page's nibble statement, brute-force integer dots, the per-sub-block
 * identity, and fp64 dequantize-then-multiply on tiny shapes.  GGUF byte-for-byte parity with real
 * model files is not pinned (no such file is available); internal consistency is.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <stdlib.h>

#define ORC_Q4_0 2
#define ORC_Q8_0 8
#define ORC_Q3_K 11
#define ORC_Q4_K 12
#define ORC_Q5_K 13
#define ORC_Q6_K 14
#define ORC_IQ4_XS 23

#define ORC_OK 0
#define ORC_ERR -1

/* ---------------------------------------------------------------------------------------------
 * IEEE 754 binary16, written from the format definition (1 sign, 5 exponent bits with bias 15,
 * 10 fraction bits; exponent 0 = subnormal with unit 2^-24; exponent 31 = inf/nan).
 * ------------------------------------------------------------------------------------------- */
double oracle_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return sign ? -v : v;
}

/* fp32 -> fp16, round to nearest, ties to even; overflow goes to inf. */
uint16_t oracle_float_to_half(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t e = (u >> 23) & 0xFFu;
    uint32_t f = u & 0x7FFFFFu;
    if (e == 0xFF) return (uint16_t)(sign | 0x7C00u | (f ? 0x200u : 0u));
    if (e == 0 && f == 0) return sign;
    /* value = sig * 2^(exp2 - 23) with a 24-bit significand (fp32 subnormals: no hidden bit) */
    uint64_t sig = (e == 0) ? f : (f | 0x800000u);
    int exp2 = (e == 0) ? -126 : (int)e - 127;
    /* number of fp16 units of 2^-24 : sig * 2^(exp2 - 23 + 24) */
    int target_exp; /* unbiased exponent of the fp16 result's leading bit */
    /* find the position of the leading bit of the exact value */
    int lead = 63;
    while (!((sig >> lead) & 1)) lead--;
    int vexp = exp2 - 23 + lead; /* value in [2^vexp, 2^(vexp+1)) */
    if (vexp >= -14) target_exp = vexp; else target_exp = -15; /* subnormal: fixed unit 2^-24 */
    /* the fp16 quantum at this exponent: normal -> 2^(target_exp-10), subnormal -> 2^-24 */
    int q_exp = (vexp >= -14) ? (target_exp - 10) : -24;
    /* express value / 2^q_exp = sig * 2^(exp2 - 23 - q_exp) */
    int sh = exp2 - 23 - q_exp;
    uint64_t n;
    if (sh >= 0) {
        n = sig << sh;
    } else {
        int r = -sh;
        if (r > 60) {
            n = 0; /* far below half of the smallest subnormal */
        } else {
            uint64_t q = sig >> r;
            uint64_t rem = sig & ((1ull << r) - 1);
            uint64_t half = 1ull << (r - 1);
            if (rem > half || (rem == half && (q & 1))) q++;
            n = q;
        }
    }
    /* n is the fp16 significand count in units of 2^q_exp; it may have carried to 2048 */
    uint32_t out;
    if (vexp >= -14) {
        int be = target_exp + 15;
        if (n >= 2048) { n >>= 1; be++; }
        if (be >= 31) return (uint16_t)(sign | 0x7C00u);
        out = ((uint32_t)be << 10) | ((uint32_t)n & 1023u);
    } else {
        /* subnormal count n in [0, 1024]; 1024 means it rounded up to the smallest normal */
        out = (uint32_t)n; /* n == 1024 encodes exponent field 1, fraction 0 -- same bits */
    }
    return (uint16_t)(sign | out);
}

static inline uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static inline void wr16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)(v & 0xFF); p[1] = (uint8_t)(v >> 8); }

/* ---------------------------------------------------------------------------------------------
 * q8_1 activation quantization (one 32-value block at a time).
 * Block bytes: d fp16 @0, s fp16 @2, q int8[32] @4 (36 bytes).
 * ------------------------------------------------------------------------------------------- */
void oracle_quantize_q8_1(const float *x, int64_t n_rows, int64_t k, uint8_t *y) {
    int64_t nb = k / 32;
    for (int64_t r = 0; r < n_rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float *xb = x + r * k + b * 32;
            uint8_t *yb = y + (r * nb + b) * 36;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float a = fabsf(xb[i]);
                if (a > amax) amax = a;
            }
            float d32 = amax / 127.0f;
            int sumq = 0;
            for (int i = 0; i < 32; ++i) {
                int q = 0;
                if (amax != 0.0f) q = (int)roundf(xb[i] / d32);
                yb[4 + i] = (uint8_t)(int8_t)q;
                sumq += q;
            }
            float s32 = d32 * (float)sumq;
            wr16(yb + 0, oracle_float_to_half(d32));
            wr16(yb + 2, oracle_float_to_half(s32));
        }
    }
}

/* ---------------------------------------------------------------------------------------------
 * Weight block decoders: integer codes and fp16 scales of one super-block / block.
 * ------------------------------------------------------------------------------------------- */

/* Q4_K, 144 bytes per 256 values. code[v] in [0,15], sc[j], m[j] in [0,63] for sub-block j = v/32. */
static void decode_q4_K(const uint8_t *blk, double *d, double *dmin, int sc[8], int m[8], int code[256]) {
    *d = oracle_half_to_double(rd16(blk + 0));
    *dmin = oracle_half_to_double(rd16(blk + 2));
    const uint8_t *s = blk + 4;
    for (int j = 0; j < 8; ++j) {
        if (j < 4) {
            sc[j] = s[j] & 63;
            m[j] = s[j + 4] & 63;
        } else {
            sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
            m[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
        }
    }
    const uint8_t *qs = blk + 16;
    for (int v = 0; v < 256; ++v) {
        int chunk = v / 64;          /* 64 values share 32 bytes */
        int l = v % 32;
        uint8_t byte = qs[32 * chunk + l];
        code[v] = (v % 64 < 32) ? (byte & 15) : (byte >> 4); /* low nibble: first sub-block of the pair */
    }
}

/* Q5_K, 176 bytes per 256 values: the Q4_K header (d, dmin, 12 scale bytes), then qh[32], then
 * qs[128] laid out as Q4_K's.  code[v] in [0,31]: Q4_K's nibble plus 16 * bit (v/32) of qh[v%32]. */
static void decode_q5_K(const uint8_t *blk, double *d, double *dmin, int sc[8], int m[8], int code[256]) {
    uint8_t q4[144];
    memcpy(q4, blk, 16);                 /* same header and scale packing as Q4_K */
    memcpy(q4 + 16, blk + 48, 128);      /* the low nibbles, in Q4_K's order */
    decode_q4_K(q4, d, dmin, sc, m, code);
    const uint8_t *qh = blk + 16;
    for (int v = 0; v < 256; ++v) code[v] += 16 * ((qh[v % 32] >> (v / 32)) & 1);
}

/* Q6_K, 210 bytes per 256 values. code[v] in [-32,31] (the 6-bit value minus 32),
 * sc[v/16] signed 8-bit. */
static void decode_q6_K(const uint8_t *blk, double *d, int sc[16], int code[256]) {
    const uint8_t *ql = blk;
    const uint8_t *qh = blk + 128;
    const int8_t *scales = (const int8_t *)(blk + 192);
    *d = oracle_half_to_double(rd16(blk + 208));
    for (int j = 0; j < 16; ++j) sc[j] = scales[j];
    for (int v = 0; v < 256; ++v) {
        int h = v / 128;
        int u = v % 128;
        int g = u / 32;
        int l = u % 32;
        uint8_t lo_byte = ql[64 * h + 32 * (g & 1) + l];
        int nib = (g < 2) ? (lo_byte & 15) : (lo_byte >> 4);
        int top = (qh[32 * h + l] >> (2 * g)) & 3;
        code[v] = (nib | (top << 4)) - 32;
    }
}

/* Q8_0, 34 bytes per 32 values. */
static void decode_q8_0(const uint8_t *blk, double *d, int code[32]) {
    *d = oracle_half_to_double(rd16(blk + 0));
    for (int i = 0; i < 32; ++i) code[i] = (int8_t)blk[2 + i];
}

/* Q4_0, 18 bytes per 32 values: {d, qs[16]}; code[i] = nibble - 8 in [-8, 7]. */
static void decode_q4_0(const uint8_t *blk, double *d, int code[32]) {
    *d = oracle_half_to_double(rd16(blk + 0));
    for (int i = 0; i < 16; ++i) {
        code[i] = (blk[2 + i] & 15) - 8;
        code[i + 16] = (blk[2 + i] >> 4) - 8;
    }
}

/* Q3_K, 110 bytes per 256 values: code[v] = 3-bit value - 4 in [-4, 3], sc[v/16] = 6-bit scale - 32. */
static void decode_q3_K(const uint8_t *blk, double *d, int sc[16], int code[256]) {
    const uint8_t *hmask = blk, *qs = blk + 32, *s = blk + 96;
    *d = oracle_half_to_double(rd16(blk + 108));
    for (int i = 0; i < 4; ++i) {
        sc[i] = ((s[i] & 15) | ((s[8 + i] & 3) << 4)) - 32;
        sc[4 + i] = ((s[4 + i] & 15) | (((s[8 + i] >> 2) & 3) << 4)) - 32;
        sc[8 + i] = ((s[i] >> 4) | (((s[8 + i] >> 4) & 3) << 4)) - 32;
        sc[12 + i] = ((s[4 + i] >> 4) | (((s[8 + i] >> 6) & 3) << 4)) - 32;
    }
    for (int v = 0; v < 256; ++v) {
        const int h = v / 128, j = (v % 128) / 32, l = v % 32;
        const int low = (qs[32 * h + l] >> (2 * j)) & 3;
        const int top = (hmask[l] >> (4 * h + j)) & 1;
        code[v] = low + 4 * top - 4;
    }
}

/* IQ4_XS, 136 bytes per 256 values: code[v] = codebook entry of its 4-bit index, sc[v/32] = 6-bit
 * scale - 32. */
static const int iq4_codebook[16] = {-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113};
static void decode_iq4_xs(const uint8_t *blk, double *d, int sc[8], int code[256]) {
    *d = oracle_half_to_double(rd16(blk + 0));
    const int sh = rd16(blk + 2);
    const uint8_t *sl = blk + 4, *qs = blk + 8;
    for (int b = 0; b < 8; ++b) {
        sc[b] = (((sl[b / 2] >> (4 * (b % 2))) & 15) | (((sh >> (2 * b)) & 3) << 4)) - 32;
        for (int i = 0; i < 16; ++i) {
            code[32 * b + i] = iq4_codebook[qs[16 * b + i] & 15];
            code[32 * b + 16 + i] = iq4_codebook[qs[16 * b + i] >> 4];
        }
    }
}

static void decode_q8_1(const uint8_t *blk, double *d, double *s, int code[32]) {
    *d = oracle_half_to_double(rd16(blk + 0));
    *s = oracle_half_to_double(rd16(blk + 2));
    for (int i = 0; i < 32; ++i) code[i] = (int8_t)blk[4 + i];
}

static int type_block_values(int type) {
    if (type == ORC_Q4_K || type == ORC_Q5_K || type == ORC_Q6_K || type == ORC_Q3_K || type == ORC_IQ4_XS) return 256;
    if (type == ORC_Q8_0 || type == ORC_Q4_0) return 32;
    return 0;
}
static int type_block_bytes(int type) {
    if (type == ORC_Q4_K) return 144;
    if (type == ORC_Q5_K) return 176;
    if (type == ORC_Q6_K) return 210;
    if (type == ORC_Q8_0) return 34;
    if (type == ORC_Q4_0) return 18;
    if (type == ORC_Q3_K) return 110;
    if (type == ORC_IQ4_XS) return 136;
    return 0;
}

int64_t oracle_row_bytes(int type, int64_t k) {
    int bv = type_block_values(type);
    if (bv == 0 || k % bv) return -1;
    return (k / bv) * type_block_bytes(type);
}

/* Number of integer sub-block dots per (row, column): Q6_K and Q3_K have 16-value sub-blocks. */
int64_t oracle_subdots_per_row(int type, int64_t k) {
    if (type == ORC_Q6_K || type == ORC_Q3_K) return k / 16;
    return k / 32;
}

/* ---------------------------------------------------------------------------------------------
 * Dequantization to fp64 (value definitions only; used by the tests' dequantize-then-multiply).
 * ------------------------------------------------------------------------------------------- */
int oracle_dequantize(int type, const uint8_t *w, int64_t rows, int64_t k, double *out) {
    int64_t rb = oracle_row_bytes(type, k);
    if (rb < 0) return ORC_ERR;
    int bv = type_block_values(type), bb = type_block_bytes(type);
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t blk = 0; blk < k / bv; ++blk) {
            const uint8_t *p = w + r * rb + blk * bb;
            double *o = out + r * k + blk * bv;
            if (type == ORC_Q4_K || type == ORC_Q5_K) {
                double d, dmin; int sc[8], m[8], code[256];
                if (type == ORC_Q4_K) decode_q4_K(p, &d, &dmin, sc, m, code);
                else decode_q5_K(p, &d, &dmin, sc, m, code);
                for (int v = 0; v < 256; ++v) o[v] = d * sc[v / 32] * code[v] - dmin * m[v / 32];
            } else if (type == ORC_Q6_K || type == ORC_Q3_K) {
                double d; int sc[16], code[256];
                if (type == ORC_Q6_K) decode_q6_K(p, &d, sc, code);
                else decode_q3_K(p, &d, sc, code);
                for (int v = 0; v < 256; ++v) o[v] = d * sc[v / 16] * code[v];
            } else if (type == ORC_IQ4_XS) {
                double d; int sc[8], code[256];
                decode_iq4_xs(p, &d, sc, code);
                for (int v = 0; v < 256; ++v) o[v] = d * sc[v / 32] * code[v];
            } else {
                double d; int code[32];
                if (type == ORC_Q8_0) decode_q8_0(p, &d, code);
                else decode_q4_0(p, &d, code);
                for (int v = 0; v < 32; ++v) o[v] = d * code[v];
            }
        }
    }
    return ORC_OK;
}

/* q8_1 blocks -> fp64 values d*q, and the per-block d and s. */
void oracle_dequantize_q8_1(const uint8_t *xq, int64_t n_rows, int64_t k, double *out, double *d_out,
                            double *s_out) {
    int64_t nb = k / 32;
    for (int64_t r = 0; r < n_rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            double d, s; int code[32];
            decode_q8_1(xq + (r * nb + b) * 36, &d, &s, code);
            for (int i = 0; i < 32; ++i) out[r * k + b * 32 + i] = d * code[i];
            if (d_out) d_out[r * nb + b] = d;
            if (s_out) s_out[r * nb + b] = s;
        }
    }
}

/* ---------------------------------------------------------------------------------------------
 * Decoded activations: per column, int codes and the fp16 d and s of every 32-value block.
 * ------------------------------------------------------------------------------------------- */
typedef struct {
    int64_t k;
    int8_t *qa;   /* [n][k] */
    double *da;   /* [n][k/32] */
    double *sa;   /* [n][k/32] */
} act_t;

static int act_decode(act_t *a, const uint8_t *xq, int64_t n, int64_t k) {
    int64_t nb = k / 32;
    a->k = k;
    a->qa = (int8_t *)malloc((size_t)(n * k) + 1);
    a->da = (double *)malloc(sizeof(double) * (size_t)(n * nb) + 8);
    a->sa = (double *)malloc(sizeof(double) * (size_t)(n * nb) + 8);
    if (!a->qa || !a->da || !a->sa) return ORC_ERR;
    for (int64_t c = 0; c < n; ++c)
        for (int64_t b = 0; b < nb; ++b) {
            int code[32];
            decode_q8_1(xq + (c * nb + b) * 36, &a->da[c * nb + b], &a->sa[c * nb + b], code);
            for (int i = 0; i < 32; ++i) a->qa[c * k + b * 32 + i] = (int8_t)code[i];
        }
    return ORC_OK;
}
static void act_free(act_t *a) { free(a->qa); free(a->da); free(a->sa); }

/* ---------------------------------------------------------------------------------------------
 * One output element: the exact integer sub-block dots, then the fp64 combine, then one round
 * to fp32.  D (optional) receives the integer dots of this (row, column).
 * ------------------------------------------------------------------------------------------- */
static float dot_row_col(int type, const uint8_t *wrow, int64_t k, const act_t *a, int64_t col, int32_t *D) {
    double acc = 0.0;
    int64_t nb32 = k / 32;
    const int8_t *qa = a->qa + col * k;
    const double *da = a->da + col * nb32;
    const double *sa = a->sa + col * nb32;

    if (type == ORC_Q4_K || type == ORC_Q5_K) {
        for (int64_t sb = 0; sb < k / 256; ++sb) {
            double d, dmin; int sc[8], m[8], code[256];
            if (type == ORC_Q4_K) decode_q4_K(wrow + sb * 144, &d, &dmin, sc, m, code);
            else decode_q5_K(wrow + sb * 176, &d, &dmin, sc, m, code);
            for (int j = 0; j < 8; ++j) {
                int64_t b = sb * 8 + j;
                int32_t Db = 0;
                for (int i = 0; i < 32; ++i) Db += code[32 * j + i] * qa[b * 32 + i];
                if (D) D[b] = Db;
                acc += d * sc[j] * da[b] * (double)Db - dmin * m[j] * sa[b];
            }
        }
    } else if (type == ORC_Q6_K || type == ORC_Q3_K) {
        for (int64_t sb = 0; sb < k / 256; ++sb) {
            double d; int sc[16], code[256];
            if (type == ORC_Q6_K) decode_q6_K(wrow + sb * 210, &d, sc, code);
            else decode_q3_K(wrow + sb * 110, &d, sc, code);
            for (int j = 0; j < 8; ++j) {           /* one q8_1 block = two 16-value sub-blocks */
                int64_t b = sb * 8 + j;
                int32_t D0 = 0, D1 = 0;
                for (int i = 0; i < 16; ++i) D0 += code[32 * j + i] * qa[b * 32 + i];
                for (int i = 16; i < 32; ++i) D1 += code[32 * j + i] * qa[b * 32 + i];
                if (D) { D[2 * b] = D0; D[2 * b + 1] = D1; }
                acc += d * da[b] * ((double)sc[2 * j] * D0 + (double)sc[2 * j + 1] * D1);
            }
        }
    } else if (type == ORC_IQ4_XS) {   /* one scale per 32-value sub-block */
        for (int64_t sb = 0; sb < k / 256; ++sb) {
            double d; int sc[8], code[256];
            decode_iq4_xs(wrow + sb * 136, &d, sc, code);
            for (int j = 0; j < 8; ++j) {
                int64_t b = sb * 8 + j;
                int32_t Db = 0;
                for (int i = 0; i < 32; ++i) Db += code[32 * j + i] * qa[b * 32 + i];
                if (D) D[b] = Db;
                acc += d * sc[j] * da[b] * (double)Db;
            }
        }
    } else { /* Q8_0, Q4_0: one scale per 32-value block */
        for (int64_t b = 0; b < nb32; ++b) {
            double d; int code[32];
            if (type == ORC_Q8_0) decode_q8_0(wrow + b * 34, &d, code);
            else decode_q4_0(wrow + b * 18, &d, code);
            int32_t Db = 0;
            for (int i = 0; i < 32; ++i) Db += code[i] * qa[b * 32 + i];
            if (D) D[b] = Db;
            acc += d * da[b] * (double)Db;
        }
    }
    return (float)acc;
}

static int check_args(int type, int64_t rows, int64_t k, int64_t n) {
    if (type_block_values(type) == 0) return ORC_ERR;
    if (rows < 0 || n < 0 || k <= 0) return ORC_ERR;
    if (k % type_block_values(type)) return ORC_ERR;
    return ORC_OK;
}

/* Y[n][rows] from weights (rows x k) and canonical q8_1 activations (n x k/32 blocks). */
int oracle_matmul_q8_1(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq,
                       int64_t n, float *y) {
    if (check_args(type, rows, k, n)) return ORC_ERR;
    int64_t rb = oracle_row_bytes(type, k);
    act_t a;
    if (act_decode(&a, xq, n, k)) { act_free(&a); return ORC_ERR; }
    int64_t total = rows * n;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t idx = 0; idx < total; ++idx) {
        int64_t r = idx % rows, c = idx / rows;
        y[c * rows + r] = dot_row_col(type, w + r * rb, k, &a, c, NULL);
    }
    act_free(&a);
    return ORC_OK;
}

/* Only the listed (column, row) outputs: out[i] = Y[cols[i]][rws[i]]. */
int oracle_matmul_q8_1_at(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq,
                          int64_t n, const int64_t *cols, const int64_t *rws, int64_t count, float *out) {
    if (check_args(type, rows, k, n)) return ORC_ERR;
    int64_t rb = oracle_row_bytes(type, k);
    for (int64_t i = 0; i < count; ++i)
        if (cols[i] < 0 || cols[i] >= n || rws[i] < 0 || rws[i] >= rows) return ORC_ERR;
    act_t a;
    if (act_decode(&a, xq, n, k)) { act_free(&a); return ORC_ERR; }
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < count; ++i)
        out[i] = dot_row_col(type, w + rws[i] * rb, k, &a, cols[i], NULL);
    act_free(&a);
    return ORC_OK;
}

/* Integer sub-block dots D[n][rows][k/32] (Q6_K: [n][rows][k/16]). */
int oracle_subdots(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n,
                   int32_t *D) {
    if (check_args(type, rows, k, n)) return ORC_ERR;
    int64_t rb = oracle_row_bytes(type, k);
    int64_t per = oracle_subdots_per_row(type, k);
    act_t a;
    if (act_decode(&a, xq, n, k)) { act_free(&a); return ORC_ERR; }
    for (int64_t c = 0; c < n; ++c)
        for (int64_t r = 0; r < rows; ++r)
            (void)dot_row_col(type, w + r * rb, k, &a, c, D + (c * rows + r) * per);
    act_free(&a);
    return ORC_OK;
}

/* Q6_K only: the scale-folded integer per 32-value q8_1 block, sc[2b]*D[2b] + sc[2b+1]*D[2b+1]
 * (the MMQ page's "Q6_K dot": two 16-value sub-blocks share one activation block).
 * Output int32 [n][rows][k/32]. */
int oracle_subdots_q6_K_folded(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n,
                               int32_t *F) {
    if (check_args(ORC_Q6_K, rows, k, n)) return ORC_ERR;
    int64_t rb = oracle_row_bytes(ORC_Q6_K, k);
    int64_t nb = k / 32;
    int32_t *D = (int32_t *)malloc(sizeof(int32_t) * (size_t)(k / 16) + 4);
    act_t a;
    if (act_decode(&a, xq, n, k)) { act_free(&a); free(D); return ORC_ERR; }
    for (int64_t c = 0; c < n; ++c)
        for (int64_t r = 0; r < rows; ++r) {
            const uint8_t *wrow = w + r * rb;
            (void)dot_row_col(ORC_Q6_K, wrow, k, &a, c, D);
            for (int64_t b = 0; b < nb; ++b) {
                const int8_t *sc = (const int8_t *)(wrow + (b / 8) * 210 + 192);
                int j = (int)(b % 8);
                F[(c * rows + r) * nb + b] = sc[2 * j] * D[2 * b] + sc[2 * j + 1] * D[2 * b + 1];
            }
        }
    act_free(&a);
    free(D);
    return ORC_OK;
}

/* Q3_K: the same folding with its scales (6-bit value - 32): sc[2b]*D[2b] + sc[2b+1]*D[2b+1]
 * per 32-value q8_1 block, D over the codes q - 4 (GP100 patch page, "How" step 3).
 * Output int32 [n][rows][k/32]. */
int oracle_subdots_q3_K_folded(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n,
                               int32_t *F) {
    if (check_args(ORC_Q3_K, rows, k, n)) return ORC_ERR;
    int64_t rb = oracle_row_bytes(ORC_Q3_K, k);
    int64_t nb = k / 32;
    int32_t *D = (int32_t *)malloc(sizeof(int32_t) * (size_t)(k / 16) + 4);
    act_t a;
    if (act_decode(&a, xq, n, k)) { act_free(&a); free(D); return ORC_ERR; }
    for (int64_t c = 0; c < n; ++c)
        for (int64_t r = 0; r < rows; ++r) {
            const uint8_t *wrow = w + r * rb;
            (void)dot_row_col(ORC_Q3_K, wrow, k, &a, c, D);
            for (int64_t sb = 0; sb < k / 256; ++sb) {
                double d; int sc[16], code[256];
                decode_q3_K(wrow + sb * 110, &d, sc, code);
                for (int j = 0; j < 8; ++j) {
                    const int64_t b = sb * 8 + j;
                    F[(c * rows + r) * nb + b] = sc[2 * j] * D[2 * b] + sc[2 * j + 1] * D[2 * b + 1];
                }
            }
        }
    act_free(&a);
    free(D);
    return ORC_OK;
}

/* fp32 activations -> q8_1 -> Y. */
int oracle_matmul(int type, const uint8_t *w, int64_t rows, int64_t k, const float *x, int64_t n,
                  float *y) {
    if (check_args(type, rows, k, n)) return ORC_ERR;
    uint8_t *xq = (uint8_t *)malloc((size_t)(n * (k / 32) * 36) + 1);
    oracle_quantize_q8_1(x, n, k, xq);
    int rc = oracle_matmul_q8_1(type, w, rows, k, xq, n, y);
    free(xq);
    return rc;
}

/* Expert-indexed product.  w: n_exp matrices of (rows x k) blocks, back to back.
 * x: fp32 [n_tok][x_per_tok][k] with x_per_tok in {1, top_k}.  ids: int32 [n_tok][top_k].
 * y: fp32 [n_tok][top_k][rows].  For each (t, slot): e = ids[t][slot]; the activation row is
 * x[t][slot] (x_per_tok == top_k) or x[t][0] (x_per_tok == 1).  An id outside [0, n_exp) leaves
 * its output row untouched and is counted in *n_invalid. */
int oracle_matmul_id(int type, const uint8_t *w, int64_t n_exp, int64_t rows, int64_t k, const float *x,
                     int64_t x_per_tok, const int32_t *ids, int64_t n_tok, int64_t top_k, float *y,
                     int64_t *n_invalid) {
    if (check_args(type, rows, k, n_tok)) return ORC_ERR;
    if (n_exp <= 0 || top_k <= 0 || (x_per_tok != 1 && x_per_tok != top_k)) return ORC_ERR;
    int64_t rb = oracle_row_bytes(type, k);
    int64_t xb = (k / 32) * 36;
    int64_t nx = n_tok * x_per_tok;
    uint8_t *xq = (uint8_t *)malloc((size_t)(nx * xb) + 1);
    oracle_quantize_q8_1(x, nx, k, xq);
    act_t a;
    if (act_decode(&a, xq, nx, k)) { act_free(&a); free(xq); return ORC_ERR; }
    int64_t bad = 0;
    for (int64_t t = 0; t < n_tok; ++t)
        for (int64_t s = 0; s < top_k; ++s) {
            int32_t e = ids[t * top_k + s];
            if (e < 0 || e >= n_exp) { bad++; continue; }
            const uint8_t *we = w + (int64_t)e * rows * rb;
            int64_t col = t * x_per_tok + (x_per_tok == 1 ? 0 : s);
            float *yo = y + (t * top_k + s) * rows;
#pragma omp parallel for schedule(static)
            for (int64_t r = 0; r < rows; ++r) yo[r] = dot_row_col(type, we + r * rb, k, &a, col, NULL);
        }
    if (n_invalid) *n_invalid = bad;
    act_free(&a);
    free(xq);
    return ORC_OK;
}

/* ---------------------------------------------------------------------------------------------
 * Gate/up products fused with SwiGLU (the "llama.cpp MMQ" page, the fusion passage after the MoE
 * dispatch: the gate and up products of one input are taken together and the GLU is applied as
 * they are written back).  The pages name SwiGLU without writing it out; read here as the usual
 *     out = silu(g) * u,   silu(g) = g / (1 + exp(-g)),
 * with g the gate product and u the up product of the same row and column.  Each product is the
 * oracle's own (above); the GLU is evaluated in fp64 from the two fp32 products and rounded once.
 * ------------------------------------------------------------------------------------------- */
static float swiglu_ref(float g, float u) {
    const double gd = (double)g;
    return (float)(gd / (1.0 + exp(-gd)) * (double)u);
}

/* y[n][rows] = silu(W_gate x) * (W_up x); both weights (rows x k) of one type. */
int oracle_matmul_glu(int type, const uint8_t *wg, const uint8_t *wu, int64_t rows, int64_t k, const float *x,
                      int64_t n, float *y) {
    if (check_args(type, rows, k, n)) return ORC_ERR;
    float *g = (float *)malloc((size_t)(n * rows) * sizeof(float) + 4);
    int rc = oracle_matmul(type, wg, rows, k, x, n, g);
    if (!rc) rc = oracle_matmul(type, wu, rows, k, x, n, y);
    if (!rc)
        for (int64_t i = 0; i < n * rows; ++i) y[i] = swiglu_ref(g[i], y[i]);
    free(g);
    return rc;
}

/* Expert form: wg, wu hold n_exp (rows x k) matrices each; x fp32 [n_tok][k] (one activation row
 * per token, shared by its top_k slots); y fp32 [n_tok][top_k][rows].  An id outside [0, n_exp)
 * leaves its output row untouched and is counted in *n_invalid. */
int oracle_matmul_id_glu(int type, const uint8_t *wg, const uint8_t *wu, int64_t n_exp, int64_t rows, int64_t k,
                         const float *x, const int32_t *ids, int64_t n_tok, int64_t top_k, float *y,
                         int64_t *n_invalid) {
    if (check_args(type, rows, k, n_tok)) return ORC_ERR;
    if (n_exp <= 0 || top_k <= 0) return ORC_ERR;
    const int64_t m = n_tok * top_k * rows;
    float *g = (float *)malloc((size_t)m * sizeof(float) + 4);
    float *u = (float *)malloc((size_t)m * sizeof(float) + 4);
    int64_t bad = 0;
    int rc = oracle_matmul_id(type, wg, n_exp, rows, k, x, 1, ids, n_tok, top_k, g, &bad);
    if (!rc) rc = oracle_matmul_id(type, wu, n_exp, rows, k, x, 1, ids, n_tok, top_k, u, NULL);
    if (!rc)
        for (int64_t p = 0; p < n_tok * top_k; ++p) {
            if (ids[p] < 0 || ids[p] >= n_exp) continue;
            for (int64_t r = 0; r < rows; ++r) y[p * rows + r] = swiglu_ref(g[p * rows + r], u[p * rows + r]);
        }
    if (n_invalid) *n_invalid = bad;
    free(g);
    free(u);
    return rc;
}

/* ---------------------------------------------------------------------------------------------
 * fp16-activation mode: encoder and product (see the header).
 * ------------------------------------------------------------------------------------------- */

/* Block prescale exponent: amax in [2^(p-1), 2^p) (frexp) -> e = 15 - p puts amax * 2^e in
 * [2^14, 2^15). */
static int f16act_exponent(double amax) {
    if (amax == 0.0) return 0;
    int p;
    frexp(amax, &p);
    return 15 - p;
}

/* x fp32 [n][k] (k % 32 == 0) -> y fp16 bit patterns [n][k], e int32 [n][k/32], block sums
 * bsum fp64 [n][k/32] (exact: 32 multiples of 2^-24 below 2^16). */
int oracle_f16act_encode(const float *x, int64_t n, int64_t k, uint16_t *y, int32_t *e, double *bsum) {
    if (n < 0 || k <= 0 || k % 32) return ORC_ERR;
    for (int64_t c = 0; c < n; ++c)
        for (int64_t b = 0; b < k / 32; ++b) {
            const float *xb = x + c * k + 32 * b;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)xb[i]));
            const int eb = f16act_exponent(amax);
            double sum = 0.0;
            for (int i = 0; i < 32; ++i) {
                const double v = ldexp((double)xb[i], eb);    /* exact */
                const uint16_t h = oracle_float_to_half((float)v);  /* v is exact as fp32 or below fp16's range */
                y[c * k + 32 * b + i] = h;
                sum += oracle_half_to_double(h);
            }
            e[c * (k / 32) + b] = eb;
            if (bsum) bsum[c * (k / 32) + b] = sum;
        }
    return ORC_OK;
}

/* Y[n][rows] = W . (fp16 activations unscaled per block), exact fp64 sums, one rounding. */
int oracle_matmul_f16act(int type, const uint8_t *w, int64_t rows, int64_t k, const float *x, int64_t n, float *y) {
    if (check_args(type, rows, k, n) || k % 32) return ORC_ERR;
    const int64_t nb = k / 32, rb = oracle_row_bytes(type, k);
    uint16_t *yh = (uint16_t *)malloc((size_t)(n * k) * 2 + 4);
    int32_t *e = (int32_t *)malloc((size_t)(n * nb) * 4 + 4);
    double *xa = (double *)malloc((size_t)(n * k) * 8 + 8);
    double *wr = (double *)malloc((size_t)k * 8);
    int rc = oracle_f16act_encode(x, n, k, yh, e, NULL);
    for (int64_t c = 0; c < n && !rc; ++c)
        for (int64_t i = 0; i < k; ++i) xa[c * k + i] = ldexp(oracle_half_to_double(yh[c * k + i]), -e[c * nb + i / 32]);
    for (int64_t r = 0; r < rows && !rc; ++r) {
        rc = oracle_dequantize(type, w + r * rb, 1, k, wr);
        for (int64_t c = 0; c < n && !rc; ++c) {
            double acc = 0.0;
            for (int64_t i = 0; i < k; ++i) acc += wr[i] * xa[c * k + i];
            y[c * rows + r] = (float)acc;
        }
    }
    free(yh);
    free(e);
    free(xa);
    free(wr);
    return rc;
}

/* ---------------------------------------------------------------------------------------------
 * Panel layout: a one-time repack of a weight matrix ("QTensor and QMatMul" page, section on the
 * 8-column Q4K repack: the blocks of adjacent rows at the same position are interleaved once, on
 * first use, into a layout the product reads faster; the original blocks are kept).  This
 * library's layout takes 16 rows and one 256-value step at a time and splits codes from scales:
 *
 *   k % 256 == 0.  G = ceil(rows / 16) row groups, S = k / 256 steps, B = bytes of 256 values in
 *   the original layout (Q4_K 144, Q5_K 176, Q6_K 210, Q8_0 272, Q4_0 144), P = 16 * B.
 *   Panel (g, s) -- rows 16g..16g+15, values 256s..256s+255 -- is the P bytes at (g*S + s) * P.
 *   Inside a panel, slab j is the 256 bytes at 256*j: one 16-byte piece for each of the 16 rows,
 *   row i's piece at 256*j + 16*i.  Slabs per type (byte ranges of the row's step in the
 *   original layout):
 *     Q4_K  slabs 0-7: qs[16j, 16j+16);   slab 8: header {d, dmin, scales[12]}
 *     Q5_K  slabs 0-1: qh[16j, +16);      slabs 2-9: qs[16(j-2), +16);  slab 10: header
 *     Q6_K  slabs 0-7: ql[16j, +16);      slabs 8-11: qh[16(j-8), +16); slab 12: scales[16];
 *           then 32 bytes: fp16 d of row i at 3328 + 2i
 *     Q8_0  slab j (0-15): qs[16(j%2), +16) of block j/2 of the step;  slab 16: the 8 blocks'
 *           fp16 d, block b at byte 2b of the row's piece
 *     Q4_0  slab j (0-7): qs[16] (nibbles) of block j;  slab 8: the 8 blocks' fp16 d as Q8_0
 *   Rows of the last group past `rows` are zero bytes.  Every byte of the original is copied
 *   unchanged (no value is re-encoded), so decoding a panel gives the original values.
 * ------------------------------------------------------------------------------------------- */
static int panel_step_bytes(int type) {
    if (type == ORC_Q4_K || type == ORC_Q4_0) return 144;
    if (type == ORC_Q5_K) return 176;
    if (type == ORC_Q6_K) return 210;
    if (type == ORC_Q8_0) return 272;
    return 0;
}

/* Offset inside a panel of byte o (0 <= o < B) of row i's step (original layout). */
static int64_t panel_offset(int type, int i, int o) {
    switch (type) {
        case ORC_Q4_K:
            if (o < 16) return 8 * 256 + 16 * i + o;
            return (o - 16) / 16 * 256 + 16 * i + (o - 16) % 16;
        case ORC_Q5_K:
            if (o < 16) return 10 * 256 + 16 * i + o;
            if (o < 48) return (o - 16) / 16 * 256 + 16 * i + (o - 16) % 16;
            return (2 + (o - 48) / 16) * 256 + 16 * i + (o - 48) % 16;
        case ORC_Q6_K:
            if (o < 128) return o / 16 * 256 + 16 * i + o % 16;
            if (o < 192) return (8 + (o - 128) / 16) * 256 + 16 * i + (o - 128) % 16;
            if (o < 208) return 12 * 256 + 16 * i + (o - 192);
            return 13 * 256 + 2 * i + (o - 208);
        case ORC_Q8_0: {
            const int b = o / 34, q = o % 34;
            if (q < 2) return 16 * 256 + 16 * i + 2 * b + q;
            return (2 * b + (q - 2) / 16) * 256 + 16 * i + (q - 2) % 16;
        }
        case ORC_Q4_0: {
            const int b = o / 18, q = o % 18;
            if (q < 2) return 8 * 256 + 16 * i + 2 * b + q;
            return b * 256 + 16 * i + (q - 2);
        }
        default:
            return -1;
    }
}

int64_t oracle_panel_bytes(int type, int64_t rows, int64_t k) {
    const int B = panel_step_bytes(type);
    if (B == 0 || rows < 1 || k < 256 || k % 256) return -1;
    return (rows + 15) / 16 * (k / 256) * 16 * B;
}

/* Offset inside a panel of byte o of row i's step: exposed for the layout pins. */
int64_t oracle_panel_offset(int type, int i, int o) {
    const int B = panel_step_bytes(type);
    if (B == 0 || i < 0 || i > 15 || o < 0 || o >= B) return -1;
    return panel_offset(type, i, o);
}

/* Original layout w [rows][k] -> panel layout out (oracle_panel_bytes bytes). */
int oracle_repack_panels(int type, const uint8_t *w, int64_t rows, int64_t k, uint8_t *out) {
    const int64_t total = oracle_panel_bytes(type, rows, k);
    if (total < 0) return ORC_ERR;
    const int64_t B = panel_step_bytes(type), S = k / 256, P = 16 * B, rb = oracle_row_bytes(type, k);
    memset(out, 0, (size_t)total);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t s = 0; s < S; ++s)
            for (int o = 0; o < B; ++o)
                out[(r / 16 * S + s) * P + panel_offset(type, (int)(r % 16), o)] = w[r * rb + s * B + o];
    return ORC_OK;
}

/* Panel layout -> fp64 values [rows][k]: each row's steps are read back from their panel
 * positions into the original byte order and decoded with the definitions above. */
int oracle_dequantize_panels(int type, const uint8_t *wp, int64_t rows, int64_t k, double *out) {
    if (oracle_panel_bytes(type, rows, k) < 0) return ORC_ERR;
    const int64_t B = panel_step_bytes(type), S = k / 256, P = 16 * B, rb = oracle_row_bytes(type, k);
    uint8_t *row = (uint8_t *)malloc((size_t)rb);
    if (!row) return ORC_ERR;
    int rc = ORC_OK;
    for (int64_t r = 0; r < rows && !rc; ++r) {
        for (int64_t s = 0; s < S; ++s)
            for (int o = 0; o < B; ++o) row[s * B + o] = wp[(r / 16 * S + s) * P + panel_offset(type, (int)(r % 16), o)];
        rc = oracle_dequantize(type, row, 1, k, out + r * k);
    }
    free(row);
    return rc;
}
