// Matrix-vector product for 1..3 activation columns with v_dot4_i32_i8 (the MMVQ regime of the
// MMQ page: "shape criteria" and the MMVQ-vs-MMQ table; "dp4a path Q4_K" section for the per
// sub-block dot and its d*sc / dmin*m*s fixup).
//
// With one to three columns a block-diagonal MFMA would spend most of its per-result fp32 fixups
// on empty columns, so this kernel works on the vector ALU and does exactly the useful work.
// A workgroup owns 16 weight rows; wave w takes the 256-value steps w, w+W, ... (W = 4, 8 or 16
// waves, chosen at launch).
// Lane 4r+g holds row r and the quarter g of the step: values 64g..64g+63, i.e. the two 32-value
// sub-blocks 2g and 2g+1 -- for Q4_K the 32 qs bytes 32g..32g+31 (low nibbles sub-block 2g, high
// nibbles 2g+1; Q5_K: the same qs bytes 32 further on, plus all 32 qh bytes, whose bits 2g and
// // 2g+1 are the fifth bits of the two sub-blocks), for Q8_0 the two 34-byte blocks, for Q4_0 the two
// 18-byte blocks (nibbles turned into int8 codes minus 8 in registers), for Q3_K the 32 qs bytes
// 32(g/2).. (2-bit codes of two 32-value rows j, shifts 2j) with all 32 hmask bytes (their third
// bits) and the 12 scale bytes, for IQ4_XS the 32 qs bytes of sub-blocks 2g and 2g+1 (4-bit
// codebook indices, looked up in registers).  Consecutive lanes of a row
// read consecutive bytes, so each quarter-wave load touches one or two cache lines.  The columns' q8_1 codes and
// fp32 (d, s) are staged once per workgroup in LDS -- read from q8_1 blocks, or, for fp32 input,
// quantized on the spot with the same arithmetic as the standalone quantize kernel (q8_1.hpp),
// which saves that kernel's launch; every lane with the same quarter reads the same LDS words (a
// broadcast).  Next step's weights load while this step computes.
//   Q4_K, Q5_K  acc += D(2g)*(d*sc)*d_a - (dmin*m)*s_a   (+ the same for sub-block 2g+1)
//   Q8_0, Q4_0  acc += D*d_w*d_a                   (both blocks)
//   IQ4_XS      acc += D*(d*(ls-32))*d_a            (both blocks)
//   Q3_K        acc += ((sc-32)*D_lo + (sc'-32)*D_hi)*d*d_a   (two 16-value sub-blocks per q8_1 block,
//               D over the codes minus 4; the GP100 patch page, "How" step 3, names the offset)
// The four quarters of a row are summed with lane shuffles, the waves in LDS in a fixed order.
// GLU (gate/up fusion, the MMQ page's fusion passage): rows 0-7 of the workgroup are 8 gate rows,
// rows 8-15 the same 8 rows of the up matrix, and the write-back applies silu(gate) * up.
// Requirements (checked by the host): K a multiple of 256; Q4_K / Q5_K weights and rows 16-byte
// aligned, Q8_0 / Q4_0 4-byte aligned, Q3_K / IQ4_XS 2-byte aligned; activations 4-byte aligned.
#include "common.hpp"
#include "launch.hpp"
#include "mv_cols.hpp"
#include "q8_1.hpp"

namespace qmm {

namespace {

constexpr int kRows = 16;
typedef u32x4 __attribute__((aligned(4))) u32x4_a4;

struct D4Args {
    int64_t rows;
    uint32_t row_bytes;   // weight bytes per row
    uint32_t nb;          // q8_1 blocks per activation row (k / 32)
    int32_t nsteps;       // 256-value steps (k / 256)
    int32_t q, r;         // steps per wave: q, plus one for waves < r
    int32_t n;            // dense column count
};

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Per-lane weight registers of one step.
template <int T> struct W4;
template <> struct W4<kQ4_K> {
    u32x4 h, q0, q1;   // header (d, dmin, scales) and qs bytes 32g..32g+31
    __device__ __forceinline__ void load(const uint8_t *base, uint32_t off, int g) {
        h = *(const u32x4 *)(base + off);
        q0 = *(const u32x4 *)(base + off + 16 + 32 * g);
        q1 = *(const u32x4 *)(base + off + 32 + 32 * g);
    }
};
template <> struct W4<kQ5_K> {
    u32x4 h, q0, q1, qh0, qh1;   // header, qs bytes 32g..32g+31 (after qh[32]), all 32 qh bytes
    __device__ __forceinline__ void load(const uint8_t *base, uint32_t off, int g) {
        h = *(const u32x4 *)(base + off);
        q0 = *(const u32x4 *)(base + off + 48 + 32 * g);
        q1 = *(const u32x4 *)(base + off + 64 + 32 * g);
        qh0 = *(const u32x4 *)(base + off + 16);
        qh1 = *(const u32x4 *)(base + off + 32);
    }
};
template <> struct W4<kQ8_0> {
    u32x4 v0, v1, v2, v3;   // bytes 68g..68g+63 of the step: {d0, q0[32], d1, q1[0..29]}
    uint32_t v4;            // bytes 68g+64..68g+67: q1[30..31] ... (the last 4 bytes)
    __device__ __forceinline__ void load(const uint8_t *base, uint32_t off, int g) {
        const uint8_t *p = base + off + 68 * g;
        v0 = *(const u32x4_a4 *)(p);
        v1 = *(const u32x4_a4 *)(p + 16);
        v2 = *(const u32x4_a4 *)(p + 32);
        v3 = *(const u32x4_a4 *)(p + 48);
        v4 = *(const uint32_t *)(p + 64);
    }
};
template <> struct W4<kQ4_0> {
    u32x4 v0, v1;   // bytes 36g..36g+31 of the step: {d0, qs0[16], d1, qs1[0..13]}
    uint32_t v4;    // bytes 36g+32..36g+35: qs1[12..15]
    __device__ __forceinline__ void load(const uint8_t *base, uint32_t off, int g) {
        const uint8_t *p = base + off + 36 * g;
        v0 = *(const u32x4_a4 *)(p);
        v1 = *(const u32x4_a4 *)(p + 16);
        v4 = *(const uint32_t *)(p + 32);
    }
};
template <> struct W4<kQ3_K> {
    u32x4 hm0, hm1, q0, q1;   // hmask[0..31]; qs[32h..32h+31], h = g/2 (values 128h + 32j + l, j = 2(g&1), +1)
    uint32_t s0, s1, s2, dbits;   // the 12 scale bytes, d
    __device__ __forceinline__ void load(const uint8_t *base, uint32_t off, int g) {
        const uint8_t *p = base + off;
        hm0 = ld16(p);
        hm1 = ld16(p + 16);
        q0 = ld16(p + 32 + 32 * (g >> 1));
        q1 = ld16(p + 48 + 32 * (g >> 1));
        s0 = ld4(p + 96);
        s1 = ld4(p + 100);
        s2 = ld4(p + 104);
        dbits = ld2(p + 108);
    }
};
template <> struct W4<kIQ4_XS> {
    uint32_t h0, h1;   // {d, scales_h}, scales_l
    u32x4 qa, qb;      // qs of sub-blocks 2g and 2g+1 (16 bytes each: low nibbles values 0-15, high 16-31)
    __device__ __forceinline__ void load(const uint8_t *base, uint32_t off, int g) {
        const uint8_t *p = base + off;
        h0 = ld4(p);
        h1 = ld4(p + 4);
        qa = ld16(p + 8 + 32 * g);
        qb = ld16(p + 24 + 32 * g);
    }
};
template <int T> struct StepBytes;
template <> struct StepBytes<kQ4_K> { static constexpr int V = 144; };
template <> struct StepBytes<kQ5_K> { static constexpr int V = 176; };
template <> struct StepBytes<kQ8_0> { static constexpr int V = 272; };
template <> struct StepBytes<kQ4_0> { static constexpr int V = 144; };
template <> struct StepBytes<kQ3_K> { static constexpr int V = 110; };
template <> struct StepBytes<kIQ4_XS> { static constexpr int V = 136; };

template <int T, int NC, bool DBG, bool EXPERT, bool F32, bool GLU>
__global__ __launch_bounds__(1024) void mmvq_dot4_kernel(const uint8_t *__restrict__ w, const uint8_t *__restrict__ w2,
                                                        const void *__restrict__ xin,
                                                        float *__restrict__ y, int32_t *__restrict__ dbg, D4Args P,
                                                        ColMap cm) {
    extern __shared__ __align__(16) uint8_t smem[];
    MvCols mc;
    if (!mv_resolve(mc, w, P.n, cm, EXPERT)) return;   // workgroup-uniform
    const int ncols = mc.ncols;                           // 1..NC
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nwaves = blockDim.x >> 6;
    const int r = lane >> 2, g = lane & 3;
    const int64_t rows = P.rows;
    const uint32_t nb = P.nb;
    static_assert(!GLU || (!DBG && !EXPERT), "the fused form is dense only");
    const int64_t row0 = (int64_t)blockIdx.x * (GLU ? kRows / 2 : kRows);
    const int rmax = (int)((rows - row0) < kRows ? (rows - row0) : kRows) - 1;
    const uint8_t *wg = mc.wbase + row0 * (int64_t)P.row_bytes;
    uint32_t woff = (uint32_t)(r < rmax ? r : rmax) * P.row_bytes;   // rows past the end re-read the last
    if constexpr (GLU) {
        // per-lane base: gate row r or up row r - 8 of output row0 + r % 8 (clamped)
        const int64_t orow = row0 + (r & 7) < rows ? row0 + (r & 7) : rows - 1;
        wg = (r < 8 ? w : w2) + orow * (int64_t)P.row_bytes;
        woff = 0;
    }
    const int my_steps = P.q + (wave < P.r ? 1 : 0);

    W4<T> cur;
    if (my_steps > 0) cur.load(wg + wave * StepBytes<T>::V, woff, g);

    // Stage the columns' q8_1 codes ([NC][nb][32 B]) and fp32 (d, s) ([NC][nb]) in LDS.
    uint8_t *acodes = smem;
    float2 *aft = (float2 *)(smem + (size_t)NC * nb * 32);
    float *red = (float *)(smem + (size_t)NC * nb * 40);   // [nwaves][16 * NC]
    if constexpr (F32) {
        // fp32 rows (dense): 4 consecutive threads quantize one block, 8 values each; nb*4 and the
        // block size are multiples of 4, so the 4 lanes of a block are active together.
        for (int c = 0; c < ncols; ++c) {
            const float *xrow = (const float *)xin + (size_t)c * nb * 32;
            for (uint32_t t = threadIdx.x; t < nb * 4; t += blockDim.x) {
                const uint32_t b = t >> 2, sub = t & 3;
                const float *src = xrow + b * 32 + 8 * sub;
                const Q81Lane4 q = quantize_q8_1_lane4(*(const float4 *)src, *(const float4 *)(src + 4));
                *(u32x2 *)(acodes + ((size_t)c * nb + b) * 32 + 8 * sub) = u32x2{q.c0, q.c1};
                if (sub == 0)
                    aft[(size_t)c * nb + b] = make_float2(h2f((uint16_t)(q.ds & 0xFFFF)), h2f((uint16_t)(q.ds >> 16)));
            }
        }
    } else {
        const uint8_t *xq = (const uint8_t *)xin;
        for (int c = 0; c < ncols; ++c) {
            const uint8_t *xrow = xq + mc.arow(c) * (int64_t)nb * kQ8_1Bytes;
            for (uint32_t b = threadIdx.x; b < nb; b += blockDim.x) {
                const uint8_t *src = xrow + (size_t)b * kQ8_1Bytes;
                const uint32_t ds = *(const uint32_t *)src;
                const u32x4 c0 = *(const u32x4_a4 *)(src + 4);
                const u32x4 c1 = *(const u32x4_a4 *)(src + 20);
                uint8_t *dst = acodes + ((size_t)c * nb + b) * 32;
                *(u32x4 *)dst = c0;
                *(u32x4 *)(dst + 16) = c1;
                aft[(size_t)c * nb + b] = make_float2(h2f((uint16_t)(ds & 0xFFFF)), h2f((uint16_t)(ds >> 16)));
            }
        }
    }
    __syncthreads();

    float acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = 0.f;
    int32_t *dbg_row = nullptr;
    int64_t dbg_ld = 0;
    constexpr int DS = kSub16<T> ? 2 : 1;   // exported dots per 32 values (Q3_K: one per 16)
    if (DBG && row0 + r < rows) {
        dbg_ld = rows * (int64_t)nb * DS;
        dbg_row = dbg + (row0 + r) * (int64_t)nb * DS;
    }

    for (int it = 0; it < my_steps; ++it) {
        const int s = wave + it * nwaves;
        const W4<T> x = cur;
        if (it + 1 < my_steps) cur.load(wg + (s + nwaves) * StepBytes<T>::V, woff, g);   // next step in flight
        const uint32_t b0 = 8 * s + 2 * g;   // q8_1 block of sub-block 2g

        if constexpr (T == kQ4_K || T == kQ5_K) {
            const float d = h2f((uint16_t)(x.h.x & 0xFFFF));
            const float dmin = h2f((uint16_t)(x.h.x >> 16));
            // 6-bit scale / min of sub-blocks 2g, 2g+1 in bytes 0, 1: sub-blocks 0-3 sit in the low
            // 6 bits of scale bytes 0-3 / 4-7, sub-blocks 4-7 in the nibbles of bytes 8-11 with
            // their top 2 bits in the top bits of bytes 0-3 / 4-7.
            const uint32_t sc_a = x.h.y & 0x3F3F3F3Fu, m_a = x.h.z & 0x3F3F3F3Fu;
            const uint32_t sc_b = (x.h.w & 0x0F0F0F0Fu) | ((x.h.y >> 2) & 0x30303030u);
            const uint32_t m_b = ((x.h.w >> 4) & 0x0F0F0F0Fu) | ((x.h.z >> 2) & 0x30303030u);
            const int sh = 16 * (g & 1);
            const uint32_t scp = (g < 2 ? sc_a : sc_b) >> sh, mp = (g < 2 ? m_a : m_b) >> sh;
            const float ws0 = d * (float)(scp & 0xFF), ws1 = d * (float)((scp >> 8) & 0xFF);
            const float wm0 = dmin * (float)(mp & 0xFF), wm1 = dmin * (float)((mp >> 8) & 0xFF);
            const uint32_t qv[8] = {x.q0.x, x.q0.y, x.q0.z, x.q0.w, x.q1.x, x.q1.y, x.q1.z, x.q1.w};
            uint32_t lo[8], hi[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                lo[i] = qv[i] & 0x0F0F0F0Fu;
                hi[i] = (qv[i] >> 4) & 0x0F0F0F0Fu;
            }
            if constexpr (T == kQ5_K) {
                // fifth bits: bit 2g (sub-block 2g) and 2g+1 of qh byte l, l = the value's position
                const uint32_t hv[8] = {x.qh0.x, x.qh0.y, x.qh0.z, x.qh0.w, x.qh1.x, x.qh1.y, x.qh1.z, x.qh1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    lo[i] |= ((hv[i] >> (2 * g)) & 0x01010101u) << 4;
                    hi[i] |= ((hv[i] >> (2 * g + 1)) & 0x01010101u) << 4;
                }
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                if (c >= ncols) break;
                const uint8_t *ab = acodes + ((size_t)c * nb + b0) * 32;
                const u32x4 a0 = *(const u32x4 *)ab, a1 = *(const u32x4 *)(ab + 16);
                const u32x4 a2 = *(const u32x4 *)(ab + 32), a3 = *(const u32x4 *)(ab + 48);
                int D0 = 0, D1 = 0;
                D0 = dot4(lo[0], a0.x, D0); D0 = dot4(lo[1], a0.y, D0); D0 = dot4(lo[2], a0.z, D0); D0 = dot4(lo[3], a0.w, D0);
                D0 = dot4(lo[4], a1.x, D0); D0 = dot4(lo[5], a1.y, D0); D0 = dot4(lo[6], a1.z, D0); D0 = dot4(lo[7], a1.w, D0);
                D1 = dot4(hi[0], a2.x, D1); D1 = dot4(hi[1], a2.y, D1); D1 = dot4(hi[2], a2.z, D1); D1 = dot4(hi[3], a2.w, D1);
                D1 = dot4(hi[4], a3.x, D1); D1 = dot4(hi[5], a3.y, D1); D1 = dot4(hi[6], a3.z, D1); D1 = dot4(hi[7], a3.w, D1);
                if (DBG) {
                    if (dbg_row) {
                        dbg_row[(int64_t)c * dbg_ld + b0] = D0;
                        dbg_row[(int64_t)c * dbg_ld + b0 + 1] = D1;
                    }
                } else {
                    const f32x4 f = *(const f32x4 *)(aft + (size_t)c * nb + b0);   // d0, s0, d1, s1
                    float a = acc[c];
                    a = fmaf((float)D0, ws0 * f.x, a);
                    a = fmaf(-wm0, f.y, a);
                    a = fmaf((float)D1, ws1 * f.z, a);
                    a = fmaf(-wm1, f.w, a);
                    acc[c] = a;
                }
            }
        } else if constexpr (T == kQ3_K) {
            // quarter g: h = g/2, j = 2(g&1) + jj for the q8_1 blocks b0 + jj (jj = 0, 1); value
            // 128h + 32j + l takes bits 2j of qs[32h + l] and bit 4h + j of hmask[l], minus 4
            // ((c + 124) ^ 128 per byte: c - 4 as int8, no carry between bytes).  Sub-block t =
            // 4g + 2jj + (l >= 16): low 4 scale bits in nibble h of scale byte 4(g&1) + 2jj + (l >= 16),
            // top 2 bits at 2g of byte 8 + 2jj + (l >= 16).
            const int h = g >> 1;
            const float d = h2f((uint16_t)x.dbits);
            const uint32_t sl = (g & 1) ? x.s1 : x.s0;
            const uint32_t qv[8] = {x.q0.x, x.q0.y, x.q0.z, x.q0.w, x.q1.x, x.q1.y, x.q1.z, x.q1.w};
            const uint32_t hv[8] = {x.hm0.x, x.hm0.y, x.hm0.z, x.hm0.w, x.hm1.x, x.hm1.y, x.hm1.z, x.hm1.w};
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int j = 2 * (g & 1) + jj, hb = 4 * h + j;
                uint32_t cv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    cv[i] = ((((qv[i] >> (2 * j)) & 0x03030303u) | (((hv[i] >> hb) & 0x01010101u) << 2)) + 0x7C7C7C7Cu) ^
                            0x80808080u;
                int sc[2];
#pragma unroll
                for (int lh = 0; lh < 2; ++lh) {
                    const int bsel = 8 * (2 * jj + lh);
                    sc[lh] = (int)(((sl >> (bsel + 4 * h)) & 15u) | (((x.s2 >> (bsel + 2 * g)) & 3u) << 4)) - 32;
                }
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    if (c >= ncols) break;
                    const uint8_t *ab = acodes + ((size_t)c * nb + b0 + jj) * 32;
                    const u32x4 a0 = *(const u32x4 *)ab, a1 = *(const u32x4 *)(ab + 16);
                    int Dl = 0, Dh = 0;
                    Dl = dot4(cv[0], a0.x, Dl); Dl = dot4(cv[1], a0.y, Dl); Dl = dot4(cv[2], a0.z, Dl); Dl = dot4(cv[3], a0.w, Dl);
                    Dh = dot4(cv[4], a1.x, Dh); Dh = dot4(cv[5], a1.y, Dh); Dh = dot4(cv[6], a1.z, Dh); Dh = dot4(cv[7], a1.w, Dh);
                    if (DBG) {
                        if (dbg_row) {
                            dbg_row[(int64_t)c * dbg_ld + 2 * (b0 + jj)] = Dl;
                            dbg_row[(int64_t)c * dbg_ld + 2 * (b0 + jj) + 1] = Dh;
                        }
                    } else {
                        // (sc_lo D_lo + sc_hi D_hi) is exact in int32 (|D| <= 16 * 4 * 127) and in fp32
                        const float da = aft[(size_t)c * nb + b0 + jj].x;
                        acc[c] = fmaf((float)(sc[0] * Dl + sc[1] * Dh), d * da, acc[c]);
                    }
                }
            }
        } else if constexpr (T == kIQ4_XS) {
            // sub-blocks 2g (qa) and 2g+1 (qb) = q8_1 blocks b0, b0 + 1; low nibbles are values
            // 0-15, high nibbles 16-31, each an index into the codebook; 6-bit scale of sub-block b:
            // nibble b&1 of scales_l byte b/2 (= g), top bits at 2b of scales_h, minus 32
            const float d = h2f((uint16_t)(x.h0 & 0xFFFF));
            const uint32_t sh = x.h0 >> 16, sl = x.h1 >> (8 * g);
            const float ws0 = d * (float)((int)((sl & 15u) | (((sh >> (4 * g)) & 3u) << 4)) - 32);
            const float ws1 = d * (float)((int)(((sl >> 4) & 15u) | (((sh >> (4 * g + 2)) & 3u) << 4)) - 32);
            const uint32_t av[4] = {x.qa.x, x.qa.y, x.qa.z, x.qa.w}, bv[4] = {x.qb.x, x.qb.y, x.qb.z, x.qb.w};
            uint32_t q0[8], q1[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                q0[i] = iq4_lookup4(av[i] & 0x0F0F0F0Fu);
                q0[4 + i] = iq4_lookup4((av[i] >> 4) & 0x0F0F0F0Fu);
                q1[i] = iq4_lookup4(bv[i] & 0x0F0F0F0Fu);
                q1[4 + i] = iq4_lookup4((bv[i] >> 4) & 0x0F0F0F0Fu);
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                if (c >= ncols) break;
                const uint8_t *ab = acodes + ((size_t)c * nb + b0) * 32;
                const u32x4 a0 = *(const u32x4 *)ab, a1 = *(const u32x4 *)(ab + 16);
                const u32x4 a2 = *(const u32x4 *)(ab + 32), a3 = *(const u32x4 *)(ab + 48);
                int D0 = 0, D1 = 0;
                D0 = dot4(q0[0], a0.x, D0); D0 = dot4(q0[1], a0.y, D0); D0 = dot4(q0[2], a0.z, D0); D0 = dot4(q0[3], a0.w, D0);
                D0 = dot4(q0[4], a1.x, D0); D0 = dot4(q0[5], a1.y, D0); D0 = dot4(q0[6], a1.z, D0); D0 = dot4(q0[7], a1.w, D0);
                D1 = dot4(q1[0], a2.x, D1); D1 = dot4(q1[1], a2.y, D1); D1 = dot4(q1[2], a2.z, D1); D1 = dot4(q1[3], a2.w, D1);
                D1 = dot4(q1[4], a3.x, D1); D1 = dot4(q1[5], a3.y, D1); D1 = dot4(q1[6], a3.z, D1); D1 = dot4(q1[7], a3.w, D1);
                if (DBG) {
                    if (dbg_row) {
                        dbg_row[(int64_t)c * dbg_ld + b0] = D0;
                        dbg_row[(int64_t)c * dbg_ld + b0 + 1] = D1;
                    }
                } else {
                    const f32x4 f = *(const f32x4 *)(aft + (size_t)c * nb + b0);   // d0, s0, d1, s1
                    float a = acc[c];
                    a = fmaf((float)D0, ws0 * f.x, a);
                    a = fmaf((float)D1, ws1 * f.z, a);
                    acc[c] = a;
                }
            }
        } else {
            // the lane's two blocks as int8 codes q0[32 B], q1[32 B] and their scales
            uint32_t q0[8], q1[8];
            float dw0, dw1;
            if constexpr (T == kQ8_0) {
                // bytes 0-1: d0; 2-33: q0; 34-35: d1; 36-67: q1 -> q0 realigned by two bytes
                const uint32_t v[17] = {x.v0.x, x.v0.y, x.v0.z, x.v0.w, x.v1.x, x.v1.y, x.v1.z, x.v1.w,
                                        x.v2.x, x.v2.y, x.v2.z, x.v2.w, x.v3.x, x.v3.y, x.v3.z, x.v3.w, x.v4};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    q0[i] = __builtin_amdgcn_alignbyte(v[i + 1], v[i], 2);
                    q1[i] = v[9 + i];
                }
                dw0 = h2f((uint16_t)(v[0] & 0xFFFF));
                dw1 = h2f((uint16_t)(v[8] >> 16));
            } else {
                // Q4_0 bytes 0-1: d0; 2-17: qs0; 18-19: d1; 20-35: qs1.  Value i of a block is the
                // low nibble of byte i, value i + 16 the high nibble; code = nibble - 8, which per
                // byte is (nibble + 120) ^ 0x80
                const uint32_t v[9] = {x.v0.x, x.v0.y, x.v0.z, x.v0.w, x.v1.x, x.v1.y, x.v1.z, x.v1.w, x.v4};
                auto c4 = [](uint32_t nib) { return (nib + 0x78787878u) ^ 0x80808080u; };
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t n0 = __builtin_amdgcn_alignbyte(v[i + 1], v[i], 2), n1 = v[5 + i];
                    q0[i] = c4(n0 & 0x0F0F0F0Fu);
                    q0[4 + i] = c4((n0 >> 4) & 0x0F0F0F0Fu);
                    q1[i] = c4(n1 & 0x0F0F0F0Fu);
                    q1[4 + i] = c4((n1 >> 4) & 0x0F0F0F0Fu);
                }
                dw0 = h2f((uint16_t)(v[0] & 0xFFFF));
                dw1 = h2f((uint16_t)(v[4] >> 16));
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                if (c >= ncols) break;
                const uint8_t *ab = acodes + ((size_t)c * nb + b0) * 32;
                const u32x4 a0 = *(const u32x4 *)ab, a1 = *(const u32x4 *)(ab + 16);
                const u32x4 a2 = *(const u32x4 *)(ab + 32), a3 = *(const u32x4 *)(ab + 48);
                int D0 = 0, D1 = 0;
                D0 = dot4(q0[0], a0.x, D0); D0 = dot4(q0[1], a0.y, D0); D0 = dot4(q0[2], a0.z, D0); D0 = dot4(q0[3], a0.w, D0);
                D0 = dot4(q0[4], a1.x, D0); D0 = dot4(q0[5], a1.y, D0); D0 = dot4(q0[6], a1.z, D0); D0 = dot4(q0[7], a1.w, D0);
                D1 = dot4(q1[0], a2.x, D1); D1 = dot4(q1[1], a2.y, D1); D1 = dot4(q1[2], a2.z, D1); D1 = dot4(q1[3], a2.w, D1);
                D1 = dot4(q1[4], a3.x, D1); D1 = dot4(q1[5], a3.y, D1); D1 = dot4(q1[6], a3.z, D1); D1 = dot4(q1[7], a3.w, D1);
                if (DBG) {
                    if (dbg_row) {
                        dbg_row[(int64_t)c * dbg_ld + b0] = D0;
                        dbg_row[(int64_t)c * dbg_ld + b0 + 1] = D1;
                    }
                } else {
                    const f32x4 f = *(const f32x4 *)(aft + (size_t)c * nb + b0);   // d0, s0, d1, s1
                    float a = acc[c];
                    a = fmaf((float)D0, dw0 * f.x, a);
                    a = fmaf((float)D1, dw1 * f.z, a);
                    acc[c] = a;
                }
            }
        }
    }
    if (DBG) return;

    // Sum the four quarters of each row (lanes 4r..4r+3), then the waves.
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        float v = acc[c];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        acc[c] = v;
    }
    if (g == 0) {
#pragma unroll
        for (int c = 0; c < NC; ++c) red[wave * (16 * NC) + r * NC + c] = acc[c];
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t >= (GLU ? 8 : 16) * NC) return;
    float v = 0.f, u = 0.f;
    for (int wv = 0; wv < nwaves; ++wv) {
        v += red[wv * (16 * NC) + t];
        if (GLU) u += red[wv * (16 * NC) + 8 * NC + t];   // the up row of the same output
    }
    const int rr = t / NC, c = t - rr * NC;
    if (c < ncols && row0 + rr < rows) y[mc.pair(c) * rows + row0 + rr] = GLU ? v / (1.0f + expf(-v)) * u : v;
}

template <int T, int NC, bool DBG, bool EXPERT, bool F32 = false, bool GLU = false>
hipError_t launch_nc(const uint8_t *w, int64_t rows, int64_t k, const void *xq, int64_t n, float *y, int32_t *dbg,
                     const ColMap &cm, int64_t n_exp, hipStream_t s, const uint8_t *w2 = nullptr) {
    const int64_t nsteps = k / kSuper;
    constexpr int RW = GLU ? kRows / 2 : kRows;   // outputs per workgroup
    const int64_t wgs = (rows + RW - 1) / RW * (EXPERT ? n_exp : 1);
    // Waves per workgroup (each takes steps w, w+W, ... with the next step's weights in flight):
    // 8 by default, 4 for two or three columns once there are two workgroups per compute unit,
    // 16 for one-column Q8_0 (its 4-byte pieces want the most loads in flight per workgroup).
    // Fewer waves per workgroup let more workgroups share a compute unit, so one workgroup's
    // staging and quantization overlaps another's weight loads (Q4_K 14336x4096 at 1 / 3 columns
    // 11.5 -> 9.9 / 21.8 -> 14.7 us against 16 waves).
    int nw = T == kQ8_0 && NC == 1 ? 16 : NC >= 2 && wgs >= 2 * (int64_t)device_cus() ? 4 : 8;
    if (nw > nsteps) nw = (int)nsteps;
    D4Args a;
    a.rows = rows;
    a.row_bytes = (uint32_t)((k / Fmt<T>::QK) * Fmt<T>::BYTES);
    a.nb = (uint32_t)(k / 32);
    a.nsteps = (int32_t)nsteps;
    a.q = (int32_t)(nsteps / nw);
    a.r = (int32_t)(nsteps % nw);
    a.n = (int32_t)n;
    const size_t smem = (size_t)NC * a.nb * 40 + (size_t)nw * 16 * NC * sizeof(float);
    // once per process (a function-local static is initialised exactly once, thread-safely)
    static const hipError_t attr_err = hipFuncSetAttribute((const void *)mmvq_dot4_kernel<T, NC, DBG, EXPERT, F32, GLU>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr_err != hipSuccess) return attr_err;
    dim3 grid((unsigned)((rows + RW - 1) / RW), EXPERT ? (unsigned)n_exp : 1u);
    hipLaunchKernelGGL((mmvq_dot4_kernel<T, NC, DBG, EXPERT, F32, GLU>), grid, dim3(64 * (unsigned)nw), smem, s, w, w2,
                       xq, y, dbg, a, cm);
    return hipGetLastError();
}

template <int T, int NC>
hipError_t dispatch_nc(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y, int32_t *dbg,
                       const ColMap *cm, int64_t n_exp, hipStream_t s) {
    const ColMap c = cm ? *cm : ColMap{};
    if (dbg) return launch_nc<T, NC, true, false>(w, rows, k, xq, n, y, dbg, c, n_exp, s);
    if (cm) return launch_nc<T, NC, false, true>(w, rows, k, xq, n, y, dbg, c, n_exp, s);
    return launch_nc<T, NC, false, false>(w, rows, k, xq, n, y, dbg, c, n_exp, s);
}

template <int T>
hipError_t dispatch(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y, int32_t *dbg,
                    const ColMap *cm, int64_t n_exp, int max_cols, hipStream_t s) {
    if (max_cols <= 1) return dispatch_nc<T, 1>(w, rows, k, xq, n, y, dbg, cm, n_exp, s);
    if (max_cols == 2) return dispatch_nc<T, 2>(w, rows, k, xq, n, y, dbg, cm, n_exp, s);
    return dispatch_nc<T, 3>(w, rows, k, xq, n, y, dbg, cm, n_exp, s);
}

}  // namespace

int mmvq_dot4_max_cols() { return 3; }

bool mmvq_dot4_supported(int type, const void *w, int64_t k, const void *xq, const ColMap *cm) {
    if (type != kQ4_K && type != kQ5_K && type != kQ8_0 && type != kQ4_0 && type != kQ3_K && type != kIQ4_XS)
        return false;
    if (k % kSuper != 0 || k < kSuper || k > 32768) return false;
    const int64_t row_bytes = type == kQ8_0   ? k / 32 * 34
                              : type == kQ4_0 ? k / 32 * 18
                                              : k / 256 * (type == kQ5_K ? 176 : type == kQ3_K ? 110 : type == kIQ4_XS ? 136 : 144);
    // Q3_K and IQ4_XS read every piece with 2-byte-aligned loads
    const int align = type == kQ8_0 || type == kQ4_0 ? 4 : type == kQ3_K || type == kIQ4_XS ? 2 : 16;
    if (row_bytes % align != 0 || (uintptr_t)w % align != 0) return false;
    if ((uintptr_t)xq % 4 != 0) return false;
    if (cm && cm->w_expert_stride % align != 0) return false;
    return true;
}

hipError_t launch_mmvq_dot4(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n,
                            float *y, int32_t *dbg, const ColMap *cm, int64_t n_exp, int max_cols, hipStream_t s) {
    if (type == kQ4_K) return dispatch<kQ4_K>(w, rows, k, xq, n, y, dbg, cm, n_exp, max_cols, s);
    if (type == kQ5_K) return dispatch<kQ5_K>(w, rows, k, xq, n, y, dbg, cm, n_exp, max_cols, s);
    if (type == kQ8_0) return dispatch<kQ8_0>(w, rows, k, xq, n, y, dbg, cm, n_exp, max_cols, s);
    if (type == kQ4_0) return dispatch<kQ4_0>(w, rows, k, xq, n, y, dbg, cm, n_exp, max_cols, s);
    if (type == kQ3_K) return dispatch<kQ3_K>(w, rows, k, xq, n, y, dbg, cm, n_exp, max_cols, s);
    if (type == kIQ4_XS) return dispatch<kIQ4_XS>(w, rows, k, xq, n, y, dbg, cm, n_exp, max_cols, s);
    return hipErrorInvalidValue;
}

hipError_t launch_mmvq_dot4_f32(int type, const uint8_t *w, int64_t rows, int64_t k, const float *x, int64_t n,
                                float *y, hipStream_t s) {
    const ColMap c{};
#define QMM_D4F(TT)                                                                                            \
    if (type == TT) {                                                                                         \
        if (n <= 1) return launch_nc<TT, 1, false, false, true>(w, rows, k, x, n, y, nullptr, c, 0, s);     \
        if (n == 2) return launch_nc<TT, 2, false, false, true>(w, rows, k, x, n, y, nullptr, c, 0, s);     \
        return launch_nc<TT, 3, false, false, true>(w, rows, k, x, n, y, nullptr, c, 0, s);                  \
    }
    QMM_D4F(kQ4_K)
    QMM_D4F(kQ5_K)
    QMM_D4F(kQ8_0)
    QMM_D4F(kQ4_0)
    QMM_D4F(kQ3_K)
    QMM_D4F(kIQ4_XS)
#undef QMM_D4F
    return hipErrorInvalidValue;
}

hipError_t launch_mmvq_dot4_glu_f32(int type, const uint8_t *wg, const uint8_t *wu, int64_t rows, int64_t k,
                                    const float *x, int64_t n, float *y, hipStream_t s) {
    const ColMap c{};
#define QMM_D4G(TT)                                                                                            \
    if (type == TT) {                                                                                         \
        if (n <= 1) return launch_nc<TT, 1, false, false, true, true>(wg, rows, k, x, n, y, nullptr, c, 0, s, wu); \
        if (n == 2) return launch_nc<TT, 2, false, false, true, true>(wg, rows, k, x, n, y, nullptr, c, 0, s, wu); \
        return launch_nc<TT, 3, false, false, true, true>(wg, rows, k, x, n, y, nullptr, c, 0, s, wu);              \
    }
    QMM_D4G(kQ4_K)
    QMM_D4G(kQ5_K)
    QMM_D4G(kQ8_0)
    QMM_D4G(kQ4_0)
    QMM_D4G(kQ3_K)
    QMM_D4G(kIQ4_XS)
#undef QMM_D4G
    return hipErrorInvalidValue;
}

}  // namespace qmm
