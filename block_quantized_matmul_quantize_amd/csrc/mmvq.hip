// Matrix-vector product for 1..8 activation columns (the MMVQ regime of the MMQ page: "shape
// criteria" and the MMVQ-vs-MMQ table -- decode is bound by how fast the weights stream, every
// weight byte is read once and serves all columns; GP100 patch page, "Coverage": multi-column
// kernels unpack each weight once and reuse it for every column).
//
// CDNA4 design.  A workgroup owns 16 weight rows and W waves; wave w handles the 256-value
// steps w, w+W, ... (SPW of them per pass), issuing every load of the pass before any math so
// the math of early steps overlaps the arrival of later ones.  Each 64-value slice of K is one
// v_mfma_i32_16x16x64_i8: B = 16 weight rows (4 lanes per row), A = activations arranged
// block-diagonally over (column, sub-block) so that all 16 result columns are useful and every
// int32 result is one exact sub-block dot D:
//   Q4_K, Q8_0: 8 columns x 2 sub-blocks of 32 values per MFMA;
//   Q6_K:       4 columns x 4 sub-blocks of 16 values per MFMA (its scale changes every 16
//               values, "Q6_K dot" section); 5..8 columns use a second MFMA.
// Weight loads: per load instruction the 4 lanes of a row read one contiguous 64-byte run; the
// K-slot assignment of each MFMA follows whatever bytes a lane holds (any consistent slot order
// gives the same contraction).  Off-diagonal activation lanes read a 16-byte zero block, and
// row indices are clamped, so the loop has no per-lane branches.
// fp32 fixups per lane ("dp4a path Q4_K" section):
//   Q4_K  acc += D * (d*sc) * d_a - (dmin*m) * s_a
//   Q6_K  acc += D * (d*sc) * d_a      with D = sum q6*q_a - 32*sum q_a (a second MFMA against a
//                                       constant -32 operand, chained through the accumulator)
//   Q8_0  acc += D * d_w * d_a
// Partial sums are combined with lane shuffles, then across waves in LDS in a fixed order.
// GLU (gate/up fusion, the MMQ page's fusion passage): the workgroup's 16 rows are 8 gate rows
// (lanes r16 < 8) and the same 8 rows of the up matrix (r16 >= 8); the write-back applies
// silu(gate) * up.
#include "common.hpp"
#include "launch.hpp"
#include "mv_cols.hpp"

namespace qmm {

constexpr int kMvRows = 16;

// 16 zero bytes: the A operand of lanes outside the block diagonal or beyond the live columns.
__device__ __attribute__((aligned(16))) uint8_t mv_zero16[16];

__device__ __forceinline__ uint32_t nib_lo(uint32_t v) { return v & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t nib_hi(uint32_t v) { return (v >> 4) & 0x0F0F0F0Fu; }
__device__ __forceinline__ u32x4 nib_lo4(u32x4 v) { return u32x4{nib_lo(v.x), nib_lo(v.y), nib_lo(v.z), nib_lo(v.w)}; }
__device__ __forceinline__ u32x4 nib_hi4(u32x4 v) { return u32x4{nib_hi(v.x), nib_hi(v.y), nib_hi(v.z), nib_hi(v.w)}; }
__device__ __forceinline__ u32x4 sel4(bool c, u32x4 a, u32x4 b) { return c ? a : b; }

// Per-lane constants shared by every step.
struct MvLane {
    int g, r16;                 // K-slot group (lane / 16) and row within the 16-row group
    uint32_t wrow_off;          // byte offset of this lane's (clamped) row from the group base
    const uint8_t *abase[2];    // activation row of this lane's A column (or the zero block)
    int64_t astride[2];         // bytes per 256-value step of that row (0 for the zero block)
    uint32_t aoff[2][4];        // byte offset, within a step, of this lane's A piece per MFMA
};

template <int T> struct MvStep;

// ------------------------------------------------------------------------------------------
// Q4_K: 144-byte super-block = {d, dmin, 12 scale bytes, qs[128]}; piece p = bytes 16p..16p+15.
// Lane g of a row loads pieces g and 4+g (two 64-byte runs per row), the last piece and the
// header (same address for the row's 4 lanes).  32 qs bytes serve 64 values: low nibbles the
// first sub-block of the pair, high nibbles the second.  MFMA j covers sub-blocks
//   j=0: {0, 2} (low nibbles of src1), j=1: {1, 3} (high, src1),
//   j=2: {4, 6} (low, src2),           j=3: {5, 7} (high, src2),
// src1 = g==0 ? piece 4 : piece g, src2 = g==0 ? piece 8 : piece 4+g; lanes g = 1, 2 carry the
// first sub-block of the pair (values 0-15 / 16-31) and g = 3, 0 the second.
// ------------------------------------------------------------------------------------------
// Q5_K (176 bytes: the Q4_K header, qh[32], then qs[128] as Q4_K's) takes the same pieces 32
// bytes further on and ORs the fifth bits in: lane g's bytes hold values 16*half(g).. of its
// sub-blocks 2*group(g) + (j&1) + 4*(j>>1) (MFMA j), whose fifth bits are bit (sub-block) of qh
// bytes 16*half(g)..16*half(g)+15.
template <int T> struct MvStepK45 {
    static constexpr int NCG = 1;
    static constexpr int BYTES = Fmt<T>::BYTES;
    static constexpr int QS = T == kQ5_K ? 48 : 16;   // qs offset in the super-block
    u32x4 pa, pb, pc, hdr, qh;
    u32x4 a[4];

    // K-slot group of lane g for the block diagonal: 0 for g in {1,2}, 1 for g in {3,0}; the half
    // of the sub-block it carries: values 0-15 for g in {1,3}, 16-31 for g in {0,2}.
    __device__ static int group(int g) { return (g == 1 || g == 2) ? 0 : 1; }
    __device__ static int half(int g) { return (g & 1) ? 0 : 1; }
    // sub-block of MFMA j for diagonal half sel
    __device__ static int subblock(int j, int sel) {
        const int base = (j >> 1) * 4 + (j & 1);
        return base + 2 * sel;
    }
    __device__ static void lane_setup(MvLane &L, int m) {
        const int sel = m >> 3;
        for (int j = 0; j < 4; ++j)
            L.aoff[0][j] = (uint32_t)(subblock(j, sel) * kQ8_1Bytes + 4 + 16 * half(L.g));
    }
    __device__ static bool a_diag(int g, int m) { return group(g) == (m >> 3); }
    __device__ static int a_col(int m, int) { return m & 7; }

    __device__ __forceinline__ void load(const uint8_t *wg, const MvLane &L, int64_t step) {
        const uint8_t *blk = wg + L.wrow_off + step * BYTES;
        pa = ld16(blk + (QS - 16) + 16 * L.g);
        pb = ld16(blk + (QS + 48) + 16 * L.g);
        pc = ld16(blk + (QS + 112));
        hdr = ld16(blk);
        if constexpr (T == kQ5_K) qh = ld16(blk + 16 + 16 * half(L.g));
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = ld16(L.abase[0] + step * L.astride[0] + L.aoff[0][j]);
    }

    template <bool DBG>
    __device__ __forceinline__ void compute(int64_t step, const MvLane &L, const float2 *sTab, float (&acc)[NCG][4],
                                            int32_t *dbg_row, int64_t dbg_ld, int ncols) const {
        const int g = L.g, sel = g >> 1;
        const float d = h2f((uint16_t)(hdr.x & 0xFFFF));
        const float dmin = h2f((uint16_t)(hdr.x >> 16));
        // 6-bit scales/mins as bytes: j<4 in the low 6 bits of bytes j / j+4, j>=4 split over the
        // low/high nibble of byte j+4 and the top bits of bytes j-4 / j.
        const uint32_t sc_lo = (hdr.y & 0x3F3F3F3Fu) >> (16 * sel);
        const uint32_t m_lo = (hdr.z & 0x3F3F3F3Fu) >> (16 * sel);
        const uint32_t sc_hi = ((hdr.w & 0x0F0F0F0Fu) | ((hdr.y >> 2) & 0x30303030u)) >> (16 * sel);
        const uint32_t m_hi = (((hdr.w >> 4) & 0x0F0F0F0Fu) | ((hdr.z >> 2) & 0x30303030u)) >> (16 * sel);
        const u32x4 src1 = sel4(g == 0, pb, pa), src2 = sel4(g == 0, pc, pb);
        u32x4 bop[4] = {nib_lo4(src1), nib_hi4(src1), nib_lo4(src2), nib_hi4(src2)};
        if constexpr (T == kQ5_K) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sbb = 2 * group(g) + (j & 1) + 4 * (j >> 1);
                bop[j].x |= ((qh.x >> sbb) & 0x01010101u) << 4;
                bop[j].y |= ((qh.y >> sbb) & 0x01010101u) << 4;
                bop[j].z |= ((qh.z >> sbb) & 0x01010101u) << 4;
                bop[j].w |= ((qh.w >> sbb) & 0x01010101u) << 4;
            }
        }
        const i32x4 zero = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const i32x4 D = mfma16x16x64(a[j], bop[j], zero);
            const int sb = subblock(j, sel);
            const int64_t blk = step * 8 + sb;
            if (DBG) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 4 * (g & 1) + e;
                    if (dbg_row && c < ncols) dbg_row[(int64_t)c * dbg_ld + blk] = D[e];
                }
            } else {
                const uint32_t scw = j < 2 ? sc_lo : sc_hi, mw = j < 2 ? m_lo : m_hi;
                const float ws = d * (float)((scw >> (8 * (j & 1))) & 0xFF);
                const float wm = dmin * (float)((mw >> (8 * (j & 1))) & 0xFF);
                const f32x4 t0 = *(const f32x4 *)(sTab + blk * 8 + 4 * (g & 1));
                const f32x4 t1 = *(const f32x4 *)(sTab + blk * 8 + 4 * (g & 1) + 2);
                acc[0][0] += (float)D[0] * (ws * t0.x) - wm * t0.y;
                acc[0][1] += (float)D[1] * (ws * t0.z) - wm * t0.w;
                acc[0][2] += (float)D[2] * (ws * t1.x) - wm * t1.y;
                acc[0][3] += (float)D[3] * (ws * t1.z) - wm * t1.w;
            }
        }
    }
};

template <> struct MvStep<kQ4_K> : MvStepK45<kQ4_K> {};
template <> struct MvStep<kQ5_K> : MvStepK45<kQ5_K> {};

// ------------------------------------------------------------------------------------------
// Q6_K: 210-byte super-block = {ql[128], qh[64], int8 scales[16], d}.  Value v: half h = v/128,
// u = v%128, quarter q = u/32, l = u%32; low 4 bits = nibble (q<2 ? low : high) of
// ql[64h + 32(q&1) + l], top 2 bits = bits 2q..2q+1 of qh[32h + l]; code = 6-bit value - 32
// (the MMQ page's Q6_K load pairs ql word txi with qh word 8*(txi/16) + txi%8 shifted by
// (txi&8)>>2, which this mapping reproduces).  Lane g of a row loads ql[16g..] and
// ql[64+16g..] and qh[16g..] (64-byte runs); MFMA p covers values 64p..64p+63, lane g the
// 16-value sub-block 4p+g, whose qh bytes sit in lane 2*(p/2) + (g&1) -- this lane or its
// xor-32 partner.
// ------------------------------------------------------------------------------------------
template <> struct MvStep<kQ6_K> {
    static constexpr int NCG = 2;
    static constexpr int BYTES = 210;
    u32x4 ql0, ql1, qh, scv;
    uint32_t dbits;
    u32x4 a[2][4];

    __device__ static void lane_setup(MvLane &L, int m) {
        const int grp = m >> 2;                  // the 16-value sub-block this A row covers
        for (int p = 0; p < 4; ++p) {
            const uint32_t off = (uint32_t)((2 * p + (grp >> 1)) * kQ8_1Bytes + 4 + 16 * (grp & 1));
            L.aoff[0][p] = off;
            L.aoff[1][p] = off;
        }
    }
    __device__ static bool a_diag(int g, int m) { return g == (m >> 2); }
    __device__ static int a_col(int m, int cg) { return (m & 3) + 4 * cg; }

    __device__ __forceinline__ void load(const uint8_t *wg, const MvLane &L, int64_t step) {
        const uint8_t *blk = wg + L.wrow_off + step * BYTES;
        ql0 = ld16(blk + 16 * L.g);
        ql1 = ld16(blk + 64 + 16 * L.g);
        qh = ld16(blk + 128 + 16 * L.g);
        scv = ld16(blk + 192);
        dbits = ld2(blk + 208);
#pragma unroll
        for (int cg = 0; cg < 2; ++cg)
#pragma unroll
            for (int p = 0; p < 4; ++p) a[cg][p] = ld16(L.abase[cg] + step * L.astride[cg] + L.aoff[cg][p]);
    }

    template <bool DBG>
    __device__ __forceinline__ void compute(int64_t step, const MvLane &L, const float2 *sTab, float (&acc)[NCG][4],
                                            int32_t *dbg_row, int64_t dbg_ld, int ncols) const {
        const int g = L.g;
        const float d = h2f((uint16_t)dbits);
        // qh bytes of half h live in lanes 2h + (g&1): fetch the partner's (xor 32) copy.
        u32x4 qh_x;
        qh_x.x = (uint32_t)__shfl_xor((int)qh.x, 32);
        qh_x.y = (uint32_t)__shfl_xor((int)qh.y, 32);
        qh_x.z = (uint32_t)__shfl_xor((int)qh.z, 32);
        qh_x.w = (uint32_t)__shfl_xor((int)qh.w, 32);
        const u32x4 qh_h0 = (g >> 1) == 0 ? qh : qh_x;     // qh[16(g&1)..] of half 0
        const u32x4 qh_h1 = (g >> 1) == 1 ? qh : qh_x;     // qh[32 + 16(g&1)..] of half 1
        const u32x4 neg32 = {0xE0E0E0E0u, 0xE0E0E0E0u, 0xE0E0E0E0u, 0xE0E0E0E0u};
        const i32x4 zero = {0, 0, 0, 0};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int odd = p & 1;
            const u32x4 L4 = (p >> 1) ? ql1 : ql0;
            const u32x4 H4 = (p >> 1) ? qh_h1 : qh_h0;
            const int tsh = 4 * odd + 2 * (g >> 1);
            u32x4 b;   // stored 6-bit values (0..63)
            b.x = ((L4.x >> (4 * odd)) & 0x0F0F0F0Fu) | (((H4.x >> tsh) << 4) & 0x30303030u);
            b.y = ((L4.y >> (4 * odd)) & 0x0F0F0F0Fu) | (((H4.y >> tsh) << 4) & 0x30303030u);
            b.z = ((L4.z >> (4 * odd)) & 0x0F0F0F0Fu) | (((H4.z >> tsh) << 4) & 0x30303030u);
            b.w = ((L4.w >> (4 * odd)) & 0x0F0F0F0Fu) | (((H4.w >> tsh) << 4) & 0x30303030u);
            const uint32_t scw = p == 0 ? scv.x : p == 1 ? scv.y : p == 2 ? scv.z : scv.w;
            const float ws = d * (float)((int32_t)(scw << (24 - 8 * g)) >> 24);   // scale of sub-block 4p+g
            const int64_t blk = step * 8 + 2 * p + (g >> 1);   // q8_1 block of this lane's sub-block
#pragma unroll
            for (int cg = 0; cg < NCG; ++cg) {
                if (cg * 4 >= ncols) break;
                i32x4 D = mfma16x16x64(a[cg][p], b, zero);
                D = mfma16x16x64(a[cg][p], neg32, D);          // - 32 * sum(q_a) over the sub-block
                if (DBG) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = 4 * cg + e;
                        if (dbg_row && c < ncols) dbg_row[(int64_t)c * dbg_ld + step * 16 + 4 * p + g] = D[e];
                    }
                } else {
                    const f32x4 t0 = *(const f32x4 *)(sTab + blk * 8 + 4 * cg);
                    const f32x4 t1 = *(const f32x4 *)(sTab + blk * 8 + 4 * cg + 2);
                    acc[cg][0] += (float)D[0] * (ws * t0.x);
                    acc[cg][1] += (float)D[1] * (ws * t0.z);
                    acc[cg][2] += (float)D[2] * (ws * t1.x);
                    acc[cg][3] += (float)D[3] * (ws * t1.z);
                }
            }
        }
    }
};

// ------------------------------------------------------------------------------------------
// Q8_0: 34-byte blocks {d, int8 q[32]}; a step is 8 blocks (256 values), MFMA p covers blocks
// 2p (lanes g = 0, 1) and 2p+1 (lanes g = 2, 3); lane g loads 16 codes of its block, so the
// 4 lanes of a row read the 64 code bytes of two adjacent blocks.  The last step of a row may be
// partial (k/32 blocks): blocks beyond it are clamped to the last block and their results dropped.
// Q4_0 (18-byte blocks {d, 16 nibble bytes}) takes the same roles: lane g reads the block's 16
// nibble bytes and keeps the low (g even: values 0-15) or high nibbles (values 16-31), minus 8.
// ------------------------------------------------------------------------------------------
template <int T> struct MvStepB32 {
    static constexpr int NCG = 1;
    static constexpr int BB = Fmt<T>::BYTES;   // bytes per 32-value block
    uint32_t dbits[4];
    u32x4 q[4];
    u32x4 a[4];

    // aoff[0][p] holds the block index 2p + sel within the step; the byte offset is formed in
    // load() after clamping to the row's last block (astride is 8 for a live lane, 0 otherwise).
    __device__ static void lane_setup(MvLane &L, int m) {
        const int sel = m >> 3;
        for (int p = 0; p < 4; ++p) L.aoff[0][p] = (uint32_t)(2 * p + sel);
    }
    __device__ static bool a_diag(int g, int m) { return (g >> 1) == (m >> 3); }
    __device__ static int a_col(int m, int) { return m & 7; }

    __device__ __forceinline__ void load(const uint8_t *wg, const MvLane &L, int64_t step, int64_t nb) {
        const int64_t live = L.astride[0] != 0 ? 1 : 0;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            int64_t bw = step * 8 + 2 * p + (L.g >> 1);
            bw = bw < nb ? bw : nb - 1;
            const uint8_t *blk = wg + L.wrow_off + bw * BB;
            dbits[p] = ld2(blk);
            if constexpr (T == kQ4_0) {
                // nibble - 8 as int8: (n + 120) ^ 0x80 per byte (no carries)
                const u32x4 v = ld16(blk + 2);
                const int sh = 4 * (L.g & 1);
                q[p] = u32x4{(((v.x >> sh) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u,
                             (((v.y >> sh) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u,
                             (((v.z >> sh) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u,
                             (((v.w >> sh) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u};
            } else {
                q[p] = ld16(blk + 2 + 16 * (L.g & 1));
            }
            int64_t ba = step * 8 + L.aoff[0][p];
            ba = ba < nb ? ba : nb - 1;
            a[p] = ld16(L.abase[0] + live * (ba * kQ8_1Bytes + 4 + 16 * (L.g & 1)));
        }
    }

    template <bool DBG>
    __device__ __forceinline__ void compute(int64_t step, const MvLane &L, const float2 *sTab, float (&acc)[NCG][4],
                                            int32_t *dbg_row, int64_t dbg_ld, int ncols, int64_t nb) const {
        const int g = L.g;
        const i32x4 zero = {0, 0, 0, 0};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            if (step * 8 + 2 * p >= nb) break;   // wave-uniform
            const i32x4 D = mfma16x16x64(a[p], q[p], zero);
            const int64_t blk = step * 8 + 2 * p + (g >> 1);
            if (blk >= nb) continue;
            if (DBG) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 4 * (g & 1) + e;
                    if (dbg_row && c < ncols) dbg_row[(int64_t)c * dbg_ld + blk] = D[e];
                }
            } else {
                const float ws = h2f((uint16_t)dbits[p]);
                const f32x4 t0 = *(const f32x4 *)(sTab + blk * 8 + 4 * (g & 1));
                const f32x4 t1 = *(const f32x4 *)(sTab + blk * 8 + 4 * (g & 1) + 2);
                acc[0][0] += (float)D[0] * (ws * t0.x);
                acc[0][1] += (float)D[1] * (ws * t0.z);
                acc[0][2] += (float)D[2] * (ws * t1.x);
                acc[0][3] += (float)D[3] * (ws * t1.z);
            }
        }
    }
};

template <> struct MvStep<kQ8_0> : MvStepB32<kQ8_0> {};
template <> struct MvStep<kQ4_0> : MvStepB32<kQ4_0> {};

// ------------------------------------------------------------------------------------------
// Q3_K: 110-byte super-block = {hmask[32], qs[64], 12 bytes of 6-bit scales, d}; value
// d * (sc - 32) * (q - 4) with a 3-bit q and one scale per 16 values (GP100 patch page, "How"
// step 3: the -4 offset).  Value v = 64p + 16g + i (MFMA p, lane group g, the 16-value sub-block
// t = 4p + g, as for Q6_K): half h = p/2, bit pair j = 2(p&1) + g/2, byte l = 16(g&1) + i; its
// low two bits are bits 2j.. of qs[32h + l], its third bit is bit 4h + j of hmask[l].  So lane g
// of a row loads hmask[16(g&1)..], qs[16(g&1)..] and qs[32 + 16(g&1)..] once per step.  Scale t:
// low nibble in byte 4(p&1) + g (p < 2: low nibble, else high), top two bits at bit 2p of byte
// 8 + g.  D = sum q*q_a - 4*sum q_a: a second MFMA against a constant -4 operand.
// ------------------------------------------------------------------------------------------
template <> struct MvStep<kQ3_K> {
    static constexpr int NCG = 2;
    static constexpr int BYTES = 110;
    u32x4 hm, qs0, qs1;
    uint32_t s0, s1, s2, dbits;
    u32x4 a[2][4];

    __device__ static void lane_setup(MvLane &L, int m) { MvStep<kQ6_K>::lane_setup(L, m); }
    __device__ static bool a_diag(int g, int m) { return g == (m >> 2); }
    __device__ static int a_col(int m, int cg) { return (m & 3) + 4 * cg; }

    __device__ __forceinline__ void load(const uint8_t *wg, const MvLane &L, int64_t step) {
        const uint8_t *blk = wg + L.wrow_off + step * BYTES;
        hm = ld16(blk + 16 * (L.g & 1));
        qs0 = ld16(blk + 32 + 16 * (L.g & 1));
        qs1 = ld16(blk + 64 + 16 * (L.g & 1));
        s0 = ld4(blk + 96);
        s1 = ld4(blk + 100);
        s2 = ld4(blk + 104);
        dbits = ld2(blk + 108);
#pragma unroll
        for (int cg = 0; cg < 2; ++cg)
#pragma unroll
            for (int p = 0; p < 4; ++p) a[cg][p] = ld16(L.abase[cg] + step * L.astride[cg] + L.aoff[cg][p]);
    }

    template <bool DBG>
    __device__ __forceinline__ void compute(int64_t step, const MvLane &L, const float2 *sTab, float (&acc)[NCG][4],
                                            int32_t *dbg_row, int64_t dbg_ld, int ncols) const {
        const int g = L.g;
        const float d = h2f((uint16_t)dbits);
        const u32x4 neg4 = {0xFCFCFCFCu, 0xFCFCFCFCu, 0xFCFCFCFCu, 0xFCFCFCFCu};
        const i32x4 zero = {0, 0, 0, 0};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const u32x4 Q = (p >> 1) ? qs1 : qs0;
            const int j = 2 * (p & 1) + (g >> 1), hb = 4 * (p >> 1) + j;
            u32x4 b;   // stored 3-bit codes (0..7)
            b.x = ((Q.x >> (2 * j)) & 0x03030303u) | (((hm.x >> hb) & 0x01010101u) << 2);
            b.y = ((Q.y >> (2 * j)) & 0x03030303u) | (((hm.y >> hb) & 0x01010101u) << 2);
            b.z = ((Q.z >> (2 * j)) & 0x03030303u) | (((hm.z >> hb) & 0x01010101u) << 2);
            b.w = ((Q.w >> (2 * j)) & 0x03030303u) | (((hm.w >> hb) & 0x01010101u) << 2);
            const uint32_t lb = (((p & 1) ? s1 : s0) >> (8 * g)) & 0xFFu;
            const int sc6 = (int)((p < 2 ? (lb & 15u) : (lb >> 4)) | (((s2 >> (8 * g + 2 * p)) & 3u) << 4));
            const float ws = d * (float)(sc6 - 32);               // scale of sub-block 4p+g
            const int64_t blk = step * 8 + 2 * p + (g >> 1);   // q8_1 block of this lane's sub-block
#pragma unroll
            for (int cg = 0; cg < NCG; ++cg) {
                if (cg * 4 >= ncols) break;
                i32x4 D = mfma16x16x64(a[cg][p], b, zero);
                D = mfma16x16x64(a[cg][p], neg4, D);           // - 4 * sum(q_a) over the sub-block
                if (DBG) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = 4 * cg + e;
                        if (dbg_row && c < ncols) dbg_row[(int64_t)c * dbg_ld + step * 16 + 4 * p + g] = D[e];
                    }
                } else {
                    const f32x4 t0 = *(const f32x4 *)(sTab + blk * 8 + 4 * cg);
                    const f32x4 t1 = *(const f32x4 *)(sTab + blk * 8 + 4 * cg + 2);
                    acc[cg][0] += (float)D[0] * (ws * t0.x);
                    acc[cg][1] += (float)D[1] * (ws * t0.z);
                    acc[cg][2] += (float)D[2] * (ws * t1.x);
                    acc[cg][3] += (float)D[3] * (ws * t1.z);
                }
            }
        }
    }
};

// ------------------------------------------------------------------------------------------
// IQ4_XS: 136-byte super-block = {d, scales_h (16 bits), scales_l[4], qs[128]}; value
// d * (ls - 32) * cb[q] with a 4-bit codebook index q and one 6-bit scale ls per 32 values
// (GP100 patch page, "How" step 3).  The lane roles are Q8_0's: MFMA p covers sub-blocks 2p (lane
// groups 0, 1) and 2p+1 (2, 3); lane g takes half g&1 of sub-block b = 2p + g/2 -- the low
// (values 0-15) or high nibbles (16-31) of qs[16b..16b+15] -- mapped through the codebook to
// int8.  ls of sub-block b: nibble b&1 of scales_l[b/2], top two bits at bit 2b of scales_h.
// ------------------------------------------------------------------------------------------
template <> struct MvStep<kIQ4_XS> {
    static constexpr int NCG = 1;
    static constexpr int BYTES = 136;
    uint32_t h0, h1;   // {d, scales_h}, scales_l
    u32x4 q[4];
    u32x4 a[4];

    __device__ static void lane_setup(MvLane &L, int m) {
        const int sel = m >> 3;
        for (int p = 0; p < 4; ++p) L.aoff[0][p] = (uint32_t)((2 * p + sel) * kQ8_1Bytes + 4 + 16 * (L.g & 1));
    }
    __device__ static bool a_diag(int g, int m) { return (g >> 1) == (m >> 3); }
    __device__ static int a_col(int m, int) { return m & 7; }

    __device__ __forceinline__ void load(const uint8_t *wg, const MvLane &L, int64_t step) {
        const uint8_t *blk = wg + L.wrow_off + step * BYTES;
        h0 = ld4(blk);
        h1 = ld4(blk + 4);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            q[p] = ld16(blk + 8 + 16 * (2 * p + (L.g >> 1)));
            a[p] = ld16(L.abase[0] + step * L.astride[0] + L.aoff[0][p]);
        }
    }

    template <bool DBG>
    __device__ __forceinline__ void compute(int64_t step, const MvLane &L, const float2 *sTab, float (&acc)[NCG][4],
                                            int32_t *dbg_row, int64_t dbg_ld, int ncols) const {
        const int g = L.g;
        const float d = h2f((uint16_t)(h0 & 0xFFFF));
        const uint32_t sh = h0 >> 16;
        const int nsh = 4 * (g & 1);
        const i32x4 zero = {0, 0, 0, 0};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int b = 2 * p + (g >> 1);
            const u32x4 c = {iq4_lookup4((q[p].x >> nsh) & 0x0F0F0F0Fu), iq4_lookup4((q[p].y >> nsh) & 0x0F0F0F0Fu),
                             iq4_lookup4((q[p].z >> nsh) & 0x0F0F0F0Fu), iq4_lookup4((q[p].w >> nsh) & 0x0F0F0F0Fu)};
            const i32x4 D = mfma16x16x64(a[p], c, zero);
            const int64_t blk = step * 8 + b;
            if (DBG) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int cc = 4 * (g & 1) + e;
                    if (dbg_row && cc < ncols) dbg_row[(int64_t)cc * dbg_ld + blk] = D[e];
                }
            } else {
                const int ls = (int)(((h1 >> (8 * (b >> 1) + 4 * (b & 1))) & 15u) | (((sh >> (2 * b)) & 3u) << 4));
                const float ws = d * (float)(ls - 32);
                const f32x4 t0 = *(const f32x4 *)(sTab + blk * 8 + 4 * (g & 1));
                const f32x4 t1 = *(const f32x4 *)(sTab + blk * 8 + 4 * (g & 1) + 2);
                acc[0][0] += (float)D[0] * (ws * t0.x);
                acc[0][1] += (float)D[1] * (ws * t0.z);
                acc[0][2] += (float)D[2] * (ws * t1.x);
                acc[0][3] += (float)D[3] * (ws * t1.z);
            }
        }
    }
};

constexpr int mv_max_waves(int spw) { return spw == 1 ? 16 : spw == 2 ? 8 : 4; }

template <int T, int SPW, bool DBG, bool EXPERT, bool GLU>
// Returns false (workgroup-uniform) when expert slot ey holds no expert, true otherwise.
__device__ __forceinline__ bool mmvq_body(const uint8_t *__restrict__ w, const uint8_t *__restrict__ w2, int64_t rows,
                                          int64_t k, const uint8_t *__restrict__ xq, int64_t n, float *__restrict__ y,
                                          int32_t *__restrict__ dbg, const ColMap &cm, int ey) {
    static_assert(!(GLU && DBG), "no debug export of the fused form");
    extern __shared__ __align__(16) uint8_t mv_smem[];
    using S = MvStep<T>;
    constexpr int NCG = S::NCG;

    MvCols mc;
    if (!mv_resolve(mc, w, n, cm, EXPERT, GLU ? w2 : nullptr, ey)) return false;   // workgroup-uniform
    const int ncols = mc.ncols;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int64_t nb = k / 32;                         // q8_1 blocks per activation row
    const int64_t row_bytes = (k / Fmt<T>::QK) * Fmt<T>::BYTES;
    const int64_t nsteps = (k + kSuper - 1) / kSuper;
    const int64_t row0 = (int64_t)blockIdx.x * (GLU ? kMvRows / 2 : kMvRows);
    const uint8_t *wg = mc.wbase + row0 * row_bytes;   // uniform base of the 16-row group
    float2 *sTab = (float2 *)mv_smem;                          // [nb][8] (d, s)
    float *sRed = (float *)(mv_smem + nb * 8 * sizeof(float2)); // [nwaves][128]

    MvLane L;
    L.g = lane >> 4;
    L.r16 = lane & 15;
    const int64_t row = row0 + (GLU ? (L.r16 & 7) : L.r16);   // GLU: output row of the lane's gate/up row
    const int64_t rclamp = row < rows ? row : rows - 1;
    if constexpr (GLU) {
        // per-lane base: gate rows for r16 < 8, up rows for r16 >= 8 (two separate matrices)
        wg = (L.r16 < 8 ? mc.wbase : mc.wbase2) + rclamp * row_bytes;
        L.wrow_off = 0;
    } else {
        L.wrow_off = (uint32_t)((rclamp - row0) * row_bytes);
    }
    const int m = L.r16;
    S::lane_setup(L, m);
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
        const int c = S::a_col(m, cg);
        const bool on = (cg < NCG) && S::a_diag(L.g, m) && c < ncols;
        L.abase[cg] = on ? xq + mc.arow(c) * nb * kQ8_1Bytes : (const uint8_t *)mv_zero16;
        L.astride[cg] = on ? 8 * kQ8_1Bytes : 0;
        if (!on)
            for (int j = 0; j < 4; ++j) L.aoff[cg][j] = 0;
    }

    // Stage the fp32 (d, s) of the workgroup's columns from their q8_1 blocks: sTab[block][column].
    if (!DBG) {
        const int c = threadIdx.x & 7;
        const uint8_t *xrow = xq + (c < ncols ? mc.arow(c) : 0) * nb * kQ8_1Bytes;
        for (int64_t i = threadIdx.x; i < nb * 8; i += blockDim.x) {
            const int64_t b = i >> 3;     // blockDim.x is a multiple of 8: column c is fixed
            float2 v = make_float2(0.f, 0.f);
            if (c < ncols) {
                const uint32_t ds = *(const uint32_t *)(xrow + b * kQ8_1Bytes);
                v = make_float2(h2f((uint16_t)(ds & 0xFFFF)), h2f((uint16_t)(ds >> 16)));
            }
            sTab[i] = v;
        }
    }

    float acc[NCG][4];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[cg][e] = 0.f;

    int32_t *dbg_row = nullptr;
    int64_t dbg_ld = 0;
    if (DBG && row < rows) {
        const int64_t per = kSub16<T> ? k / 16 : nb;
        dbg_ld = rows * per;
        dbg_row = dbg + row * per;
    }

    // Passes of SPW steps per wave; within a pass every load is issued before the first math.
    bool synced = false;
    for (int64_t base = 0; base < nsteps; base += (int64_t)SPW * nwaves) {
        S st[SPW];
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int64_t s = base + wave + (int64_t)i * nwaves;
            if (s < nsteps) {
                if constexpr (T == kQ8_0 || T == kQ4_0) st[i].load(wg, L, s, nb);
                else st[i].load(wg, L, s);
            }
        }
        if (!synced) { __syncthreads(); synced = true; }   // scale table ready
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int64_t s = base + wave + (int64_t)i * nwaves;
            if (s < nsteps) {
                if constexpr (T == kQ8_0 || T == kQ4_0) st[i].template compute<DBG>(s, L, sTab, acc, dbg_row, dbg_ld, ncols, nb);
                else st[i].template compute<DBG>(s, L, sTab, acc, dbg_row, dbg_ld, ncols);
            }
        }
    }
    if (DBG) return true;

    // Combine the sub-block slots held by lane groups: Q4_K/Q8_0 lanes g and g^2 (the two halves
    // of the block diagonal), Q6_K lanes g = 0..3 (the four 16-value sub-blocks).
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = acc[cg][e];
            if (kSub16<T>) v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            acc[cg][e] = v;
        }
    // Lanes holding the wave's values: Q4_K/Q8_0 g in {0,1} (columns 4g..4g+3), Q6_K g == 0
    // (columns 4cg..4cg+3); 128 floats per wave.
    const bool holder = kSub16<T> ? (L.g == 0) : (L.g < 2);
    if (holder) {
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
            for (int e = 0; e < 4; ++e) sRed[wave * 128 + lane * (4 * NCG) + cg * 4 + e] = acc[cg][e];
    }
    __syncthreads();
    if (wave != 0 || !holder || row >= rows || (GLU && L.r16 >= 8)) return true;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = 0.f, u = 0.f;
            for (int wv = 0; wv < nwaves; ++wv) {
                v += sRed[wv * 128 + lane * (4 * NCG) + cg * 4 + e];
                if (GLU) u += sRed[wv * 128 + (lane + 8) * (4 * NCG) + cg * 4 + e];   // the up row
            }
            const int c = kSub16<T> ? 4 * cg + e : 4 * L.g + e;
            if (c < ncols) y[mc.pair(c) * rows + row] = GLU ? v / (1.0f + expf(-v)) * u : v;
        }
    return true;
}

// Dense: one row group per workgroup.  Expert mode: grid row blockIdx.y takes the listed small
// experts blockIdx.y, blockIdx.y + gridDim.y, ... until the compacted list ends (see
// mmvq_stream_kernel).
template <int T, int SPW, bool DBG, bool EXPERT, bool GLU>
__global__ __launch_bounds__(64 * mv_max_waves(SPW)) void mmvq_kernel(const uint8_t *__restrict__ w,
                                                    const uint8_t *__restrict__ w2, int64_t rows, int64_t k,
                                                    const uint8_t *__restrict__ xq, int64_t n, float *__restrict__ y,
                                                    int32_t *__restrict__ dbg, ColMap cm) {
    if constexpr (!EXPERT) {
        mmvq_body<T, SPW, DBG, EXPERT, GLU>(w, w2, rows, k, xq, n, y, dbg, cm, -1);
    } else {
        if (gridDim.y == (unsigned)cm.n_exp) {   // one expert slot per grid row: no loop
            mmvq_body<T, SPW, DBG, EXPERT, GLU>(w, w2, rows, k, xq, n, y, dbg, cm, (int)blockIdx.y);
            return;
        }
        for (int ey = blockIdx.y;;) {
            if (!mmvq_body<T, SPW, DBG, EXPERT, GLU>(w, w2, rows, k, xq, n, y, dbg, cm, ey)) break;
            ey += gridDim.y;
            if (ey >= cm.n_exp) break;
            __syncthreads();   // the next expert reuses the LDS
        }
    }
}

template <int T, int SPW, bool DBG, bool EXPERT, bool GLU = false>
static hipError_t launch_mmvq_spw(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y,
                                  int32_t *dbg, const ColMap &c, int64_t n_exp, hipStream_t s,
                                  const uint8_t *w2 = nullptr) {
    const int64_t nsteps = (k + kSuper - 1) / kSuper;
    int64_t nw = (nsteps + SPW - 1) / SPW;
    if (nw > mv_max_waves(SPW)) nw = mv_max_waves(SPW);
    if (nw < 1) nw = 1;
    constexpr int RW = GLU ? kMvRows / 2 : kMvRows;   // outputs per workgroup
    const int64_t groups = (rows + RW - 1) / RW;
    dim3 grid((unsigned)groups, EXPERT ? (unsigned)mv_expert_slots(groups, n_exp, c.pairs) : 1u);
    const size_t smem = (size_t)(k / 32) * 8 * sizeof(float2) + (size_t)nw * 128 * sizeof(float);
    // once per process (a function-local static is initialised exactly once, thread-safely)
    static const hipError_t attr_err = hipFuncSetAttribute((const void *)mmvq_kernel<T, SPW, DBG, EXPERT, GLU>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr_err != hipSuccess) return attr_err;
    hipLaunchKernelGGL((mmvq_kernel<T, SPW, DBG, EXPERT, GLU>), grid, dim3(64 * (unsigned)nw), smem, s, w, w2, rows, k,
                       xq, n, y, dbg, c);
    return hipGetLastError();
}

template <int T, bool DBG, bool EXPERT>
static hipError_t launch_mmvq_t(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y,
                                int32_t *dbg, const ColMap *cm, int64_t n_exp, int spw, hipStream_t s) {
    ColMap c = cm ? *cm : ColMap{};
    if (spw == 0) spw = 2;
    if (spw == 1) return launch_mmvq_spw<T, 1, DBG, EXPERT>(w, rows, k, xq, n, y, dbg, c, n_exp, s);
    if (spw == 4) return launch_mmvq_spw<T, 4, DBG, EXPERT>(w, rows, k, xq, n, y, dbg, c, n_exp, s);
    return launch_mmvq_spw<T, 2, DBG, EXPERT>(w, rows, k, xq, n, y, dbg, c, n_exp, s);
}

// Largest column count the automatic choice sends to the dot4 kernel, per type and weight rows:
// up to three columns from 8192 rows on (Q8_0: one column from 8192 rows, three from 12288), none
// below.  Measured with the weights rotated over > 512 MB (graph-replayed calls, fp32 input, K =
// 4096, the LDS-staged kernel against dot4 at 1 / 2 / 3 columns): Q4_K 4096 rows 5.1 / 5.3 / 6.1
// against 5.3 / 6.1 / 6.8 us, 8192 rows 8.7 / 9.0 / 10.4 against 6.7 / 8.6 / 9.7, 14336 rows
// 15.3 / 15.8 / 18.8 against 9.8 / 12.1 / 14.5 (the LDS-staged kernel's 16-row workgroups each
// quantize all of x and run one step per wave, while dot4's 4-8-wave workgroups share a compute
// unit and stream several steps per wave); Q5_K and Q4_0 alike; Q8_0 8192 rows 10.7 / 10.9 /
// 11.8 against 9.3 / 11.7 / 12.9, 14336 rows 18.9 / 19.3 / 20.8 against 14.9 / 17.3 / 18.3.
// Q3_K and IQ4_XS, which the LDS-staged kernel does not serve, take dot4 up to three columns at
// any row count: their alternative is a separate quantize launch and the register-streamed kernel.
constexpr int64_t kDot4MinRows = 8192;
constexpr int64_t kDot4Q8MultiRows = 12288;
static int dot4_auto_cols(int type, int64_t rows) {
    if (type == kQ3_K || type == kIQ4_XS) return 3;
    if (rows < kDot4MinRows) return 0;
    if (type == kQ8_0) return rows >= kDot4Q8MultiRows ? 3 : 1;
    return type == kQ4_K || type == kQ5_K || type == kQ4_0 ? 3 : 0;
}

// Which fused kernel serves an fp32-input call: 3 dot4, 2 LDS-staged MFMA, 0 none.  Override
// o.mv_kernel: 0 automatic, 1 register-streamed (never fused), 2 LDS-staged only, 3 dot4 only.
static int fused_kernel(int type, const void *w, int64_t rows, int64_t k, const float *x, int64_t n, const Ovr &o) {
    const int kc = o.mv_kernel;
    if (n < 1 || (uintptr_t)x % 16 != 0) return 0;
    if (kc == 0 || kc == 3) {
        const int lim = kc == 3 ? mmvq_dot4_max_cols() : dot4_auto_cols(type, rows);
        if (n <= lim && mmvq_dot4_supported(type, w, k, x, nullptr)) return 3;
        if (kc == 3) return 0;
    }
    // The LDS-staged kernel quantizes a step's blocks with 4 lanes per block; every workgroup
    // quantizes all of x, so the cost grows with n while a separate quantize launch costs a
    // fixed ~2-3 us.  Measured at 4096 x 4096 (graph-replayed calls), fused is faster for every
    // n <= 8 and type: 1.9-2.4 us at n = 1, 0.3-0.7 us at n = 8.
    const int lim = o.fuse_cols > 0 ? o.fuse_cols : 8;
    if ((kc == 0 || kc == 2) && n <= lim && mmvq_stream_supported(type, w, k, x, nullptr)) return 2;
    return 0;
}

hipError_t launch_mmvq_fused(int choice, int type, const uint8_t *w, int64_t rows, int64_t k, const float *x, int64_t n,
                             float *y, hipStream_t s) {
    switch (choice) {
        case 3: return launch_mmvq_dot4_f32(type, w, rows, k, x, n, y, s);
        case 2: return launch_mmvq_stream_f32(type, w, rows, k, x, n, y, s);
        default: return hipErrorInvalidValue;
    }
}

int mmvq_kernel_choice(int type, const void *w, int64_t rows, int64_t k, const void *xq, int64_t n, const ColMap *cm,
                       const Ovr &o) {
    const int kc = o.mv_kernel;
    if (kc == 3 || kc == 0) {
        const int lim = kc == 3 ? mmvq_dot4_max_cols() : dot4_auto_cols(type, rows);
        if (!cm && n <= lim && mmvq_dot4_supported(type, w, k, xq, cm)) return 3;
        if (kc == 3) return 0;
    }
    if (kc != 1 && mmvq_stream_supported(type, w, k, xq, cm)) return 2;
    if (kc == 2) return 0;
    return 1;
}

int mmvq_fused_choice(int type, const void *w, int64_t rows, int64_t k, const float *x, int64_t n, const Ovr &o) {
    return fused_kernel(type, w, rows, k, x, n, o);
}

hipError_t launch_mmvq(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y,
                       int32_t *dbg, const ColMap *cm, int64_t n_exp, const Ovr &o, hipStream_t s) {
    switch (mmvq_kernel_choice(type, w, rows, k, xq, n, cm, o)) {
        case 3: return launch_mmvq_dot4(type, w, rows, k, xq, n, y, dbg, cm, n_exp, (int)n, s);
        case 2: return launch_mmvq_stream(type, w, rows, k, xq, n, y, dbg, cm, n_exp, s);
        case 1: break;
        default: return hipErrorInvalidValue;
    }
    const bool expert = cm != nullptr;
    const bool d = dbg != nullptr;
#define QMM_MV(TT)                                                                                       \
    if (type == TT) {                                                                                  \
        if (d) return launch_mmvq_t<TT, true, false>(w, rows, k, xq, n, y, dbg, cm, n_exp, o.mv_steps, s); \
        if (expert) return launch_mmvq_t<TT, false, true>(w, rows, k, xq, n, y, dbg, cm, n_exp, o.mv_steps, s); \
        return launch_mmvq_t<TT, false, false>(w, rows, k, xq, n, y, dbg, cm, n_exp, o.mv_steps, s);   \
    }
    QMM_MV(kQ4_K)
    QMM_MV(kQ5_K)
    QMM_MV(kQ6_K)
    QMM_MV(kQ8_0)
    QMM_MV(kQ4_0)
    QMM_MV(kQ3_K)
    QMM_MV(kIQ4_XS)
#undef QMM_MV
    return hipErrorInvalidValue;
}

}  // namespace qmm

namespace qmm {

// Gate/up fusion from q8_1 columns (dense or the small experts): the LDS-staged kernel where both
// matrices meet its alignment rules (and no override forces the register-streamed one), else the
// register-streamed kernel.
hipError_t launch_mmvq_glu(int type, const uint8_t *wg, const uint8_t *wu, int64_t rows, int64_t k, const uint8_t *xq,
                           int64_t n, float *y, const ColMap *cm, int64_t n_exp, const Ovr &o, hipStream_t s) {
    if (o.mv_kernel != 1 && o.mv_kernel != 3 && mmvq_stream_supported(type, wg, k, xq, cm) &&
        mmvq_stream_supported(type, wu, k, xq, cm))
        return launch_mmvq_stream_glu(type, wg, wu, rows, k, xq, false, n, y, cm, n_exp, s);
    const ColMap c = cm ? *cm : ColMap{};
#define QMM_MVG(TT)                                                                                      \
    if (type == TT) {                                                                                  \
        if (cm) return launch_mmvq_spw<TT, 2, false, true, true>(wg, rows, k, xq, n, y, nullptr, c, n_exp, s, wu); \
        return launch_mmvq_spw<TT, 2, false, false, true>(wg, rows, k, xq, n, y, nullptr, c, n_exp, s, wu);     \
    }
    QMM_MVG(kQ4_K)
    QMM_MVG(kQ5_K)
    QMM_MVG(kQ6_K)
    QMM_MVG(kQ8_0)
    QMM_MVG(kQ4_0)
    QMM_MVG(kQ3_K)
    QMM_MVG(kIQ4_XS)
#undef QMM_MVG
    return hipErrorInvalidValue;
}

// Kernel for a dense fp32-input gate/up call of n <= 8 columns, as fused_kernel decides for one
// matrix, with both matrices checked: 3 dot4, 2 LDS-staged (both quantize x themselves), 0 none
// (quantize first, then launch_mmvq_glu).  The kernel streams both matrices: 2 * rows weight rows.
int mmvq_glu_f32_choice(int type, const void *wg, const void *wu, int64_t rows, int64_t k, const float *x, int64_t n,
                        const Ovr &o) {
    const int a = fused_kernel(type, wg, 2 * rows, k, x, n, o), b = fused_kernel(type, wu, 2 * rows, k, x, n, o);
    return a == b ? a : 0;
}

}  // namespace qmm
