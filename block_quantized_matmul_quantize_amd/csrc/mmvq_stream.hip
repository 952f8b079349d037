// Matrix-vector product for 1..8 activation columns, streamed through LDS (the MMVQ regime of
// the MMQ page: "shape criteria" and the MMVQ-vs-MMQ table -- decode is bound by how fast the
// weights stream, every weight byte is read once and serves all columns).
//
// CDNA4 design.  A workgroup owns 16 weight rows; wave w takes the 256-value steps w, w+W, ...
// (up to 16 waves, so a 4096-wide K gives every wave one step and a CU 16 waves to hide HBM
// latency with).  For each step the wave loads the 16 rows' bytes of that step and the step's
// activations with coalesced loads, parks them in its own LDS stage, and loads the next step
// while it computes.  No workgroup barrier in the loop.  Operands are then read from LDS in the
// MFMA lane layout: one v_mfma_i32_16x16x64_i8 per 64-value slice, B = 16 weight rows, A =
// activations placed block-diagonally over (column, sub-block) so every int32 result is one exact
// sub-block dot D (the same contraction as the register-streamed kernel in mmvq.hip, which serves
// the shapes this one does not).  Fixups per D in fp32 ("dp4a path Q4_K" section of the MMQ page):
//   Q4_K, Q5_K  acc += D * (d*sc) * d_a - (dmin*m) * s_a   (Q5_K: fifth bits from qh ORed in)
//   Q6_K  acc += D * (d*sc) * d_a      (D includes -32 * sum q_a via a second MFMA)
//   Q8_0  acc += D * d_w * d_a
// Every 16-byte LDS operand sits at a 16-byte aligned address (a misaligned ds_read_b128 runs at
// a quarter to an eighth of the aligned rate), so parking reshapes what the loads return: q8_1
// blocks (36 bytes) are split into 32 aligned code bytes per block and an fp32 (d, s) table; a Q6_K
// super-block (210 bytes, at an even offset) is shifted into place with a lane exchange and
// v_alignbyte; Q8_0 blocks (34 bytes) are loaded two at a time (68 bytes, 4-byte aligned) and
// split into aligned codes and fp32 scales.  For fp32 activations (dense) the wave quantizes its
// step's blocks itself, 4 lanes per block with the arithmetic of the standalone quantize kernel
// (q8_1.hpp) -- one launch instead of two.
// Requirements (checked by the host): K a multiple of 256; Q4_K, Q5_K and Q6_K weights and rows 16-byte
// aligned, Q8_0 weights 4-byte aligned; q8_1 activations 4-byte aligned (fp32: 16-byte).
// GLU (gate/up fusion, the MMQ page's fusion passage): the 16 rows are 8 gate rows (load
// instructions 0-1) and the same 8 rows of the up matrix (instructions 2-3); the write-back applies
// silu(gate) * up.
#include "common.hpp"
#include "launch.hpp"
#include "mv_cols.hpp"
#include "q8_1.hpp"

namespace qmm {

namespace {

constexpr int kRows = 16;
constexpr int kActStep = 8 * kQ8_1Bytes;   // one column's q8_1 bytes per 256-value step (288)
// Per-wave LDS head before its stage: 208 zero bytes (the off-diagonal A operand: a lane's
// operand pointer for slice j is its base plus a fixed offset of at most 192, and lanes off the
// diagonal take the zero block as base) and a 48-byte sink that lanes with nothing to park write
// to, so every load and store is unconditional (no divergent branches around memory operations).
constexpr int kHead = 256;
constexpr int kZeroBytes = 208;

typedef u32x4 __attribute__((aligned(4))) u32x4_a4;

// Per-type step geometry.  Q4_K / Q6_K: PPR 16-byte pieces per row per step (Q6_K: the
// 16-byte-aligned window around a 210-byte super-block that starts at an even offset -- always
// 14 pieces), STEP bytes per row per step.  RSTR is the LDS row stride (16 rows read in one MFMA
// operand fetch fall in distinct banks); Q8_0 rows hold 8 blocks x 32 aligned code bytes, WD its
// fp32 block scales [16 rows][8 blocks].
template <int T> struct Geo;
template <> struct Geo<kQ4_K> { static constexpr int PPR = 9, STEP = 144, RSTR = 144, WD = 0; };
template <> struct Geo<kQ5_K> { static constexpr int PPR = 11, STEP = 176, RSTR = 176, WD = 0; };
// Q4_K and Q5_K (the Q4_K header and nibbles, qs 32 bytes further on after qh[32]) share a path.
template <int T> constexpr bool kK45 = T == kQ4_K || T == kQ5_K;
template <> struct Geo<kQ6_K> { static constexpr int PPR = 14, STEP = 210, RSTR = 240, WD = 0; };
template <> struct Geo<kQ8_0> { static constexpr int PPR = 0, STEP = 272, RSTR = 272, WD = 16 * 8 * 4; };
// Q4_0 (18-byte blocks {d, 16 nibble bytes}): loaded as 36-byte block pairs, parked as Q8_0's codes.
template <> struct Geo<kQ4_0> { static constexpr int PPR = 0, STEP = 144, RSTR = 272, WD = 16 * 8 * 4; };

// Panel layout (repack.hip): the bytes of 16 rows x 256 values, parked in LDS as they are.
// B: bytes of 256 values of a row (a panel is 16 * B bytes, B pieces).  HDR: the slab after the
// code slabs (the K-quant header, the Q8_0 / Q4_0 fp16 scales); QS: the first qs slab (Q5_K's
// qh comes first).
template <int T> struct PanelGeo {
    static constexpr int B = T == kQ5_K ? 176 : T == kQ6_K ? 210 : T == kQ8_0 ? 272 : 144;
    static constexpr int HDR = B / 16 - 1, QS = T == kQ5_K ? 2 : 0;
};

// Weights loaded straight into the registers of the lanes whose MFMA operands they are, none
// parked in LDS: the panel layout (every type it serves), and Q4_K in the original layout, whose
// 144-byte super-blocks keep the header and every qs piece 16-byte aligned, so that lane (row r,
// group g) reads the same three pieces the panel form hands it (the four lanes of a row read one
// 64-byte run of its qs).  Measured 2-5 % faster at 4096 x 4096 than parking the rows in LDS;
// Q5_K, a fourth piece per lane (qh), 0-6 % slower, so it keeps the parked rows.
template <int T, bool PK> constexpr bool kRegW = PK || T == kQ4_K;

template <int T, bool REG = false> struct Stage {
    // weights (+ Q8_0 scales); weights in registers: none are parked, the space holds the
    // cross-wave partial sums at the end (up to 2 KB)
    static constexpr int WB = REG ? 2048 : kRows * Geo<T>::RSTR + Geo<T>::WD;
    static constexpr int AB = 8 * 256;                             // activation codes: [column][block][32]
    static constexpr int FB = 64 * 8;                              // fp32 (d, s): [block][column]
    static constexpr int BYTES = WB + AB + FB;
};

__device__ __forceinline__ uint32_t nib_lo(uint32_t v) { return v & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t nib_hi(uint32_t v) { return (v >> 4) & 0x0F0F0F0Fu; }
__device__ __forceinline__ u32x4 nib_lo4(u32x4 v) { return u32x4{nib_lo(v.x), nib_lo(v.y), nib_lo(v.z), nib_lo(v.w)}; }
__device__ __forceinline__ u32x4 nib_hi4(u32x4 v) { return u32x4{nib_hi(v.x), nib_hi(v.y), nib_hi(v.z), nib_hi(v.w)}; }
__device__ __forceinline__ u32x4 lds16(const uint8_t *p) { return *(const u32x4 *)p; }   // 16-byte aligned
__device__ __forceinline__ uint32_t abyte(uint32_t hi, uint32_t lo, uint32_t sh) {
    return __builtin_amdgcn_alignbyte(hi, lo, sh);
}

// The same register of the next lane within a row of 16 lanes (DPP row_shl:1; the last lane of a
// row keeps its own value, which no caller uses).
__device__ __forceinline__ uint32_t from_next_lane(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x101, 0xF, 0xF, false);
}

// Bytes [16j + 4Q + r, +16) of a row whose 16-byte pieces j (this lane) and j+1 are c and n.
template <int Q> __device__ __forceinline__ u32x4 shift_piece(u32x4 c, u32x4 n, uint32_t r) {
    const uint32_t D[8] = {c.x, c.y, c.z, c.w, n.x, n.y, n.z, n.w};
    return u32x4{abyte(D[Q + 1], D[Q], r), abyte(D[Q + 2], D[Q + 1], r), abyte(D[Q + 3], D[Q + 2], r),
                 abyte(D[Q + 4], D[Q + 3], r)};
}
template <int V> struct IC { static constexpr int value = V; };

// Q4_K block diagonal (as in mmvq.hip): MFMA j covers sub-blocks {(j>>1)*4 + (j&1) + 2*sel};
// lanes g in {1,2} carry diagonal half 0, g in {3,0} half 1; g odd holds values 0-15 of its
// sub-block, g even values 16-31.
__device__ __forceinline__ int q4_group(int g) { return (g == 1 || g == 2) ? 0 : 1; }
__device__ __forceinline__ int q4_half(int g) { return (g & 1) ? 0 : 1; }
__device__ __forceinline__ int q4_sub(int j, int sel) { return (j >> 1) * 4 + (j & 1) + 2 * sel; }

// Launch constants computed on the host (no 64-bit or variable-divisor arithmetic on the GPU).
struct MvArgs {
    int64_t rows;
    uint32_t row_bytes;   // weight bytes per row
    uint32_t col_bytes;   // q8_1 bytes per activation row (k/32 blocks)
    int32_t nsteps;       // 256-value steps (k / 256)
    int32_t q, r;         // steps per wave: q, plus one for waves < r
    int32_t n;            // dense column count
};

// PK: w is in the panel layout (repack.hip): workgroup b reads panels (b, s).  A slab (256
// bytes, one 16-byte piece per row) is exactly a 16-row MFMA operand slice, so each lane loads the
// pieces its operands need straight into registers -- 16 lanes read 256 contiguous bytes -- and
// only the activations go through LDS (measured 3-5 % faster than parking the panel in LDS).
template <int T, bool DBG, bool EXPERT, bool F32, bool GLU, bool PK>
// Returns false (workgroup-uniform) when expert slot ey holds no expert, true otherwise.
__device__ __forceinline__ bool mmvq_stream_body(const uint8_t *__restrict__ w, const uint8_t *__restrict__ w2,
                                                 const void *__restrict__ xin, float *__restrict__ y,
                                                 int32_t *__restrict__ dbg, const MvArgs &P, const ColMap &cm, int ey) {
    static_assert(!PK || !(GLU || EXPERT || DBG), "the panel layout serves the dense product");
    constexpr bool REG = kRegW<T, PK>, DR = REG && !PK;   // DR: Q4_K pieces from the original rows
    using S = Stage<T, REG>;
    constexpr int PPR = Geo<T>::PPR, RSTR = Geo<T>::RSTR, WB = S::WB, SB = S::BYTES;
    constexpr int A0 = WB, F0 = WB + S::AB;   // activation codes and (d, s) table within a stage
    constexpr int NCG = (T == kQ6_K) ? 2 : 1;
    extern __shared__ __align__(16) uint8_t smem[];

    MvCols mc;
    static_assert(!(GLU && DBG), "no debug export of the fused form");
    if (!mv_resolve(mc, w, P.n, cm, EXPERT, GLU ? w2 : nullptr, ey)) return false;   // workgroup-uniform
    const int ncols = mc.ncols;                           // >= 1
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nwaves = blockDim.x >> 6;
    const int64_t rows = P.rows;
    const uint32_t row_bytes = P.row_bytes, col_bytes = P.col_bytes;
    constexpr int RW = GLU ? kRows / 2 : kRows;   // outputs per workgroup
    const int64_t row0 = (int64_t)blockIdx.x * RW;
    const int rmax = (int)((rows - row0) < RW ? (rows - row0) : RW) - 1;   // last live output row of the group
    constexpr int PB = 16 * PanelGeo<T>::B;   // panel bytes
    const uint8_t *wg = PK ? w + (int64_t)blockIdx.x * P.nsteps * PB : mc.wbase + row0 * (int64_t)row_bytes;
    const uint8_t *wg2 = GLU ? mc.wbase2 + row0 * (int64_t)row_bytes : wg;   // up rows (GLU)
    uint8_t *zero = smem + (size_t)wave * (kHead + SB);   // zero block (off-diagonal A lanes)
    uint8_t *st = zero + kHead;                            // this wave's stage
    constexpr int kSink = kZeroBytes - kHead;              // sink offset relative to st
    const int my_steps = P.q + (wave < P.r ? 1 : 0);

    // Weight loads.  Q4_K / Q6_K: instruction i covers rows 4i..4i+3, 16 lanes per row, lane piece
    // j = lane % 16 (j < PPR) of the step's aligned window.  Q8_0: lane (row lane/4, pair lane%4)
    // reads the 68 bytes of blocks 2p, 2p+1 of the step.  Lanes past PPR re-read piece 0 and rows
    // past the end re-read the last row (valid addresses, no predicate); their copies go to the
    // sink (pieces) or to rows whose outputs are never written.
    constexpr int PM = PPR < 16 ? PPR : 16;
    const int rq = lane >> 4, jq = lane & 15;
    const int r8 = lane >> 2, p8 = lane & 3;   // Q8_0 lane roles
    uint32_t wofs[4];
    int32_t pofs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + rq, ro = GLU ? (r & 7) : r;
        wofs[i] = (uint32_t)(ro < rmax ? ro : rmax) * row_bytes + 16u * (jq < PM ? jq : 0);
        pofs[i] = jq < PM ? r * RSTR + 16 * jq : kSink;
    }
    const int ro8 = GLU ? (r8 & 7) : r8;
    const uint32_t wofs8 = (uint32_t)(ro8 < rmax ? ro8 : rmax) * row_bytes + (T == kQ4_0 ? 36u : 68u) * p8;
    const uint8_t *wg8 = (GLU && r8 >= 8) ? wg2 : wg;
    // DR: this lane's row (r16 = lane % 16; GLU: rows 8.. are the up rows)
    const int rd = lane & 15, rdo = GLU ? (rd & 7) : rd;
    const uint8_t *wrd = ((GLU && rd >= 8) ? wg2 : wg) + (uint32_t)(rdo < rmax ? rdo : rmax) * row_bytes;

    u32x4 wv[4];
    uint32_t wv4 = 0;
    // panel layout: the pieces this lane's MFMA operands need, straight into registers (slab j,
    // row r16 at 256 j + 16 r16 of the panel)
    u32x4 pw[REG ? 5 : 1] = {};
    uint16_t pwd = 0;
    auto load_w = [&](int s) __attribute__((always_inline)) {
        if constexpr (PK) {
            const uint8_t *src = wg + (uint32_t)(s * PB) + 16 * (lane & 15);
            const int gg = lane >> 4;
            if constexpr (kK45<T>) {
                constexpr int QS = PanelGeo<T>::QS, HDR = PanelGeo<T>::HDR;
                const int qa = (gg + 3) & 3;
                pw[0] = *(const u32x4 *)(src + 256 * HDR);
                pw[1] = *(const u32x4 *)(src + 256 * (QS + qa));
                pw[2] = *(const u32x4 *)(src + 256 * (QS + 4 + qa));
                if constexpr (T == kQ5_K) pw[3] = *(const u32x4 *)(src + 256 * q4_half(gg));
            } else if constexpr (T == kQ6_K) {
                pw[0] = *(const u32x4 *)(src + 256 * gg);
                pw[1] = *(const u32x4 *)(src + 256 * (4 + gg));
                pw[2] = *(const u32x4 *)(src + 256 * (8 + (gg & 1)));
                pw[3] = *(const u32x4 *)(src + 256 * (10 + (gg & 1)));
                pw[4] = *(const u32x4 *)(src + 256 * 12);
                pwd = *(const uint16_t *)(wg + (uint32_t)(s * PB) + 13 * 256 + 2 * (lane & 15));
            } else {
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    pw[p] = *(const u32x4 *)(src + 256 * (T == kQ4_0 ? 2 * p + (gg >> 1) : 4 * p + gg));
                pw[4] = *(const u32x4 *)(src + 256 * PanelGeo<T>::HDR);
            }
        } else if constexpr (DR) {
            // super-block s of the row: header (d, dmin, scales) at 0, qs at 16
            static_assert(T == kQ4_K, "original-layout pieces in registers: Q4_K");
            const uint8_t *src = wrd + (uint32_t)(s * 144);
            const int gd = lane >> 4, qa = (gd + 3) & 3;
            pw[0] = *(const u32x4 *)src;
            pw[1] = *(const u32x4 *)(src + 16 + 16 * qa);
            pw[2] = *(const u32x4 *)(src + 16 + 16 * (4 + qa));
        } else if constexpr (T == kQ8_0) {
            const uint8_t *src = wg8 + (uint32_t)(s * 272) + wofs8;
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[i] = *(const u32x4_a4 *)(src + 16 * i);
            wv4 = *(const uint32_t *)(src + 64);
        } else if constexpr (T == kQ4_0) {
            const uint8_t *src = wg8 + (uint32_t)(s * 144) + wofs8;
            wv[0] = *(const u32x4_a4 *)src;
            wv[1] = *(const u32x4_a4 *)(src + 16);
            wv4 = *(const uint32_t *)(src + 32);
        } else {
            const uint32_t so = (uint32_t)(s * Geo<T>::STEP) & ~15u;
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[i] = *(const u32x4 *)(((GLU && i >= 2) ? wg2 : wg) + so + wofs[i]);
        }
    };

    // q8_1 activation loads.  Codes: instruction i covers columns 4i..4i+3, lane (column 4i +
    // lane/16, block (lane/2)%8, half lane%2) reads 16 code bytes; scales: lane (column lane/8,
    // block lane%8) reads the block's (d, s).  Missing columns re-read the last column and park
    // in the sink.
    const int nic = (ncols + 3) >> 2;
    int64_t acoff[2];
    int32_t acdst[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = 4 * i + (lane >> 4), b = (lane >> 1) & 7, h = lane & 1;
        const int ce = c < ncols ? c : ncols - 1;
        acoff[i] = (EXPERT ? mc.arow(ce) : (int64_t)ce) * (int64_t)col_bytes + 36 * b + 4 + 16 * h;
        acdst[i] = c < ncols ? A0 + c * 256 + 32 * b + 16 * h : kSink;
    }
    int64_t asoff;
    int32_t asdst;
    {
        const int c = lane >> 3, b = lane & 7;
        const int ce = c < ncols ? c : ncols - 1;
        asoff = (EXPERT ? mc.arow(ce) : (int64_t)ce) * (int64_t)col_bytes + 36 * b;
        asdst = c < ncols ? F0 + 8 * (8 * b + c) : kSink;
    }
    u32x4 av[2];
    uint32_t ads = 0;

    // fp32 input: a column's 256 step values are 8 blocks of 4 lanes, 8 values per lane, so a
    // pass covers columns 2i + lane/32; the first NPF passes are fetched ahead into registers
    // (one for Q6_K, whose unpacking needs registers, three for Q5_K, whose fifth bits do: four
    // would spill at the 128 registers 16 waves allow), the rest at park time.  Lanes of a
    // missing odd column quantize a copy of the last column and park it in the sink.
    constexpr int NPF = T == kQ6_K ? 1 : T == kQ5_K ? 3 : 4;
    const int cq = lane >> 5, ja = lane & 31;
    const size_t xstride = (size_t)P.nsteps * kSuper;
    const float *xf = (const float *)xin + 8 * ja;
    size_t xcol[4];
    int32_t xdst[4], xfd[4];
    const int qb = (lane >> 2) & 7, qsub = lane & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = 2 * i + cq;
        xcol[i] = (size_t)(c < ncols ? c : ncols - 1) * xstride;
        xdst[i] = c < ncols ? A0 + c * 256 + 32 * qb + 8 * qsub : kSink;
        xfd[i] = c < ncols && qsub == 0 ? F0 + 8 * (8 * qb + c) : kSink;
    }
    float4 xa[4], xb[4];   // prefetched passes (constant indices only: kept in registers)
    auto load8 = [&](int s, int i, float4 &a, float4 &b) __attribute__((always_inline)) {
        const float *src = xf + xcol[i] + s * kSuper;
        a = *(const float4 *)src;
        b = *(const float4 *)(src + 4);
    };
    auto load_a = [&](int s) __attribute__((always_inline)) {
        if constexpr (F32) {
#pragma unroll
            for (int i = 0; i < NPF; ++i)
                if (2 * i < ncols) load8(s, i, xa[i], xb[i]);   // wave-uniform test
        } else {
            const uint8_t *astep = (const uint8_t *)xin + (uint32_t)(s * kActStep);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                if (i < nic) av[i] = *(const u32x4_a4 *)(astep + acoff[i]);   // wave-uniform test
            ads = *(const uint32_t *)(astep + asoff);
        }
    };
    // Activations first: they come from L2, so their wait (loads retire in order) does not wait
    // for the weights, and quantizing or re-laying them overlaps the weights' flight.
    if (my_steps > 0) {
        load_a(wave);
        load_w(wave);
    }

    auto park = [&](int s) __attribute__((always_inline)) {
        if constexpr (F32) {
            // quantized before the weights are parked so late loads overlap the weights' arrival
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (2 * i < ncols) {   // wave-uniform
                    float4 a, bv;
                    if (i < NPF) {
                        a = xa[i];
                        bv = xb[i];
                    } else {
                        load8(s, i, a, bv);
                    }
                    const Q81Lane4 q = quantize_q8_1_lane4(a, bv);
                    *(u32x2 *)(st + xdst[i]) = u32x2{q.c0, q.c1};
                    *(float2 *)(st + xfd[i]) = make_float2(h2f((uint16_t)(q.ds & 0xFFFF)), h2f((uint16_t)(q.ds >> 16)));
                }
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                if (i < nic) *(u32x4 *)(st + acdst[i]) = av[i];
            *(float2 *)(st + asdst) = make_float2(h2f((uint16_t)(ads & 0xFFFF)), h2f((uint16_t)(ads >> 16)));
        }
        if constexpr (REG) {
            // weights stay in registers (pw)
        } else if constexpr (kK45<T>) {
#pragma unroll
            for (int i = 0; i < 4; ++i) *(u32x4 *)(st + pofs[i]) = wv[i];
        } else if constexpr (T == kQ6_K) {
            // the super-block starts a6 bytes into the aligned window: shift every piece by a6
            // (wave-uniform) so that LDS row r holds super-block bytes 0..209 at offset 0
            const uint32_t a6 = (uint32_t)(s * 210) & 15u;
            u32x4 nx[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                nx[i] = u32x4{from_next_lane(wv[i].x), from_next_lane(wv[i].y), from_next_lane(wv[i].z),
                              from_next_lane(wv[i].w)};
            auto put = [&](auto QC) __attribute__((always_inline)) {
                constexpr int Q = decltype(QC)::value;
#pragma unroll
                for (int i = 0; i < 4; ++i) *(u32x4 *)(st + pofs[i]) = shift_piece<Q>(wv[i], nx[i], a6 & 3u);
            };
            switch (a6 >> 2) {
                case 0: put(IC<0>{}); break;
                case 1: put(IC<1>{}); break;
                case 2: put(IC<2>{}); break;
                default: put(IC<3>{}); break;
            }
        } else if constexpr (T == kQ4_0) {
            // bytes 0..35 of blocks 2p, 2p+1 = {d0, qs0[16], d1, qs1[16]}: qs0 sits 2 bytes off a
            // dword boundary, qs1 on one; nibble - 8 as int8 is (n + 120) ^ 0x80 per byte
            const uint32_t D[9] = {wv[0].x, wv[0].y, wv[0].z, wv[0].w, wv[1].x, wv[1].y, wv[1].z, wv[1].w, wv4};
            const uint32_t q0[4] = {abyte(D[1], D[0], 2), abyte(D[2], D[1], 2), abyte(D[3], D[2], 2), abyte(D[4], D[3], 2)};
            const uint32_t q1[4] = {D[5], D[6], D[7], D[8]};
            auto c4 = [](uint32_t nib) { return (nib + 0x78787878u) ^ 0x80808080u; };
            uint8_t *dst = st + r8 * RSTR + 64 * p8;
            *(u32x4 *)dst = u32x4{c4(q0[0] & 0x0F0F0F0Fu), c4(q0[1] & 0x0F0F0F0Fu), c4(q0[2] & 0x0F0F0F0Fu), c4(q0[3] & 0x0F0F0F0Fu)};
            *(u32x4 *)(dst + 16) = u32x4{c4((q0[0] >> 4) & 0x0F0F0F0Fu), c4((q0[1] >> 4) & 0x0F0F0F0Fu),
                                         c4((q0[2] >> 4) & 0x0F0F0F0Fu), c4((q0[3] >> 4) & 0x0F0F0F0Fu)};
            *(u32x4 *)(dst + 32) = u32x4{c4(q1[0] & 0x0F0F0F0Fu), c4(q1[1] & 0x0F0F0F0Fu), c4(q1[2] & 0x0F0F0F0Fu), c4(q1[3] & 0x0F0F0F0Fu)};
            *(u32x4 *)(dst + 48) = u32x4{c4((q1[0] >> 4) & 0x0F0F0F0Fu), c4((q1[1] >> 4) & 0x0F0F0F0Fu),
                                         c4((q1[2] >> 4) & 0x0F0F0F0Fu), c4((q1[3] >> 4) & 0x0F0F0F0Fu)};
            *(float2 *)(st + kRows * RSTR + 4 * (8 * r8 + 2 * p8)) =
                make_float2(h2f((uint16_t)(D[0] & 0xFFFF)), h2f((uint16_t)(D[4] >> 16)));
        } else {
            // Q8_0: bytes 0..67 of blocks 2p, 2p+1 = {d0, q0[32], d1, q1[32]}; q0 sits 2 bytes off
            // a dword boundary, q1 on one
            const uint32_t D[17] = {wv[0].x, wv[0].y, wv[0].z, wv[0].w, wv[1].x, wv[1].y, wv[1].z, wv[1].w,
                                    wv[2].x, wv[2].y, wv[2].z, wv[2].w, wv[3].x, wv[3].y, wv[3].z, wv[3].w, wv4};
            uint8_t *dst = st + r8 * RSTR + 64 * p8;
            *(u32x4 *)dst = u32x4{abyte(D[1], D[0], 2), abyte(D[2], D[1], 2), abyte(D[3], D[2], 2), abyte(D[4], D[3], 2)};
            *(u32x4 *)(dst + 16) = u32x4{abyte(D[5], D[4], 2), abyte(D[6], D[5], 2), abyte(D[7], D[6], 2), abyte(D[8], D[7], 2)};
            *(u32x4 *)(dst + 32) = u32x4{D[9], D[10], D[11], D[12]};
            *(u32x4 *)(dst + 48) = u32x4{D[13], D[14], D[15], D[16]};
            *(float2 *)(st + kRows * RSTR + 4 * (8 * r8 + 2 * p8)) =
                make_float2(h2f((uint16_t)(D[0] & 0xFFFF)), h2f((uint16_t)(D[8] >> 16)));
        }
    };
    if (lane < kZeroBytes / 4) ((uint32_t *)zero)[lane] = 0u;     // read only by this wave
    ((float2 *)(st + F0))[lane] = make_float2(0.f, 0.f);          // columns past ncols stay zero

    // Per-lane operand addresses (offsets within a stage).
    const int g = lane >> 4, r16 = lane & 15;
    const int m = r16;   // this lane's A row
    const int wrow = r16 * RSTR;
    // A operand of slice j for column group cg: abase[cg] + aoffj(j); abase is the zero block
    // for lanes off the diagonal or past the last column.
    const uint8_t *abase[NCG];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
        int c, blk0, half;
        bool on;
        if (kK45<T>) {
            const int sel = m >> 3;
            c = m & 7;
            on = q4_group(g) == sel;
            blk0 = q4_sub(0, sel);
            half = q4_half(g);
        } else if (T == kQ6_K) {
            const int grp = m >> 2;
            c = (m & 3) + 4 * cg;
            on = g == grp;
            blk0 = grp >> 1;
            half = grp & 1;
        } else {
            const int sel = m >> 3;
            c = m & 7;
            on = (g >> 1) == sel;
            blk0 = sel;
            half = g & 1;
        }
        abase[cg] = on && c < ncols ? st + A0 + c * 256 + blk0 * 32 + 16 * half : zero;
    }
    // Q4_K: slice j covers sub-blocks (j>>1)*4 + (j&1) + 2*sel; Q6_K / Q8_0: blocks 2j + ...
    auto aoffj = [](int j) { return kK45<T> ? 32 * ((j >> 1) * 4 + (j & 1)) : 64 * j; };
    static_assert(!kK45<T> || 32 * 5 + 16 <= kZeroBytes, "zero block too small");
    static_assert(64 * 3 + 16 <= kZeroBytes, "zero block too small");

    float acc[NCG][4];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[cg][e] = 0.f;

    int32_t *dbg_row = nullptr;
    int64_t dbg_ld = 0;
    const int64_t row = row0 + r16;
    if (DBG && row < rows) {
        const int64_t per = (T == kQ6_K) ? (int64_t)P.nsteps * 16 : (int64_t)P.nsteps * 8;
        dbg_ld = rows * per;
        dbg_row = dbg + row * per;
    }
    const i32x4 zero4 = {0, 0, 0, 0};
    const float2 *ftab = (const float2 *)(st + F0);

    for (int it = 0; it < my_steps; ++it) {
        const int s = wave + it * nwaves;
        park(s);
        // weights in registers: step s's pieces, taken before the next step's loads refill pw
        u32x4 pc[REG ? 5 : 1];
        uint16_t pcd = 0;
        if constexpr (REG) {
#pragma unroll
            for (int i = 0; i < 5; ++i) pc[i] = pw[i];
            pcd = pwd;
        }
        if (it + 1 < my_steps) {   // the next step's loads fly during this step's math
            load_a(s + nwaves);
            load_w(s + nwaves);
        }

        auto aop = [&](int cg, int j) -> u32x4 { return lds16(abase[cg] + aoffj(j)); };
        if constexpr (kK45<T>) {
            constexpr int QS = T == kQ5_K ? 32 : 0;   // Q5_K: qs after qh[32]
            const uint8_t *wr = st + wrow;
            // this lane's qs pieces: (g + 3) % 4 and 4 + (g + 3) % 4 of the row's eight
            const int qa = (g + 3) & 3;
            const u32x4 hdr = REG ? pc[0] : lds16(wr);
            const u32x4 src1 = REG ? pc[1] : lds16(wr + QS + 16 + 16 * qa);
            const u32x4 src2 = REG ? pc[2] : lds16(wr + QS + 16 + 16 * (4 + qa));
            const int sel = g >> 1;
            const float d = h2f((uint16_t)(hdr.x & 0xFFFF));
            const float dmin = h2f((uint16_t)(hdr.x >> 16));
            const uint32_t sc_lo = (hdr.y & 0x3F3F3F3Fu) >> (16 * sel);
            const uint32_t m_lo = (hdr.z & 0x3F3F3F3Fu) >> (16 * sel);
            const uint32_t sc_hi = ((hdr.w & 0x0F0F0F0Fu) | ((hdr.y >> 2) & 0x30303030u)) >> (16 * sel);
            const uint32_t m_hi = (((hdr.w >> 4) & 0x0F0F0F0Fu) | ((hdr.z >> 2) & 0x30303030u)) >> (16 * sel);
            u32x4 bop[4] = {nib_lo4(src1), nib_hi4(src1), nib_lo4(src2), nib_hi4(src2)};
            if constexpr (T == kQ5_K) {
                // fifth bits: this lane's bytes are values 16*half.. of sub-blocks
                // 2*group + (j&1) + 4*(j>>1); bit (sub-block) of qh bytes 16*half..
                const u32x4 qh = REG ? pc[REG ? 3 : 0] : lds16(wr + 16 + 16 * q4_half(g));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int sbb = 2 * q4_group(g) + (j & 1) + 4 * (j >> 1);
                    bop[j].x |= ((qh.x >> sbb) & 0x01010101u) << 4;
                    bop[j].y |= ((qh.y >> sbb) & 0x01010101u) << 4;
                    bop[j].z |= ((qh.z >> sbb) & 0x01010101u) << 4;
                    bop[j].w |= ((qh.w >> sbb) & 0x01010101u) << 4;
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const i32x4 D = mfma16x16x64(aop(0, j), bop[j], zero4);
                const int sb = q4_sub(j, sel);
                if (DBG) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = 4 * (g & 1) + e;
                        if (dbg_row && c < ncols) dbg_row[(int64_t)c * dbg_ld + s * 8 + sb] = D[e];
                    }
                } else {
                    const uint32_t scw = j < 2 ? sc_lo : sc_hi, mw = j < 2 ? m_lo : m_hi;
                    const float ws = d * (float)((scw >> (8 * (j & 1))) & 0xFF);
                    const float wm = dmin * (float)((mw >> (8 * (j & 1))) & 0xFF);
                    const f32x4 t0 = *(const f32x4 *)(ftab + sb * 8 + 4 * (g & 1));
                    const f32x4 t1 = *(const f32x4 *)(ftab + sb * 8 + 4 * (g & 1) + 2);
                    acc[0][0] = fmaf(-wm, t0.y, fmaf((float)D[0], ws * t0.x, acc[0][0]));
                    acc[0][1] = fmaf(-wm, t0.w, fmaf((float)D[1], ws * t0.z, acc[0][1]));
                    acc[0][2] = fmaf(-wm, t1.y, fmaf((float)D[2], ws * t1.x, acc[0][2]));
                    acc[0][3] = fmaf(-wm, t1.w, fmaf((float)D[3], ws * t1.z, acc[0][3]));
                }
            }
        } else if constexpr (T == kQ6_K) {
            const uint8_t *wr = st + wrow;
            // original super-block bytes / panel slabs: ql pieces g and 4+g, qh pieces (g&1) and
            // 2+(g&1), the 16 scales, d
            const uint8_t *pr = st + 16 * r16;
            const u32x4 ql0 = PK ? pc[0] : lds16(wr + 16 * g);
            const u32x4 ql1 = PK ? pc[PK ? 1 : 0] : lds16(wr + 64 + 16 * g);
            const u32x4 qh0 = PK ? pc[PK ? 2 : 0] : lds16(wr + 128 + 16 * (g & 1));   // half 0
            const u32x4 qh1 = PK ? pc[PK ? 3 : 0] : lds16(wr + 160 + 16 * (g & 1));  // half 1
            const u32x4 scv = PK ? pc[PK ? 4 : 0] : lds16(wr + 192);
            const float d = h2f(PK ? pcd : *(const uint16_t *)(wr + 208));
            const u32x4 neg32 = {0xE0E0E0E0u, 0xE0E0E0E0u, 0xE0E0E0E0u, 0xE0E0E0E0u};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int odd = p & 1;
                const u32x4 L4 = (p >> 1) ? ql1 : ql0;
                const u32x4 H4 = (p >> 1) ? qh1 : qh0;
                const int tsh = 4 * odd + 2 * (g >> 1);
                u32x4 b;
                b.x = ((L4.x >> (4 * odd)) & 0x0F0F0F0Fu) | (((H4.x >> tsh) << 4) & 0x30303030u);
                b.y = ((L4.y >> (4 * odd)) & 0x0F0F0F0Fu) | (((H4.y >> tsh) << 4) & 0x30303030u);
                b.z = ((L4.z >> (4 * odd)) & 0x0F0F0F0Fu) | (((H4.z >> tsh) << 4) & 0x30303030u);
                b.w = ((L4.w >> (4 * odd)) & 0x0F0F0F0Fu) | (((H4.w >> tsh) << 4) & 0x30303030u);
                const uint32_t scw = p == 0 ? scv.x : p == 1 ? scv.y : p == 2 ? scv.z : scv.w;
                const float ws = d * (float)((int32_t)(scw << (24 - 8 * g)) >> 24);
                const int blk = 2 * p + (g >> 1);
#pragma unroll
                for (int cg = 0; cg < NCG; ++cg) {
                    if (cg * 4 >= ncols) break;
                    const u32x4 a = aop(cg, p);
                    i32x4 D = mfma16x16x64(a, b, zero4);
                    D = mfma16x16x64(a, neg32, D);
                    if (DBG) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int c = 4 * cg + e;
                            if (dbg_row && c < ncols) dbg_row[(int64_t)c * dbg_ld + s * 16 + 4 * p + g] = D[e];
                        }
                    } else {
                        const f32x4 t0 = *(const f32x4 *)(ftab + blk * 8 + 4 * cg);
                        const f32x4 t1 = *(const f32x4 *)(ftab + blk * 8 + 4 * cg + 2);
                        acc[cg][0] = fmaf((float)D[0], ws * t0.x, acc[cg][0]);
                        acc[cg][1] = fmaf((float)D[1], ws * t0.z, acc[cg][1]);
                        acc[cg][2] = fmaf((float)D[2], ws * t1.x, acc[cg][2]);
                        acc[cg][3] = fmaf((float)D[3], ws * t1.z, acc[cg][3]);
                    }
                }
            }
        } else {
            const uint8_t *wr = st + wrow;
            const float *wd = (const float *)(st + kRows * RSTR) + 8 * r16;
            const uint32_t wdw[4] = {pc[PK ? 4 : 0].x, pc[PK ? 4 : 0].y, pc[PK ? 4 : 0].z, pc[PK ? 4 : 0].w};   // panel: fp16 d
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int blk = 2 * p + (g >> 1);
                u32x4 q;
                if constexpr (PK && T == kQ4_0) {
                    // block blk's 16 nibble bytes; this lane's half (g & 1) of its 32 values as
                    // int8 nibble - 8: (n + 120) ^ 0x80 per byte
                    const u32x4 nb = pc[p];
                    const uint32_t sh = 4 * (g & 1);
                    auto c4 = [sh](uint32_t v) { return (((v >> sh) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u; };
                    q = u32x4{c4(nb.x), c4(nb.y), c4(nb.z), c4(nb.w)};
                } else if constexpr (PK) {
                    q = pc[p];
                } else {
                    q = lds16(wr + 64 * p + 16 * g);
                }
                const i32x4 D = mfma16x16x64(aop(0, p), q, zero4);
                if (DBG) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = 4 * (g & 1) + e;
                        if (dbg_row && c < ncols) dbg_row[(int64_t)c * dbg_ld + s * 8 + blk] = D[e];
                    }
                } else {
                    const float ws = PK ? h2f((uint16_t)(wdw[blk >> 1] >> (16 * (blk & 1)))) : wd[blk];
                    const f32x4 t0 = *(const f32x4 *)(ftab + blk * 8 + 4 * (g & 1));
                    const f32x4 t1 = *(const f32x4 *)(ftab + blk * 8 + 4 * (g & 1) + 2);
                    acc[0][0] = fmaf((float)D[0], ws * t0.x, acc[0][0]);
                    acc[0][1] = fmaf((float)D[1], ws * t0.z, acc[0][1]);
                    acc[0][2] = fmaf((float)D[2], ws * t1.x, acc[0][2]);
                    acc[0][3] = fmaf((float)D[3], ws * t1.z, acc[0][3]);
                }
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
            if (T == kQ6_K) v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            acc[cg][e] = v;
        }
    // Each wave leaves its 16 rows x 8 columns (128 floats) at the start of its own stage:
    // Q4_K/Q8_0 lanes g < 2 hold columns 4g..4g+3 of row r16 (index 4*lane + e), Q6_K lanes
    // g == 0 hold columns 4cg + e (index 8*lane + 4cg + e).
    const bool holder = (T == kQ6_K) ? (g == 0) : (g < 2);
    float *red = (float *)st;
    if (holder) {
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[lane * (4 * NCG) + cg * 4 + e] = acc[cg][e];
    }
    __syncthreads();
    // Each of the 128 (row, column) sums over the waves is one thread's, all loads in flight at
    // once; a one-wave workgroup (K = 256) takes two per thread.
    for (int t = threadIdx.x; t < 128; t += blockDim.x) {
        int rr, c;
        if (T == kQ6_K) { rr = t >> 3; c = t & 7; }
        else { rr = (t >> 2) & 15; c = 4 * (t >> 6) + (t & 3); }
        if (GLU && rr >= 8) continue;
        // GLU: the up value of (rr, c) sits at row rr + 8: index t + 64 (Q6_K) or t + 32
        constexpr int kUp = T == kQ6_K ? 64 : 32;
        float v = 0.f, u = 0.f;
        for (int wv = 0; wv < nwaves; ++wv) {
            const float *rb = (const float *)(smem + (size_t)wv * (kHead + SB) + kHead);
            v += rb[t];
            if (GLU) u += rb[t + kUp];
        }
        if (c < ncols && row0 + rr < rows) y[mc.pair(c) * rows + row0 + rr] = GLU ? v / (1.0f + expf(-v)) * u : v;
    }
    return true;
}

// Dense: one row group per workgroup.  Expert mode: the workgroups of grid row blockIdx.y take the
// listed small experts blockIdx.y, blockIdx.y + gridDim.y, ... until the list ends (it is compacted,
// -1 after the last), so the launch holds a few workgroups per row group rather than one per
// expert, most of which would find no expert to run.
template <int T, bool DBG, bool EXPERT, bool F32, bool GLU, bool PK = false>
__global__ __launch_bounds__(1024) void mmvq_stream_kernel(const uint8_t *__restrict__ w, const uint8_t *__restrict__ w2,
                                                          const void *__restrict__ xin,
                                                          float *__restrict__ y, int32_t *__restrict__ dbg,
                                                          MvArgs P, ColMap cm) {
    if constexpr (!EXPERT) {
        mmvq_stream_body<T, DBG, EXPERT, F32, GLU, PK>(w, w2, xin, y, dbg, P, cm, -1);
    } else {
        if (gridDim.y == (unsigned)cm.n_exp) {   // one expert slot per grid row: no loop
            mmvq_stream_body<T, DBG, EXPERT, F32, GLU, PK>(w, w2, xin, y, dbg, P, cm, (int)blockIdx.y);
            return;
        }
        for (int ey = blockIdx.y;;) {
            if (!mmvq_stream_body<T, DBG, EXPERT, F32, GLU, PK>(w, w2, xin, y, dbg, P, cm, ey)) break;
            ey += gridDim.y;
            if (ey >= cm.n_exp) break;
            __syncthreads();   // the next expert reuses the LDS stages
        }
    }
}

template <int T, bool DBG, bool EXPERT, bool F32 = false, bool GLU = false, bool PK = false>
hipError_t launch_t(const uint8_t *w, int64_t rows, int64_t k, const void *xq, int64_t n, float *y,
                    int32_t *dbg, const ColMap &c, int64_t n_exp, hipStream_t s, const uint8_t *w2 = nullptr) {
    const int64_t nsteps = k / kSuper;
    const int nw = (int)(nsteps < 16 ? nsteps : 16);
    const size_t smem = (size_t)nw * (kHead + Stage<T, kRegW<T, PK>>::BYTES);
    MvArgs a;
    a.rows = rows;
    a.row_bytes = (uint32_t)((k / Fmt<T>::QK) * Fmt<T>::BYTES);
    a.col_bytes = (uint32_t)(k / 32 * kQ8_1Bytes);
    a.nsteps = (int32_t)nsteps;
    a.q = (int32_t)(nsteps / nw);
    a.r = (int32_t)(nsteps % nw);
    a.n = (int32_t)n;
    // once per process (a function-local static is initialised exactly once, thread-safely)
    static const hipError_t attr_err = hipFuncSetAttribute((const void *)mmvq_stream_kernel<T, DBG, EXPERT, F32, GLU, PK>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr_err != hipSuccess) return attr_err;
    constexpr int RW = GLU ? kRows / 2 : kRows;
    const int64_t groups = (rows + RW - 1) / RW;
    dim3 grid((unsigned)groups, EXPERT ? (unsigned)mv_expert_slots(groups, n_exp, c.pairs) : 1u);
    hipLaunchKernelGGL((mmvq_stream_kernel<T, DBG, EXPERT, F32, GLU, PK>), grid, dim3(64 * (unsigned)nw), smem, s, w, w2,
                       xq, y, dbg, a, c);
    return hipGetLastError();
}

template <int T>
hipError_t dispatch(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y, int32_t *dbg,
                    const ColMap *cm, int64_t n_exp, hipStream_t s) {
    const ColMap c = cm ? *cm : ColMap{};
    if (dbg) return launch_t<T, true, false>(w, rows, k, xq, n, y, dbg, c, n_exp, s);
    if (cm) return launch_t<T, false, true>(w, rows, k, xq, n, y, dbg, c, n_exp, s);
    return launch_t<T, false, false>(w, rows, k, xq, n, y, dbg, c, n_exp, s);
}

}  // namespace

bool mmvq_stream_supported(int type, const void *w, int64_t k, const void *xq, const ColMap *cm) {
    if (type != kQ4_K && type != kQ5_K && type != kQ6_K && type != kQ8_0 && type != kQ4_0) return false;
    if (k % kSuper != 0 || k < kSuper) return false;
    const int64_t row_bytes = type == kQ8_0   ? k / 32 * 34
                              : type == kQ4_0 ? k / 32 * 18
                                              : k / 256 * (type == kQ4_K ? 144 : type == kQ5_K ? 176 : 210);
    // Q8_0 / Q4_0: 68- / 36-byte block pairs; else aligned windows
    const int64_t walign = type == kQ8_0 || type == kQ4_0 ? 4 : 16;
    if (row_bytes % walign != 0 || (uintptr_t)w % walign != 0) return false;
    if ((uintptr_t)xq % 4 != 0) return false;
    if (cm && cm->w_expert_stride % walign != 0) return false;
    return true;
}

hipError_t launch_mmvq_stream_f32(int type, const uint8_t *w, int64_t rows, int64_t k, const float *x, int64_t n,
                                  float *y, hipStream_t s) {
    const ColMap c{};
    if (type == kQ4_K) return launch_t<kQ4_K, false, false, true>(w, rows, k, x, n, y, nullptr, c, 0, s);
    if (type == kQ5_K) return launch_t<kQ5_K, false, false, true>(w, rows, k, x, n, y, nullptr, c, 0, s);
    if (type == kQ6_K) return launch_t<kQ6_K, false, false, true>(w, rows, k, x, n, y, nullptr, c, 0, s);
    if (type == kQ8_0) return launch_t<kQ8_0, false, false, true>(w, rows, k, x, n, y, nullptr, c, 0, s);
    if (type == kQ4_0) return launch_t<kQ4_0, false, false, true>(w, rows, k, x, n, y, nullptr, c, 0, s);
    return hipErrorInvalidValue;
}

hipError_t launch_mmvq_stream_panel_f32(int type, const uint8_t *wp, int64_t rows, int64_t k, const float *x, int64_t n,
                                        float *y, hipStream_t s) {
    const ColMap c{};
#define QMM_SP(TT) \
    if (type == TT) return launch_t<TT, false, false, true, false, true>(wp, rows, k, x, n, y, nullptr, c, 0, s);
    QMM_SP(kQ4_K)
    QMM_SP(kQ5_K)
    QMM_SP(kQ6_K)
    QMM_SP(kQ8_0)
    QMM_SP(kQ4_0)
#undef QMM_SP
    return hipErrorInvalidValue;
}

hipError_t launch_mmvq_stream(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n,
                              float *y, int32_t *dbg, const ColMap *cm, int64_t n_exp, hipStream_t s) {
    if (type == kQ4_K) return dispatch<kQ4_K>(w, rows, k, xq, n, y, dbg, cm, n_exp, s);
    if (type == kQ5_K) return dispatch<kQ5_K>(w, rows, k, xq, n, y, dbg, cm, n_exp, s);
    if (type == kQ6_K) return dispatch<kQ6_K>(w, rows, k, xq, n, y, dbg, cm, n_exp, s);
    if (type == kQ8_0) return dispatch<kQ8_0>(w, rows, k, xq, n, y, dbg, cm, n_exp, s);
    if (type == kQ4_0) return dispatch<kQ4_0>(w, rows, k, xq, n, y, dbg, cm, n_exp, s);
    return hipErrorInvalidValue;
}

hipError_t launch_mmvq_stream_glu(int type, const uint8_t *wg, const uint8_t *wu, int64_t rows, int64_t k,
                                  const void *x, bool x_fp32, int64_t n, float *y, const ColMap *cm, int64_t n_exp,
                                  hipStream_t s) {
    const ColMap c = cm ? *cm : ColMap{};
#define QMM_SG(TT)                                                                                                   \
    if (type == TT) {                                                                                                \
        if (cm) return launch_t<TT, false, true, false, true>(wg, rows, k, x, n, y, nullptr, c, n_exp, s, wu);     \
        if (x_fp32) return launch_t<TT, false, false, true, true>(wg, rows, k, x, n, y, nullptr, c, 0, s, wu);     \
        return launch_t<TT, false, false, false, true>(wg, rows, k, x, n, y, nullptr, c, 0, s, wu);                \
    }
    QMM_SG(kQ4_K)
    QMM_SG(kQ5_K)
    QMM_SG(kQ6_K)
    QMM_SG(kQ8_0)
    QMM_SG(kQ4_0)
#undef QMM_SG
    return hipErrorInvalidValue;
}

}  // namespace qmm
