// Tiled product for many activation columns (the MMQ regime of the MMQ page: "tiling skeleton",
// "J runtime selection", "tile efficiency", "stream-K", "fixup", "expert bounds").
//
// CDNA4 design.  A workgroup of 4 waves (8 for J = 128) owns a 128-row x J-column output tile
// (J = 32/64/128) and walks K in 256-value steps.  Each step's weight and activation tiles are
// fetched from HBM into registers while an earlier step computes (software pipelining: the loads
// of the next step are issued right after a step is parked in LDS; Q4_K 8-wave tiles keep two
// LDS step buffers and fetch two steps ahead), then parked in LDS: Q4_K as packed qs bytes plus
// per-(row, sub-block) scales d*sc (fp32) and mins -dmin*m (as exact bf16 pieces), Q8_0 as int8
// codes plus fp32 d, Q6_K unpacked (below); activations, read from the step-tiled q8_1 layout, as
// int8 codes plus fp32 (d, s) per 32-value block (the MMQ page's
// "why not dequantize": stay quantized and reuse each unpacked tile for J columns).  Each wave
// owns 32 rows; per 32-value block it runs one v_mfma_i32_32x32x32_i8 per 32 columns -- K = 32
// is exactly one q8_1 block, so every int32 result is one exact sub-block dot D -- and folds it
// into its fp32 accumulators with one multiply-add, the per-element scale coming from an
// outer-product MFMA:
//   Q4_K  acc += D * (d*sc * d_a);  the min term -(dmin*m) * s_a is a rank-8 product per step,
//         three v_mfma_f32_32x32x16_bf16 per column block over exact bf16 pieces
//   Q8_0  acc += D * (d_w * d_a)
//   Q6_K  acc += (sc0*D0 + sc1*D1) * (d * d_a)
// Q6_K changes scale every 16 values, so its int8 scale is folded into the codes at unpack time:
// v = sc*(q-32) lies in [-4064, 4096] and is split as v = 128*hi + lo with lo in [0,127] and hi
// in [-32, 32]; two MFMAs give D_hi and D_lo and sc0*D0 + sc1*D1 = 128*D_hi + D_lo exactly.
//
// Work split: `units` workgroups; the first dp_tiles = floor(ntiles/units)*units tiles go whole,
// unit u taking tiles u, u + units, ... (data-parallel rounds), and the units share the remaining
// tiles' W = (ntiles - dp_tiles)*k_iters (tile, step) items, unit u owning [u*W/units,
// (u+1)*W/units) (stream-K).  A unit that covers a whole tile writes it to y; a partial tile goes
// to the unit's slot (0: its first tile, 1: its last), and the last covering unit to finish --
// an atomic counter per split tile tells -- adds the slots in ascending unit order and writes the
// tile (finish_split: deterministic, no unit waits for another, no separate fixup launch).
// Splitting only the remainder keeps the partial round trip to the tiles that need it (at 448
// tiles on 256 units: 192 split tiles instead of nearly all 448).  Without stream-K, units ==
// ntiles and every unit is exactly one tile.  Tiles are numbered in bands of 8 row
// tiles walked column by column (tile_coords), units are contiguous per XCD.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace qmm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float bf16_val(uint32_t b) { return __builtin_bit_cast(float, b << 16); }

constexpr int kTI = 128;        // rows per tile
constexpr int kLd = 272;        // LDS bytes per 256-value row of int8 codes (+16 to spread banks)
constexpr int kLd4 = 144;       // LDS bytes per row of packed Q4_K qs (128 + 16)

struct MmqArgs {
    int64_t ntiles, n_ct, k_iters, units;
    float *partials;            // [units][2] slots of 128 x J floats
    int32_t *counters;          // [ntiles - dp_tiles] arrivals per split tile, zero when a call starts
    int32_t write_partials;     // stream-K active
    int64_t dp_tiles;           // tiles 0..dp_tiles-1 go whole, one per unit per round (data-parallel)
};

// Tile order: bands of kBand row tiles, each walked column by column, so that consecutive tiles
// (the ones an XCD runs at the same time, units being contiguous per XCD) share kBand weight row
// tiles and a few activation column tiles in that XCD's L2, instead of every XCD sweeping all
// column tiles for each pair of row tiles (which re-fetches the activations for every pair).
constexpr int64_t kBand = 8;
__device__ __forceinline__ void tile_coords(int64_t t, int64_t ntiles, int64_t n_ct, int64_t &rt, int64_t &ct) {
    const int64_t n_rt = ntiles / n_ct;
    const int64_t band = t / (kBand * n_ct), i = t - band * kBand * n_ct;
    const int64_t rows_in_band = n_rt - band * kBand < kBand ? n_rt - band * kBand : kBand;
    ct = i / rows_in_band;
    rt = band * kBand + (i - ct * rows_in_band);
}

// Threads per tile: 4 row waves (32 rows each) times J/64 column waves (J = 128: two 64-column
// halves, so every wave keeps at most 64 columns of accumulators and two waves fit per SIMD).
template <int J> struct Cfg {
    static constexpr int NWC = J == 128 ? 2 : 1;   // column waves
    static constexpr int NT = 256 * NWC;            // threads
    static constexpr int JW = J / NWC;              // columns per wave
    static constexpr int NCB = JW / 32;             // 32-column MFMA blocks per wave
};

// Q4_K and Q5_K share the super-block header, the scale/min packing and the fixup (the MMQ page
// pairs them in its "Q4_K load" section); Q5_K adds a fifth code bit per value.
template <int T> constexpr bool kK45 = T == kQ4_K || T == kQ5_K;
// Q8_0, Q4_0 and IQ4_XS: one scale per 32-value block; parked alike (int8 codes + fp32 scale).
template <int T> constexpr bool kB32 = T == kQ8_0 || T == kQ4_0 || T == kIQ4_XS;
// Q6_K and Q3_K: a scale per 16 values, folded into the codes at park time (two int8 planes).
template <int T> constexpr bool kQ6like = T == kQ6_K || T == kQ3_K;
// Types whose K need only be a multiple of 32 (the last step may be partial).
template <int T> constexpr bool kRaggedK = T == kQ8_0 || T == kQ4_0;
// Types the panel layout (repack.hip) serves.
template <int T> constexpr bool kPanel = T == kQ4_K || T == kQ5_K || T == kQ6_K || T == kQ8_0 || T == kQ4_0;

// LDS layout of one step: a weight part and an activation part, each in buffers of its own.
template <int T, int J> struct Smem {
    // weight part (offsets from a weight buffer)
    static constexpr int W_BYTES = kK45<T> ? kTI * kLd4 + (T == kQ5_K ? kTI * 32 : 0)   // qs (+ Q5_K qh)
                                          : (kQ6like<T> ? 2 * kTI * kLd : kTI * kLd);
    static constexpr int W_OFF = 0;
    static constexpr int QH_OFF = kTI * kLd4;                                     // Q5_K qh [128][32]
    static constexpr int WS_OFF = W_OFF + W_BYTES;                               // float [8][128]
    static constexpr int WM_OFF = WS_OFF + 8 * kTI * 4;                          // Q4_K: bf16 pieces of -dmin*m,
    static constexpr int W_PART = WM_OFF + (kK45<T> ? kTI * 48 : 0);            // [128][half][piece][4]
    // activation part (offsets from an activation buffer), an image of the tiled layout's records
    // (tiled_act.hpp): codes [J][kLd] (a column's 256 codes and 16 bytes of padding, so that the
    // rows of a B-operand read fall in distinct banks); d [8][J] fp32; s parts [J][8] (K-quants
    // with a min term)
    static constexpr int A_OFF = 0;
    static constexpr int X_OFF = A_OFF + J * kLd;
    static constexpr int XB_OFF = X_OFF + 8 * J * 4;
    static constexpr int A_PART = XB_OFF + (kK45<T> ? 8 * J * 4 : 0);
};

// Two LDS weight buffers where they fit beside the occupancy the tile runs at: K-quant 8-wave
// tiles (one workgroup per CU either way).  The activation part is always double-buffered.
template <int T, int J> constexpr bool kDoubleBuffer = kK45<T> && J == 128;
template <int T, int J> constexpr int kSmemBytes = (kDoubleBuffer<T, J> ? 2 : 1) * Smem<T, J>::W_PART + 2 * Smem<T, J>::A_PART;

typedef __attribute__((address_space(3))) void lds_void;

// ---------------------------------------------------------------------------------------------
// Activation tile: J columns of a step, copied from the tiled layout (tiled_act.hpp) into an
// activation buffer with direct global-to-LDS loads -- no registers, no vector ALU work and no
// LDS stores of the waves.  One wave instruction fills 64 consecutive LDS slots of 16 (or 4)
// bytes, lane l slot l, from sources the lane picks: code slot q is part q % 17 of column q / 17
// (parts 0-15 the column's 16-byte chunks, part 16 its padding, loaded with chunk 15 again); d
// slot x is block x / J of column x % J; s-part slot q is half q % 2 of column q / 2.  Each lane
// keeps the byte offsets of its slots' records (fixed for a tile: the step only moves the uniform
// table bases).  colrow(c) names the activation row of tile column c, always a valid row (columns
// past the end repeat one and are never written out).
// ---------------------------------------------------------------------------------------------
template <int T, int J> struct ActDirect {
    static constexpr int NT = Cfg<J>::NT, NW = NT / 64;
    static constexpr int NSLOT = J * 17;                      // code slots
    static constexpr int NI = (NSLOT + 63) / 64;              // code instructions (the last one partial for J = 32)
    static constexpr int NA = (NI + NW - 1) / NW;             // code instructions per wave, at most
    static constexpr int NX = J * 8 / 64 / NW;                // d slots (4 B) per lane
    static constexpr int NBW = kK45<T> ? J * 2 / 64 : 0;      // waves with one s-part instruction
    static_assert(NX * 64 * NW == J * 8 && NBW <= NW && kLd == 272, "activation slots");
    uint32_t ao[NA], xo[NX], bo;
    template <class CR> __device__ __forceinline__ void init(const CR &colrow) {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
        for (int m = 0; m < NA; ++m) {
            const int q = 64 * (w + NW * m) + lane;
            const int c = q / 17, part = q - 17 * c;
            ao[m] = q < NSLOT ? (uint32_t)colrow(c) * 256u + 16u * (uint32_t)(part < 16 ? part : 15) : 0u;
        }
#pragma unroll
        for (int m = 0; m < NX; ++m) {
            const int x = 64 * (w + NW * m) + lane, blk = x / J, c = x - blk * J;
            xo[m] = (uint32_t)colrow(c) * 32u + 4u * (uint32_t)blk;
        }
        bo = 0u;
        if constexpr (NBW > 0) {
            const int q = 64 * (w < NBW ? w : 0) + lane;
            bo = (uint32_t)colrow(q >> 1) * 32u + 16u * (uint32_t)(q & 1);
        }
    }
    // Step kb into the activation buffer at xsm (act_rows rows, nsteps steps in the layout).
    __device__ __forceinline__ void issue(uint8_t *xsm, const uint8_t *xq, int64_t kb, int64_t act_rows,
                                          int64_t nsteps) const {
        using L = Smem<T, J>;
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        const int64_t cells = nsteps * act_rows, cell0 = kb * act_rows;
        const uint8_t *codes = xq + cell0 * 256, *dtab = xq + cells * 256 + cell0 * 32;
#pragma unroll
        for (int m = 0; m < NA; ++m) {
            const int j = w + NW * m;
            if (j < NI && 64 * j + lane < NSLOT)   // wave-uniform but for the partial last instruction
                __builtin_amdgcn_global_load_lds((const void *)(codes + ao[m]), (lds_void *)(xsm + L::A_OFF + 1024 * j),
                                                 16, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < NX; ++m)
            __builtin_amdgcn_global_load_lds((const void *)(dtab + xo[m]), (lds_void *)(xsm + L::X_OFF + 256 * (w + NW * m)),
                                             4, 0, 0);
        if constexpr (NBW > 0) {
            if (w < NBW) {
                const uint8_t *ptab = xq + cells * 288 + cell0 * 32;
                __builtin_amdgcn_global_load_lds((const void *)(ptab + bo), (lds_void *)(xsm + L::XB_OFF + 1024 * w), 16, 0, 0);
            }
        }
    }
};

// The same tile through registers, for the Q4_K / Q5_K kernels: fetched ahead and stored by the
// waves in one burst, where direct loads (landing while a step computes) measured slower.  Thread
// tid owns (column, block) pairs i = tid + NT*it: column i/8, block i%8.
template <int T, int J> struct ActRegs {
    static constexpr int NT = Cfg<J>::NT, N = J * 8 / NT;
    uint32_t po[N];       // byte offset of the pair's column record in each table (times 1, 8 or 32)
    u32x4 c0[N], c1[N];   // the block's 32 codes
    float d[N];
    uint32_t sp[N];       // s parts
    template <class CR> __device__ __forceinline__ void init(const CR &colrow) {
#pragma unroll
        for (int it = 0; it < N; ++it) po[it] = (uint32_t)colrow((threadIdx.x + NT * it) >> 3);
    }
    __device__ __forceinline__ void fetch(const uint8_t *xq, int64_t kb, int64_t act_rows, int64_t nsteps) {
        const int64_t cells = nsteps * act_rows, cell0 = kb * act_rows;
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int blk = (threadIdx.x + NT * it) & 7;
            const uint8_t *src = xq + (cell0 + po[it]) * 256 + 32 * blk;
            c0[it] = *(const u32x4 *)src;
            c1[it] = *(const u32x4 *)(src + 16);
            d[it] = ((const float *)(xq + cells * 256))[(cell0 + po[it]) * 8 + blk];
            if constexpr (kK45<T>) sp[it] = ((const uint32_t *)(xq + cells * 288))[(cell0 + po[it]) * 8 + blk];
        }
    }
    __device__ __forceinline__ void store(uint8_t *xsm) const {
        using L = Smem<T, J>;
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int i = threadIdx.x + NT * it, col = i >> 3, blk = i & 7;
            uint8_t *cbase = xsm + L::A_OFF + col * kLd + 32 * blk;
            *(u32x4 *)cbase = c0[it];
            *(u32x4 *)(cbase + 16) = c1[it];
            ((float *)(xsm + L::X_OFF))[blk * J + col] = d[it];
            if constexpr (kK45<T>) ((uint32_t *)(xsm + L::XB_OFF))[col * 8 + blk] = sp[it];
        }
    }
};

// Waits until this wave's direct loads (and every earlier global load) have landed.
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------------------------
// Weight rows of a tile.  Plain: tile row t is matrix row r0 + t.  GLU (gate/up fusion, the MMQ
// page's fusion passage): the tile's 128 rows hold 64 outputs, alternating in groups of 8 between
// the gate (w0) and up (w1) matrices -- tile row t is row r0 + 8*(t/16) + t%8 of w1 if t & 8, else
// of w0 -- which in the accumulator layout puts the gate and up values of one output in elements
// e and e + 4 of the same lane.  Rows past the end repeat the last row (never written out).
// ---------------------------------------------------------------------------------------------
template <bool GLU> struct WRows {
    const uint8_t *w0;
    int64_t d01;   // GLU: byte distance from w0 to w1 (an offset, not a select: a select between two
                   // fields makes the compiler keep the struct in scratch memory)
    int64_t row_bytes, r0, rows;
    __device__ __forceinline__ WRows(const uint8_t *w0_, const uint8_t *w1_, int64_t rb, int64_t r0_, int64_t rows_)
        : w0(w0_), d01(GLU ? (int64_t)((uintptr_t)w1_ - (uintptr_t)w0_) : 0), row_bytes(rb), r0(r0_), rows(rows_) {}
    __device__ __forceinline__ const uint8_t *row(int t) const {
        int64_t r = GLU ? r0 + 8 * (t >> 4) + (t & 7) : r0 + t;
        r = r < rows ? r : rows - 1;
        return w0 + (GLU ? (int64_t)((t >> 3) & 1) * d01 : 0) + r * row_bytes;
    }
    // Byte o of tile row t's 256-value step kb (o counts from the step's first byte in the row).
    template <int T> __device__ __forceinline__ const uint8_t *at(int t, int64_t kb, int o) const {
        return row(t) + kb * (kSuper / Fmt<T>::QK * Fmt<T>::BYTES) + o;
    }
};

// ---------------------------------------------------------------------------------------------
// Weight rows in the panel layout (repack.hip): rows 16g..16g+15 x values 256s..256s+255 are the
// 16*B contiguous bytes of panel (g, s) at (g*nsteps + s) * 16*B; slab j (256 bytes at 256*j)
// holds a 16-byte piece per row.  panel_off maps byte o of a row's step in the original layout to
// its panel offset for row i of the group; every fetch below reads a run that stays inside one
// piece (or, for the fp16 scales, one 2-byte unit), so the run is contiguous in both layouts.
// ---------------------------------------------------------------------------------------------
template <int T> __device__ __forceinline__ int panel_off(int o, int i) {
    if constexpr (T == kQ4_K) {
        return o < 16 ? 8 * 256 + 16 * i + o : ((o - 16) >> 4) * 256 + 16 * i + ((o - 16) & 15);
    } else if constexpr (T == kQ5_K) {
        return o < 16 ? 10 * 256 + 16 * i + o
               : o < 48 ? ((o - 16) >> 4) * 256 + 16 * i + ((o - 16) & 15)
                        : (2 + ((o - 48) >> 4)) * 256 + 16 * i + ((o - 48) & 15);
    } else if constexpr (T == kQ6_K) {
        return o < 192 ? (o >> 4) * 256 + 16 * i + (o & 15)   // ql: slabs 0-7, qh: slabs 8-11
               : o < 208 ? 12 * 256 + 16 * i + (o - 192)
                         : 13 * 256 + 2 * i + (o - 208);
    } else if constexpr (T == kQ8_0) {
        const int b = o / 34, q = o - 34 * b;
        return q < 2 ? 16 * 256 + 16 * i + 2 * b + q : (2 * b + ((q - 2) >> 4)) * 256 + 16 * i + ((q - 2) & 15);
    } else {
        static_assert(T == kQ4_0, "the panel layout serves Q4_K, Q5_K, Q6_K, Q8_0 and Q4_0");
        const int b = o / 18, q = o - 18 * b;
        return q < 2 ? 8 * 256 + 16 * i + 2 * b + q : b * 256 + 16 * i + (q - 2);
    }
}

struct WPanels {
    const uint8_t *w;
    int64_t group_bytes;   // nsteps * panel bytes: one row group's panels
    int64_t r0, rows;
    template <int T> __device__ __forceinline__ const uint8_t *at(int t, int64_t kb, int o) const {
        int64_t r = r0 + t;
        r = r < rows ? r : rows - 1;   // rows past the end repeat the last row (never written out)
        return w + (r >> 4) * group_bytes + kb * (16 * (kSuper / Fmt<T>::QK * Fmt<T>::BYTES)) +
               panel_off<T>(o, (int)(r & 15));
    }
};

// ---------------------------------------------------------------------------------------------
// Weight tile fetch / park: the tile's 128 rows (WRows) of step kb.
// ---------------------------------------------------------------------------------------------
template <int T, int NT> struct WFetch;

// Q4_K: qs pieces (row i/8, 16-byte piece i%8 of the 128 qs bytes) and the row headers (threads
// below 128, whole waves).
// Q5_K: the same, with the qs bytes 32 bytes further (after qh[32]) and the two 16-byte qh pieces
// of each row (threads below 256, whole waves) parked beside the qs.
template <int T, int NT> struct WFetchK45 {
    static constexpr int N = 1024 / NT, NH = T == kQ5_K ? (256 + NT - 1) / NT : 0;
    static constexpr int BB = Fmt<T>::BYTES, QS = T == kQ5_K ? 48 : 16;   // block bytes, qs offset
    u32x4 q[N], h, qh[NH > 0 ? NH : 1];
    template <class WR>
    __device__ __forceinline__ void fetch(const WR &wr, int64_t kb, int64_t) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int i = tid + NT * it;
            q[it] = ld16(wr.template at<T>(i >> 3, kb, QS + 16 * (i & 7)));
        }
        if (tid < kTI) h = ld16(wr.template at<T>(tid, kb, 0));
#pragma unroll
        for (int it = 0; it < NH; ++it) {
            const int i = tid + NT * it;
            if (i < 256) qh[it] = ld16(wr.template at<T>(i >> 1, kb, 16 + 16 * (i & 1)));
        }
    }
    template <int J, class WR>
    __device__ __forceinline__ void store(uint8_t *sm, const WR &, int64_t, int64_t) const {
        const int tid = threadIdx.x;
        uint8_t *sW = sm + Smem<T, J>::W_OFF;
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int i = tid + NT * it;
            *(u32x4 *)(sW + (i >> 3) * kLd4 + 16 * (i & 7)) = q[it];
        }
#pragma unroll
        for (int it = 0; it < NH; ++it) {
            const int i = tid + NT * it;
            if (i < 256) *(u32x4 *)(sm + Smem<T, J>::QH_OFF + (i >> 1) * 32 + 16 * (i & 1)) = qh[it];
        }
        if (tid < kTI) {
            float *sWs = (float *)(sm + Smem<T, J>::WS_OFF);
            const float d = h2f((uint16_t)(h.x & 0xFFFF)), dmin = h2f((uint16_t)(h.x >> 16));
            const uint32_t sc_lo = h.y & 0x3F3F3F3Fu, m_lo = h.z & 0x3F3F3F3Fu;
            const uint32_t sc_hi = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
            const uint32_t m_hi = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
            // c = -dmin*m has at most 17 significant bits (exact in fp32) and splits exactly into
            // three bf16 pieces p0 + p1 + p2 (8 + 8 + 1 bits), with fp32's exponent range
            uint32_t pc[3][8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t scw = j < 4 ? sc_lo : sc_hi, mw = j < 4 ? m_lo : m_hi;
                const int sh = 8 * (j & 3);
                sWs[j * kTI + tid] = d * (float)((scw >> sh) & 0xFF);
                const float c = -(dmin * (float)((mw >> sh) & 0xFF));
                pc[0][j] = bf16_bits(c);
                const float r = c - bf16_val(pc[0][j]);
                pc[1][j] = bf16_bits(r);
                pc[2][j] = bf16_bits(r - bf16_val(pc[1][j]));
            }
            // row layout [half][piece][4 sub-blocks]: the 24 bytes a lane of a half reads
            uint32_t wv[12];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int m = 0; m < 3; ++m) {
                    wv[6 * hf + 2 * m] = pc[m][4 * hf] | (pc[m][4 * hf + 1] << 16);
                    wv[6 * hf + 2 * m + 1] = pc[m][4 * hf + 2] | (pc[m][4 * hf + 3] << 16);
                }
            u32x4 *dst = (u32x4 *)(sm + Smem<T, J>::WM_OFF + tid * 48);
            dst[0] = u32x4{wv[0], wv[1], wv[2], wv[3]};
            dst[1] = u32x4{wv[4], wv[5], wv[6], wv[7]};
            dst[2] = u32x4{wv[8], wv[9], wv[10], wv[11]};
        }
    }
};

template <int NT> struct WFetch<kQ4_K, NT> : WFetchK45<kQ4_K, NT> {};
template <int NT> struct WFetch<kQ5_K, NT> : WFetchK45<kQ5_K, NT> {};

// Q8_0: 16 code bytes per (row, block, half) and the fp16 d per (row, block); blocks past the end
// of a ragged last step read as zero.
template <int NT> struct WFetch<kQ8_0, NT> {
    static constexpr int NQ = 2048 / NT, ND = 1024 / NT;
    u32x4 q[NQ];
    uint16_t d[ND];
    template <class WR>
    __device__ __forceinline__ void fetch(const WR &wr, int64_t kb, int64_t nb32) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int it = 0; it < NQ; ++it) {
            const int i = tid + NT * it;
            const int bs = (i >> 1) & 7;   // block within the step
            const int64_t b = kb * 8 + bs;
            q[it] = b < nb32 ? ld16(wr.template at<kQ8_0>(i >> 4, kb, 34 * bs + 2 + 16 * (i & 1))) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int it = 0; it < ND; ++it) {
            const int i = tid + NT * it;
            const int64_t b = kb * 8 + (i & 7);
            d[it] = b < nb32 ? ld2(wr.template at<kQ8_0>(i >> 3, kb, 34 * (i & 7))) : (uint16_t)0;
        }
    }
    template <int J, class WR>
    __device__ __forceinline__ void store(uint8_t *sm, const WR &, int64_t, int64_t) const {
        const int tid = threadIdx.x;
        uint8_t *sW = sm + Smem<kQ8_0, J>::W_OFF;
        float *sWs = (float *)(sm + Smem<kQ8_0, J>::WS_OFF);
#pragma unroll
        for (int it = 0; it < NQ; ++it) {
            const int i = tid + NT * it;
            *(u32x4 *)(sW + (i >> 4) * kLd + 32 * ((i >> 1) & 7) + 16 * (i & 1)) = q[it];
        }
#pragma unroll
        for (int it = 0; it < ND; ++it) {
            const int i = tid + NT * it;
            sWs[(i & 7) * kTI + (i >> 3)] = h2f(d[it]);
        }
    }
};

// Q4_0: the 16 nibble bytes and the fp16 d per (row, block), parked as Q8_0's int8 codes
// (nibble - 8; low nibbles are values 0-15, high 16-31) and fp32 d; blocks past the end of a
// ragged last step get d = 0.
template <int NT> struct WFetch<kQ4_0, NT> {
    static constexpr int N = 1024 / NT;
    u32x4 q[N];
    uint16_t d[N];
    template <class WR>
    __device__ __forceinline__ void fetch(const WR &wr, int64_t kb, int64_t nb32) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int i = tid + NT * it;   // (row i/8, block i%8)
            const int64_t b = kb * 8 + (i & 7);
            q[it] = b < nb32 ? ld16(wr.template at<kQ4_0>(i >> 3, kb, 18 * (i & 7) + 2)) : u32x4{0u, 0u, 0u, 0u};
            d[it] = b < nb32 ? ld2(wr.template at<kQ4_0>(i >> 3, kb, 18 * (i & 7))) : (uint16_t)0;
        }
    }
    // nibble - 8 as int8, four bytes at a time: (n + 120) has bit 7 set iff n >= 8, so flipping
    // bit 7 gives n - 8 in two's complement; no byte carries (n + 120 <= 135)
    static __device__ __forceinline__ uint32_t code4(uint32_t nib) { return (nib + 0x78787878u) ^ 0x80808080u; }
    template <int J, class WR>
    __device__ __forceinline__ void store(uint8_t *sm, const WR &, int64_t, int64_t) const {
        const int tid = threadIdx.x;
        uint8_t *sW = sm + Smem<kQ4_0, J>::W_OFF;
        float *sWs = (float *)(sm + Smem<kQ4_0, J>::WS_OFF);
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int i = tid + NT * it;
            uint8_t *dst = sW + (i >> 3) * kLd + 32 * (i & 7);
            const u32x4 v = q[it];
            *(u32x4 *)dst = u32x4{code4(v.x & 0x0F0F0F0Fu), code4(v.y & 0x0F0F0F0Fu), code4(v.z & 0x0F0F0F0Fu),
                                  code4(v.w & 0x0F0F0F0Fu)};
            *(u32x4 *)(dst + 16) = u32x4{code4((v.x >> 4) & 0x0F0F0F0Fu), code4((v.y >> 4) & 0x0F0F0F0Fu),
                                         code4((v.z >> 4) & 0x0F0F0F0Fu), code4((v.w >> 4) & 0x0F0F0F0Fu)};
            sWs[(i & 7) * kTI + (i >> 3)] = h2f(d[it]);
        }
    }
};

// Q6_K scale folding for four codes c (the bytes of c6, each in [0, 63]) of one 16-value group:
// v = sc * (c - 32) in [-4064, 4096], split as v = 128 * hi + lo with lo in [0, 127] and hi in
// [-32, 32], returned as the byte vectors lo and hi.  Two codes per 32-bit lane pair: packed
// 16-bit integer multiply-add and arithmetic shift, then v_perm gathers the bytes.
typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void q6_split4(uint32_t c6, s16x2 sc2, s16x2 off2, uint32_t &lo, uint32_t &hi) {
    const uint32_t ce = c6 & 0x00FF00FFu;                          // codes 0, 2
    const uint32_t co = __builtin_amdgcn_perm(0u, c6, 0x0c030c01u);  // codes 1, 3
    const s16x2 ve = __builtin_bit_cast(s16x2, ce) * sc2 + off2;   // sc * c - 32 * sc
    const s16x2 vo = __builtin_bit_cast(s16x2, co) * sc2 + off2;
    const uint32_t ue = __builtin_bit_cast(uint32_t, ve), uo = __builtin_bit_cast(uint32_t, vo);
    lo = __builtin_amdgcn_perm(uo, ue, 0x06020400u) & 0x7F7F7F7Fu;
    const uint32_t he = __builtin_bit_cast(uint32_t, ve >> (short)7), ho = __builtin_bit_cast(uint32_t, vo >> (short)7);
    hi = __builtin_amdgcn_perm(ho, he, 0x06020400u);
}

// Q6_K with 4-wave tiles (J <= 64): unpacked straight from HBM into the two planes at park time
// (no register prefetch: the registers are taken by the accumulators).
template <int NT> struct WFetchQ6Direct {
    template <class WR>
    __device__ __forceinline__ void fetch(const WR &, int64_t, int64_t) {}
    template <int J, class WR>
    __device__ __forceinline__ void store(uint8_t *sm, const WR &wr, int64_t kb, int64_t) const {
        const int tid = threadIdx.x;
        int8_t *sLo = (int8_t *)(sm + Smem<kQ6_K, J>::W_OFF);
        int8_t *sHi = sLo + kTI * kLd;
#pragma unroll 2
        for (int it = 0; it < 2048 / NT; ++it) {
            const int i = tid + NT * it;               // (row, 16-value group G): 128 x 16
            const int r = i >> 4, G = i & 15;
            uint32_t lo_w[4], hi_w[4];
            {
                const int hh = G >> 3, gq = (G & 7) >> 1, l0 = 16 * (G & 1);
                const u32x4 ql = ld16(wr.template at<kQ6_K>(r, kb, 64 * hh + 32 * (gq & 1) + l0));
                const u32x4 qh = ld16(wr.template at<kQ6_K>(r, kb, 128 + 32 * hh + l0));
                const int sc = (int)(int8_t)*wr.template at<kQ6_K>(r, kb, 192 + G);
                const s16x2 sc2 = {(short)sc, (short)sc}, off2 = {(short)(-32 * sc), (short)(-32 * sc)};
                const int nsh = gq < 2 ? 0 : 4, tsh = 2 * gq;
                const uint32_t qlw[4] = {ql.x, ql.y, ql.z, ql.w}, qhw[4] = {qh.x, qh.y, qh.z, qh.w};
#pragma unroll
                for (int dd = 0; dd < 4; ++dd) {
                    const uint32_t code6 = ((qlw[dd] >> nsh) & 0x0F0F0F0Fu) | (((qhw[dd] >> tsh) & 0x03030303u) << 4);
                    q6_split4(code6, sc2, off2, lo_w[dd], hi_w[dd]);
                }
            }
            *(u32x4 *)(sLo + r * kLd + 16 * G) = u32x4{lo_w[0], lo_w[1], lo_w[2], lo_w[3]};
            *(u32x4 *)(sHi + r * kLd + 16 * G) = u32x4{hi_w[0], hi_w[1], hi_w[2], hi_w[3]};
        }
        if (tid < kTI) {
            float *sWs = (float *)(sm + Smem<kQ6_K, J>::WS_OFF);
            sWs[tid] = h2f(ld2(wr.template at<kQ6_K>(tid, kb, 208)));
        }
    }
};

// Q6_K with 8-wave tiles (J = 128): thread u owns row u/4 and, of its 16 sixteen-value groups,
// the four with G/8 = (u/2)%2 and G%2 = u%2 (gq = 0..3).  It prefetches exactly the pieces those
// groups need -- the two 16-byte ql pieces (low nibbles: gq 0/1, high: gq 2/3), the 16-byte qh
// piece (2-bit fields gq) and the 16 scale bytes (the thread takes its four), plus the fp16 d for
// one thread per row -- and unpacks them from registers into the two planes at park time.
template <int NT> struct WFetchQ6Reg {
    static_assert(NT == 512, "one (row, half, group-parity) unit per thread");
    u32x4 ql0, ql1, qh, sc;
    uint16_t d;
    template <class WR>
    __device__ __forceinline__ void fetch(const WR &wr, int64_t kb, int64_t) {
        const int u = threadIdx.x;
        const int r = u >> 2, hh = (u >> 1) & 1, l0 = 16 * (u & 1);
        ql0 = ld16(wr.template at<kQ6_K>(r, kb, 64 * hh + l0));
        ql1 = ld16(wr.template at<kQ6_K>(r, kb, 64 * hh + 32 + l0));
        qh = ld16(wr.template at<kQ6_K>(r, kb, 128 + 32 * hh + l0));
        sc = ld16(wr.template at<kQ6_K>(r, kb, 192));
        d = (u & 3) == 0 ? ld2(wr.template at<kQ6_K>(r, kb, 208)) : (uint16_t)0;
    }
    template <int J, class WR>
    __device__ __forceinline__ void store(uint8_t *sm, const WR &, int64_t, int64_t) const {
        const int u = threadIdx.x;
        const int r = u >> 2, hh = (u >> 1) & 1, half = u & 1;
        int8_t *sLo = (int8_t *)(sm + Smem<kQ6_K, J>::W_OFF);
        int8_t *sHi = sLo + kTI * kLd;
        const uint32_t scw[4] = {sc.x, sc.y, sc.z, sc.w};
        const uint32_t qlw0[4] = {ql0.x, ql0.y, ql0.z, ql0.w}, qlw1[4] = {ql1.x, ql1.y, ql1.z, ql1.w};
        const uint32_t qhw[4] = {qh.x, qh.y, qh.z, qh.w};
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int G = 8 * hh + 2 * gq + half;
            const int scv = (int)(int8_t)((scw[G >> 2] >> (8 * (G & 3))) & 0xFF);
            const s16x2 sc2 = {(short)scv, (short)scv}, off2 = {(short)(-32 * scv), (short)(-32 * scv)};
            const int nsh = gq < 2 ? 0 : 4, tsh = 2 * gq;
            uint32_t lo_w[4], hi_w[4];
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) {
                const uint32_t q = (gq & 1) ? qlw1[dd] : qlw0[dd];
                const uint32_t code6 = ((q >> nsh) & 0x0F0F0F0Fu) | (((qhw[dd] >> tsh) & 0x03030303u) << 4);
                q6_split4(code6, sc2, off2, lo_w[dd], hi_w[dd]);
            }
            *(u32x4 *)(sLo + r * kLd + 16 * G) = u32x4{lo_w[0], lo_w[1], lo_w[2], lo_w[3]};
            *(u32x4 *)(sHi + r * kLd + 16 * G) = u32x4{hi_w[0], hi_w[1], hi_w[2], hi_w[3]};
        }
        if ((u & 3) == 0) {
            float *sWs = (float *)(sm + Smem<kQ6_K, J>::WS_OFF);
            sWs[r] = h2f(d);
        }
    }
};

template <int NT> struct WFetch<kQ6_K, NT> : std::conditional<(NT >= 512), WFetchQ6Reg<NT>, WFetchQ6Direct<NT>>::type {};

// Q3_K (GP100 patch page, "How" step 3: 3-bit codes with a -4 offset; a 6-bit scale - 32 per 16
// values): parked like Q6_K, v = (sc - 32) * (q - 4) in [-124, 128] split into the two planes, the
// fp16 d per row in the scale slot.  Unit (row, 16-value group G), unpacked straight from HBM at
// park time: values 16G.. sit in half h = G/8, bit pair j = (G%8)/2, bytes l = 16(G&1)..: low bits
// 2j.. of qs[32h + l], third bit 4h + j of hmask[l]; scale G: low nibble in byte G%8 of the 12
// scale bytes (G < 8: low nibble, else high), top two bits at bit 2(G/4) of byte 8 + G%4.
template <int NT> struct WFetchQ3 {
    template <class WR>
    __device__ __forceinline__ void fetch(const WR &, int64_t, int64_t) {}
    template <int J, class WR>
    __device__ __forceinline__ void store(uint8_t *sm, const WR &wr, int64_t kb, int64_t) const {
        const int tid = threadIdx.x;
        int8_t *sLo = (int8_t *)(sm + Smem<kQ3_K, J>::W_OFF);
        int8_t *sHi = sLo + kTI * kLd;
#pragma unroll 2
        for (int it = 0; it < 2048 / NT; ++it) {
            const int i = tid + NT * it;               // (row, 16-value group G): 128 x 16
            const int r = i >> 4, G = i & 15;
            const int h = G >> 3, j = (G & 7) >> 1, l0 = 16 * (G & 1);
            const u32x4 qs = ld16(wr.template at<kQ3_K>(r, kb, 32 + 32 * h + l0));
            const u32x4 hm = ld16(wr.template at<kQ3_K>(r, kb, l0));
            const uint32_t lb = *wr.template at<kQ3_K>(r, kb, 96 + (G & 7));
            const uint32_t tb = *wr.template at<kQ3_K>(r, kb, 104 + (G & 3));
            const int sc = (int)((G < 8 ? (lb & 15u) : (lb >> 4)) | (((tb >> (2 * (G >> 2))) & 3u) << 4)) - 32;
            const s16x2 sc2 = {(short)sc, (short)sc}, off2 = {(short)(-4 * sc), (short)(-4 * sc)};
            const uint32_t qw[4] = {qs.x, qs.y, qs.z, qs.w}, hw[4] = {hm.x, hm.y, hm.z, hm.w};
            uint32_t lo_w[4], hi_w[4];
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) {
                const uint32_t code3 = ((qw[dd] >> (2 * j)) & 0x03030303u) | (((hw[dd] >> (4 * h + j)) & 0x01010101u) << 2);
                q6_split4(code3, sc2, off2, lo_w[dd], hi_w[dd]);
            }
            *(u32x4 *)(sLo + r * kLd + 16 * G) = u32x4{lo_w[0], lo_w[1], lo_w[2], lo_w[3]};
            *(u32x4 *)(sHi + r * kLd + 16 * G) = u32x4{hi_w[0], hi_w[1], hi_w[2], hi_w[3]};
        }
        if (tid < kTI) {
            float *sWs = (float *)(sm + Smem<kQ3_K, J>::WS_OFF);
            sWs[tid] = h2f(ld2(wr.template at<kQ3_K>(tid, kb, 108)));
        }
    }
};
// Q3_K with 8-wave tiles (J = 128), as Q6_K's: thread u owns row u/4 and the four 16-value groups
// G = 8h + 2j + half with h = (u/2)%2, half = u%2, j = 0..3 -- all four read the same 16 qs
// bytes 32h + 16 half.. (bit pairs j) and the same 16 hmask bytes 16 half.. (bits 4h + j) -- so it
// prefetches those two pieces, the 12 scale bytes and (one thread per row) d in the previous step,
// and unpacks them from registers at park time.
template <int NT> struct WFetchQ3Reg {
    static_assert(NT == 512, "one (row, half, group-parity) unit per thread");
    u32x4 qs, hm;
    uint32_t s0, s1, s2;
    uint16_t d;
    template <class WR>
    __device__ __forceinline__ void fetch(const WR &wr, int64_t kb, int64_t) {
        const int u = threadIdx.x;
        const int r = u >> 2, h = (u >> 1) & 1, l0 = 16 * (u & 1);
        qs = ld16(wr.template at<kQ3_K>(r, kb, 32 + 32 * h + l0));
        hm = ld16(wr.template at<kQ3_K>(r, kb, l0));
        s0 = ld4(wr.template at<kQ3_K>(r, kb, 96));
        s1 = ld4(wr.template at<kQ3_K>(r, kb, 100));
        s2 = ld4(wr.template at<kQ3_K>(r, kb, 104));
        d = (u & 3) == 0 ? ld2(wr.template at<kQ3_K>(r, kb, 108)) : (uint16_t)0;
    }
    template <int J, class WR>
    __device__ __forceinline__ void store(uint8_t *sm, const WR &, int64_t, int64_t) const {
        const int u = threadIdx.x;
        const int r = u >> 2, h = (u >> 1) & 1, half = u & 1;
        int8_t *sLo = (int8_t *)(sm + Smem<kQ3_K, J>::W_OFF);
        int8_t *sHi = sLo + kTI * kLd;
        const uint32_t qw[4] = {qs.x, qs.y, qs.z, qs.w}, hw[4] = {hm.x, hm.y, hm.z, hm.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int G = 8 * h + 2 * j + half, t = 2 * j + half;   // t = G % 8
            // low nibble of scale G in byte G%8 (nibble G/8 = h), top bits at 2(G/4) of byte 8 + G%4
            const uint32_t lb = ((t < 4 ? s0 : s1) >> (8 * (t & 3) + 4 * h)) & 15u;
            const uint32_t tb = (s2 >> (8 * (t & 3) + 2 * (2 * h + (j >> 1)))) & 3u;
            const int sc = (int)(lb | (tb << 4)) - 32;
            const s16x2 sc2 = {(short)sc, (short)sc}, off2 = {(short)(-4 * sc), (short)(-4 * sc)};
            uint32_t lo_w[4], hi_w[4];
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) {
                const uint32_t code3 = ((qw[dd] >> (2 * j)) & 0x03030303u) | (((hw[dd] >> (4 * h + j)) & 0x01010101u) << 2);
                q6_split4(code3, sc2, off2, lo_w[dd], hi_w[dd]);
            }
            *(u32x4 *)(sLo + r * kLd + 16 * G) = u32x4{lo_w[0], lo_w[1], lo_w[2], lo_w[3]};
            *(u32x4 *)(sHi + r * kLd + 16 * G) = u32x4{hi_w[0], hi_w[1], hi_w[2], hi_w[3]};
        }
        if ((u & 3) == 0) {
            float *sWs = (float *)(sm + Smem<kQ3_K, J>::WS_OFF);
            sWs[r] = h2f(d);
        }
    }
};

template <int NT> struct WFetch<kQ3_K, NT> : std::conditional<(NT >= 512), WFetchQ3Reg<NT>, WFetchQ3<NT>>::type {};

// IQ4_XS (GP100 patch page, "How" step 3: a 4-bit codebook index and a 6-bit scale - 32 per 32
// values): unit (row, sub-block b) -- the 16 index bytes qs[16b..] (low nibbles: values 0-15,
// high: 16-31), mapped through the codebook to int8 codes and parked as Q8_0's; the fp32 scale
// d * (ls - 32) with ls from nibble b&1 of scales_l[b/2] and bits 2b.. of scales_h.
template <int NT> struct WFetch<kIQ4_XS, NT> {
    static constexpr int N = 1024 / NT;
    u32x4 q[N];
    uint32_t h0[N], h1[N];
    template <class WR>
    __device__ __forceinline__ void fetch(const WR &wr, int64_t kb, int64_t) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int i = tid + NT * it;   // (row i/8, sub-block i%8)
            q[it] = ld16(wr.template at<kIQ4_XS>(i >> 3, kb, 8 + 16 * (i & 7)));
            h0[it] = ld4(wr.template at<kIQ4_XS>(i >> 3, kb, 0));
            h1[it] = ld4(wr.template at<kIQ4_XS>(i >> 3, kb, 4));
        }
    }
    template <int J, class WR>
    __device__ __forceinline__ void store(uint8_t *sm, const WR &, int64_t, int64_t) const {
        const int tid = threadIdx.x;
        uint8_t *sW = sm + Smem<kIQ4_XS, J>::W_OFF;
        float *sWs = (float *)(sm + Smem<kIQ4_XS, J>::WS_OFF);
#pragma unroll
        for (int it = 0; it < N; ++it) {
            const int i = tid + NT * it, b = i & 7;
            uint8_t *dst = sW + (i >> 3) * kLd + 32 * b;
            const u32x4 v = q[it];
            *(u32x4 *)dst = u32x4{iq4_lookup4(v.x & 0x0F0F0F0Fu), iq4_lookup4(v.y & 0x0F0F0F0Fu),
                                  iq4_lookup4(v.z & 0x0F0F0F0Fu), iq4_lookup4(v.w & 0x0F0F0F0Fu)};
            *(u32x4 *)(dst + 16) = u32x4{iq4_lookup4((v.x >> 4) & 0x0F0F0F0Fu), iq4_lookup4((v.y >> 4) & 0x0F0F0F0Fu),
                                         iq4_lookup4((v.z >> 4) & 0x0F0F0F0Fu), iq4_lookup4((v.w >> 4) & 0x0F0F0F0Fu)};
            const int ls = (int)(((h1[it] >> (8 * (b >> 1) + 4 * (b & 1))) & 15u) | (((h0[it] >> (16 + 2 * b)) & 3u) << 4));
            sWs[b * kTI + (i >> 3)] = h2f((uint16_t)(h0[it] & 0xFFFF)) * (float)(ls - 32);
        }
    }
};

// ---------------------------------------------------------------------------------------------
// One 256-value step of MFMAs + fixups for this wave's 32 rows x JW columns.  Wave wid: row wave
// rw = wid % 4 (rows 32*rw..), column wave cw = wid / 4 (columns JW*cw..).  Accumulator block cb,
// element e of lane l: row 32*rw + 8*(e/4) + 4*(l/32) + e%4, column JW*cw + 32*cb + l%32.
// The per-element scale w_scale[row] * d_a[col] of a 32x32 block is their outer product, made
// on the matrix pipe, so the vector ALU does two operations per result: int->float (Q4_K: an
// exact subtraction, see BIAS below) and a multiply-add.
// ---------------------------------------------------------------------------------------------
// Q4_K dots satisfy |D| <= 32 * 15 * 127 < 2^22, so an integer MFMA whose accumulator starts at
// the bits of 1.5 * 2^23 (cinit) returns the float 1.5 * 2^23 + D exactly and one exact
// subtraction recovers D (cheaper on the vector ALU than the int -> float conversion: ~9 % of the
// Q4_K tile time).  The tile loop builds the seed once and makes it opaque, so that it stays in
// registers instead of being rebuilt every step.  Q8_0, Q4_0 and IQ4_XS (|D| <= 32 * 127 * 127)
// take it in their 8-wave (J = 128) tiles, 2-3 % faster; their 64-column tiles run out of
// registers with the 16 seed registers.  Q6_K's scale-folded dots can exceed the range.
template <int T, int J> constexpr bool kSeeded = kK45<T> || (kB32<T> && J == 128);   // Q5_K: |D| <= 32*31*127 too
constexpr int32_t kBiasBits = 0x4B400000;
constexpr float kBias = 12582912.0f;   // 1.5 * 2^23

// DBG (the integer-dot export) runs the same loads, LDS layout, MFMAs and seeded accumulators; it
// differs only where an integer dot would be folded into the fp32 accumulators: there it stores
// the exact integer the production fold consumes (the seeded value minus the seed for Q4_K /
// Q5_K, the scale-folded 128*D_hi + D_lo for Q6_K, D for Q8_0 / Q4_0).
template <int T, int J, bool DBG>
__device__ __forceinline__ void tile_step(const uint8_t *wsm, const uint8_t *xsm, f32x16 (&acc)[Cfg<J>::NCB],
                                          const i32x16 &cinit,
                                          int64_t kb, int64_t nb32, int32_t *dbg, int64_t rows, int64_t n, int64_t r0,
                                          int64_t c0) {
    using L = Smem<T, J>;
    constexpr int NCB = Cfg<J>::NCB, JW = Cfg<J>::JW;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int rw = wid & 3, cw = wid >> 2;
    const int8_t *sA = (const int8_t *)(xsm + L::A_OFF);
    const float *sWs = (const float *)(wsm + L::WS_OFF);
    const float *sX = (const float *)(xsm + L::X_OFF);
    const int arow = 32 * rw + (lane & 31);
    const int h = lane >> 5, koff = 16 * h;
    const int colw = JW * cw + (lane & 31);   // + 32*cb
    const i32x16 zero = {};
    const f32x16 fzero = {};

    // Debug export of the integer dot v of element e of column block cb, sub-block sb.
    auto export_dot = [&](int cb, int sb, int e, int32_t v) {
        const int64_t col = c0 + colw + 32 * cb;
        const int64_t row = r0 + 32 * rw + 4 * h + 8 * (e >> 2) + (e & 3);
        if (row < rows && col < n) dbg[(col * rows + row) * nb32 + kb * 8 + sb] = v;
    };

    // Per-element scales of sub-block sb: the outer product of this wave's 32 row scales and its
    // columns' d_a.  Two 32-column blocks come from one two-block v_mfma_f32_32x32x1_f32 (block b
    // takes rows from lanes 32b.. and columns from lanes 32b..: here the same rows, the block's
    // columns); a single block from v_mfma_f32_32x32x2_f32 with the second K slot zero.
    auto scales = [&](int sb, float wsr, f32x16 (&S)[NCB]) {
        if constexpr (NCB == 2) {
            const float da = sX[sb * J + JW * cw + 32 * h + (lane & 31)];
            const f32x32 S2 = __builtin_amdgcn_mfma_f32_32x32x1f32(wsr, da, f32x32{}, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                S[0][e] = S2[e];
                S[1][e] = S2[16 + e];
            }
        } else {
            const float da = h ? 0.f : sX[sb * J + colw];
            S[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(h ? 0.f : wsr, da, fzero, 0, 0, 0);
        }
    };
    // D of block (sb, cb) folded into the accumulators with its scales (or exported)
    auto fix = [&](int cb, int sb, const i32x16 &D, const f32x16 &S) {
        if constexpr (kSeeded<T, J>) {
            const f32x16 Df = __builtin_bit_cast(f32x16, D);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float dv = Df[e] - kBias;   // exact: |D| < 2^22
                if constexpr (DBG) export_dot(cb, sb, e, (int32_t)dv);
                else acc[cb][e] = fmaf(dv, S[e], acc[cb][e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                if constexpr (DBG) export_dot(cb, sb, e, D[e]);
                else acc[cb][e] = fmaf((float)D[e], S[e], acc[cb][e]);
            }
        }
    };

    // Seeded tiles: per 32-value block, t = D * d_a by one multiply-add on the seeded value
    // ((1.5 * 2^23 + D) * d_a - 1.5 * 2^23 * d_a, the second product exact: d_a has 11 significant
    // bits), then acc += t * w[row] -- the lane's 16 row scales are read from LDS and its column's
    // d_a is one scalar, so no scale-product MFMA is needed.
    auto seeded_fold = [&](int sb, const u32x4 &aop) __attribute__((always_inline)) {
        f32x4 wr[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) wr[q] = *(const f32x4 *)(sWs + sb * kTI + 32 * rw + 8 * q + 4 * h);
        auto fold = [&](int cb, const i32x16 &D) __attribute__((always_inline)) {
            const float da = sX[sb * J + colw + 32 * cb];
            const float nb = -kBias * da;
            const f32x16 Df = __builtin_bit_cast(f32x16, D);
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[cb][e] = fmaf(fmaf(Df[e], da, nb), wr[e >> 2][e & 3], acc[cb][e]);
        };
        auto bop = [&](int cb) __attribute__((always_inline)) {
            return *(const u32x4 *)(sA + (colw + 32 * cb) * kLd + 32 * sb + koff);
        };
        if constexpr (T != kQ5_K && J == 128) {
            // every column block's MFMA is issued before the first fold, so the matrix pipe works
            // while the vector ALU folds (8-wave tiles; Q5_K's fifth bits and the 4-wave tiles'
            // other state leave no registers for it)
            i32x16 Ds[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) Ds[cb] = mfma32x32x32(aop, bop(cb), cinit);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) fold(cb, Ds[cb]);
        } else {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) fold(cb, mfma32x32x32(aop, bop(cb), cinit));
        }
    };

    if constexpr (kK45<T>) {
        const uint8_t *sW = wsm + L::W_OFF;
        // Q5_K: qh bytes 16h..16h+15 of the lane's row; bit sb of byte l is the fifth bit of value
        // l of sub-block sb
        u32x4 qh = {0u, 0u, 0u, 0u};
        if constexpr (T == kQ5_K) qh = *(const u32x4 *)(wsm + L::QH_OFF + arow * 32 + koff);
#pragma unroll 2
        for (int sb = 0; sb < 8; ++sb) {
            // qs bytes 32*(sb/2)+16h .. +15: low nibbles = values 16h.. of the even sub-block of
            // the pair, high nibbles = of the odd one
            const u32x4 q = *(const u32x4 *)(sW + arow * kLd4 + 32 * (sb >> 1) + koff);
            const int sh = 4 * (sb & 1);
            u32x4 aop = {(q.x >> sh) & 0x0F0F0F0Fu, (q.y >> sh) & 0x0F0F0F0Fu, (q.z >> sh) & 0x0F0F0F0Fu,
                         (q.w >> sh) & 0x0F0F0F0Fu};
            if constexpr (T == kQ5_K) {
                aop.x |= ((qh.x >> sb) & 0x01010101u) << 4;
                aop.y |= ((qh.y >> sb) & 0x01010101u) << 4;
                aop.z |= ((qh.z >> sb) & 0x01010101u) << 4;
                aop.w |= ((qh.w >> sb) & 0x01010101u) << 4;
            }
            if constexpr (!DBG) {
                seeded_fold(sb, aop);
            } else {
                f32x16 S[NCB];
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const u32x4 b = *(const u32x4 *)(sA + (colw + 32 * cb) * kLd + 32 * sb + koff);
                    fix(cb, sb, mfma32x32x32(aop, b, cinit), S[cb]);
                }
            }
        }
    } else if constexpr (kB32<T>) {
        const int8_t *sW = (const int8_t *)(wsm + L::W_OFF);
#pragma unroll 2
        for (int j = 0; j < 8; ++j) {
            if (kb * 8 + j >= nb32) break;   // ragged last step (workgroup-uniform)
            const u32x4 a = *(const u32x4 *)(sW + arow * kLd + 32 * j + koff);
            if constexpr (!DBG && kSeeded<T, J>) {
                seeded_fold(j, a);
            } else {
                f32x16 S[NCB];
                if constexpr (!DBG) scales(j, sWs[j * kTI + arow], S);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const u32x4 b = *(const u32x4 *)(sA + (colw + 32 * cb) * kLd + 32 * j + koff);
                    fix(cb, j, mfma32x32x32(a, b, cinit), S[cb]);
                }
            }
        }
    } else {
        // Q6_K: the weight scale d is one per row for the whole step and every accumulator
        // element of a lane is in the lane's column, so the per-element scale factors as
        // d[row] * d_a[col]: T += D * d_a with d_a a per-lane scalar, then acc += d[row] * T once
        // per step (no scale-product MFMAs).
        const int8_t *sW = (const int8_t *)(wsm + L::W_OFF);
        f32x16 Tc[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) Tc[cb] = fzero;
#pragma unroll 2
        for (int j = 0; j < 8; ++j) {
            const u32x4 a = *(const u32x4 *)(sW + arow * kLd + 32 * j + koff);
            const u32x4 a_hi = *(const u32x4 *)(sW + kTI * kLd + arow * kLd + 32 * j + koff);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const u32x4 b = *(const u32x4 *)(sA + (colw + 32 * cb) * kLd + 32 * j + koff);
                const float da = sX[j * J + colw + 32 * cb];
                const i32x16 D = mfma32x32x32(a, b, zero);
                const i32x16 Dh = mfma32x32x32(a_hi, b, zero);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int32_t v = (Dh[e] << 7) + D[e];   // sc0*D0 + sc1*D1
                    if constexpr (DBG) export_dot(cb, j, e, v);
                    else Tc[cb][e] = fmaf((float)v, da, Tc[cb][e]);
                }
            }
        }
        if constexpr (!DBG) {
            // row scales of the lane's elements: rows 32*rw + 8*q + 4*h + (0..3), q = e/4
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 dr = *(const f32x4 *)(sWs + 32 * rw + 8 * q + 4 * h);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[cb][4 * q + i] = fmaf(dr[i], Tc[cb][4 * q + i], acc[cb][4 * q + i]);
            }
        }
    }
}

// Q4_K min term of one step: acc += sum over the 8 sub-blocks of (-dmin*m)[row] * s_a[col], a
// rank-8 product, on the matrix pipe in bf16 (fp32's exponent range, so no coefficient can
// overflow): -dmin*m = p0 + p1 + p2 and s_a = t1 + t2 exactly, every product p*t is exact in fp32,
// and three K = 16 MFMAs per column block sum them -- MFMA m, lane (row, h), slots 2q and 2q+1
// hold p_m of sub-block 4h+q against t1 and t2 of the same sub-block.
template <int T, int J>
__device__ __forceinline__ void q4k_min_term(const uint8_t *wsm, const uint8_t *xsm, f32x16 (&acc)[Cfg<J>::NCB]) {
    using L = Smem<T, J>;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int rw = wid & 3, cw = wid >> 2, h = lane >> 5;
    const int arow = 32 * rw + (lane & 31), colw = Cfg<J>::JW * cw + (lane & 31);
    const uint8_t *wp = wsm + L::WM_OFF + arow * 48 + 24 * h;
    u32x4 bs[Cfg<J>::NCB];
#pragma unroll
    for (int cb = 0; cb < Cfg<J>::NCB; ++cb) bs[cb] = *(const u32x4 *)(xsm + L::XB_OFF + (colw + 32 * cb) * 32 + 16 * h);
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const u32x2 p = *(const u32x2 *)(wp + 8 * m);
        const u32x4 a = {__builtin_amdgcn_perm(p.x, p.x, 0x01000100u), __builtin_amdgcn_perm(p.x, p.x, 0x03020302u),
                         __builtin_amdgcn_perm(p.y, p.y, 0x01000100u), __builtin_amdgcn_perm(p.y, p.y, 0x03020302u)};
#pragma unroll
        for (int cb = 0; cb < Cfg<J>::NCB; ++cb)
            acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                             __builtin_bit_cast(bf16x8, bs[cb]), acc[cb], 0, 0, 0);
    }
}

// One tile's steps [kb0, kb1), software-pipelined: the loads of a later step are in flight while
// a step computes.  Two weight buffers (kDoubleBuffer): weights and activations are fetched into
// registers two steps ahead and step kb+1 is parked while step kb computes, so a step needs one
// barrier (it publishes the parked step and retires the buffers computed before).  One weight
// buffer: step kb's weights (fetched a step ahead) are parked between two barriers; the
// activations of Q6_K, Q3_K and the 32-value types, double-buffered, come by direct loads issued
// before step kb computes and awaited (each wave its own, then the first barrier) before step
// kb+1, those of Q4_K / Q5_K through registers like the weights (measured faster for them).  A
// barrier waits for every load the wave has in flight, so no load is issued just before one.
template <int T, int J, bool DBG, class WR, class CR>
__device__ __forceinline__ void run_tile(uint8_t *sm, f32x16 (&acc)[Cfg<J>::NCB], const WR &wr, int64_t kb0,
                                         int64_t kb1, int64_t nb32, const uint8_t *xq, const CR &colrow,
                                         int32_t *dbg, int64_t n, int64_t c0, int64_t act_rows) {
    using L = Smem<T, J>;
    constexpr bool DB = kDoubleBuffer<T, J>;
    i32x16 cinit = {};
    if constexpr (kSeeded<T, J>) {
#pragma unroll
        for (int e = 0; e < 16; ++e) cinit[e] = kBiasBits;
        asm volatile("" : "+v"(cinit));
    }
    const int64_t nsteps = (nb32 + 7) / 8;
    uint8_t *const wb0 = sm, *const wb1 = sm + (DB ? L::W_PART : 0);
    uint8_t *const xb0 = sm + (DB ? 2 : 1) * L::W_PART, *const xb1 = xb0 + L::A_PART;
    WFetch<T, Cfg<J>::NT> wf;
    if constexpr (DB) {
        ActRegs<T, J> ar;
        ar.init(colrow);
        wf.fetch(wr, kb0, nb32);
        ar.fetch(xq, kb0, act_rows, nsteps);
        __syncthreads();   // the previous tile's reads of every buffer are done
        wf.template store<J>(wb0, wr, kb0, nb32);
        ar.store(xb0);
        if (kb0 + 1 < kb1) {
            wf.fetch(wr, kb0 + 1, nb32);
            ar.fetch(xq, kb0 + 1, act_rows, nsteps);
        }
        for (int64_t kb = kb0; kb < kb1; ++kb) {
            const bool odd = (kb - kb0) & 1;
            __syncthreads();   // publishes step kb; step kb-1 is retired
            if (kb + 1 < kb1) {
                wf.template store<J>(odd ? wb0 : wb1, wr, kb + 1, nb32);
                ar.store(odd ? xb0 : xb1);
                if (kb + 2 < kb1) {
                    wf.fetch(wr, kb + 2, nb32);
                    ar.fetch(xq, kb + 2, act_rows, nsteps);
                }
            }
            const uint8_t *wcur = odd ? wb1 : wb0, *xcur = odd ? xb1 : xb0;
            if constexpr (kK45<T> && !DBG) q4k_min_term<T, J>(wcur, xcur, acc);   // acc only
            tile_step<T, J, DBG>(wcur, xcur, acc, cinit, kb, nb32, dbg, wr.rows, n, wr.r0, c0);
        }
    } else if constexpr (kK45<T>) {
        // one weight buffer, activations through registers: step kb parked between two barriers
        ActRegs<T, J> ar;
        ar.init(colrow);
        wf.fetch(wr, kb0, nb32);
        ar.fetch(xq, kb0, act_rows, nsteps);
        for (int64_t kb = kb0; kb < kb1; ++kb) {
            __syncthreads();   // the previous step's (or tile's) LDS reads are done
            wf.template store<J>(wb0, wr, kb, nb32);
            ar.store(xb0);
            __syncthreads();
            if (kb + 1 < kb1) {
                wf.fetch(wr, kb + 1, nb32);
                ar.fetch(xq, kb + 1, act_rows, nsteps);
            }
            if constexpr (!DBG) q4k_min_term<T, J>(wb0, xb0, acc);   // acc only
            tile_step<T, J, DBG>(wb0, xb0, acc, cinit, kb, nb32, dbg, wr.rows, n, wr.r0, c0);
        }
    } else {
        ActDirect<T, J> ad;
        ad.init(colrow);
        __syncthreads();   // the previous tile's reads of every buffer are done
        ad.issue(xb0, xq, kb0, act_rows, nsteps);
        wf.fetch(wr, kb0, nb32);
        for (int64_t kb = kb0; kb < kb1; ++kb) {
            const bool odd = (kb - kb0) & 1;
            uint8_t *const xcur = odd ? xb1 : xb0, *const xnxt = odd ? xb0 : xb1;
            wait_loads();      // this wave's direct loads of step kb (and the weights fetched since) landed
            __syncthreads();   // ... every wave's: step kb's activations are in LDS; step kb-1 is retired
            wf.template store<J>(wb0, wr, kb, nb32);
            __syncthreads();   // step kb's weights are parked (a barrier waits for every load in flight,
                               // so the next step's loads are issued after it)
            if (kb + 1 < kb1) {
                ad.issue(xnxt, xq, kb + 1, act_rows, nsteps);
                wf.fetch(wr, kb + 1, nb32);
            }
            if constexpr (kK45<T> && !DBG) q4k_min_term<T, J>(wb0, xcur, acc);   // acc only
            tile_step<T, J, DBG>(wb0, xcur, acc, cinit, kb, nb32, dbg, wr.rows, n, wr.r0, c0);
        }
    }
}

// Writes a tile's accumulators to dst (column-major with leading dimension ld), rows < rlim and
// columns < clim.
template <int J>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[Cfg<J>::NCB], float *dst, int64_t ld, int64_t rlim,
                                           int64_t clim) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int rw = wid & 3, cw = wid >> 2;
#pragma unroll
    for (int cb = 0; cb < Cfg<J>::NCB; ++cb) {
        const int col = Cfg<J>::JW * cw + 32 * cb + (lane & 31);
        if (col >= clim) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int r = 32 * rw + 4 * (lane >> 5) + 8 * (e >> 2) + (e & 3);
            if (r < rlim) dst[(int64_t)col * ld + r] = acc[cb][e];
        }
    }
}

// SwiGLU of a gate value g and an up value u: silu(g) * u, silu(g) = g / (1 + e^-g).
__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// GLU tile (WRows<true>): 64 outputs; element e (e % 8 < 4) of a lane is the gate value and e + 4
// the up value of output row 16*rw + 8*(e/8) + 4*(lane/32) + e%4.  dst[col * ld + row], rows <
// rlim, columns < clim.
template <int J>
__device__ __forceinline__ void store_tile_glu(const f32x16 (&acc)[Cfg<J>::NCB], float *dst, int64_t ld,
                                               int64_t rlim, int64_t clim) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int rw = wid & 3, cw = wid >> 2;
#pragma unroll
    for (int cb = 0; cb < Cfg<J>::NCB; ++cb) {
        const int col = Cfg<J>::JW * cw + 32 * cb + (lane & 31);
        if (col >= clim) continue;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int e = (q & 3) + 8 * (q >> 2);
            const int r = 16 * rw + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
            if (r < rlim) dst[(int64_t)col * ld + r] = swiglu(acc[cb][e], acc[cb][e + 4]);
        }
    }
}

// Stream-K unit owning item i of the W stream-K items: the largest u with floor(u*W/units) <= i.
__device__ __forceinline__ int64_t unit_of(int64_t i, int64_t W, int64_t units) {
    const int64_t u = ((i + 1) * units - 1) / W;
    return u < units - 1 ? u : units - 1;
}

// Epilogue of a unit's piece of a split tile (stream-K tile ts, the unit's partial slot `slot`).
// Every covering unit stores its accumulators to its slot (in register order: element e of column
// block cb of thread tid at (cb*16 + e)*NT + tid, so the stores and loads are coalesced) and counts
// itself in; the unit that arrives last adds the covering units' partials in ascending unit order
// -- its own from registers -- and writes the tile to y.  The slots are written through to memory
// and read past the caches (system-scope accesses), and each thread waits for its stores to
// complete before the unit counts in, so no cache-wide fence is needed (a device-scope fence
// writes back and invalidates a whole L2, which measured twice as slow).  The order of the sum
// does not depend on which unit arrives last (deterministic, bitwise reruns), and no unit waits
// for another.
template <int J>
__device__ __forceinline__ void finish_split(const f32x16 (&acc)[Cfg<J>::NCB], const MmqArgs &args, int64_t u,
                                             int64_t ts, int64_t slot, float *y, int64_t rows, int64_t n,
                                             int64_t r0, int64_t c0) {
    constexpr int NT = Cfg<J>::NT, NCB = Cfg<J>::NCB;
    const int tid = threadIdx.x;
    const int64_t S = (int64_t)kTI * J;
    float *mine = args.partials + slot * S;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            __hip_atomic_store(mine + (cb * 16 + e) * NT + tid, acc[cb][e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's slot stores have completed
    // covering units: u0..u1, those with an empty range (fewer items than units) excepted
    const int64_t W = (args.ntiles - args.dp_tiles) * args.k_iters, U = args.units, K = args.k_iters;
    const int64_t u0 = unit_of(ts * K, W, U), u1 = unit_of((ts + 1) * K - 1, W, U);
    __shared__ int32_t last;
    __syncthreads();
    if (tid == 0) {
        int32_t cover = 0;
        for (int64_t v = u0; v <= u1; ++v) cover += ((v + 1) * W) / U != (v * W) / U;
        last = atomicAdd(args.counters + ts, 1) == cover - 1;
    }
    __syncthreads();
    if (!last) return;   // workgroup-uniform: the other units' slots were complete before they counted in
    f32x16 tot[NCB];
    bool started = false;
    for (int64_t v = u0; v <= u1; ++v) {
        const int64_t start = (v * W) / U;
        if (((v + 1) * W) / U == start) continue;   // empty range: not a covering unit
        const float *src = args.partials + (2 * v + (start / K == ts ? 0 : 1)) * S;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = v == u ? acc[cb][e]
                                       : __hip_atomic_load(src + (cb * 16 + e) * NT + tid, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_SYSTEM);
                tot[cb][e] = started ? tot[cb][e] + p : p;
            }
        started = true;
    }
    store_tile<J>(tot, y + c0 * rows + r0, rows, rows - r0, n - c0);
}

// ---------------------------------------------------------------------------------------------
// Dense kernel: persistent over the unit's (tile, step) range.
// ---------------------------------------------------------------------------------------------
// PK: w in the panel layout (repack.hip).
template <int T, int J, bool DBG, bool PK = false>
__global__ __launch_bounds__(Cfg<J>::NT, 2) void mmq_kernel(const uint8_t *__restrict__ w, int64_t rows, int64_t k,
                                                         const uint8_t *__restrict__ xq, int64_t n,
                                                         float *__restrict__ y, int32_t *__restrict__ dbg,
                                                         MmqArgs args) {
    extern __shared__ __align__(16) uint8_t sm[];
    const int64_t nb32 = k / 32;
    const int64_t row_bytes = (k / Fmt<T>::QK) * Fmt<T>::BYTES;
    const int64_t u = xcd_remap(blockIdx.x, args.units);
    // Data-parallel rounds first (tiles u, u + units, ... below dp_tiles, each whole), then the
    // unit's stream-K range over the remaining tiles' (tile, step) items.
    const int64_t W = (args.ntiles - args.dp_tiles) * args.k_iters;
    int64_t tdp = u;
    int64_t pos = (u * W) / args.units;
    const int64_t end = ((u + 1) * W) / args.units;
    const int64_t first = pos;

    for (;;) {
        int64_t t, kb0, kb1, ts = 0, slot = -1;   // slot < 0: the tile is whole here (or stream-K is off)
        if (tdp < args.dp_tiles) {
            t = tdp;
            kb0 = 0;
            kb1 = args.k_iters;
            tdp += args.units;
        } else if (pos < end) {
            ts = pos / args.k_iters;
            t = args.dp_tiles + ts;
            kb0 = pos - ts * args.k_iters;
            kb1 = (kb0 + (end - pos) < args.k_iters) ? kb0 + (end - pos) : args.k_iters;
            if (args.write_partials && !(kb0 == 0 && kb1 == args.k_iters)) slot = 2 * u + (pos == first ? 0 : 1);
            pos += kb1 - kb0;
        } else {
            break;
        }
        int64_t rt, ct;
        tile_coords(t, args.ntiles, args.n_ct, rt, ct);
        const int64_t r0 = rt * kTI, c0 = ct * J;

        // columns past the end repeat the last (never written out)
        auto colrow = [&](int c) -> int64_t { return c0 + c < n ? c0 + c : n - 1; };
        f32x16 acc[Cfg<J>::NCB];
#pragma unroll
        for (int cb = 0; cb < Cfg<J>::NCB; ++cb) acc[cb] = f32x16{};

        if constexpr (PK) {
            const WPanels wr{w, args.k_iters * 16 * (kSuper / Fmt<T>::QK * Fmt<T>::BYTES), r0, rows};
            run_tile<T, J, DBG>(sm, acc, wr, kb0, kb1, nb32, xq, colrow, dbg, n, c0, n);
        } else {
            const WRows<false> wr{w, w, row_bytes, r0, rows};
            run_tile<T, J, DBG>(sm, acc, wr, kb0, kb1, nb32, xq, colrow, dbg, n, c0, n);
        }

        if (!DBG) {
            if (slot < 0) store_tile<J>(acc, y + c0 * rows + r0, rows, rows - r0, n - c0);
            else finish_split<J>(acc, args, u, ts, slot, y, rows, n, r0, c0);
        }
    }
}

// Dense gate/up kernel (GLU tiles of 64 outputs): one tile per workgroup over the whole K range
// (the two products of an output must meet in one workgroup, so no stream-K split).
template <int T, int J>
__global__ __launch_bounds__(Cfg<J>::NT, 2) void mmq_glu_kernel(const uint8_t *__restrict__ wg,
                                                             const uint8_t *__restrict__ wu, int64_t rows, int64_t k,
                                                             const uint8_t *__restrict__ xq, int64_t n,
                                                             float *__restrict__ y, int64_t ntiles, int64_t n_ct) {
    extern __shared__ __align__(16) uint8_t sm[];
    const int64_t nb32 = k / 32;
    const int64_t row_bytes = (k / Fmt<T>::QK) * Fmt<T>::BYTES;
    const int64_t t = xcd_remap(blockIdx.x, ntiles);
    int64_t rt, ct;
    tile_coords(t, ntiles, n_ct, rt, ct);
    const int64_t r0 = rt * (kTI / 2), c0 = ct * J;
    auto colrow = [&](int c) -> int64_t { return c0 + c < n ? c0 + c : n - 1; };
    f32x16 acc[Cfg<J>::NCB];
#pragma unroll
    for (int cb = 0; cb < Cfg<J>::NCB; ++cb) acc[cb] = f32x16{};
    const WRows<true> wr{wg, wu, row_bytes, r0, rows};
    run_tile<T, J, false>(sm, acc, wr, 0, (k + kSuper - 1) / kSuper, nb32, xq, colrow, nullptr, n, c0, n);
    store_tile_glu<J>(acc, y + c0 * rows + r0, rows, rows - r0, n - c0);
}

// Sum of the partial slots of every split tile, in ascending unit order.

// ---------------------------------------------------------------------------------------------
// Expert kernel: one tile per workgroup, full K; grid (row tiles, column-tile slots).
// ---------------------------------------------------------------------------------------------
template <int T, int J, bool GLU>
__global__ __launch_bounds__(Cfg<J>::NT, 2) void mmq_id_kernel(const uint8_t *__restrict__ w,
                                                            const uint8_t *__restrict__ w2, int64_t rows, int64_t k,
                                                            const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                            ColMap cm, int32_t n_exp) {
    extern __shared__ __align__(16) uint8_t sm[];
    // The grid is sized for the most column tiles the call can have; the valid ones are
    // tile_start[n_exp] (device).  Valid (row tile, column tile) pairs are numbered in the dense
    // kernel's banded order and dealt out in contiguous ranges per XCD (hardware workgroup b runs
    // on XCD b % 8), so an XCD walks an expert's column tiles back to back with that expert's
    // weight rows in its L2; workgroups past the valid count exit.
    const int64_t V = cm.tile_start[n_exp];
    const int64_t total = (int64_t)gridDim.x * V;
    const int64_t b = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    const int64_t xcd = b % 8, slot = b / 8, q8 = total / 8, r8 = total % 8;
    if (slot >= q8 + (xcd < r8 ? 1 : 0)) return;
    int64_t rt, ct;
    tile_coords(xcd * q8 + (xcd < r8 ? xcd : r8) + slot, total, V, rt, ct);
    // expert owning column tile ct: largest e with tile_start[e] <= ct
    int lo = 0, hi = n_exp - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (cm.tile_start[mid] <= ct) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int64_t jt = ct - cm.tile_start[e];
    const int64_t seg = cm.bounds[e];
    const int64_t cnt = cm.bounds[e + 1] - seg;
    const int64_t nb32 = k / 32;
    const int64_t row_bytes = (k / Fmt<T>::QK) * Fmt<T>::BYTES;
    const int64_t r0 = rt * (GLU ? kTI / 2 : kTI);
    const int64_t c0 = jt * J;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

    auto arow_of = [&](int64_t c) -> int64_t {
        const int64_t pr = cm.sorted[seg + c];
        const int64_t t = pr / cm.top_k, s = pr - t * cm.top_k;
        return t * cm.x_per_tok + (cm.x_per_tok > 1 ? s : 0);
    };
    // past the end: the last column (never written out)
    auto colrow = [&](int c) -> int64_t { return arow_of(c0 + c < cnt ? c0 + c : cnt - 1); };
    f32x16 acc[Cfg<J>::NCB];
#pragma unroll
    for (int cb = 0; cb < Cfg<J>::NCB; ++cb) acc[cb] = f32x16{};

    const int64_t k_iters = (k + kSuper - 1) / kSuper;
    const WRows<GLU> wr{w + (int64_t)e * cm.w_expert_stride, GLU ? w2 + (int64_t)e * cm.w_expert_stride : nullptr,
                        row_bytes, r0, rows};
    run_tile<T, J, false>(sm, acc, wr, 0, k_iters, nb32, xq, colrow, nullptr, cnt, c0, cm.act_rows);
    const int rw = wid & 3, cw = wid >> 2;
#pragma unroll
    for (int cb = 0; cb < Cfg<J>::NCB; ++cb) {
        const int64_t c = c0 + Cfg<J>::JW * cw + 32 * cb + (lane & 31);
        if (c >= cnt) continue;
        const int64_t orow = cm.sorted[seg + c];
        if constexpr (GLU) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int e2 = (q & 3) + 8 * (q >> 2);
                const int64_t r = r0 + 16 * rw + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                if (r < rows) y[orow * rows + r] = swiglu(acc[cb][e2], acc[cb][e2 + 4]);
            }
        } else {
#pragma unroll
            for (int e2 = 0; e2 < 16; ++e2) {
                const int64_t r = r0 + 32 * rw + 4 * (lane >> 5) + 8 * (e2 >> 2) + (e2 & 3);
                if (r < rows) y[orow * rows + r] = acc[cb][e2];
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------------
template <int T, int J, bool DBG, bool PK = false>
static hipError_t launch_mmq_t(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y,
                               int32_t *dbg, const MmqLaunch &p, hipStream_t s) {
    // whole rounds of tiles run data-parallel; stream-K splits only the remainder (without stream-K
    // units == ntiles: one round)
    const int64_t dp = p.units > 0 ? (p.ntiles / p.units) * p.units : 0;
    MmqArgs a{p.ntiles, p.n_ct, p.k_iters, p.units, p.partials, p.counters, p.stream_k ? 1 : 0, dp};
    constexpr int smem = kSmemBytes<T, J>;
    auto kern = mmq_kernel<T, J, DBG, PK>;
    // once per process (a function-local static is initialised exactly once, thread-safely)
    static const hipError_t attr_err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (attr_err != hipSuccess) return attr_err;
    hipLaunchKernelGGL(kern, dim3((unsigned)p.units), dim3(Cfg<J>::NT), smem, s, w, rows, k, xq, n, y, dbg, a);
    return hipGetLastError();
}

template <int T, bool DBG, bool PK = false>
static hipError_t launch_mmq_j(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y,
                               int32_t *dbg, const MmqLaunch &p, hipStream_t s) {
    if (p.tile_j == 32) return launch_mmq_t<T, 32, DBG, PK>(w, rows, k, xq, n, y, dbg, p, s);
    if (p.tile_j == 64) return launch_mmq_t<T, 64, DBG, PK>(w, rows, k, xq, n, y, dbg, p, s);
    if (p.tile_j == 128) return launch_mmq_t<T, 128, DBG, PK>(w, rows, k, xq, n, y, dbg, p, s);
    return hipErrorInvalidValue;
}

template <int T>
static hipError_t launch_mmq_panels(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y,
                                    const MmqLaunch &p, hipStream_t s) {
    if constexpr (kPanel<T>) return launch_mmq_j<T, false, true>(w, rows, k, xq, n, y, nullptr, p, s);
    else return hipErrorInvalidValue;
}

hipError_t launch_mmq(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y,
                      int32_t *dbg, const MmqLaunch &p, hipStream_t s) {
    const bool d = dbg != nullptr;
    if (p.packed && d) return hipErrorInvalidValue;   // no integer-dot export from panel weights
#define QMM_MQ(TT)                                                                                    \
    if (type == TT) {                                                                                 \
        if (p.packed) return launch_mmq_panels<TT>(w, rows, k, xq, n, y, p, s);                       \
        return d ? launch_mmq_j<TT, true>(w, rows, k, xq, n, y, dbg, p, s)                           \
                 : launch_mmq_j<TT, false>(w, rows, k, xq, n, y, dbg, p, s);                          \
    }
    QMM_MQ(kQ4_K)
    QMM_MQ(kQ5_K)
    QMM_MQ(kQ6_K)
    QMM_MQ(kQ8_0)
    QMM_MQ(kQ4_0)
    QMM_MQ(kQ3_K)
    QMM_MQ(kIQ4_XS)
#undef QMM_MQ
    return hipErrorInvalidValue;
}

template <int T, int J>
static hipError_t launch_mmq_glu_t(const uint8_t *wg, const uint8_t *wu, int64_t rows, int64_t k, const uint8_t *xq,
                                   int64_t n, float *y, hipStream_t s) {
    constexpr int smem = kSmemBytes<T, J>;
    auto kern = mmq_glu_kernel<T, J>;
    // once per process (a function-local static is initialised exactly once, thread-safely)
    static const hipError_t attr_err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (attr_err != hipSuccess) return attr_err;
    const int64_t n_ct = (n + J - 1) / J;
    const int64_t ntiles = ((rows + kTI / 2 - 1) / (kTI / 2)) * n_ct;
    hipLaunchKernelGGL(kern, dim3((unsigned)ntiles), dim3(Cfg<J>::NT), smem, s, wg, wu, rows, k, xq, n, y, ntiles, n_ct);
    return hipGetLastError();
}

hipError_t launch_mmq_glu(int type, const uint8_t *wg, const uint8_t *wu, int64_t rows, int64_t k, const uint8_t *xq,
                          int64_t n, float *y, int tile_j, hipStream_t s) {
#define QMM_MG(TT)                                                                                    \
    if (type == TT) {                                                                                 \
        if (tile_j == 32) return launch_mmq_glu_t<TT, 32>(wg, wu, rows, k, xq, n, y, s);             \
        if (tile_j == 64) return launch_mmq_glu_t<TT, 64>(wg, wu, rows, k, xq, n, y, s);             \
        if (tile_j == 128) return launch_mmq_glu_t<TT, 128>(wg, wu, rows, k, xq, n, y, s);           \
    }
    QMM_MG(kQ4_K)
    QMM_MG(kQ5_K)
    QMM_MG(kQ6_K)
    QMM_MG(kQ8_0)
    QMM_MG(kQ4_0)
    QMM_MG(kQ3_K)
    QMM_MG(kIQ4_XS)
#undef QMM_MG
    return hipErrorInvalidValue;
}

template <int T, int J, bool GLU>
static hipError_t launch_mmq_id_t(const uint8_t *w, const uint8_t *w2, int64_t rows, int64_t k, const uint8_t *xq,
                                  float *y, const ColMap &cm, int32_t n_exp, int64_t max_ct, hipStream_t s) {
    constexpr int smem = kSmemBytes<T, J>;
    auto kern = mmq_id_kernel<T, J, GLU>;
    // once per process (a function-local static is initialised exactly once, thread-safely)
    static const hipError_t attr_err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (attr_err != hipSuccess) return attr_err;
    if (max_ct <= 0) return hipSuccess;
    constexpr int64_t TR = GLU ? kTI / 2 : kTI;   // outputs per row tile
    dim3 grid((unsigned)((rows + TR - 1) / TR), (unsigned)max_ct);
    hipLaunchKernelGGL(kern, grid, dim3(Cfg<J>::NT), smem, s, w, w2, rows, k, xq, y, cm, n_exp);
    return hipGetLastError();
}

template <int T, bool GLU>
static hipError_t launch_mmq_id_j(const uint8_t *w, const uint8_t *w2, int64_t rows, int64_t k, const uint8_t *xq,
                                  float *y, const ColMap &cm, int tile_j, int64_t max_ct, hipStream_t s) {
    if (tile_j == 32) return launch_mmq_id_t<T, 32, GLU>(w, w2, rows, k, xq, y, cm, cm.n_exp, max_ct, s);
    if (tile_j == 64) return launch_mmq_id_t<T, 64, GLU>(w, w2, rows, k, xq, y, cm, cm.n_exp, max_ct, s);
    if (tile_j == 128) return launch_mmq_id_t<T, 128, GLU>(w, w2, rows, k, xq, y, cm, cm.n_exp, max_ct, s);
    return hipErrorInvalidValue;
}

hipError_t launch_mmq_id(int type, const uint8_t *w, const uint8_t *w_up, int64_t rows, int64_t k,
                         const uint8_t *xq, float *y, const ColMap &cm, int tile_j, int64_t max_col_tiles,
                         hipStream_t s) {
#define QMM_MQI(TT)                                                                                   \
    if (type == TT) {                                                                                 \
        return w_up ? launch_mmq_id_j<TT, true>(w, w_up, rows, k, xq, y, cm, tile_j, max_col_tiles, s)    \
                    : launch_mmq_id_j<TT, false>(w, nullptr, rows, k, xq, y, cm, tile_j, max_col_tiles, s); \
    }
    QMM_MQI(kQ4_K)
    QMM_MQI(kQ5_K)
    QMM_MQI(kQ6_K)
    QMM_MQI(kQ8_0)
    QMM_MQI(kQ4_0)
    QMM_MQI(kQ3_K)
    QMM_MQI(kIQ4_XS)
#undef QMM_MQI
    return hipErrorInvalidValue;
}

}  // namespace qmm
