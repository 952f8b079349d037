// Tiled product for many activation columns (the MMQ regime of the MMQ page: "tiling skeleton",
// "J runtime selection", "tile efficiency", "stream-K", "fixup", "expert bounds").
//
// CDNA4 design.  A 256-thread workgroup owns a 128-row x J-column output tile (J = 32/64/128)
// and walks K in 256-value steps.  Each step stages the weight tile into LDS already unpacked to
// int8 codes (the MMQ page's "why not dequantize": stay quantized, unpack once per tile and
// reuse it for J columns) together with fp32 per-row scales, and the activation tile (int8 codes
// plus fp32 (d, s) per 32-value block).  Each wave owns 32 rows; per 32-value block it runs one
// v_mfma_i32_32x32x32_i8 per 32 columns -- K = 32 is exactly one q8_1 block, so every int32
// result is one exact sub-block dot D -- and applies the fp32 fixup to its 16 accumulators:
//   Q4_K  acc += D * (d*sc) * d_a - (dmin*m) * s_a
//   Q8_0  acc += D * d_w * d_a
//   Q6_K  acc += (sc0*D0 + sc1*D1) * d * d_a
// Q6_K changes scale every 16 values, so its int8 scale is folded into the codes at unpack time:
// v = sc*(q-32) lies in [-4064, 4096] and is split as v = 128*hi + lo with lo in [0,127] and hi
// in [-32, 32]; two MFMAs give D_hi and D_lo and sc0*D0 + sc1*D1 = 128*D_hi + D_lo exactly.
//
// Work split: `units` workgroups share ntiles*k_iters (tile, step) items; unit u owns
// [u*W/units, (u+1)*W/units).  A unit that covers a whole tile writes it to y; a partial tile
// goes to the unit's slot (0: its first tile, 1: its last) and the fixup kernel adds the slots
// of a split tile in ascending unit order (deterministic, no atomics).  Without stream-K,
// units == ntiles and every unit is exactly one tile.
#include "common.hpp"
#include "launch.hpp"

namespace qmm {

constexpr int kTI = 128;        // rows per tile
constexpr int kLd = 272;        // LDS bytes per 256-value row (+16 to spread banks)

struct MmqArgs {
    int64_t ntiles, n_ct, k_iters, units;
    float *partials;
    int32_t write_partials;     // stream-K active
};

template <int T, int J> struct Smem {
    static constexpr int NW = (T == kQ6_K) ? 2 : 1;               // weight planes
    static constexpr int W_OFF = 0;
    static constexpr int A_OFF = W_OFF + NW * kTI * kLd;
    static constexpr int WS_OFF = A_OFF + J * kLd;                 // float [8][128]
    static constexpr int WM_OFF = WS_OFF + 8 * kTI * 4;            // float [8][128]
    static constexpr int X_OFF = WM_OFF + 8 * kTI * 4;             // float2 [8][J]
    static constexpr int BYTES = X_OFF + 8 * J * 8;
};

// ---------------------------------------------------------------------------------------------
// Weight tile staging: rows [r0, r0+128) of the step's 256 values -> int8 codes + fp32 scales.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void stage_weights_q4_k(uint8_t *sm, const uint8_t *wbase, int64_t row_bytes,
                                                   int64_t r0, int64_t rows, int64_t kb) {
    const int tid = threadIdx.x;
    int8_t *sW = (int8_t *)sm;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int i = tid + 256 * it;              // (row, 16-byte piece of qs): 128 x 8
        const int r = i >> 3, piece = i & 7;
        const int64_t row = r0 + r;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row < rows) v = ld16(wbase + row * row_bytes + kb * 144 + 16 + 16 * piece);
        // 32 qs bytes serve 64 values: low nibbles the first sub-block of the pair, high the second
        const int c = piece >> 1, l0 = 16 * (piece & 1);
        u32x4 lo, hi;
        lo.x = v.x & 0x0F0F0F0Fu; hi.x = (v.x >> 4) & 0x0F0F0F0Fu;
        lo.y = v.y & 0x0F0F0F0Fu; hi.y = (v.y >> 4) & 0x0F0F0F0Fu;
        lo.z = v.z & 0x0F0F0F0Fu; hi.z = (v.z >> 4) & 0x0F0F0F0Fu;
        lo.w = v.w & 0x0F0F0F0Fu; hi.w = (v.w >> 4) & 0x0F0F0F0Fu;
        *(u32x4 *)(sW + r * kLd + 64 * c + l0) = lo;
        *(u32x4 *)(sW + r * kLd + 64 * c + 32 + l0) = hi;
    }
}

template <int T, int J>
__device__ __forceinline__ void stage_weight_scales(uint8_t *sm, const uint8_t *wbase, int64_t row_bytes,
                                                    int64_t r0, int64_t rows, int64_t kb, int64_t nb32) {
    const int tid = threadIdx.x;
    float *sWs = (float *)(sm + Smem<T, J>::WS_OFF);
    float *sWm = (float *)(sm + Smem<T, J>::WM_OFF);
    if constexpr (T == kQ4_K) {
        if (tid < kTI) {
            const int64_t row = r0 + tid;
            u32x4 h = {0u, 0u, 0u, 0u};
            if (row < rows) h = ld16(wbase + row * row_bytes + kb * 144);
            const float d = h2f((uint16_t)(h.x & 0xFFFF)), dmin = h2f((uint16_t)(h.x >> 16));
            const uint32_t sc_lo = h.y & 0x3F3F3F3Fu, m_lo = h.z & 0x3F3F3F3Fu;
            const uint32_t sc_hi = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
            const uint32_t m_hi = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t scw = j < 4 ? sc_lo : sc_hi, mw = j < 4 ? m_lo : m_hi;
                const int sh = 8 * (j & 3);
                sWs[j * kTI + tid] = d * (float)((scw >> sh) & 0xFF);
                sWm[j * kTI + tid] = dmin * (float)((mw >> sh) & 0xFF);
            }
        }
    } else if constexpr (T == kQ8_0) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int i = tid + 256 * it;          // (row, block) pairs: 128 x 8
            const int r = i >> 3, j = i & 7;
            const int64_t row = r0 + r, b = kb * 8 + j;
            float d = 0.f;
            if (row < rows && b < nb32) d = h2f(ld2(wbase + row * row_bytes + b * 34));
            sWs[j * kTI + r] = d;
        }
    } else {   // Q6_K: the per-row super-block scale d
        if (tid < kTI) {
            const int64_t row = r0 + tid;
            float d = 0.f;
            if (row < rows) d = h2f(ld2(wbase + row * row_bytes + kb * 210 + 208));
            sWs[tid] = d;
        }
    }
}

template <int J>
__device__ __forceinline__ void stage_weights_q8_0(uint8_t *sm, const uint8_t *wbase, int64_t row_bytes,
                                                   int64_t r0, int64_t rows, int64_t kb, int64_t nb32) {
    const int tid = threadIdx.x;
    int8_t *sW = (int8_t *)sm;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int i = tid + 256 * it;              // (row, block, half): 128 x 8 x 2
        const int r = i >> 4, j = (i >> 1) & 7, half = i & 1;
        const int64_t row = r0 + r, b = kb * 8 + j;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row < rows && b < nb32) v = ld16(wbase + row * row_bytes + b * 34 + 2 + 16 * half);
        *(u32x4 *)(sW + r * kLd + 32 * j + 16 * half) = v;
    }
}

// Q6_K: codes folded with their int8 scale, split into lo (plane 0) and hi (plane 1).
__device__ __forceinline__ void stage_weights_q6_k(uint8_t *sm, const uint8_t *wbase, int64_t row_bytes,
                                                   int64_t r0, int64_t rows, int64_t kb) {
    const int tid = threadIdx.x;
    int8_t *sLo = (int8_t *)sm;
    int8_t *sHi = (int8_t *)sm + kTI * kLd;
#pragma unroll 2
    for (int it = 0; it < 8; ++it) {
        const int i = tid + 256 * it;              // (row, 16-value group G): 128 x 16
        const int r = i >> 4, G = i & 15;
        const int64_t row = r0 + r;
        uint32_t lo_w[4] = {0u, 0u, 0u, 0u}, hi_w[4] = {0u, 0u, 0u, 0u};
        if (row < rows) {
            const uint8_t *blk = wbase + row * row_bytes + kb * 210;
            const int h = G >> 3, gq = (G & 7) >> 1, l0 = 16 * (G & 1);
            const u32x4 ql = ld16(blk + 64 * h + 32 * (gq & 1) + l0);
            const u32x4 qh = ld16(blk + 128 + 32 * h + l0);
            const int sc = (int)(int8_t)blk[192 + G];
            const int nsh = gq < 2 ? 0 : 4, tsh = 2 * gq;
            const uint32_t qlw[4] = {ql.x, ql.y, ql.z, ql.w}, qhw[4] = {qh.x, qh.y, qh.z, qh.w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t code6 = ((qlw[d] >> nsh) & 0x0F0F0F0Fu) | (((qhw[d] >> tsh) & 0x03030303u) << 4);
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int bi = 0; bi < 4; ++bi) {
                    const int v = sc * ((int)((code6 >> (8 * bi)) & 0xFF) - 32);
                    lo |= (uint32_t)(v & 127) << (8 * bi);
                    hi |= (uint32_t)((v >> 7) & 0xFF) << (8 * bi);
                }
                lo_w[d] = lo;
                hi_w[d] = hi;
            }
        }
        const u32x4 lo4 = {lo_w[0], lo_w[1], lo_w[2], lo_w[3]};
        const u32x4 hi4 = {hi_w[0], hi_w[1], hi_w[2], hi_w[3]};
        *(u32x4 *)(sLo + r * kLd + 16 * G) = lo4;
        *(u32x4 *)(sHi + r * kLd + 16 * G) = hi4;
    }
}

// ---------------------------------------------------------------------------------------------
// Activation tile staging: J columns of the step's 8 q8_1 blocks -> int8 codes + fp32 (d, s).
// acol[] holds this thread's activation rows (or -1 for columns beyond the tile's range).
// ---------------------------------------------------------------------------------------------
template <int T, int J>
__device__ __forceinline__ void stage_acts(uint8_t *sm, const uint8_t *xq, int64_t nb32, int64_t kb,
                                           const int64_t (&acol)[J / 16], const int64_t (&tcol)[J / 32]) {
    const int tid = threadIdx.x;
    int8_t *sA = (int8_t *)(sm + Smem<T, J>::A_OFF);
    float2 *sX = (float2 *)(sm + Smem<T, J>::X_OFF);
#pragma unroll
    for (int it = 0; it < J / 16; ++it) {
        const int i = tid + 256 * it;              // (column, block, half): J x 8 x 2
        const int c = i >> 4, j = (i >> 1) & 7, half = i & 1;
        const int64_t b = kb * 8 + j;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (acol[it] >= 0 && b < nb32) v = ld16(xq + (acol[it] * nb32 + b) * kQ8_1Bytes + 4 + 16 * half);
        *(u32x4 *)(sA + c * kLd + 32 * j + 16 * half) = v;
    }
#pragma unroll
    for (int it = 0; it < J / 32; ++it) {
        const int i = tid + 256 * it;              // (block, column): 8 x J
        const int j = i / J, c = i % J;
        const int64_t b = kb * 8 + j;
        float2 v = make_float2(0.f, 0.f);
        if (tcol[it] >= 0 && b < nb32) {
            const uint32_t ds = *(const uint32_t *)(xq + (tcol[it] * nb32 + b) * kQ8_1Bytes);
            v = make_float2(h2f((uint16_t)(ds & 0xFFFF)), h2f((uint16_t)(ds >> 16)));
        }
        sX[j * J + c] = v;
    }
}

// ---------------------------------------------------------------------------------------------
// One 256-value step of MFMAs + fixups for this wave's 32 rows and all J columns.
// ---------------------------------------------------------------------------------------------
template <int T, int J, bool DBG>
__device__ __forceinline__ void tile_step(const uint8_t *sm, float (&acc)[J / 32][16], int64_t kb, int64_t nb32,
                                          int32_t *dbg, int64_t rows, int64_t n, int64_t r0, int64_t c0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int8_t *sW = (const int8_t *)sm;
    const int8_t *sA = (const int8_t *)(sm + Smem<T, J>::A_OFF);
    const float *sWs = (const float *)(sm + Smem<T, J>::WS_OFF);
    const float *sWm = (const float *)(sm + Smem<T, J>::WM_OFF);
    const float2 *sX = (const float2 *)(sm + Smem<T, J>::X_OFF);
    const int arow = 32 * wave + (lane & 31);
    const int koff = 16 * (lane >> 5);
    const int rbase = 32 * wave + 4 * (lane >> 5);   // + 8*(e/4) + e%4
    float d6[16];
    if constexpr (T == kQ6_K) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 v = *(const f32x4 *)(sWs + rbase + 8 * q);
            d6[4 * q] = v.x; d6[4 * q + 1] = v.y; d6[4 * q + 2] = v.z; d6[4 * q + 3] = v.w;
        }
    }
#pragma unroll 1
    for (int j = 0; j < 8; ++j) {
        if (kb * 8 + j >= nb32) break;   // Q8_0 ragged last step (workgroup-uniform)
        const u32x4 a = *(const u32x4 *)(sW + arow * kLd + 32 * j + koff);
        u32x4 a_hi;
        if constexpr (T == kQ6_K) a_hi = *(const u32x4 *)(sW + kTI * kLd + arow * kLd + 32 * j + koff);
        float ws[16], wm[16];
        if constexpr (T != kQ6_K) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = *(const f32x4 *)(sWs + j * kTI + rbase + 8 * q);
                ws[4 * q] = v.x; ws[4 * q + 1] = v.y; ws[4 * q + 2] = v.z; ws[4 * q + 3] = v.w;
                if constexpr (T == kQ4_K) {
                    const f32x4 u = *(const f32x4 *)(sWm + j * kTI + rbase + 8 * q);
                    wm[4 * q] = u.x; wm[4 * q + 1] = u.y; wm[4 * q + 2] = u.z; wm[4 * q + 3] = u.w;
                }
            }
        }
#pragma unroll
        for (int cb = 0; cb < J / 32; ++cb) {
            const int bcol = 32 * cb + (lane & 31);
            const u32x4 b = *(const u32x4 *)(sA + bcol * kLd + 32 * j + koff);
            const i32x16 zero = {};
            i32x16 D = mfma32x32x32(a, b, zero);
            if constexpr (T == kQ6_K) {
                const i32x16 Dh = mfma32x32x32(a_hi, b, zero);
#pragma unroll
                for (int e = 0; e < 16; ++e) D[e] = (Dh[e] << 7) + D[e];
            }
            if (DBG) {
                const int64_t col = c0 + bcol;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t row = r0 + rbase + 8 * (e >> 2) + (e & 3);
                    if (row < rows && col < n) dbg[(col * rows + row) * nb32 + kb * 8 + j] = D[e];
                }
            } else {
                const float2 x = sX[j * J + bcol];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    if constexpr (T == kQ4_K) acc[cb][e] += (float)D[e] * (ws[e] * x.x) - wm[e] * x.y;
                    else if constexpr (T == kQ8_0) acc[cb][e] += (float)D[e] * (ws[e] * x.x);
                    else acc[cb][e] += (float)D[e] * (d6[e] * x.x);
                }
            }
        }
    }
}

template <int T, int J>
__device__ __forceinline__ void stage_step(uint8_t *sm, const uint8_t *wbase, int64_t row_bytes, int64_t r0,
                                           int64_t rows, int64_t kb, int64_t nb32, const uint8_t *xq,
                                           const int64_t (&acol)[J / 16], const int64_t (&tcol)[J / 32]) {
    if constexpr (T == kQ4_K) stage_weights_q4_k(sm, wbase, row_bytes, r0, rows, kb);
    else if constexpr (T == kQ8_0) stage_weights_q8_0<J>(sm, wbase, row_bytes, r0, rows, kb, nb32);
    else stage_weights_q6_k(sm, wbase, row_bytes, r0, rows, kb);
    stage_weight_scales<T, J>(sm, wbase, row_bytes, r0, rows, kb, nb32);
    stage_acts<T, J>(sm, xq, nb32, kb, acol, tcol);
}

// Accumulator (lane, e) -> tile coordinates.
__device__ __forceinline__ int acc_row(int e) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    return 32 * wave + 4 * (lane >> 5) + 8 * (e >> 2) + (e & 3);
}

// ---------------------------------------------------------------------------------------------
// Dense kernel: persistent over the unit's (tile, step) range.
// ---------------------------------------------------------------------------------------------
template <int T, int J, bool DBG>
__global__ __launch_bounds__(256) void mmq_kernel(const uint8_t *__restrict__ w, int64_t rows, int64_t k,
                                                  const uint8_t *__restrict__ xq, int64_t n, float *__restrict__ y,
                                                  int32_t *__restrict__ dbg, MmqArgs args) {
    extern __shared__ __align__(16) uint8_t sm[];
    const int64_t nb32 = k / 32;
    const int64_t row_bytes = (k / Fmt<T>::QK) * Fmt<T>::BYTES;
    const int64_t u = xcd_remap(blockIdx.x, args.units);
    const int64_t W = args.ntiles * args.k_iters;
    int64_t pos = (u * W) / args.units;
    const int64_t end = ((u + 1) * W) / args.units;
    const int64_t first = pos;
    const int tid = threadIdx.x, lane = tid & 63;

    while (pos < end) {
        const int64_t t = pos / args.k_iters;
        const int64_t kb0 = pos - t * args.k_iters;
        const int64_t kb1 = (kb0 + (end - pos) < args.k_iters) ? kb0 + (end - pos) : args.k_iters;
        const int64_t rt = t / args.n_ct, ct = t - rt * args.n_ct;
        const int64_t r0 = rt * kTI, c0 = ct * J;

        int64_t acol[J / 16], tcol[J / 32];
#pragma unroll
        for (int it = 0; it < J / 16; ++it) {
            const int64_t c = c0 + ((tid + 256 * it) >> 4);
            acol[it] = c < n ? c : -1;
        }
#pragma unroll
        for (int it = 0; it < J / 32; ++it) {
            const int64_t c = c0 + (tid + 256 * it) % J;
            tcol[it] = (c < n && !DBG) ? c : -1;   // the debug export needs no scales
        }
        float acc[J / 32][16];
#pragma unroll
        for (int cb = 0; cb < J / 32; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[cb][e] = 0.f;

        for (int64_t kb = kb0; kb < kb1; ++kb) {
            __syncthreads();
            stage_step<T, J>(sm, w, row_bytes, r0, rows, kb, nb32, xq, acol, tcol);
            __syncthreads();
            tile_step<T, J, DBG>(sm, acc, kb, nb32, dbg, rows, n, r0, c0);
        }

        if (!DBG) {
            const bool whole = kb0 == 0 && kb1 == args.k_iters;
            float *dst;
            int64_t ld, rlim, clim;
            if (whole || !args.write_partials) {
                dst = y + c0 * rows + r0; ld = rows; rlim = rows - r0; clim = n - c0;
            } else {
                const int64_t slot = 2 * u + (pos == first ? 0 : 1);
                dst = args.partials + slot * (int64_t)kTI * J; ld = kTI; rlim = kTI; clim = J;
            }
#pragma unroll
            for (int cb = 0; cb < J / 32; ++cb) {
                const int col = 32 * cb + (lane & 31);
                if (col >= clim) continue;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int r = acc_row(e);
                    if (r < rlim) dst[(int64_t)col * ld + r] = acc[cb][e];
                }
            }
        }
        pos += kb1 - kb0;
    }
}

// Sum of the partial slots of every split tile, in ascending unit order.
__device__ __forceinline__ int64_t unit_of(int64_t item, int64_t W, int64_t units) {
    // largest u with floor(u*W/units) <= item
    int64_t lo = 0, hi = units - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) / 2;
        if ((mid * W) / units <= item) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <int J>
__global__ __launch_bounds__(256) void streamk_fixup_kernel(float *__restrict__ y, int64_t rows, int64_t n,
                                                            MmqArgs args) {
    const int64_t t = blockIdx.x;
    const int64_t W = args.ntiles * args.k_iters;
    const int64_t u0 = unit_of(t * args.k_iters, W, args.units);
    const int64_t u1 = unit_of((t + 1) * args.k_iters - 1, W, args.units);
    if (u0 == u1) return;                         // one unit covered the whole tile
    const int64_t rt = t / args.n_ct, ct = t - rt * args.n_ct;
    const int64_t r0 = rt * kTI, c0 = ct * J;
    for (int i = threadIdx.x; i < kTI * J; i += blockDim.x) {
        const int c = i / kTI, r = i - c * kTI;
        if (r0 + r >= rows || c0 + c >= n) continue;
        float v = 0.f;
        for (int64_t u = u0; u <= u1; ++u) {
            const int64_t first_tile = ((u * W) / args.units) / args.k_iters;
            const int64_t slot = 2 * u + (first_tile == t ? 0 : 1);
            v += args.partials[slot * (int64_t)kTI * J + (int64_t)c * kTI + r];
        }
        y[(c0 + c) * rows + r0 + r] = v;
    }
}

// ---------------------------------------------------------------------------------------------
// Expert kernel: one tile per workgroup, full K; grid (row tiles, column-tile slots).
// ---------------------------------------------------------------------------------------------
template <int T, int J>
__global__ __launch_bounds__(256) void mmq_id_kernel(const uint8_t *__restrict__ w, int64_t rows, int64_t k,
                                                     const uint8_t *__restrict__ xq, float *__restrict__ y,
                                                     ColMap cm, int32_t n_exp) {
    extern __shared__ __align__(16) uint8_t sm[];
    const int64_t ct = blockIdx.y;
    if (ct >= cm.tile_start[n_exp]) return;
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
    const uint8_t *wbase = w + (int64_t)e * cm.w_expert_stride;
    const int64_t r0 = (int64_t)blockIdx.x * kTI;
    const int64_t c0 = jt * J;
    const int tid = threadIdx.x, lane = tid & 63;

    auto arow_of = [&](int64_t c) -> int64_t {
        const int64_t pr = cm.sorted[seg + c];
        const int64_t t = pr / cm.top_k, s = pr - t * cm.top_k;
        return t * cm.x_per_tok + (cm.x_per_tok > 1 ? s : 0);
    };
    int64_t acol[J / 16], tcol[J / 32];
#pragma unroll
    for (int it = 0; it < J / 16; ++it) {
        const int64_t c = c0 + ((tid + 256 * it) >> 4);
        acol[it] = c < cnt ? arow_of(c) : -1;
    }
#pragma unroll
    for (int it = 0; it < J / 32; ++it) {
        const int64_t c = c0 + (tid + 256 * it) % J;
        tcol[it] = c < cnt ? arow_of(c) : -1;
    }
    float acc[J / 32][16];
#pragma unroll
    for (int cb = 0; cb < J / 32; ++cb)
#pragma unroll
        for (int e2 = 0; e2 < 16; ++e2) acc[cb][e2] = 0.f;

    const int64_t k_iters = (k + kSuper - 1) / kSuper;
    for (int64_t kb = 0; kb < k_iters; ++kb) {
        __syncthreads();
        stage_step<T, J>(sm, wbase, row_bytes, r0, rows, kb, nb32, xq, acol, tcol);
        __syncthreads();
        tile_step<T, J, false>(sm, acc, kb, nb32, nullptr, rows, cnt, r0, c0);
    }
#pragma unroll
    for (int cb = 0; cb < J / 32; ++cb) {
        const int64_t c = c0 + 32 * cb + (lane & 31);
        if (c >= cnt) continue;
        const int64_t orow = cm.sorted[seg + c];
#pragma unroll
        for (int e2 = 0; e2 < 16; ++e2) {
            const int64_t r = r0 + acc_row(e2);
            if (r < rows) y[orow * rows + r] = acc[cb][e2];
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------------
template <int T, int J, bool DBG>
static hipError_t launch_mmq_t(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y,
                               int32_t *dbg, const MmqLaunch &p, hipStream_t s) {
    MmqArgs a{p.ntiles, p.n_ct, p.k_iters, p.units, p.partials, p.stream_k ? 1 : 0};
    constexpr int smem = Smem<T, J>::BYTES;
    auto kern = mmq_kernel<T, J, DBG>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)p.units), dim3(256), smem, s, w, rows, k, xq, n, y, dbg, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || DBG || !p.stream_k) return e;
    hipLaunchKernelGGL(streamk_fixup_kernel<J>, dim3((unsigned)p.ntiles), dim3(256), 0, s, y, rows, n, a);
    return hipGetLastError();
}

template <int T, bool DBG>
static hipError_t launch_mmq_j(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y,
                               int32_t *dbg, const MmqLaunch &p, hipStream_t s) {
    if (p.tile_j == 32) return launch_mmq_t<T, 32, DBG>(w, rows, k, xq, n, y, dbg, p, s);
    if (p.tile_j == 64) return launch_mmq_t<T, 64, DBG>(w, rows, k, xq, n, y, dbg, p, s);
    if (p.tile_j == 128) return launch_mmq_t<T, 128, DBG>(w, rows, k, xq, n, y, dbg, p, s);
    return hipErrorInvalidValue;
}

hipError_t launch_mmq(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y,
                      int32_t *dbg, const MmqLaunch &p, hipStream_t s) {
    const bool d = dbg != nullptr;
#define QMM_MQ(TT)                                                                                    \
    if (type == TT) return d ? launch_mmq_j<TT, true>(w, rows, k, xq, n, y, dbg, p, s)    \
                             : launch_mmq_j<TT, false>(w, rows, k, xq, n, y, dbg, p, s);
    QMM_MQ(kQ4_K)
    QMM_MQ(kQ6_K)
    QMM_MQ(kQ8_0)
#undef QMM_MQ
    return hipErrorInvalidValue;
}

template <int T, int J>
static hipError_t launch_mmq_id_t(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, float *y,
                                  const ColMap &cm, int32_t n_exp, int64_t max_ct, hipStream_t s) {
    constexpr int smem = Smem<T, J>::BYTES;
    auto kern = mmq_id_kernel<T, J>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    if (max_ct <= 0) return hipSuccess;
    dim3 grid((unsigned)((rows + kTI - 1) / kTI), (unsigned)max_ct);
    hipLaunchKernelGGL(kern, grid, dim3(256), smem, s, w, rows, k, xq, y, cm, n_exp);
    return hipGetLastError();
}

hipError_t launch_mmq_id(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, float *y,
                         const ColMap &cm, int tile_j, int64_t max_col_tiles, hipStream_t s) {
#define QMM_MQI(TT)                                                                                   \
    if (type == TT) {                                                                                 \
        if (tile_j == 32) return launch_mmq_id_t<TT, 32>(w, rows, k, xq, y, cm, cm.n_exp, max_col_tiles, s); \
        if (tile_j == 64) return launch_mmq_id_t<TT, 64>(w, rows, k, xq, y, cm, cm.n_exp, max_col_tiles, s); \
        if (tile_j == 128) return launch_mmq_id_t<TT, 128>(w, rows, k, xq, y, cm, cm.n_exp, max_col_tiles, s); \
    }
    QMM_MQI(kQ4_K)
    QMM_MQI(kQ6_K)
    QMM_MQI(kQ8_0)
#undef QMM_MQI
    return hipErrorInvalidValue;
}

}  // namespace qmm
