// Expert grouping for the expert-indexed product (MMQ page, "expert bounds": per-expert segments
// of the expert-sorted column list, built on the GPU so that nothing is read back; "MoE skew":
// sorting by expert makes each expert's columns contiguous).
//
// One workgroup runs a stable counting sort of the (token, slot) pairs by expert id:
//   1. thread t counts its contiguous chunk of pairs per expert into an LDS table cnt[e][t]
//      (ids read in batches of independent loads);
//   2. per expert row e, the wave that owns it sums cnt[e][*] into bounds[e]; a scan over the
//      experts turns these into the segment starts; the row is then scanned in thread order, so
//      that (e, t) holds the first output position of thread t's pairs of expert e;
//   3. each thread walks its chunk again and writes pair indices to their positions, so the
//      order inside an expert is ascending pair index (token-major, then slot).
// It also emits the per-expert dispatch: experts with 1..small_max columns go to the
// matrix-vector kernel (list `small`), larger ones get ceil(count / tile_j) column tiles whose
// prefix is tile_start[].  Ids outside [0, n_exp) are skipped and counted in invalid[0].
#include "common.hpp"
#include "launch.hpp"

namespace qmm {

constexpr int kGroupThreads = 256;
constexpr int kGroupTableInts = 32768;   // LDS table: n_exp * threads_used <= 32768
constexpr int kGroupBatch = 16;          // ids in flight per thread

__device__ __forceinline__ int32_t wave_sum(int32_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    return v;
}

__global__ __launch_bounds__(kGroupThreads) void moe_group_kernel(const int32_t *__restrict__ ids, int64_t pairs,
                                                                  int32_t n_exp, int32_t nthr, int32_t tile_j,
                                                                  int32_t small_max, int32_t *__restrict__ sorted,
                                                                  int32_t *__restrict__ bounds,
                                                                  int32_t *__restrict__ tile_start,
                                                                  int32_t *__restrict__ small,
                                                                  int32_t *__restrict__ invalid) {
    __shared__ int32_t tab[kGroupTableInts];
    __shared__ int32_t part[kGroupThreads];
    __shared__ int32_t bad_sh[kGroupThreads];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    constexpr int NW = kGroupThreads / 64;
    const bool active = t < nthr;
    const int64_t chunk = (pairs + nthr - 1) / nthr;
    const int64_t lo = active ? (int64_t)t * chunk : 0;
    const int64_t hi = active ? (lo + chunk < pairs ? lo + chunk : pairs) : 0;

    for (int i = t; i < n_exp * nthr; i += kGroupThreads) tab[i] = 0;
    __syncthreads();
    int bad = 0;
    for (int64_t p0 = lo; p0 < hi; p0 += kGroupBatch) {
        int32_t ev[kGroupBatch];
#pragma unroll
        for (int j = 0; j < kGroupBatch; ++j) ev[j] = p0 + j < hi ? ids[p0 + j] : -1;
#pragma unroll
        for (int j = 0; j < kGroupBatch; ++j) {
            if (p0 + j >= hi) break;
            const int32_t e = ev[j];
            if (e >= 0 && e < n_exp) tab[e * nthr + t] += 1;
            else bad++;
        }
    }
    bad_sh[t] = bad;
    __syncthreads();

    // per-expert totals into bounds[e] (expert rows e = wid, wid + NW, ...; lanes stride the row)
    for (int e = wid; e < n_exp; e += NW) {
        int32_t v = 0;
        for (int i = lane; i < nthr; i += 64) v += tab[e * nthr + i];
        v = wave_sum(v);
        if (lane == 0) bounds[e] = v;
    }
    __syncthreads();
    // exclusive scan of the totals over the experts: thread t takes experts [t*ce, t*ce + ce)
    {
        const int ce = (n_exp + kGroupThreads - 1) / kGroupThreads;
        const int e0 = t * ce, e1 = e0 + ce < n_exp ? e0 + ce : n_exp;
        int32_t sum = 0;
        for (int e = e0; e < e1; ++e) sum += bounds[e];
        part[t] = sum;
        __syncthreads();
        if (t == 0) {
            int32_t run = 0, nbad = 0;
            for (int i = 0; i < kGroupThreads; ++i) {
                const int32_t v = part[i];
                part[i] = run;
                run += v;
                nbad += bad_sh[i];
            }
            bounds[n_exp] = run;
            invalid[0] = nbad;
        }
        __syncthreads();
        int32_t run = part[t];
        for (int e = e0; e < e1; ++e) {
            const int32_t v = bounds[e];
            bounds[e] = run;
            run += v;
        }
    }
    __syncthreads();
    // each expert row scanned in thread order: lane l takes threads [l*q, l*q + q), q = nthr/64
    // (nthr >= 64) or one thread per lane for l < nthr (nthr < 64)
    for (int e = wid; e < n_exp; e += NW) {
        const int q = nthr >= 64 ? nthr / 64 : 1;
        const int t0 = lane * q;
        int32_t loc[4];
        int32_t sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            loc[j] = (j < q && t0 + j < nthr) ? tab[e * nthr + t0 + j] : 0;
            sum += loc[j];
        }
        int32_t run = wave_incl_scan(sum) - sum + bounds[e];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < q && t0 + j < nthr) tab[e * nthr + t0 + j] = run;
            run += loc[j];
        }
    }
    __syncthreads();
    // the per-expert dispatch, from the segment starts
    if (t == 0) {
        int32_t tiles = 0, ns = 0;
        for (int e = 0; e < n_exp; ++e) {
            const int32_t c = bounds[e + 1] - bounds[e];
            tile_start[e] = tiles;
            if (c > small_max) tiles += (c + tile_j - 1) / tile_j;
            else if (c > 0) small[ns++] = e;
        }
        tile_start[n_exp] = tiles;
        for (int e = ns; e < n_exp; ++e) small[e] = -1;
    }
    // scatter (the table is not read by the dispatch above, so no barrier is needed here)
    for (int64_t p0 = lo; p0 < hi; p0 += kGroupBatch) {
        int32_t ev[kGroupBatch];
#pragma unroll
        for (int j = 0; j < kGroupBatch; ++j) ev[j] = p0 + j < hi ? ids[p0 + j] : -1;
#pragma unroll
        for (int j = 0; j < kGroupBatch; ++j) {
            if (p0 + j >= hi) break;
            const int32_t e = ev[j];
            if (e >= 0 && e < n_exp) {
                const int32_t pos = tab[e * nthr + t]++;
                sorted[pos] = (int32_t)(p0 + j);
            }
        }
    }
}

hipError_t launch_moe_group(const int32_t *ids, int64_t pairs, int32_t n_exp, int32_t tile_j, int32_t small_max,
                            int32_t *sorted, int32_t *bounds, int32_t *tile_start, int32_t *small, int32_t *invalid,
                            hipStream_t s) {
    int32_t nthr = kGroupThreads;
    while (nthr > 1 && (int64_t)nthr * n_exp > kGroupTableInts) nthr >>= 1;
    if ((int64_t)nthr * n_exp > kGroupTableInts) return hipErrorInvalidValue;
    hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(kGroupThreads), 0, s, ids, pairs, n_exp, nthr, tile_j,
                       small_max, sorted, bounds, tile_start, small, invalid);
    return hipGetLastError();
}

}  // namespace qmm
