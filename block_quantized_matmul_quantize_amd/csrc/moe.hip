// Expert grouping for the expert-indexed product (MMQ page, "expert bounds": per-expert segments
// of the expert-sorted column list, built on the GPU so that nothing is read back; "MoE skew":
// sorting by expert makes each expert's columns contiguous).
//
// One workgroup runs a stable counting sort of the (token, slot) pairs by expert id:
//   1. thread t counts its contiguous chunk of pairs per expert into an LDS table cnt[e][t]
//      (ids read in batches of independent loads, counted with LDS atomics on its own column);
//   2. thread e sums row e into bounds[e]; a scan over the experts turns these into the segment
//      starts; thread e then scans row e in thread order, so that (e, t) holds the first output
//      position of thread t's pairs of expert e (rows are padded to nthr + 1 entries, so the
//      threads of a wave walking their rows in step hit distinct LDS banks);
//   3. each thread walks its chunk again and writes pair indices to their positions, so the
//      order inside an expert is ascending pair index (token-major, then slot).
// It also emits the per-expert dispatch: experts with 1..small_max columns go to the
// matrix-vector kernel (list `small`), larger ones get ceil(count / tile_j) column tiles whose
// prefix is tile_start[].  Ids outside [0, n_exp) are skipped and counted in invalid[0].
#include "common.hpp"
#include "launch.hpp"

namespace qmm {

constexpr int kGroupThreads = 256;
constexpr int kGroupTableInts = 36864;   // LDS table: n_exp * row_stride(nthr) <= 36864 (144 KB)
constexpr int kGroupBatch = 32;          // ids in flight per thread

__host__ __device__ constexpr int group_row_stride(int nthr) { return nthr == 1 ? 1 : nthr + 1; }

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
    const int t = threadIdx.x;
    const int rs = group_row_stride(nthr);
    const bool active = t < nthr;
    const int64_t chunk = (pairs + nthr - 1) / nthr;
    const int64_t lo = active ? (int64_t)t * chunk : 0;
    const int64_t hi = active ? (lo + chunk < pairs ? lo + chunk : pairs) : 0;

    for (int i = t; i < n_exp * rs; i += kGroupThreads) tab[i] = 0;
    __syncthreads();
    int bad = 0;
    for (int64_t p0 = lo; p0 < hi; p0 += kGroupBatch) {
        int32_t ev[kGroupBatch];
#pragma unroll
        for (int j = 0; j < kGroupBatch; ++j) ev[j] = p0 + j < hi ? ids[p0 + j] : -1;
#pragma unroll
        for (int j = 0; j < kGroupBatch; ++j) {
            const int32_t e = ev[j];
            if (e >= 0 && e < n_exp) atomicAdd(&tab[e * rs + t], 1);
            else if (p0 + j < hi) bad++;
        }
    }
    bad_sh[t] = bad;
    __syncthreads();

    // row totals into bounds[e] (thread e, e + 256, ...)
    for (int e = t; e < n_exp; e += kGroupThreads) {
        int32_t v = 0;
        for (int i = 0; i < nthr; ++i) v += tab[e * rs + i];
        bounds[e] = v;
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
    // each row scanned in thread order from its segment start
    for (int e = t; e < n_exp; e += kGroupThreads) {
        int32_t run = bounds[e];
        for (int i = 0; i < nthr; ++i) {
            const int32_t v = tab[e * rs + i];
            tab[e * rs + i] = run;
            run += v;
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
    // scatter (the table is not read by the dispatch above, so no barrier is needed here); each
    // thread advances only its own column, in pair order
    for (int64_t p0 = lo; p0 < hi; p0 += kGroupBatch) {
        int32_t ev[kGroupBatch];
#pragma unroll
        for (int j = 0; j < kGroupBatch; ++j) ev[j] = p0 + j < hi ? ids[p0 + j] : -1;
#pragma unroll
        for (int j = 0; j < kGroupBatch; ++j) {
            const int32_t e = ev[j];
            if (e >= 0 && e < n_exp) sorted[atomicAdd(&tab[e * rs + t], 1)] = (int32_t)(p0 + j);
        }
    }
}

hipError_t launch_moe_group(const int32_t *ids, int64_t pairs, int32_t n_exp, int32_t tile_j, int32_t small_max,
                            int32_t *sorted, int32_t *bounds, int32_t *tile_start, int32_t *small, int32_t *invalid,
                            hipStream_t s) {
    int32_t nthr = kGroupThreads;
    while (nthr > 1 && (int64_t)group_row_stride(nthr) * n_exp > kGroupTableInts) nthr >>= 1;
    if ((int64_t)group_row_stride(nthr) * n_exp > kGroupTableInts) return hipErrorInvalidValue;
    hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(kGroupThreads), 0, s, ids, pairs, n_exp, nthr, tile_j,
                       small_max, sorted, bounds, tile_start, small, invalid);
    return hipGetLastError();
}

}  // namespace qmm
