// Expert grouping for the expert-indexed product (MMQ page, "expert bounds": per-expert segments
// of the expert-sorted column list, built on the GPU so that nothing is read back; "MoE skew":
// sorting by expert makes each expert's columns contiguous).
//
// One workgroup runs a stable counting sort of the (token, slot) pairs by expert id:
//   1. thread t counts its contiguous chunk of pairs per expert into an LDS table cnt[e][t];
//   2. an exclusive scan of the table in (expert, thread) order gives each (e, t) its first
//      output position, and expert e's segment start bounds[e];
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
    __shared__ int32_t total_sh;
    const int t = threadIdx.x;
    const bool active = t < nthr;
    const int64_t chunk = (pairs + nthr - 1) / nthr;
    const int64_t lo = active ? (int64_t)t * chunk : 0;
    const int64_t hi = active ? (lo + chunk < pairs ? lo + chunk : pairs) : 0;

    if (active)
        for (int e = 0; e < n_exp; ++e) tab[e * nthr + t] = 0;
    int bad = 0;
    for (int64_t p = lo; p < hi; ++p) {
        const int32_t e = ids[p];
        if (e >= 0 && e < n_exp) tab[e * nthr + t] += 1;
        else bad++;
    }
    bad_sh[t] = bad;
    __syncthreads();

    // Exclusive scan over tab in linear (expert-major) order: thread t owns entries
    // [t*n_exp, (t+1)*n_exp) of the nthr*n_exp table.
    int32_t s = 0;
    if (active)
        for (int i = 0; i < n_exp; ++i) s += tab[t * n_exp + i];
    part[t] = active ? s : 0;
    __syncthreads();
    if (t == 0) {
        int32_t run = 0, nbad = 0;
        for (int i = 0; i < nthr; ++i) {
            const int32_t v = part[i];
            part[i] = run;
            run += v;
        }
        for (int i = 0; i < kGroupThreads; ++i) nbad += bad_sh[i];
        bounds[n_exp] = run;
        total_sh = run;
        invalid[0] = nbad;
    }
    __syncthreads();
    if (active) {
        int32_t run = part[t];
        for (int i = 0; i < n_exp; ++i) {
            const int32_t v = tab[t * n_exp + i];
            tab[t * n_exp + i] = run;
            run += v;
        }
    }
    __syncthreads();
    // Segment starts and the per-expert dispatch, read from the scanned table before the
    // scatter advances it.
    for (int e = t; e < n_exp; e += blockDim.x) bounds[e] = tab[e * nthr];
    if (t == 0) {
        const int32_t total = total_sh;
        int32_t tiles = 0, ns = 0;
        for (int e = 0; e < n_exp; ++e) {
            const int32_t start = tab[e * nthr];
            const int32_t stop = (e + 1 < n_exp) ? tab[(e + 1) * nthr] : total;
            const int32_t c = stop - start;
            tile_start[e] = tiles;
            if (c > small_max) tiles += (c + tile_j - 1) / tile_j;
            else if (c > 0) small[ns++] = e;
        }
        tile_start[n_exp] = tiles;
        for (int e = ns; e < n_exp; ++e) small[e] = -1;
    }
    __syncthreads();
    // scatter
    for (int64_t p = lo; p < hi; ++p) {
        const int32_t e = ids[p];
        if (e >= 0 && e < n_exp) {
            const int32_t pos = tab[e * nthr + t]++;
            sorted[pos] = (int32_t)p;
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
