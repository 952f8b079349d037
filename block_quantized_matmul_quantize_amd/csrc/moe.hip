// Expert grouping for the expert-indexed product (MMQ page, "expert bounds": per-expert segments
// of the expert-sorted column list, built on the GPU so that nothing is read back; "MoE skew":
// sorting by expert makes each expert's columns contiguous).
//
// One workgroup runs a counting sort of the (token, slot) pairs by expert id; up to 2304 experts it
// shares its launch with the quantization of the activations (moe_prologue_kernel, below), which
// the other workgroups do meanwhile.  Up to 2304 experts
// the slots come from per-wave LDS atomics (moe_group_wave_kernel, below: each expert's segment
// holds exactly its pairs, in an order not fixed within a wave's share); for more experts, a
// stable sort from per-thread counts:
//   1. thread t counts its contiguous chunk of pairs per expert into an LDS table cnt[e][t]
//      (ids read in batches of independent loads, counted with LDS atomics on its own column);
//   2. thread t owns the experts [t*ce, t*ce + ce): it sums their rows, a block scan over the
//      threads gives each expert its segment start bounds[e], and the thread scans each of its
//      rows in thread order, so that (e, t') holds the first output position of thread t''s
//      pairs of expert e (rows are padded to nthr + 1 entries, so the threads of a wave walking
//      their rows in step hit distinct LDS banks);
//   3. each thread writes its pair indices to their positions (scanned start of (e, t) plus the
//      pair's rank from the count pass, kept in registers for chunks up to 64 pairs; longer
//      chunks walk again with atomics), so the order inside an expert is ascending pair index
//      (token-major, then slot).
// It also emits the per-expert dispatch: experts with 1..small_max columns go to the
// matrix-vector kernel (list `small`), larger ones get ceil(count / tile_j) column tiles whose
// prefix is tile_start[] (two more block scans).  Ids outside [0, n_exp) are skipped and counted
// in invalid[0].  No step loops over all experts or all threads in one thread.
#include "common.hpp"
#include "launch.hpp"
#include "q8_1.hpp"
#include "tiled_act.hpp"

namespace qmm {

constexpr int kGroupThreads = 256;
constexpr int kGroupTableInts = 36864;   // LDS table: n_exp * row_stride(nthr) <= 36864 (144 KB)
constexpr int kGroupBatch = 32;          // ids in flight per thread
constexpr int kGroupKeep = 64;           // chunk length up to which ids and ranks stay in registers

__host__ __device__ constexpr int group_row_stride(int nthr) { return nthr == 1 ? 1 : nthr + 1; }

// ids [p0, p0 + kGroupBatch) of a chunk ending at hi into ev (-1 past hi): 16-byte loads where
// the ids are 16-byte aligned (chunks start at multiples of 4 pairs), single ids otherwise.
__device__ __forceinline__ void load_ids(const int32_t *ids, int64_t p0, int64_t hi, bool vec,
                                         int32_t (&ev)[kGroupBatch]) {
#pragma unroll
    for (int v = 0; v < kGroupBatch / 4; ++v) {
        const int64_t q = p0 + 4 * v;
        if (vec && q + 4 <= hi) {
            const u32x4 w = *(const u32x4 *)(ids + q);
            ev[4 * v] = (int32_t)w.x;
            ev[4 * v + 1] = (int32_t)w.y;
            ev[4 * v + 2] = (int32_t)w.z;
            ev[4 * v + 3] = (int32_t)w.w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) ev[4 * v + i] = q + i < hi ? ids[q + i] : -1;
        }
    }
}

// Exclusive scan of one value per thread over the workgroup (Hillis-Steele in LDS); returns the
// thread's exclusive prefix and writes the total to *total.  buf: 2 * kGroupThreads ints.
__device__ __forceinline__ int32_t block_excl_scan(int32_t v, int32_t *buf, int32_t *total) {
    const int t = threadIdx.x;
    int cur = 0;
    buf[t] = v;
    __syncthreads();
#pragma unroll
    for (int d = 1; d < kGroupThreads; d <<= 1) {
        const int32_t x = buf[cur * kGroupThreads + t] + (t >= d ? buf[cur * kGroupThreads + t - d] : 0);
        buf[(cur ^ 1) * kGroupThreads + t] = x;
        cur ^= 1;
        __syncthreads();
    }
    const int32_t incl = buf[cur * kGroupThreads + t];
    *total = buf[cur * kGroupThreads + kGroupThreads - 1];
    __syncthreads();   // buf is reused by the next scan
    return incl - v;
}

__global__ __launch_bounds__(kGroupThreads) void moe_group_kernel(const int32_t *__restrict__ ids, int64_t pairs,
                                                                  int32_t n_exp, int32_t nthr, int32_t tile_j,
                                                                  int32_t small_max, int32_t *__restrict__ sorted,
                                                                  int32_t *__restrict__ bounds,
                                                                  int32_t *__restrict__ tile_start,
                                                                  int32_t *__restrict__ small,
                                                                  int32_t *__restrict__ invalid) {
    __shared__ __align__(16) int32_t tab[kGroupTableInts];
    __shared__ int32_t sbuf[2 * kGroupThreads];
    __shared__ int32_t bad_sh;
    const int t = threadIdx.x;
    const int rs = group_row_stride(nthr);
    const bool active = t < nthr;
    const int64_t chunk = ((pairs + nthr - 1) / nthr + 3) & ~(int64_t)3;   // a multiple of 4 pairs
    const bool vec = (((uintptr_t)ids) & 15) == 0;
    const int64_t lo0 = (int64_t)t * chunk;
    const bool has = active && lo0 < pairs;                  // threads past the last chunk count nothing
    const int64_t lo = has ? lo0 : 0, hi = has ? (lo0 + chunk < pairs ? lo0 + chunk : pairs) : 0;
    const int ce = (n_exp + kGroupThreads - 1) / kGroupThreads;
    const int e0 = t * ce < n_exp ? t * ce : n_exp, e1 = e0 + ce < n_exp ? e0 + ce : n_exp;

    if (t == 0) bad_sh = 0;
    {   // zero the table, 16 bytes per store (kGroupTableInts is a multiple of 4 * kGroupThreads)
        u32x4 *tab4 = (u32x4 *)tab;
        const int n4 = (n_exp * rs + 3) / 4;
        for (int i = t; i < n4; i += kGroupThreads) tab4[i] = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    int bad = 0;
    // Chunks of at most kGroupKeep pairs (every chunk of the call: the chunk length is uniform)
    // keep their ids and their ranks inside (expert, thread) in registers, so the scatter needs
    // neither a second read of the ids nor a second atomic per pair.
    const bool keep = chunk <= kGroupKeep;
    int32_t kid[kGroupKeep], krank[kGroupKeep];
    if (keep) {
#pragma unroll
        for (int b = 0; b < kGroupKeep / kGroupBatch; ++b) {
            const int64_t p0 = lo + b * kGroupBatch;
            int32_t ev[kGroupBatch];
            load_ids(ids, p0, hi, vec, ev);
#pragma unroll
            for (int j = 0; j < kGroupBatch; ++j) {
                const int32_t e = ev[j];
                kid[b * kGroupBatch + j] = e;
                // out-of-range ids (and the -1 past the chunk) skip the table; only real ones
                // count as bad
                krank[b * kGroupBatch + j] = (uint32_t)e < (uint32_t)n_exp ? atomicAdd(&tab[e * rs + t], 1) : 0;
                if ((uint32_t)e >= (uint32_t)n_exp) bad += p0 + j < hi ? 1 : 0;
            }
        }
    } else {
        for (int64_t p0 = lo; p0 < hi; p0 += kGroupBatch) {
            int32_t ev[kGroupBatch];
            load_ids(ids, p0, hi, vec, ev);
#pragma unroll
            for (int j = 0; j < kGroupBatch; ++j) {
                const int32_t e = ev[j];
                if ((uint32_t)e < (uint32_t)n_exp) atomicAdd(&tab[e * rs + t], 1);
                else bad += p0 + j < hi ? 1 : 0;
            }
        }
    }
    if (bad) atomicAdd(&bad_sh, bad);
    __syncthreads();

    // row totals of the thread's experts (kept in bounds[e] until the scan below)
    int32_t mine = 0;
    for (int e = e0; e < e1; ++e) {
        const int32_t *row = tab + e * rs;
        int32_t a0 = 0, a1 = 0, a2 = 0, a3 = 0;
        int i = 0;
        for (; i + 4 <= nthr; i += 4) {
            a0 += row[i];
            a1 += row[i + 1];
            a2 += row[i + 2];
            a3 += row[i + 3];
        }
        for (; i < nthr; ++i) a0 += row[i];
        const int32_t v = a0 + a1 + a2 + a3;
        bounds[e] = v;
        mine += v;
    }
    int32_t total = 0;
    int32_t run = block_excl_scan(mine, sbuf, &total);
    // segment starts, row scans, and the thread's dispatch counts
    int32_t my_tiles = 0, my_small = 0;
    for (int e = e0; e < e1; ++e) {
        const int32_t c = bounds[e];
        bounds[e] = run;
        int32_t *row = tab + e * rs;
        int32_t r = run;
        int i = 0;
        for (; i + 4 <= nthr; i += 4) {
            const int32_t v0 = row[i], v1 = row[i + 1], v2 = row[i + 2], v3 = row[i + 3];
            row[i] = r;
            row[i + 1] = r + v0;
            row[i + 2] = r + v0 + v1;
            row[i + 3] = r + v0 + v1 + v2;
            r += v0 + v1 + v2 + v3;
        }
        for (; i < nthr; ++i) {
            const int32_t v0 = row[i];
            row[i] = r;
            r += v0;
        }
        run += c;
        // count of tiles, or -1 for an expert the matrix-vector kernel takes (prefixes below)
        const int32_t nt = c > small_max ? (c + tile_j - 1) / tile_j : (c > 0 ? -1 : 0);
        tile_start[e] = nt;
        my_tiles += nt > 0 ? nt : 0;
        my_small += nt < 0 ? 1 : 0;
    }
    int32_t tiles_total = 0, small_total = 0;
    int32_t trun = block_excl_scan(my_tiles, sbuf, &tiles_total);
    int32_t srun = block_excl_scan(my_small, sbuf, &small_total);
    for (int e = e0; e < e1; ++e) {
        const int32_t nt = tile_start[e];
        if (nt < 0) small[srun++] = e;
        tile_start[e] = trun;
        trun += nt > 0 ? nt : 0;
    }
    for (int i = small_total + t; i < n_exp; i += kGroupThreads) small[i] = -1;
    if (t == 0) {
        bounds[n_exp] = total;
        tile_start[n_exp] = tiles_total;
        invalid[0] = bad_sh;
    }
    __syncthreads();
    // scatter: position = the (expert, thread) start from the scan + the pair's rank there
    if (keep) {
#pragma unroll
        for (int j = 0; j < kGroupKeep; ++j) {
            const int32_t e = kid[j];
            if ((uint32_t)e < (uint32_t)n_exp) sorted[tab[e * rs + t] + krank[j]] = (int32_t)(lo + j);
        }
        return;
    }
    // longer chunks: each thread advances its own column, in pair order
    for (int64_t p0 = lo; p0 < hi; p0 += kGroupBatch) {
        int32_t ev[kGroupBatch];
        load_ids(ids, p0, hi, vec, ev);
        // positions first (LDS atomics in pair order on the thread's own column), then the stores
        int32_t pos[kGroupBatch];
#pragma unroll
        for (int j = 0; j < kGroupBatch; ++j) {
            const int32_t e = ev[j];
            pos[j] = (uint32_t)e < (uint32_t)n_exp ? atomicAdd(&tab[e * rs + t], 1) : -1;
        }
#pragma unroll
        for (int j = 0; j < kGroupBatch; ++j)
            if (pos[j] >= 0) sorted[pos[j]] = (int32_t)(p0 + j);
    }
}

// ---------------------------------------------------------------------------------------------
// The grouping for up to kWaveMaxExperts experts, with LDS atomics instead of per-thread rows.
// 16 waves; wave w owns the contiguous pairs [w*chunk, (w+1)*chunk) and counts them per expert
// into its own row hist[w][e] with LDS atomics (lanes of a wave with the same expert serialise on
// one address); the value an atomic returns is the pair's rank among wave w's pairs of expert e.
// The rows are scanned expert-major -- expert e's segment start plus the counts of waves w' < w --
// so a pair's slot is hist[w][e] + its rank.  Chunks of up to 1024 pairs (every call up to 16384
// pairs) keep their ids and ranks in registers, so the ids are read once and each pair costs one
// atomic; longer chunks read their ids again and take slots with a second atomic per pair.  Each
// expert's segment holds exactly its pairs, the pairs of wave w before those of wave w + 1
// (ascending blocks of pair indices), but the order among one wave's pairs of an expert is the
// order the atomics were served in, which need not be the same from run to run.  Any order is
// correct: every column of an expert is computed on its own, with the same arithmetic whatever
// its place in the segment, so the products are bitwise the same.  (The earlier per-thread form
// spent most of its time in serial row scans of an n_exp x 256 table on one compute unit.)
// ---------------------------------------------------------------------------------------------
constexpr int kWaveGroupWaves = 16;
constexpr int kWaveMaxExperts = kGroupTableInts / kWaveGroupWaves;   // 2304
constexpr int kWaveGroupBatches = 16;                                // 64-id batches loaded together

// Exclusive scans of three values per thread over the 1024-thread workgroup in one pass: lane
// prefixes by shuffles, then the 16 wave totals of each (wsum, 3 x 16 ints of LDS).  v[i] becomes
// the thread's exclusive prefix, tot[i] the workgroup total.
__device__ __forceinline__ void wave_block_excl_scan3(int32_t (&v)[3], int32_t *wsum, int32_t (&tot)[3]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t x[3] = {v[0], v[1], v[2]};
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int32_t y = __shfl_up(x[i], d);
            if (lane >= d) x[i] += y;
        }
    }
    if (lane == 63) {
#pragma unroll
        for (int i = 0; i < 3; ++i) wsum[i * kWaveGroupWaves + wave] = x[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        int32_t pre = 0, t = 0;
#pragma unroll
        for (int w = 0; w < kWaveGroupWaves; ++w) {
            const int32_t sv = wsum[i * kWaveGroupWaves + w];
            pre += w < wave ? sv : 0;
            t += sv;
        }
        tot[i] = t;
        v[i] = pre + x[i] - v[i];
    }
}

// The grouping itself, run by one 1024-thread workgroup; hist / wsum / bad_sh are its LDS.
__device__ __forceinline__ void moe_group_wave(const int32_t *__restrict__ ids, int64_t pairs, int32_t n_exp,
                                               int32_t tile_j, int32_t small_max, int32_t *__restrict__ sorted,
                                               int32_t *__restrict__ bounds, int32_t *__restrict__ tile_start,
                                               int32_t *__restrict__ small, int32_t *__restrict__ invalid,
                                               int32_t *hist, int32_t *wsum, int32_t &bad_sh) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    constexpr int NT = 64 * kWaveGroupWaves;
    const int64_t chunk = ((pairs + kWaveGroupWaves - 1) / kWaveGroupWaves + 63) & ~(int64_t)63;
    const int64_t lo = (int64_t)wave * chunk < pairs ? (int64_t)wave * chunk : pairs;
    const int64_t hi = lo + chunk < pairs ? lo + chunk : pairs;
    int32_t *my = hist + wave * n_exp;
    // chunk is uniform over the waves, so every wave takes the same branch below
    const bool keep = chunk <= 64 * kWaveGroupBatches;

    // The wave's ids, kWaveGroupBatches batches of 64 at a time, every load issued before the
    // first is used (one memory latency per group, not per batch).
    auto load_group = [&](int64_t g0, int32_t (&ev)[kWaveGroupBatches]) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < kWaveGroupBatches; ++b) {
            const int64_t p = g0 + 64 * b + lane;
            ev[b] = p < hi ? ids[p] : -1;
        }
    };

    // The first group's loads go out before the table is cleared.
    int32_t ev[kWaveGroupBatches], rank[kWaveGroupBatches];
    load_group(lo, ev);
    if (t == 0) bad_sh = 0;
    for (int i = t; i < kWaveGroupWaves * n_exp; i += NT) hist[i] = 0;
    __syncthreads();

    // pass 1: per-wave counts (and, for a kept chunk, each pair's rank)
    int bad = 0;
    for (int64_t g0 = lo; g0 < hi; g0 += 64 * kWaveGroupBatches) {
        if (g0 != lo) load_group(g0, ev);
#pragma unroll
        for (int b = 0; b < kWaveGroupBatches; ++b) {
            const int32_t e = ev[b];
            if ((uint32_t)e < (uint32_t)n_exp) rank[b] = atomicAdd(&my[e], 1);
            else bad += g0 + 64 * b + lane < hi ? 1 : 0;
        }
    }
    if (bad) atomicAdd(&bad_sh, bad);
    __syncthreads();

    // scan: thread t owns the experts [t*ce, t*ce + ce) (contiguous, so the workgroup scan of the
    // per-thread totals orders them); hist[w][e] becomes the first position of wave w's pairs of e
    const int ce = (n_exp + NT - 1) / NT;
    const int e0 = t * ce < n_exp ? t * ce : n_exp, e1 = e0 + ce < n_exp ? e0 + ce : n_exp;
    // per thread: pairs, column tiles, and matrix-vector (small) experts of its experts
    int32_t acc[3] = {0, 0, 0};
    for (int e = e0; e < e1; ++e) {
        int32_t c = 0;
#pragma unroll
        for (int w = 0; w < kWaveGroupWaves; ++w) c += hist[w * n_exp + e];
        acc[0] += c;
        acc[1] += c > small_max ? (c + tile_j - 1) / tile_j : 0;
        acc[2] += c > 0 && c <= small_max ? 1 : 0;
    }
    int32_t tot[3];
    wave_block_excl_scan3(acc, wsum, tot);
    int32_t run = acc[0], trun = acc[1], srun = acc[2];
    for (int e = e0; e < e1; ++e) {
        bounds[e] = run;
        tile_start[e] = trun;
        int32_t r = run;
#pragma unroll
        for (int w = 0; w < kWaveGroupWaves; ++w) {
            const int32_t v = hist[w * n_exp + e];
            hist[w * n_exp + e] = r;
            r += v;
        }
        const int32_t c = r - run;
        run = r;
        if (c > small_max) trun += (c + tile_j - 1) / tile_j;
        else if (c > 0) small[srun++] = e;
    }
    for (int i = tot[2] + t; i < n_exp; i += NT) small[i] = -1;
    if (t == 0) {
        bounds[n_exp] = tot[0];
        tile_start[n_exp] = tot[1];
        invalid[0] = bad_sh;
    }
    __syncthreads();

    // pass 2: each pair's slot.  A kept chunk whose whole sorted list fits in LDS beside the table
    // is placed there first and then written out with contiguous 16-byte stores: scattered 4-byte
    // stores from the one compute unit cost more than all the rest of the kernel.
    if (keep) {
        const int soff = (kWaveGroupWaves * n_exp + 3) & ~3;   // 16-byte aligned staging area
        if (soff + pairs <= kGroupTableInts) {
            int32_t *stage = hist + soff;
#pragma unroll
            for (int b = 0; b < kWaveGroupBatches; ++b) {
                const int32_t e = ev[b];
                if ((uint32_t)e < (uint32_t)n_exp) stage[my[e] + rank[b]] = (int32_t)(lo + 64 * b + lane);
            }
            __syncthreads();
            const int32_t n = tot[0], n4 = n >> 2;
            const u32x4 *s4 = (const u32x4 *)stage;
            u32x4 *d4 = (u32x4 *)sorted;   // sorted is 256-byte aligned (workspace layout)
            for (int i = t; i < n4; i += NT) d4[i] = s4[i];
            for (int i = 4 * n4 + t; i < n; i += NT) sorted[i] = stage[i];
        } else {
#pragma unroll
            for (int b = 0; b < kWaveGroupBatches; ++b) {
                const int32_t e = ev[b];
                if ((uint32_t)e < (uint32_t)n_exp) sorted[my[e] + rank[b]] = (int32_t)(lo + 64 * b + lane);
            }
        }
        return;
    }
    for (int64_t g0 = lo; g0 < hi; g0 += 64 * kWaveGroupBatches) {
        load_group(g0, ev);
        int32_t pos[kWaveGroupBatches];
#pragma unroll
        for (int b = 0; b < kWaveGroupBatches; ++b) {
            const int32_t e = ev[b];
            pos[b] = (uint32_t)e < (uint32_t)n_exp ? atomicAdd(&my[e], 1) : -1;
        }
#pragma unroll
        for (int b = 0; b < kWaveGroupBatches; ++b)
            if (pos[b] >= 0) sorted[pos[b]] = (int32_t)(g0 + 64 * b + lane);
    }
}

__global__ __launch_bounds__(64 * kWaveGroupWaves) void moe_group_wave_kernel(
    const int32_t *__restrict__ ids, int64_t pairs, int32_t n_exp, int32_t tile_j, int32_t small_max,
    int32_t *__restrict__ sorted, int32_t *__restrict__ bounds, int32_t *__restrict__ tile_start,
    int32_t *__restrict__ small, int32_t *__restrict__ invalid) {
    __shared__ __align__(16) int32_t hist[kGroupTableInts];   // [wave][expert]
    __shared__ int32_t wsum[3 * kWaveGroupWaves];
    __shared__ int32_t bad_sh;
    moe_group_wave(ids, pairs, n_exp, tile_j, small_max, sorted, bounds, tile_start, small, invalid, hist, wsum, bad_sh);
}

// The expert call's prologue in one launch: workgroup 0 groups the pairs (moe_group_wave), the
// others quantize the fp32 activation rows into the tiled and the canonical q8_1 layouts with the
// arithmetic of quantize_q8_1_tiled_kernel (q8_1.hpp), a 4-lane group per 32-value block, striding
// over the blocks.  The two jobs are independent, so the grouping's latency -- one compute unit
// working through a chain of loads, LDS atomics, scans and barriers -- hides under the
// quantization instead of adding to it.
__global__ __launch_bounds__(64 * kWaveGroupWaves) void moe_prologue_kernel(
    const int32_t *__restrict__ ids, int64_t pairs, int32_t n_exp, int32_t tile_j, int32_t small_max,
    int32_t *__restrict__ sorted, int32_t *__restrict__ bounds, int32_t *__restrict__ tile_start,
    int32_t *__restrict__ small, int32_t *__restrict__ invalid, const float *__restrict__ x, int64_t n_rows,
    int64_t k, uint8_t *__restrict__ tiled, uint8_t *__restrict__ canon) {
    __shared__ __align__(16) int32_t hist[kGroupTableInts];
    __shared__ int32_t wsum[3 * kWaveGroupWaves];
    __shared__ int32_t bad_sh;
    if (blockIdx.x == 0) {
        moe_group_wave(ids, pairs, n_exp, tile_j, small_max, sorted, bounds, tile_start, small, invalid, hist, wsum,
                       bad_sh);
        return;
    }
    const int64_t nb = k / 32;
    const int64_t total = n_rows * nb * 4;   // a multiple of 4: the 4 lanes of a block loop together
    const int64_t stride = (int64_t)(gridDim.x - 1) * blockDim.x;
    for (int64_t gid = (int64_t)(blockIdx.x - 1) * blockDim.x + threadIdx.x; gid < total; gid += stride) {
        const int64_t blk = gid >> 2;
        const int sub = (int)(gid & 3);
        const int64_t row = blk / nb, bi = blk - row * nb;
        const float *src = x + row * k + bi * 32 + 8 * sub;
        const Q81Lane4 q = quantize_q8_1_lane4(*(const float4 *)src, *(const float4 *)(src + 4));
        tiled_act_put(tiled, (nb + 7) / 8, n_rows, row, bi, sub, q.c0, q.c1, q.ds);
        uint8_t *yb = canon + blk * kQ8_1Bytes;
        *(u32x2_a4 *)(yb + 4 + 8 * sub) = u32x2{q.c0, q.c1};
        if (sub == 0) *(uint32_t *)yb = q.ds;
    }
}

hipError_t launch_moe_group(const int32_t *ids, int64_t pairs, int32_t n_exp, int32_t tile_j, int32_t small_max,
                            int32_t *sorted, int32_t *bounds, int32_t *tile_start, int32_t *small, int32_t *invalid,
                            hipStream_t s) {
    if (n_exp >= 1 && n_exp <= kWaveMaxExperts) {
        hipLaunchKernelGGL(moe_group_wave_kernel, dim3(1), dim3(64 * kWaveGroupWaves), 0, s, ids, pairs, n_exp,
                           tile_j, small_max, sorted, bounds, tile_start, small, invalid);
        return hipGetLastError();
    }
    int32_t nthr = kGroupThreads;
    while (nthr > 1 && (int64_t)group_row_stride(nthr) * n_exp > kGroupTableInts) nthr >>= 1;
    if ((int64_t)group_row_stride(nthr) * n_exp > kGroupTableInts) return hipErrorInvalidValue;
    hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(kGroupThreads), 0, s, ids, pairs, n_exp, nthr, tile_j,
                       small_max, sorted, bounds, tile_start, small, invalid);
    return hipGetLastError();
}

bool moe_prologue_fused(int32_t n_exp) { return n_exp >= 1 && n_exp <= kWaveMaxExperts; }

hipError_t launch_moe_prologue(const int32_t *ids, int64_t pairs, int32_t n_exp, int32_t tile_j, int32_t small_max,
                               int32_t *sorted, int32_t *bounds, int32_t *tile_start, int32_t *small, int32_t *invalid,
                               const float *x, int64_t n_rows, int64_t k, uint8_t *tiled, uint8_t *canon,
                               int32_t cus, hipStream_t s) {
    if (!moe_prologue_fused(n_exp)) return hipErrorInvalidValue;
    // one quantizing workgroup per remaining compute unit (each holds the grouping's LDS, so one
    // workgroup per compute unit), at most one per 1024 threads of work
    const int64_t work = n_rows * (k / 32) * 4;
    int64_t q = (work + 64 * kWaveGroupWaves - 1) / (64 * kWaveGroupWaves);
    const int64_t qmax = cus > 1 ? cus - 1 : 1;
    if (q > qmax) q = qmax;
    if (q < 1) q = 1;
    hipLaunchKernelGGL(moe_prologue_kernel, dim3((unsigned)(1 + q)), dim3(64 * kWaveGroupWaves), 0, s, ids, pairs,
                       n_exp, tile_j, small_max, sorted, bounds, tile_start, small, invalid, x, n_rows, k, tiled, canon);
    return hipGetLastError();
}

}  // namespace qmm
