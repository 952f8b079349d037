// Column resolution shared by the matrix-vector kernels.
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace qmm {

// Resolve the workgroup's columns: dense -> column c is activation row c and output row c;
// expert mode -> expert small[blockIdx.y], columns are its (token, slot) pairs.
struct MvCols {
    int ncols;
    int lo;
    const uint8_t *wbase;
    const uint8_t *wbase2;   // gate/up fusion: the up matrix (wbase the gate)
    bool expert;
    ColMap cm;
    __device__ __forceinline__ int64_t pair(int c) const { return expert ? cm.sorted[lo + c] : c; }
    __device__ __forceinline__ int64_t arow(int c) const {
        if (!expert) return c;
        const int64_t pr = cm.sorted[lo + c];
        const int64_t t = pr / cm.top_k, s = pr - t * cm.top_k;
        return t * cm.x_per_tok + (cm.x_per_tok > 1 ? s : 0);
    }
};

__device__ __forceinline__ bool mv_resolve(MvCols &mc, const uint8_t *w, int64_t n, const ColMap &cm,
                                           bool expert, const uint8_t *w2 = nullptr) {
    mc.wbase = w;
    mc.wbase2 = w2;
    mc.expert = expert;
    mc.cm = cm;
    mc.lo = 0;
    if (!expert) {
        mc.ncols = (int)n;
        return true;
    }
    const int e = cm.small[blockIdx.y];
    if (e < 0) return false;
    mc.lo = cm.bounds[e];
    mc.ncols = cm.bounds[e + 1] - mc.lo;
    mc.wbase = w + (int64_t)e * cm.w_expert_stride;
    if (w2) mc.wbase2 = w2 + (int64_t)e * cm.w_expert_stride;
    return true;
}

}  // namespace qmm
