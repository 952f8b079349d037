// Column resolution shared by the matrix-vector kernels.
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace qmm {

// Resolve the workgroup's columns: dense -> column c is activation row c and output row c;
// expert mode -> expert small[ey] (ey: the workgroup's place in the small-expert list, default
// blockIdx.y), columns are its (token, slot) pairs.
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
                                           bool expert, const uint8_t *w2 = nullptr, int ey = -1) {
    mc.wbase = w;
    mc.wbase2 = w2;
    mc.expert = expert;
    mc.cm = cm;
    mc.lo = 0;
    if (!expert) {
        mc.ncols = (int)n;
        return true;
    }
    const int e = cm.small[ey < 0 ? (int)blockIdx.y : ey];
    if (e < 0) return false;
    mc.lo = cm.bounds[e];
    mc.ncols = cm.bounds[e + 1] - mc.lo;
    mc.wbase = w + (int64_t)e * cm.w_expert_stride;
    if (w2) mc.wbase2 = w2 + (int64_t)e * cm.w_expert_stride;
    return true;
}

// Grid rows of an expert-mode matrix-vector launch (each row walks the small-expert list with a
// stride of the row count).  Where the experts average more than 16 pairs, few if any are small and
// most workgroups would only find the list's end: about four workgroups per compute unit over the
// row groups then suffice.  Otherwise (sparse routing, many small experts) one row per expert, so
// the small experts run side by side rather than one after another in a workgroup.
inline int64_t mv_expert_slots(int64_t row_groups, int64_t n_exp, int64_t pairs) {
    if (pairs <= 16 * n_exp) return n_exp;
    const int64_t target = 4 * (int64_t)device_cus();
    int64_t y = (target + row_groups - 1) / row_groups;
    if (y < 1) y = 1;
    return y < n_exp ? y : n_exp;
}

}  // namespace qmm
