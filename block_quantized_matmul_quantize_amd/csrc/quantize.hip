// q8_1 activation quantization kernel: one block of 32 values per 4 consecutive lanes, each lane
// owning 8 values (two 16-byte loads, one 8-byte store of codes); the arithmetic and its readings
// are in q8_1.hpp.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"
#include "q8_1.hpp"
#include "tiled_act.hpp"

namespace qmm {

__global__ __launch_bounds__(256) void quantize_q8_1_kernel(const float *__restrict__ x, int64_t n_rows,
                                                            int64_t k, uint8_t *__restrict__ y) {
    const int64_t nb = k / 32;
    const int64_t total = n_rows * nb;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t blk = gid >> 2;
    const int sub = (int)(gid & 3);
    const bool live = blk < total;   // the whole 4-lane group shares this predicate
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (live) {
        const int64_t row = blk / nb;
        const float *src = x + row * k + (blk - row * nb) * 32 + 8 * sub;
        a = *(const float4 *)src;
        b = *(const float4 *)(src + 4);
    }
    const Q81Lane4 q = quantize_q8_1_lane4(a, b);
    if (!live) return;
    uint8_t *yb = y + blk * kQ8_1Bytes;
    *(u32x2_a4 *)(yb + 4 + 8 * sub) = u32x2{q.c0, q.c1};
    if (sub == 0) *(uint32_t *)yb = q.ds;
}

// Same quantization, written in the tiled kernel's layout (tiled_act.hpp), optionally also as
// canonical blocks.
__global__ __launch_bounds__(256) void quantize_q8_1_tiled_kernel(const float *__restrict__ x, int64_t n_rows,
                                                                  int64_t k, uint8_t *__restrict__ tiled,
                                                                  uint8_t *__restrict__ canon,
                                                                  int32_t *__restrict__ zero, int64_t nzero) {
    const int64_t nb = k / 32;
    const int64_t total = n_rows * nb;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t i = gid; i < nzero; i += (int64_t)gridDim.x * blockDim.x) zero[i] = 0;
    const int64_t blk = gid >> 2;
    const int sub = (int)(gid & 3);
    const bool live = blk < total;   // the whole 4-lane group shares this predicate
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    int64_t row = 0, bi = 0;
    if (live) {
        row = blk / nb;
        bi = blk - row * nb;
        const float *src = x + row * k + bi * 32 + 8 * sub;
        a = *(const float4 *)src;
        b = *(const float4 *)(src + 4);
    }
    const Q81Lane4 q = quantize_q8_1_lane4(a, b);
    if (!live) return;
    tiled_act_put(tiled, (nb + 7) / 8, n_rows, row, bi, sub, q.c0, q.c1, q.ds);
    if (canon) {
        uint8_t *yb = canon + blk * kQ8_1Bytes;
        *(u32x2_a4 *)(yb + 4 + 8 * sub) = u32x2{q.c0, q.c1};
        if (sub == 0) *(uint32_t *)yb = q.ds;
    }
}

// Canonical q8_1 blocks -> tiled layout: 4 threads per block, 8 code bytes each.
__global__ __launch_bounds__(256) void relayout_q8_1_tiled_kernel(const uint8_t *__restrict__ xq, int64_t n_rows,
                                                                  int64_t k, uint8_t *__restrict__ tiled,
                                                                  int32_t *__restrict__ zero, int64_t nzero) {
    const int64_t nb = k / 32;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t i = gid; i < nzero; i += (int64_t)gridDim.x * blockDim.x) zero[i] = 0;
    const int64_t blk = gid >> 2;
    const int sub = (int)(gid & 3);
    if (blk >= n_rows * nb) return;
    const int64_t row = blk / nb, bi = blk - row * nb;
    const uint8_t *src = xq + blk * kQ8_1Bytes;
    const u32x2 c = *(const u32x2_a4 *)(src + 4 + 8 * sub);
    tiled_act_put(tiled, (nb + 7) / 8, n_rows, row, bi, sub, c.x, c.y, *(const uint32_t *)src);
}

// Plain fill kernel (used instead of a memset so that the call sequence stays capturable).
__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *__restrict__ p, int64_t n, uint32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = i; j < n; j += stride) p[j] = v;
}

hipError_t launch_quantize_q8_1(const float *x, int64_t n_rows, int64_t k, uint8_t *y, hipStream_t s) {
    const int64_t threads = n_rows * (k / 32) * 4;
    if (threads == 0) return hipSuccess;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(quantize_q8_1_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, n_rows, k, y);
    return hipGetLastError();
}

hipError_t launch_quantize_q8_1_tiled(const float *x, int64_t n_rows, int64_t k, uint8_t *tiled, uint8_t *canon,
                                      hipStream_t s, int32_t *zero, int64_t nzero) {
    const int64_t threads = n_rows * (k / 32) * 4;
    if (threads == 0 && nzero <= 0) return hipSuccess;
    const int64_t blocks = (std::max<int64_t>(threads, nzero) + 255) / 256;
    hipLaunchKernelGGL(quantize_q8_1_tiled_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, n_rows, k, tiled, canon,
                       zero, nzero);
    return hipGetLastError();
}

hipError_t launch_relayout_q8_1_tiled(const uint8_t *xq, int64_t n_rows, int64_t k, uint8_t *tiled, hipStream_t s,
                                      int32_t *zero, int64_t nzero) {
    const int64_t threads = n_rows * (k / 32) * 4;
    if (threads == 0 && nzero <= 0) return hipSuccess;
    const int64_t blocks = (std::max<int64_t>(threads, nzero) + 255) / 256;
    hipLaunchKernelGGL(relayout_q8_1_tiled_kernel, dim3((unsigned)blocks), dim3(256), 0, s, xq, n_rows, k, tiled,
                       zero, nzero);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

}  // namespace qmm
