// q8_1 activation quantization (MMQ page, introduction and "dp4a path Q4_K" section: 32 int8
// codes per block with the half2 (d, s), s = d * sum(q)).
//
// Readings where the page is silent: d32 = amax / 127 (fp32 IEEE divide), q = round half away
// from zero of x / d32 (divide by the unrounded d32), d = fp16(d32), s = fp16(d32 * sum(q));
// an all-zero block yields d = s = 0 and q = 0.  Device division and roundf are the correctly
// rounded IEEE operations (no fast-math), so the bytes match a plain CPU implementation.
//
// One block of 32 values is handled by 8 consecutive lanes, each owning 4 values (one 16-byte
// load, one 4-byte store of codes); max and sum reduce over the 8 lanes with xor shuffles.
#include "common.hpp"
#include "launch.hpp"

namespace qmm {

__global__ __launch_bounds__(256) void quantize_q8_1_kernel(const float *__restrict__ x, int64_t n_rows,
                                                            int64_t k, uint8_t *__restrict__ y) {
    const int64_t nb = k / 32;
    const int64_t total = n_rows * nb;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t blk = gid >> 3;
    const int sub = (int)(gid & 7);
    const bool live = blk < total;   // the whole 8-lane group shares this predicate
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    int64_t row = 0, b = 0;
    if (live) {
        row = blk / nb;
        b = blk - row * nb;
        v = *(const float4 *)(x + row * k + b * 32 + 4 * sub);
    }
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
    const float d32 = amax / 127.0f;
    int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    if (amax != 0.0f) {
        q0 = (int)roundf(v.x / d32);
        q1 = (int)roundf(v.y / d32);
        q2 = (int)roundf(v.z / d32);
        q3 = (int)roundf(v.w / d32);
    }
    int sum = q0 + q1 + q2 + q3;
    sum += __shfl_xor(sum, 1, 8);
    sum += __shfl_xor(sum, 2, 8);
    sum += __shfl_xor(sum, 4, 8);
    if (!live) return;
    uint8_t *yb = y + blk * kQ8_1Bytes;
    const uint32_t packed = (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) |
                            ((uint32_t)(q2 & 0xFF) << 16) | ((uint32_t)(q3 & 0xFF) << 24);
    *(uint32_t *)(yb + 4 + 4 * sub) = packed;
    if (sub == 0) {
        const __half hd = __float2half_rn(d32);
        // s is the fp32 product d32 * sum(q) rounded to fp16.  The empty asm pins the fp32 product
        // in a register so it cannot be fused into a single-rounding multiply-to-fp16
        // (v_fma_mixlo_f16), which differs from the double rounding in the last bit.
        float s32 = d32 * (float)sum;
        asm volatile("" : "+v"(s32));
        const __half hs = __float2half_rn(s32);
        *(uint32_t *)yb = (uint32_t)__half_as_ushort(hd) | ((uint32_t)__half_as_ushort(hs) << 16);
    }
}

// Plain fill kernel (used instead of a memset so that the call sequence stays capturable).
__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *__restrict__ p, int64_t n, uint32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = i; j < n; j += stride) p[j] = v;
}

hipError_t launch_quantize_q8_1(const float *x, int64_t n_rows, int64_t k, uint8_t *y, hipStream_t s) {
    const int64_t threads = n_rows * (k / 32) * 8;
    if (threads == 0) return hipSuccess;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(quantize_q8_1_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, n_rows, k, y);
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
