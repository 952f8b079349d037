// Measurement probes (include/qmm_probe.h): the streaming-read and int8 matrix-core ceilings the
// benchmark reports its kernels against.  Not used by the product path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qmm_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

// One 16-byte streaming load per thread per pass of the grid stride; the loads of a pass are
// independent, so every wave has its whole share in flight at once.
__global__ void probe_read_kernel(const u32x4 *__restrict__ p, uint64_t n16, uint32_t *__restrict__ sink) {
    uint32_t acc = 0;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u && threadIdx.x == 0) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void probe_mfma_i8_kernel(int32_t iters, int32_t *__restrict__ sink) {
    i32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const i32x4 a = {(int)threadIdx.x, 1, 2, 3}, b = {5, (int)threadIdx.x, 7, 8};
    for (int32_t i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c3, 0, 0, 0);
    }
    int32_t s = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c0[e] ^ c1[e] ^ c2[e] ^ c3[e];
    if (s == 0x7FFFFFFF) sink[0] = s;
}

}  // namespace

extern "C" int qmm_probe_read(const void *buf, uint64_t bytes, uint32_t *sink, int32_t wgs, int32_t threads,
                              void *stream) {
    if (!buf || !sink || bytes == 0 || (bytes & 15) || (((uintptr_t)buf) & 15)) return -1;
    if (wgs <= 0 || threads < 64 || threads > 1024 || (threads & 63)) return -1;
    hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)wgs), dim3((unsigned)threads), 0, (hipStream_t)stream,
                       (const u32x4 *)buf, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int qmm_probe_mfma_i8(int32_t iters, int32_t wgs, int32_t *sink, void *stream) {
    if (!sink || iters <= 0 || wgs <= 0) return -1;
    hipLaunchKernelGGL(probe_mfma_i8_kernel, dim3((unsigned)wgs), dim3(256), 0, (hipStream_t)stream, iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
