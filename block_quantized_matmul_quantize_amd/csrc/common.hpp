// Shared device/host definitions for libqmm (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace qmm {

constexpr int kQ4_0 = 2;
constexpr int kQ8_0 = 8;
constexpr int kQ3_K = 11;
constexpr int kQ4_K = 12;
constexpr int kQ5_K = 13;
constexpr int kQ6_K = 14;
constexpr int kIQ4_XS = 23;

// GGUF block geometry.
template <int T> struct Fmt;
template <> struct Fmt<kQ4_K> { static constexpr int QK = 256, BYTES = 144; };
template <> struct Fmt<kQ5_K> { static constexpr int QK = 256, BYTES = 176; };
template <> struct Fmt<kQ6_K> { static constexpr int QK = 256, BYTES = 210; };
template <> struct Fmt<kQ8_0> { static constexpr int QK = 32, BYTES = 34; };
template <> struct Fmt<kQ4_0> { static constexpr int QK = 32, BYTES = 18; };
template <> struct Fmt<kQ3_K> { static constexpr int QK = 256, BYTES = 110; };
template <> struct Fmt<kIQ4_XS> { static constexpr int QK = 256, BYTES = 136; };

// Types whose scale changes every 16 values (Q6_K, Q3_K): their integer dots are per 16-value
// sub-block.
template <int T> constexpr bool kSub16 = T == kQ6_K || T == kQ3_K;

// IQ4_XS: the format's 16-entry non-linear codebook (GP100 patch page, "How" step 3, names the
// codebook; the values are GGUF's table), as int8 bytes in four dwords for a v_perm lookup.
constexpr int8_t kIq4Codebook[16] = {-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113};
constexpr uint32_t iq4_table_dword(int i) {
    return (uint32_t)(uint8_t)kIq4Codebook[4 * i] | ((uint32_t)(uint8_t)kIq4Codebook[4 * i + 1] << 8) |
           ((uint32_t)(uint8_t)kIq4Codebook[4 * i + 2] << 16) | ((uint32_t)(uint8_t)kIq4Codebook[4 * i + 3] << 24);
}
// Four 4-bit indices (one per byte, values 0..15) -> their four int8 codebook entries: v_perm picks
// entries 0-7 and 8-15 by the low three bits, bit 3 chooses between the two.
__device__ __forceinline__ uint32_t iq4_lookup4(uint32_t idx) {
    const uint32_t sel = idx & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(iq4_table_dword(1), iq4_table_dword(0), sel);
    const uint32_t hi = __builtin_amdgcn_perm(iq4_table_dword(3), iq4_table_dword(2), sel);
    const uint32_t mask = ((idx >> 3) & 0x01010101u) * 0xFFu;
    return (hi & mask) | (lo & ~mask);
}

constexpr int kQ8_1Bytes = 36;       // {fp16 d, fp16 s, int8 q[32]}
constexpr int kSuper = 256;          // K values per planning step (one K-quant super-block)

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x32 __attribute__((ext_vector_type(32)));
// 16-byte vector with only 2-byte alignment guaranteed: Q6_K (210 B) and Q8_0 (34 B) blocks
// and the q8_1 code arrays sit at 2- or 4-byte offsets.  gfx950 global loads accept these.
typedef u32x4 __attribute__((aligned(2))) u32x4_a2;
typedef uint32_t __attribute__((aligned(2))) u32_a2;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef u32x2 __attribute__((aligned(4))) u32x2_a4;   // 8 bytes at a 4-byte offset (q8_1 codes)

__device__ __forceinline__ u32x4 ld16(const uint8_t *p) { return *(const u32x4_a2 *)p; }
__device__ __forceinline__ uint32_t ld4(const uint8_t *p) { return *(const u32_a2 *)p; }
__device__ __forceinline__ uint16_t ld2(const uint8_t *p) { return *(const uint16_t *)p; }

__device__ __forceinline__ float h2f(uint16_t bits) {
    return __half2float(__ushort_as_half(bits));
}

// MFMA wrappers.  16x16x64: A lane l holds row l%16, B lane l column l%16, each 16 int8 of the
// K slots owned by lane group l/16; C lane l holds C[4*(l/16)+e][l%16], e = 0..3.
__device__ __forceinline__ i32x4 mfma16x16x64(u32x4 a, u32x4 b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8((i32x4)a, (i32x4)b, c, 0, 0, 0);
}
// 32x32x32: A lane l holds row l%32, B lane l column l%32, 16 int8 each of the K slots owned by
// lane group l/32; C lane l holds C[8*(e/4) + 4*(l/32) + e%4][l%32], e = 0..15.
__device__ __forceinline__ i32x16 mfma32x32x32(u32x4 a, u32x4 b, i32x16 c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8((i32x4)a, (i32x4)b, c, 0, 0, 0);
}

// Per-byte x - 32 for bytes in [0, 63] (no borrow crosses a byte: each byte first gets its top
// bit set, and the top bit is flipped back afterwards).
__device__ __forceinline__ uint32_t sub32_bytes(uint32_t x) {
    return ((x | 0x80808080u) - 0x20202020u) ^ 0x80808080u;
}

// Workgroup index -> work index such that each XCD (workgroups are dealt round-robin over the
// 8 XCDs) gets one contiguous range of work, keeping neighbouring tiles in one L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t n) {
    const int64_t q = n / 8, r = n % 8;
    const int64_t x = b % 8, i = b / 8;
    return x * q + (x < r ? x : r) + i;
}

}  // namespace qmm
