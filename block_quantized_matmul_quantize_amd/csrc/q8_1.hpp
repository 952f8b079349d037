// q8_1 block quantization shared by the standalone quantize kernel and the fused matrix-vector
// kernel (MMQ page, introduction and "dp4a path Q4_K" section: 32 int8 codes per block with the
// half2 (d, s), s = d * sum(q)).
//
// Readings where the page is silent: d32 = amax / 127 (fp32 IEEE divide), q = round half away
// from zero of x / d32 (divide by the unrounded d32), d = fp16(d32), s = fp16(d32 * sum(q));
// an all-zero block yields d = s = 0 and q = 0.  Device division and roundf are the correctly
// rounded IEEE operations (no fast-math), so the bytes match a plain CPU implementation.
#pragma once
#include "common.hpp"

namespace qmm {

struct Q81Lane {
    uint32_t codes;   // this lane's 4 codes, little-endian bytes
    uint32_t ds;      // fp16 d | fp16 s << 16 of the whole block (same on all 8 lanes)
};

// Lane exchange within aligned groups of 8 lanes by DPP (a modifier on a vector ALU operation,
// no LDS round trip): quad_perm [1,0,3,2] (xor 1), quad_perm [2,3,0,1] (xor 2), row_half_mirror
// (lane i of the group <-> lane 7-i, which pairs the two quads).  After the three steps every
// lane of the group holds the max / sum of all eight.
template <int CTRL> __device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141;

// One block of 32 values held by 8 consecutive lanes (lane l of the group owns values 4l..4l+3,
// the group starts at a lane index divisible by 8); max and sum reduce over the group, so all 8
// lanes must call it together.
//
// q = round-half-away(RN(x / d32)).  Fast path: t = x * rcp(d32) (hardware reciprocal, 1 ulp)
// is within 2^-15 + 2^-17 of x / d32 for |x| <= amax, and q = trunc(t + copysign(0.5, t)) equals
// the exact answer unless x / d32 lies within a few ulps of a half-integer -- which the
// |fract(|t|) - 0.5| < 2^-13 test catches (it also covers the rounding of t + 0.5).  Those values,
// and blocks whose d32 is outside [2^-100, 2^100] (or not finite), take the IEEE division, so the
// codes are always those of the plain definition.
__device__ __forceinline__ int q81_round_div(float x, float d32) { return (int)roundf(x / d32); }

__device__ __forceinline__ Q81Lane quantize_q8_1_lane(float4 v) {
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = fmaxf(amax, dpp_f<kDppXor1>(amax));
    amax = fmaxf(amax, dpp_f<kDppXor2>(amax));
    amax = fmaxf(amax, dpp_f<kDppHalfMirror>(amax));
    const float d32 = amax / 127.0f;
    int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    if (amax != 0.0f) {
        bool slow = !(d32 >= 0x1p-100f && d32 <= 0x1p100f);
        if (!slow) {
            const float r = __builtin_amdgcn_rcpf(d32);
            const float t0 = v.x * r, t1 = v.y * r, t2 = v.z * r, t3 = v.w * r;
            const float m = 0x1p-13f;
            slow = fabsf(__builtin_amdgcn_fractf(fabsf(t0)) - 0.5f) < m ||
                   fabsf(__builtin_amdgcn_fractf(fabsf(t1)) - 0.5f) < m ||
                   fabsf(__builtin_amdgcn_fractf(fabsf(t2)) - 0.5f) < m ||
                   fabsf(__builtin_amdgcn_fractf(fabsf(t3)) - 0.5f) < m;
            q0 = (int)(t0 + copysignf(0.5f, t0));
            q1 = (int)(t1 + copysignf(0.5f, t1));
            q2 = (int)(t2 + copysignf(0.5f, t2));
            q3 = (int)(t3 + copysignf(0.5f, t3));
        }
        if (slow) {
            q0 = q81_round_div(v.x, d32);
            q1 = q81_round_div(v.y, d32);
            q2 = q81_round_div(v.z, d32);
            q3 = q81_round_div(v.w, d32);
        }
    }
    int sum = q0 + q1 + q2 + q3;
    sum += dpp_i<kDppXor1>(sum);
    sum += dpp_i<kDppXor2>(sum);
    sum += dpp_i<kDppHalfMirror>(sum);
    Q81Lane out;
    out.codes = (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) | ((uint32_t)(q2 & 0xFF) << 16) |
                ((uint32_t)(q3 & 0xFF) << 24);
    const __half hd = __float2half_rn(d32);
    // s is the fp32 product d32 * sum(q) rounded to fp16.  The empty asm pins the fp32 product in a
    // register so it cannot be fused into a single-rounding multiply-to-fp16 (v_fma_mixlo_f16),
    // which differs from the double rounding in the last bit.
    float s32 = d32 * (float)sum;
    asm volatile("" : "+v"(s32));
    const __half hs = __float2half_rn(s32);
    out.ds = (uint32_t)__half_as_ushort(hd) | ((uint32_t)__half_as_ushort(hs) << 16);
    return out;
}

}  // namespace qmm
