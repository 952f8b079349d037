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

// Lane exchange within aligned groups of 4 lanes by DPP (a modifier on a vector ALU operation,
// no LDS round trip): quad_perm [1,0,3,2] (xor 1), quad_perm [2,3,0,1] (xor 2).  After the two
// steps every lane of the quad holds the max / sum of all four.
template <int CTRL> __device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL> __device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E;

// q = round-half-away(RN(x / d32)).  Fast path: x * rcp(d32) (hardware reciprocal, 1 ulp) is
// within E = 2^-15 + 2^-17 of x / d32 for |x| <= amax, so rounding it to the nearest integer gives
// the exact answer unless the two lie on opposite sides of a half-integer (or x / d32 is one:
// ties to even and ties away from zero differ only there), and then x * rcp(d32) is within E of
// that half-integer.  One fma with 1.5 * 2^23 rounds x * rcp(d32) to an integer whose low byte is
// the int8 code; a second gives the residual e = x * rcp(d32) - q, and |e| > 0.5 - 2^-14 (> 0.5 -
// E) sends the lane to the IEEE division, as do blocks whose d32 is outside [2^-100, 2^100] (or
// not finite), so the codes are always those of the plain definition.
__device__ __forceinline__ int q81_round_div(float x, float d32) { return (int)roundf(x / d32); }

__device__ __forceinline__ uint32_t pack4(int q0, int q1, int q2, int q3) {
    const uint32_t lo = __builtin_amdgcn_perm((uint32_t)q1, (uint32_t)q0, 0x0c0c0400u);   // q0.b0, q1.b0
    const uint32_t hi = __builtin_amdgcn_perm((uint32_t)q3, (uint32_t)q2, 0x04000c0cu);   // q2.b0, q3.b0 in bytes 2, 3
    return lo | hi;
}

// One block of 32 values held by 4 consecutive lanes (lane l of the group owns values 8l..8l+7
// as a and b, the group starts at a lane index divisible by 4); max and sum reduce over the
// group, so all 4 lanes must call it together.
struct Q81Lane4 {
    uint32_t c0, c1;   // this lane's 8 codes, little-endian bytes
    uint32_t ds;       // fp16 d | fp16 s << 16 of the whole block (same on all 4 lanes)
};

__device__ __forceinline__ Q81Lane4 quantize_q8_1_lane4(float4 a, float4 b) {
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    // max |v| over the lane (three v_max3 with |.| operand modifiers), then over the quad with the
    // DPP exchange as an operand modifier (finite inputs: no NaN canonicalisation is needed)
    float m0, m1, amax;
    asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(m0) : "v"(v[0]), "v"(v[1]), "v"(v[2]));
    asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(m1) : "v"(v[3]), "v"(v[4]), "v"(v[5]));
    asm("v_max_f32 %0, %1, %2" : "=v"(amax) : "v"(m0), "v"(m1));
    asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(amax) : "v"(v[6]), "v"(v[7]), "v"(amax));
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" : "=v"(m0) : "v"(amax));
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf" : "=v"(amax) : "v"(m0));
    // d32 = amax / 127 by one multiply and an fma correction: with c = RN(1/127), the corrected
    // quotient equals the IEEE quotient for every amax whose quotient lies in [2^-101, 2^101]
    // (checked exhaustively over all such floats); outside that range the division below runs.
    const float c127 = 1.0f / 127.0f;
    const float q1 = amax * c127;
    float d32 = fmaf(fmaf(-q1, 127.0f, amax), c127, q1);
    uint32_t c0 = 0u, c1 = 0u;
    if (amax != 0.0f) {
        bool slow = !(d32 >= 0x1p-100f && d32 <= 0x1p100f);
        if (!slow) {
            const float r = __builtin_amdgcn_rcpf(d32);
            constexpr float kRound = 12582912.0f;   // 1.5 * 2^23: sums in [2^23, 2^24) are integers
            int q[8];
            float dev = 0.0f;   // largest distance of a quotient from its nearest integer
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float m = fmaf(v[i], r, kRound);        // 1.5 * 2^23 + q, |q| <= 127: exact
                const float e = fmaf(v[i], r, kRound - m);    // x * rcp(d32) - q, one rounding
                dev = fmaxf(dev, fabsf(e));
                q[i] = __float_as_int(m);                     // low byte: q (two's complement)
            }
            slow = dev > 0.5f - 0x1p-14f;
            c0 = pack4(q[0], q[1], q[2], q[3]);
            c1 = pack4(q[4], q[5], q[6], q[7]);
        }
        if (slow) {
            d32 = amax / 127.0f;
            c0 = pack4(q81_round_div(v[0], d32), q81_round_div(v[1], d32), q81_round_div(v[2], d32),
                       q81_round_div(v[3], d32));
            c1 = pack4(q81_round_div(v[4], d32), q81_round_div(v[5], d32), q81_round_div(v[6], d32),
                       q81_round_div(v[7], d32));
        }
    } else {
        d32 = 0.0f;
    }
    // sum of the 8 codes by two byte dot products with ones, then over the 4 lanes
    int sum = __builtin_amdgcn_sdot4((int)c1, 0x01010101, __builtin_amdgcn_sdot4((int)c0, 0x01010101, 0, false), false);
    sum += dpp_i<kDppXor1>(sum);
    sum += dpp_i<kDppXor2>(sum);
    Q81Lane4 out;
    out.c0 = c0;
    out.c1 = c1;
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
