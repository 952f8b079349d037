// fp16-activation matrix-vector mode (GP100 MMVQ page, "How": activations converted once to fp16
// with a power-of-two prescale per 32 values so that max|y| < 2^15, exact fp32 block sums for the
// min / offset terms; the page's accuracy paragraph: about ten times lower error than q8_1).
//
// Encoder: one lane per value, 32 lanes per block.  The block's max |x| (lane exchanges) gives the
// exponent e = 15 - p with max|x| in [2^(p-1), 2^p), read off the fp32 bits (exact for
// subnormals too); y = fp16(x * 2^e) with one round to nearest even; the block sum of the y in
// fp32.
//
// Product (below): lane l of a row's wave takes the row's 32-value blocks l, l+64, ...  Each
// block's weights are an affine map of small unsigned integer codes u: value = A*u + B (Q4_K /
// Q5_K: A = d*sc, B = -dmin*m; Q8_0: u = q + 128, B = -128 d; Q4_0: B = -8 d; Q6_K per 16 values:
// u = 6-bit code, B = -32 A).  The codes become exact fp16 integers (bit pattern 0x6400 | u is
// 1024 + u; minus 1024), v_dot2_f32_f16 sums u*y in fp32, and the block adds
// 2^-e * (A * sum(u*y) + B * sum(y)).  The columns (1..8) reuse each lane's decoded codes; the
// 64 lanes of a row are summed with lane exchanges in a fixed order.
#include "common.hpp"
#include "launch.hpp"

namespace qmm {
namespace {

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int f16act_exp(float amax) {
    const uint32_t u = __float_as_uint(amax);
    const int E = (int)(u >> 23);
    if (u == 0u) return 0;
    const int p = E > 0 ? E - 126 : (32 - __clz((int)u)) - 149;
    return 15 - p;
}

__global__ __launch_bounds__(256) void f16act_encode_kernel(const float *__restrict__ x, int64_t total,
                                                            uint16_t *__restrict__ y, int32_t *__restrict__ e,
                                                            float *__restrict__ bsum) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;   // total % 32 == 0: a block's 32 lanes leave together
    const float v = x[t];
    float amax = fabsf(v);
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const int eb = f16act_exp(amax);
    const _Float16 h = (_Float16)ldexpf(v, eb);
    y[t] = __builtin_bit_cast(uint16_t, h);
    float s = (float)h;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) s += __shfl_xor(s, o);
    if ((t & 31) == 0) {
        e[t >> 5] = eb;
        bsum[t >> 5] = s;
    }
}

// Four bytes -> two half2 of exact integers (bytes 0,1 and 2,3).
__device__ __forceinline__ void bytes_to_h2(uint32_t w, h2v &lo, h2v &hi) {
    const uint32_t a = (w & 0xFFu) | ((w & 0xFF00u) << 8) | 0x64006400u;
    const uint32_t b = ((w >> 16) & 0xFFu) | ((w >> 8) & 0x00FF0000u) | 0x64006400u;
    const h2v k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    lo = __builtin_bit_cast(h2v, a) - k1024;
    hi = __builtin_bit_cast(h2v, b) - k1024;
}

__device__ __forceinline__ float dot16(const h2v *u, const u32x4 *yv, int first) {
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const u32x4 q = yv[(first + i) >> 2];
        const uint32_t wv = ((first + i) & 3) == 0 ? q.x : ((first + i) & 3) == 1 ? q.y : ((first + i) & 3) == 2 ? q.z : q.w;
        p = __builtin_amdgcn_fdot2(u[first + i], __builtin_bit_cast(h2v, wv), p, false);
    }
    return p;
}

// Decoded block: 16 half2 codes (values 2i, 2i+1 in u[i]) and the affine terms of each 16-value half.
struct Blk {
    h2v u[16];
    float A0, B0, A1, B1;
};

template <int T>
__device__ __forceinline__ void decode(const uint8_t *row, int jg, Blk &o) {
    uint32_t c[8];   // 32 code bytes, value i in byte i
    if constexpr (T == kQ4_K || T == kQ5_K) {
        constexpr int SB = T == kQ4_K ? 144 : 176, QS = T == kQ4_K ? 16 : 48;
        const uint8_t *sb = row + (jg >> 3) * SB;
        const int j = jg & 7;
        const u32x4 h = *(const u32x4 *)sb;
        const float d = h2f((uint16_t)(h.x & 0xFFFF)), dmin = h2f((uint16_t)(h.x >> 16));
        const uint32_t s03 = h.y, s47 = h.z, s811 = h.w;   // scales[0..3], [4..7], [8..11]
        auto byte = [](uint32_t w, int i) { return (int)((w >> (8 * i)) & 0xFF); };
        int sc, m;
        if (j < 4) {
            sc = byte(s03, j) & 63;
            m = byte(s47, j) & 63;
        } else {
            sc = (byte(s811, j - 4) & 15) | ((byte(s03, j - 4) >> 6) << 4);
            m = (byte(s811, j - 4) >> 4) | ((byte(s47, j - 4) >> 6) << 4);
        }
        const u32x4 q0 = *(const u32x4 *)(sb + QS + 32 * (j >> 1));
        const u32x4 q1 = *(const u32x4 *)(sb + QS + 32 * (j >> 1) + 16);
        const uint32_t qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        const int sh = 4 * (j & 1);
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = (qq[i] >> sh) & 0x0F0F0F0Fu;
        if constexpr (T == kQ5_K) {
            const u32x4 g0 = *(const u32x4 *)(sb + 16), g1 = *(const u32x4 *)(sb + 32);
            const uint32_t gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] |= ((gg[i] >> j) & 0x01010101u) << 4;
        }
        o.A0 = o.A1 = d * (float)sc;
        o.B0 = o.B1 = -dmin * (float)m;
    } else if constexpr (T == kQ6_K) {
        const uint8_t *sb = row + (jg >> 3) * 210;
        const int j = jg & 7, h = j >> 2, g = j & 3;
        const u32x4 l0 = *(const u32x4_a2 *)(sb + 64 * h + 32 * (g & 1));
        const u32x4 l1 = *(const u32x4_a2 *)(sb + 64 * h + 32 * (g & 1) + 16);
        const u32x4 h0 = *(const u32x4_a2 *)(sb + 128 + 32 * h);
        const u32x4 h1 = *(const u32x4_a2 *)(sb + 128 + 32 * h + 16);
        const uint32_t ll[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        const uint32_t hh[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
        const int lsh = g < 2 ? 0 : 4;
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = ((ll[i] >> lsh) & 0x0F0F0F0Fu) | (((hh[i] >> (2 * g)) & 0x03030303u) << 4);
        const float d = h2f(*(const uint16_t *)(sb + 208));
        const int8_t *scl = (const int8_t *)(sb + 192);
        o.A0 = d * (float)scl[2 * j];
        o.A1 = d * (float)scl[2 * j + 1];
        o.B0 = -32.f * o.A0;
        o.B1 = -32.f * o.A1;
    } else if constexpr (T == kQ8_0) {
        const uint8_t *b = row + jg * 34;
        const float d = h2f(*(const uint16_t *)b);
        const u32x4 q0 = *(const u32x4_a2 *)(b + 2), q1 = *(const u32x4_a2 *)(b + 18);
        const uint32_t qq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = qq[i] ^ 0x80808080u;   // q + 128
        o.A0 = o.A1 = d;
        o.B0 = o.B1 = -128.f * d;
    } else {   // Q4_0
        const uint8_t *b = row + jg * 18;
        const float d = h2f(*(const uint16_t *)b);
        const u32x4 q = *(const u32x4_a2 *)(b + 2);
        const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c[i] = qq[i] & 0x0F0F0F0Fu;
            c[4 + i] = (qq[i] >> 4) & 0x0F0F0F0Fu;
        }
        o.A0 = o.A1 = d;
        o.B0 = o.B1 = -8.f * d;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) bytes_to_h2(c[i], o.u[2 * i], o.u[2 * i + 1]);
}

// Product: a workgroup of 16 waves (Q6_K: 8, whose two scales per block need more registers than
// 16 waves per compute unit leave) owns one weight row per wave and walks K in chunks of 64
// blocks (2048 values).  Each chunk's fp16 activations of all columns, with their exponents and
// block sums, are parked in LDS once per workgroup (64 + 16 bytes per block and column, so the 16
// lanes of a row read group hit distinct banks) and serve the workgroup's 16 rows: the columns are
// read from L2 once per 16 rows instead of once per row.  Within a chunk lane l takes block l of
// every row of its wave, so a lane still accumulates its blocks l, l + 64, ... in order and the
// 64 lanes of a row are summed with the same lane exchanges.
template <int T> constexpr int kF16Rows = T == kQ6_K ? 8 : 16;   // rows (= waves) per workgroup
constexpr int kF16RowsPerWave = 1;
constexpr int kF16Chunk = 64;          // 32-value blocks per K chunk
constexpr int kF16YStride = 80;        // LDS bytes per (column, block): 32 fp16 + 16 pad

template <int T>
__global__ __launch_bounds__(64 * kF16Rows<T>) void mmvq_f16act_kernel(const uint8_t *__restrict__ w, int64_t rows,
                                                                  int64_t row_bytes, int64_t k,
                                                                  const uint16_t *__restrict__ y16,
                                                                  const int32_t *__restrict__ e,
                                                                  const float *__restrict__ bsum, int n,
                                                                  float *__restrict__ out) {
    __shared__ __align__(16) uint8_t ys[8 * kF16Chunk * kF16YStride];
    __shared__ int32_t es[8 * kF16Chunk];
    __shared__ float bs[8 * kF16Chunk];
    constexpr int kF16Threads = 64 * kF16Rows<T>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t rbase = (int64_t)blockIdx.x * kF16Rows<T> + wave * kF16RowsPerWave;
    const int nb = (int)(k >> 5);
    float acc[kF16RowsPerWave][8];
#pragma unroll
    for (int rr = 0; rr < kF16RowsPerWave; ++rr)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[rr][c] = 0.f;

    for (int jb0 = 0; jb0 < nb; jb0 += kF16Chunk) {
        const int cnt = nb - jb0 < kF16Chunk ? nb - jb0 : kF16Chunk;
        __syncthreads();   // the previous chunk's LDS reads are done
        // 16-byte pieces (column c, block b, quarter q) of the chunk
        for (int p = tid; p < n * cnt * 4; p += kF16Threads) {
            const int c = p / (cnt * 4), rem = p - c * cnt * 4, b = rem >> 2, q = rem & 3;
            *(u32x4 *)(ys + (c * kF16Chunk + b) * kF16YStride + 16 * q) =
                *(const u32x4 *)(y16 + (int64_t)c * k + (int64_t)(jb0 + b) * 32 + 8 * q);
        }
        for (int p = tid; p < n * cnt; p += kF16Threads) {
            const int c = p / cnt, b = p - c * cnt;
            es[c * kF16Chunk + b] = e[(int64_t)c * nb + jb0 + b];
            bs[c * kF16Chunk + b] = bsum[(int64_t)c * nb + jb0 + b];
        }
        __syncthreads();
        if (lane >= cnt) continue;   // the last chunk may be partial (no barrier until the next chunk)
        const int jg = jb0 + lane;
#pragma unroll
        for (int rr = 0; rr < kF16RowsPerWave; ++rr) {
            const int64_t r = rbase + rr;
            if (r >= rows) break;   // wave-uniform
            Blk b;
            decode<T>(w + r * row_bytes, jg, b);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                if (c >= n) break;
                const uint8_t *yp = ys + (c * kF16Chunk + lane) * kF16YStride;
                const u32x4 yy[4] = {*(const u32x4 *)yp, *(const u32x4 *)(yp + 16), *(const u32x4 *)(yp + 32),
                                     *(const u32x4 *)(yp + 48)};
                const int eb = es[c * kF16Chunk + lane];
                float t;
                if constexpr (T == kQ6_K) {
                    // the two 16-value halves' sums of y (the offset term of each half's scale)
                    const h2v one = {(_Float16)1.0f, (_Float16)1.0f};
                    const h2v ones[16] = {one, one, one, one, one, one, one, one, one, one, one, one, one, one, one, one};
                    const float s0 = dot16(ones, yy, 0), s1 = dot16(ones, yy, 8);
                    t = b.A0 * dot16(b.u, yy, 0) + b.B0 * s0 + (b.A1 * dot16(b.u, yy, 8) + b.B1 * s1);
                } else {
                    const float pp = dot16(b.u, yy, 0) + dot16(b.u, yy, 8);
                    t = b.A0 * pp + b.B0 * bs[c * kF16Chunk + lane];
                }
                acc[rr][c] += ldexpf(t, -eb);
            }
        }
    }
#pragma unroll
    for (int rr = 0; rr < kF16RowsPerWave; ++rr) {
        const int64_t r = rbase + rr;
        if (r >= rows) break;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            if (c >= n) break;
            float v = acc[rr][c];
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
            if (lane == 0) out[(int64_t)c * rows + r] = v;
        }
    }
}

template <int T>
hipError_t launch_t(const uint8_t *w, int64_t rows, int64_t k, const uint16_t *y16, const int32_t *e,
                    const float *bsum, int64_t n, float *out, hipStream_t s) {
    const int64_t row_bytes = k / Fmt<T>::QK * Fmt<T>::BYTES;
    hipLaunchKernelGGL(mmvq_f16act_kernel<T>, dim3((unsigned)((rows + kF16Rows<T> - 1) / kF16Rows<T>)),
                       dim3(64 * kF16Rows<T>), 0, s, w,
                       rows, row_bytes, k, y16, e, bsum, (int)n, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_f16act_encode(const float *x, int64_t n, int64_t k, uint16_t *y16, int32_t *e, float *bsum,
                                hipStream_t s) {
    const int64_t total = n * k;
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL(f16act_encode_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, x, total, y16, e,
                       bsum);
    return hipGetLastError();
}

hipError_t launch_mmvq_f16act(int type, const uint8_t *w, int64_t rows, int64_t k, const uint16_t *y16,
                              const int32_t *e, const float *bsum, int64_t n, float *out, hipStream_t s) {
    switch (type) {
        case kQ4_K: return launch_t<kQ4_K>(w, rows, k, y16, e, bsum, n, out, s);
        case kQ5_K: return launch_t<kQ5_K>(w, rows, k, y16, e, bsum, n, out, s);
        case kQ6_K: return launch_t<kQ6_K>(w, rows, k, y16, e, bsum, n, out, s);
        case kQ8_0: return launch_t<kQ8_0>(w, rows, k, y16, e, bsum, n, out, s);
        case kQ4_0: return launch_t<kQ4_0>(w, rows, k, y16, e, bsum, n, out, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
