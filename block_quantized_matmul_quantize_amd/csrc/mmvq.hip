// Matrix-vector product for 1..8 activation columns (the MMVQ regime of the MMQ page: "shape
// criteria" and the MMVQ-vs-MMQ table -- decode is bound by how fast the weights stream, every
// weight byte is read once and serves all columns; GP100 patch page, "Coverage": multi-column
// kernels unpack each weight once and reuse it for every column).
//
// CDNA4 design.  A workgroup owns 16 weight rows; its waves split K (one 256-value step per wave
// per iteration, the next step's weight and code loads are issued before the current step's
// math).  Each 64-value slice of K is one v_mfma_i32_16x16x64_i8 whose B operand is 16 weight
// rows and whose A operand is block-diagonal over activation (column, sub-block) pairs, so every
// one of the 16 result columns is useful:
//   Q4_K, Q8_0: A row m = (column m%8, sub-block m/8); K slots 0-31 hold sub-block 2p, slots
//               32-63 sub-block 2p+1; the off-diagonal halves are zero.  -> 8 columns.
//   Q6_K:       A row m = (column m%4, 16-value sub-block m/4), four diagonal 16-slot blocks,
//               because Q6_K scales change every 16 values ("Q6_K dot" section).  -> 4 columns
//               per MFMA, two MFMAs for 5..8 columns.
// The int32 result of each lane is then one exact sub-block dot D for one (row, column,
// sub-block), and the fp32 fixup ("dp4a path Q4_K" section) is applied per lane:
//   Q4_K  acc += D * (d*sc) * d_a - (dmin*m) * s_a
//   Q6_K  acc += D * (d*sc) * d_a
//   Q8_0  acc += D * d_w * d_a
// Partial sums over sub-blocks are combined with lane shuffles, then across waves in LDS in a
// fixed order (bitwise reproducible).
#include "common.hpp"
#include "launch.hpp"

namespace qmm {

constexpr int kMvRows = 16;
constexpr int kMvMaxWaves1 = 16;     // one step per wave up to K = 4096
constexpr int kMvMaxWaves2 = 8;      // longer K: 8 waves, two register buffers each
constexpr int kMvMaxBlocks = 1024;   // K <= 32768 (the activation scale table is staged in LDS)

template <int T> struct MvStep;

// ------------------------------------------------------------------------------------------
// Q4_K: one step = one 144-byte super-block per row = 4 MFMAs (sub-block pairs 2p, 2p+1).
// ------------------------------------------------------------------------------------------
template <> struct MvStep<kQ4_K> {
    static constexpr int NCG = 1;
    u32x4 hdr;
    u32x4 q[4];
    u32x4 a[4][1];

    __device__ __forceinline__ void load(const uint8_t *wrow, bool row_ok, int64_t step, int g,
                                         const uint8_t *arow, bool a_ok, int asel) {
        const uint8_t *blk = wrow + step * 144;
        const u32x4 z = {0u, 0u, 0u, 0u};
        hdr = row_ok ? ld16(blk) : z;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            q[p] = row_ok ? ld16(blk + 16 + 32 * p + 16 * (g & 1)) : z;
            a[p][0] = a_ok ? ld16(arow + (step * 8 + 2 * p + asel) * kQ8_1Bytes + 4 + 16 * (g & 1)) : z;
        }
    }

    template <bool DBG>
    __device__ __forceinline__ void compute(int64_t step, int g, const float2 *sTab, float acc[NCG][4],
                                           int32_t *dbg_row, int dbg_ld, int ncols) const {
        const int sel = g >> 1;
        const float d = h2f((uint16_t)(hdr.x & 0xFFFF));
        const float dmin = h2f((uint16_t)(hdr.x >> 16));
        // 6-bit scales/mins of sub-blocks 0..7 as bytes: j<4 in the low 6 bits of bytes j / j+4,
        // j>=4 split over the low/high nibble of byte j+4 and the top bits of bytes j-4 / j.
        uint32_t sc_lo = hdr.y & 0x3F3F3F3Fu;
        uint32_t m_lo = hdr.z & 0x3F3F3F3Fu;
        uint32_t sc_hi = (hdr.w & 0x0F0F0F0Fu) | ((hdr.y >> 2) & 0x30303030u);
        uint32_t m_hi = ((hdr.w >> 4) & 0x0F0F0F0Fu) | ((hdr.z >> 2) & 0x30303030u);
        // this lane's sub-blocks are 2p + sel: shift so that byte 2*(p%2) is the one needed
        sc_lo >>= 8 * sel; m_lo >>= 8 * sel; sc_hi >>= 8 * sel; m_hi >>= 8 * sel;
        const int shift = 4 * sel;   // low nibbles: first sub-block of the pair
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t scw = p < 2 ? sc_lo : sc_hi;
            const uint32_t mw = p < 2 ? m_lo : m_hi;
            const int bsh = 16 * (p & 1);
            const float ws = d * (float)((scw >> bsh) & 0xFF);
            const float wm = dmin * (float)((mw >> bsh) & 0xFF);
            u32x4 b;
            b.x = (q[p].x >> shift) & 0x0F0F0F0Fu;
            b.y = (q[p].y >> shift) & 0x0F0F0F0Fu;
            b.z = (q[p].z >> shift) & 0x0F0F0F0Fu;
            b.w = (q[p].w >> shift) & 0x0F0F0F0Fu;
            const i32x4 zero = {0, 0, 0, 0};
            const i32x4 D = mfma16x16x64(a[p][0], b, zero);
            const int64_t blk = step * 8 + 2 * p + sel;
            if (DBG) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 4 * (g & 1) + e;
                    if (dbg_row && c < ncols) dbg_row[(int64_t)c * dbg_ld + blk] = D[e];
                }
            } else {
                const f32x4 t0 = *(const f32x4 *)(sTab + blk * 8 + 4 * (g & 1));
                const f32x4 t1 = *(const f32x4 *)(sTab + blk * 8 + 4 * (g & 1) + 2);
                acc[0][0] += (float)D[0] * (ws * t0.x) - wm * t0.y;
                acc[0][1] += (float)D[1] * (ws * t0.z) - wm * t0.w;
                acc[0][2] += (float)D[2] * (ws * t1.x) - wm * t1.y;
                acc[0][3] += (float)D[3] * (ws * t1.z) - wm * t1.w;
            }
        }
    }
};

// ------------------------------------------------------------------------------------------
// Q6_K: one step = one 210-byte super-block per row = 4 MFMAs per 4-column group.
// Value v of a super-block: half h = v/128, u = v%128, quarter g = u/32, l = u%32; the low 4 bits
// are nibble (g<2 ? low : high) of ql[64h + 32(g&1) + l], the top 2 bits are bits 2g..2g+1 of
// qh[32h + l], and the code is that 6-bit value minus 32 (the MMQ page's Q6_K load pairs ql word
// txi with qh word 8*(txi/16) + txi%8 shifted by (txi&8)>>2, which this mapping reproduces).
// ------------------------------------------------------------------------------------------
template <> struct MvStep<kQ6_K> {
    static constexpr int NCG = 2;
    u32x4 scv;
    uint32_t dbits;
    u32x4 ql[2], qh[2];     // per 128-value half: ql serves two quarters (low/high nibble)
    u32x4 a[4][2];

    __device__ __forceinline__ void load(const uint8_t *wrow, bool row_ok, int64_t step, int g,
                                         const uint8_t *arow0, const uint8_t *arow1, bool a_ok0, bool a_ok1) {
        const uint8_t *blk = wrow + step * 210;
        const u32x4 z = {0u, 0u, 0u, 0u};
        scv = row_ok ? ld16(blk + 192) : z;
        dbits = row_ok ? (uint32_t)ld2(blk + 208) : 0u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            ql[h] = row_ok ? ld16(blk + 64 * h + 16 * g) : z;
            qh[h] = row_ok ? ld16(blk + 128 + 32 * h + 16 * (g & 1)) : z;
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int64_t off = (step * 8 + 2 * p + (g >> 1)) * kQ8_1Bytes + 4 + 16 * (g & 1);
            a[p][0] = a_ok0 ? ld16(arow0 + off) : z;
            a[p][1] = a_ok1 ? ld16(arow1 + off) : z;
        }
    }

    template <bool DBG>
    __device__ __forceinline__ void compute(int64_t step, int g, const float2 *sTab, float acc[NCG][4],
                                            int32_t *dbg_row, int dbg_ld, int ncols) const {
        const float d = h2f((uint16_t)dbits);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int odd = p & 1;
            const uint32_t scw = p == 0 ? scv.x : p == 1 ? scv.y : p == 2 ? scv.z : scv.w;
            const float ws = d * (float)((int32_t)(scw << (24 - 8 * g)) >> 24);   // scale of 16-value block 4p+g
            const int tsh = 4 * odd + 2 * (g >> 1);
            u32x4 b;
            const u32x4 L = ql[p >> 1], H = qh[p >> 1];
            b.x = sub32_bytes(((L.x >> (4 * odd)) & 0x0F0F0F0Fu) | (((H.x >> tsh) & 0x03030303u) << 4));
            b.y = sub32_bytes(((L.y >> (4 * odd)) & 0x0F0F0F0Fu) | (((H.y >> tsh) & 0x03030303u) << 4));
            b.z = sub32_bytes(((L.z >> (4 * odd)) & 0x0F0F0F0Fu) | (((H.z >> tsh) & 0x03030303u) << 4));
            b.w = sub32_bytes(((L.w >> (4 * odd)) & 0x0F0F0F0Fu) | (((H.w >> tsh) & 0x03030303u) << 4));
            const int64_t blk = step * 8 + 2 * p + (g >> 1);   // q8_1 block of this lane's sub-block
#pragma unroll
            for (int cg = 0; cg < NCG; ++cg) {
                if (cg * 4 >= ncols) break;
                const i32x4 zero = {0, 0, 0, 0};
                const i32x4 D = mfma16x16x64(a[p][cg], b, zero);
                if (DBG) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = 4 * cg + e;
                        if (dbg_row && c < ncols) dbg_row[(int64_t)c * dbg_ld + step * 16 + 4 * p + g] = D[e];
                    }
                } else {
                    const f32x4 t0 = *(const f32x4 *)(sTab + blk * 8 + 4 * cg);
                    const f32x4 t1 = *(const f32x4 *)(sTab + blk * 8 + 4 * cg + 2);
                    acc[cg][0] += (float)D[0] * (ws * t0.x);
                    acc[cg][1] += (float)D[1] * (ws * t0.z);
                    acc[cg][2] += (float)D[2] * (ws * t1.x);
                    acc[cg][3] += (float)D[3] * (ws * t1.z);
                }
            }
        }
    }
};

// ------------------------------------------------------------------------------------------
// Q8_0: one step = 8 blocks of 34 bytes (256 values) = 4 MFMAs; a final partial step masks the
// blocks beyond k/32.
// ------------------------------------------------------------------------------------------
template <> struct MvStep<kQ8_0> {
    static constexpr int NCG = 1;
    uint32_t dbits[4];
    u32x4 q[4];
    u32x4 a[4][1];

    __device__ __forceinline__ void load(const uint8_t *wrow, bool row_ok, int64_t step, int g, int64_t nb,
                                         const uint8_t *arow, bool a_ok, int asel) {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int64_t bw = step * 8 + 2 * p + (g >> 1);    // this lane's weight block
            const bool ok = row_ok && bw < nb;
            const uint8_t *blk = wrow + bw * 34;
            dbits[p] = ok ? (uint32_t)ld2(blk) : 0u;
            q[p] = ok ? ld16(blk + 2 + 16 * (g & 1)) : z;
            const int64_t ba = step * 8 + 2 * p + asel;        // this lane's activation block
            a[p][0] = (a_ok && ba < nb) ? ld16(arow + ba * kQ8_1Bytes + 4 + 16 * (g & 1)) : z;
        }
    }

    template <bool DBG>
    __device__ __forceinline__ void compute(int64_t step, int g, const float2 *sTab, float acc[NCG][4],
                                            int32_t *dbg_row, int dbg_ld, int ncols, int64_t nb) const {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int64_t blk = step * 8 + 2 * p + (g >> 1);
            if (step * 8 + 2 * p >= nb) break;   // wave-uniform
            const i32x4 zero = {0, 0, 0, 0};
            const i32x4 D = mfma16x16x64(a[p][0], q[p], zero);
            if (blk >= nb) continue;
            if (DBG) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 4 * (g & 1) + e;
                    if (dbg_row && c < ncols) dbg_row[(int64_t)c * dbg_ld + blk] = D[e];
                }
            } else {
                const float ws = h2f((uint16_t)dbits[p]);
                const f32x4 t0 = *(const f32x4 *)(sTab + blk * 8 + 4 * (g & 1));
                const f32x4 t1 = *(const f32x4 *)(sTab + blk * 8 + 4 * (g & 1) + 2);
                acc[0][0] += (float)D[0] * (ws * t0.x);
                acc[0][1] += (float)D[1] * (ws * t0.z);
                acc[0][2] += (float)D[2] * (ws * t1.x);
                acc[0][3] += (float)D[3] * (ws * t1.z);
            }
        }
    }
};

// Resolve the workgroup's columns: dense -> column c is activation row c and output row c;
// expert mode -> expert small[blockIdx.y], columns are its (token, slot) pairs.
struct MvCols {
    int ncols;
    int lo;
    const uint8_t *wbase;
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
                                           bool expert) {
    mc.wbase = w;
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
    return true;
}

// NB = 1: every wave owns at most one 256-value step (up to 16 waves), so all of a workgroup's
// weight loads are in flight at once.  NB = 2: 8 waves walk K with two explicitly unrolled
// register buffers, the loads of step s + 2*nwaves issued right after step s is consumed.
template <int T, bool DBG, bool EXPERT, int NB>
__global__ __launch_bounds__(NB == 1 ? 1024 : 512) void mmvq_kernel(
    const uint8_t *__restrict__ w, int64_t rows, int64_t k, const uint8_t *__restrict__ xq, int64_t n,
    float *__restrict__ y, int32_t *__restrict__ dbg, ColMap cm) {
    extern __shared__ __align__(16) uint8_t mv_smem[];
    using S = MvStep<T>;
    constexpr int NCG = S::NCG;

    MvCols mc;
    if (!mv_resolve(mc, w, n, cm, EXPERT)) return;   // workgroup-uniform
    const int ncols = mc.ncols;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int g = lane >> 4;
    const int r16 = lane & 15;
    const int64_t row = (int64_t)blockIdx.x * kMvRows + r16;
    const bool row_ok = row < rows;
    const int64_t nb = k / 32;                         // q8_1 blocks per activation row
    const int64_t row_bytes = (k / Fmt<T>::QK) * Fmt<T>::BYTES;
    const uint8_t *wrow = mc.wbase + (row_ok ? row : 0) * row_bytes;
    const int64_t nsteps = (k + kSuper - 1) / kSuper;
    float2 *sTab = (float2 *)mv_smem;                          // [nb][8] (d, s)
    float *sRed = (float *)(mv_smem + nb * 8 * sizeof(float2)); // [nwaves][128]

    // This lane's A-operand column (one per column group).
    const int m = r16;
    int acol0, acol1, asel;
    if (T == kQ6_K) { acol0 = m & 3; acol1 = 4 + (m & 3); asel = m >> 2; }
    else { acol0 = m & 7; acol1 = 0; asel = m >> 3; }
    const bool a_diag = (T == kQ6_K) ? (g == asel) : ((g >> 1) == asel);
    const bool a_ok0 = a_diag && acol0 < ncols;
    const bool a_ok1 = a_diag && acol1 < ncols;
    const uint8_t *arow0 = xq + (a_ok0 ? mc.arow(acol0) : 0) * nb * kQ8_1Bytes;
    const uint8_t *arow1 = xq + (a_ok1 ? mc.arow(acol1) : 0) * nb * kQ8_1Bytes;

    auto do_load = [&](S &st, int64_t s) {
        if constexpr (T == kQ6_K) st.load(wrow, row_ok, s, g, arow0, arow1, a_ok0, a_ok1);
        else if constexpr (T == kQ8_0) st.load(wrow, row_ok, s, g, nb, arow0, a_ok0, asel);
        else st.load(wrow, row_ok, s, g, arow0, a_ok0, asel);
    };
    // Weight and code loads first: nothing below waits on them until the first compute.
    S b0, b1;
    const int64_t s0 = wave, s1 = wave + nwaves;
    if (s0 < nsteps) do_load(b0, s0);
    if (NB == 2 && s1 < nsteps) do_load(b1, s1);

    // Stage the fp32 (d, s) of the workgroup's columns from their q8_1 blocks: sTab[block][column].
    if (!DBG) {
        const int c = threadIdx.x & 7;
        const uint8_t *xrow = xq + (c < ncols ? mc.arow(c) : 0) * nb * kQ8_1Bytes;
        for (int64_t i = threadIdx.x; i < nb * 8; i += blockDim.x) {
            const int64_t b = i >> 3;     // blockDim.x is a multiple of 8: column c is fixed
            float2 v = make_float2(0.f, 0.f);
            if (c < ncols) {
                const uint32_t ds = *(const uint32_t *)(xrow + b * kQ8_1Bytes);
                v = make_float2(h2f((uint16_t)(ds & 0xFFFF)), h2f((uint16_t)(ds >> 16)));
            }
            sTab[i] = v;
        }
    }

    float acc[NCG][4];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[cg][e] = 0.f;

    int32_t *dbg_row = nullptr;
    int dbg_ld = 0;
    if (DBG && row_ok) {
        const int per = (T == kQ6_K) ? (int)(k / 16) : (int)nb;
        dbg_ld = (int)(rows * per);
        dbg_row = dbg + row * per;
    }
    auto do_compute = [&](const S &st, int64_t s) {
        if constexpr (T == kQ8_0) st.template compute<DBG>(s, g, sTab, acc, dbg_row, dbg_ld, ncols, nb);
        else st.template compute<DBG>(s, g, sTab, acc, dbg_row, dbg_ld, ncols);
    };
    __syncthreads();
    if (NB == 1) {
        if (s0 < nsteps) do_compute(b0, s0);
    } else {
        for (int64_t s = s0; s < nsteps; s += 2 * nwaves) {
            do_compute(b0, s);
            if (s + 2 * nwaves < nsteps) do_load(b0, s + 2 * nwaves);
            if (s + nwaves < nsteps) {
                do_compute(b1, s + nwaves);
                if (s + 3 * nwaves < nsteps) do_load(b1, s + 3 * nwaves);
            }
        }
    }
    if (DBG) return;

    // Combine the sub-block slots held by lane groups: Q4_K/Q8_0 lanes g and g^2 (sub-blocks
    // 2p and 2p+1), Q6_K lanes g = 0..3 (the four 16-value sub-blocks).
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = acc[cg][e];
            if (T == kQ6_K) v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            acc[cg][e] = v;
        }
    // Lanes holding the wave's values: Q4_K/Q8_0 g in {0,1} (columns 4g..4g+3), Q6_K g == 0
    // (columns 4cg..4cg+3); 128 floats per wave.
    const bool holder = (T == kQ6_K) ? (g == 0) : (g < 2);
    if (holder) {
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
            for (int e = 0; e < 4; ++e) sRed[wave * 128 + lane * (4 * NCG) + cg * 4 + e] = acc[cg][e];
    }
    __syncthreads();
    if (wave != 0 || !holder || !row_ok) return;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = 0.f;
            for (int wv = 0; wv < nwaves; ++wv) v += sRed[wv * 128 + lane * (4 * NCG) + cg * 4 + e];
            const int c = (T == kQ6_K) ? 4 * cg + e : 4 * g + e;
            if (c < ncols) y[mc.pair(c) * rows + row] = v;
        }
}

template <int T, bool DBG, bool EXPERT>
static hipError_t launch_mmvq_t(const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y,
                                int32_t *dbg, const ColMap *cm, int64_t n_exp, hipStream_t s) {
    const int64_t nsteps = (k + kSuper - 1) / kSuper;
    ColMap c = cm ? *cm : ColMap{};
    dim3 grid((unsigned)((rows + kMvRows - 1) / kMvRows), EXPERT ? (unsigned)n_exp : 1u);
    const size_t smem_tab = (size_t)(k / 32) * 8 * sizeof(float2);
    if (nsteps <= kMvMaxWaves1) {
        const int nw = (int)nsteps;
        const size_t smem = smem_tab + (size_t)nw * 128 * sizeof(float);
        static bool attr1 = false;
        if (!attr1) {
            hipError_t e = hipFuncSetAttribute((const void *)mmvq_kernel<T, DBG, EXPERT, 1>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
            if (e != hipSuccess) return e;
            attr1 = true;
        }
        hipLaunchKernelGGL((mmvq_kernel<T, DBG, EXPERT, 1>), grid, dim3(64 * nw), smem, s, w, rows, k, xq, n, y,
                           dbg, c);
    } else {
        const int nw = kMvMaxWaves2;
        const size_t smem = smem_tab + (size_t)nw * 128 * sizeof(float);
        static bool attr2 = false;
        if (!attr2) {
            hipError_t e = hipFuncSetAttribute((const void *)mmvq_kernel<T, DBG, EXPERT, 2>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
            if (e != hipSuccess) return e;
            attr2 = true;
        }
        hipLaunchKernelGGL((mmvq_kernel<T, DBG, EXPERT, 2>), grid, dim3(64 * nw), smem, s, w, rows, k, xq, n, y,
                           dbg, c);
    }
    return hipGetLastError();
}

hipError_t launch_mmvq(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y,
                       int32_t *dbg, const ColMap *cm, int64_t n_exp, hipStream_t s) {
    const bool expert = cm != nullptr;
    const bool d = dbg != nullptr;
#define QMM_MV(TT)                                                                                       \
    if (type == TT) {                                                                                  \
        if (d) return launch_mmvq_t<TT, true, false>(w, rows, k, xq, n, y, dbg, cm, n_exp, s); \
        if (expert) return launch_mmvq_t<TT, false, true>(w, rows, k, xq, n, y, dbg, cm, n_exp, s); \
        return launch_mmvq_t<TT, false, false>(w, rows, k, xq, n, y, dbg, cm, n_exp, s);   \
    }
    QMM_MV(kQ4_K)
    QMM_MV(kQ6_K)
    QMM_MV(kQ8_0)
#undef QMM_MV
    return hipErrorInvalidValue;
}

}  // namespace qmm
