// One-time repack of a weight matrix into the panel layout ("QTensor and QMatMul" page, section
// on the 8-column Q4K repack: the blocks of adjacent rows are interleaved once, on first use, into
// a layout the product reads faster, and the original blocks are kept).  Here the unit is a panel
// of 16 rows x 256 values -- the row group of the matrix-vector kernel and a sixteenth of the
// tiled kernel's row tile -- stored as 256-byte slabs, each holding one 16-byte piece per row, with
// the codes split from the scales (the slab table is in qmm.h).  Every piece sits at a 16-byte
// aligned address and a panel is one contiguous run, so a kernel fetches a whole panel with
// coalesced 16-byte loads and parks it in LDS as it is: reading a slab in the MFMA operand layout
// (16 rows x 16 bytes) touches 256 consecutive bytes, free of bank conflicts.  No value is
// re-encoded: every byte of the original is copied once, rows past the end are zero.
#include "common.hpp"
#include "launch.hpp"

namespace qmm {

namespace {

// Original bytes of 256 values of one row (a panel holds 16 of these, i.e. B pieces of 16 bytes).
template <int T> struct PanelB;
template <> struct PanelB<kQ4_K> { static constexpr int B = 144; };
template <> struct PanelB<kQ5_K> { static constexpr int B = 176; };
template <> struct PanelB<kQ6_K> { static constexpr int B = 210; };
template <> struct PanelB<kQ8_0> { static constexpr int B = 272; };
template <> struct PanelB<kQ4_0> { static constexpr int B = 144; };

// Source of 2-byte unit t (0..7) of panel piece pc: the row within the group and the byte offset
// within that row's 256-value step of the original layout.  Piece pc < 16 * slabs is slab pc/16,
// row pc%16; Q6_K's last two pieces hold the fp16 d of rows 0-7 and 8-15.
template <int T> __device__ __forceinline__ void piece_src(int pc, int t, int &row, int &off) {
    const int j = pc >> 4;
    row = pc & 15;
    if constexpr (T == kQ4_K) {
        off = j < 8 ? 16 + 16 * j + 2 * t : 2 * t;
    } else if constexpr (T == kQ5_K) {
        off = j < 2 ? 16 + 16 * j + 2 * t : j < 10 ? 48 + 16 * (j - 2) + 2 * t : 2 * t;
    } else if constexpr (T == kQ6_K) {
        if (pc >= 208) {
            row = 8 * (pc - 208) + t;
            off = 208;
        } else {
            off = j < 8 ? 16 * j + 2 * t : j < 12 ? 128 + 16 * (j - 8) + 2 * t : 192 + 2 * t;
        }
    } else if constexpr (T == kQ8_0) {
        off = j < 16 ? 34 * (j >> 1) + 2 + 16 * (j & 1) + 2 * t : 34 * t;
    } else {   // Q4_0
        off = j < 8 ? 18 * j + 2 + 2 * t : 18 * t;
    }
}

// One thread per 16-byte piece of the output, pieces in output order (coalesced stores).
template <int T>
__global__ __launch_bounds__(256) void repack_panels_kernel(const uint8_t *__restrict__ w, int64_t rows,
                                                            int64_t row_bytes, int64_t nsteps, int64_t npieces,
                                                            uint8_t *__restrict__ wp) {
    constexpr int B = PanelB<T>::B;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < npieces; q += (int64_t)gridDim.x * 256) {
        const int64_t panel = q / B;
        const int pc = (int)(q - panel * B);
        const int64_t g = panel / nsteps, s = panel - g * nsteps;
        uint32_t u[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            uint32_t pair = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                int row, off;
                piece_src<T>(pc, 2 * h + e, row, off);
                const int64_t r = 16 * g + row;
                const uint32_t v = r < rows ? ld2(w + r * row_bytes + s * B + off) : 0u;
                pair |= v << (16 * e);
            }
            u[h] = pair;
        }
        *(u32x4 *)(wp + q * 16) = u32x4{u[0], u[1], u[2], u[3]};
    }
}

template <int T>
hipError_t launch_t(const uint8_t *w, int64_t rows, int64_t k, uint8_t *wp, hipStream_t s) {
    constexpr int B = PanelB<T>::B;
    const int64_t nsteps = k / 256, groups = (rows + 15) / 16;
    const int64_t npieces = groups * nsteps * B;   // 16 * B bytes per panel = B pieces
    const int64_t row_bytes = (k / Fmt<T>::QK) * Fmt<T>::BYTES;
    const int64_t blocks = (npieces + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 16384 ? blocks : 16384);
    hipLaunchKernelGGL(repack_panels_kernel<T>, dim3(grid), dim3(256), 0, s, w, rows, row_bytes, nsteps, npieces, wp);
    return hipGetLastError();
}

}  // namespace

int64_t panel_bytes(int type, int64_t rows, int64_t k) {
    const int B = type == kQ4_K || type == kQ4_0 ? 144 : type == kQ5_K ? 176 : type == kQ6_K ? 210
                  : type == kQ8_0 ? 272 : 0;
    if (B == 0 || rows < 1 || k < 256 || k % 256 != 0) return -1;
    return (rows + 15) / 16 * (k / 256) * 16 * B;
}

hipError_t launch_repack_panels(int type, const uint8_t *w, int64_t rows, int64_t k, uint8_t *wp, hipStream_t s) {
    switch (type) {
        case kQ4_K: return launch_t<kQ4_K>(w, rows, k, wp, s);
        case kQ5_K: return launch_t<kQ5_K>(w, rows, k, wp, s);
        case kQ6_K: return launch_t<kQ6_K>(w, rows, k, wp, s);
        case kQ8_0: return launch_t<kQ8_0>(w, rows, k, wp, s);
        case kQ4_0: return launch_t<kQ4_0>(w, rows, k, wp, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
