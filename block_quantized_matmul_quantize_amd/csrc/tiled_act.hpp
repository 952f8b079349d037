// Activation layout of the tiled kernel: q8_1 blocks (the MMQ page, "activation quantization")
// regrouped per 256-value step so that a step of one activation row is three fixed-size records
// the tiled kernel copies into LDS with direct global-to-LDS loads, unchanged:
//   codes   [nsteps][n_rows][256] int8   -- the 8 blocks' codes of the step, block b at 32*b
//   d       [nsteps][n_rows][8]   fp32   -- each block's fp16 scale d, widened to fp32
//   s parts [nsteps][n_rows][8]   uint32 -- each block's fp16 s = t1 + t2 exactly, t1 and t2 bf16
//                                           (t1 in the low half): the B operand of the K-quant
//                                           min term
// 320 bytes per (step, row).  Blocks past K in a partial last step are left unwritten: the tiled
// kernel never reads them.
#pragma once

#include "common.hpp"
#include "q8_1.hpp"

namespace qmm {

constexpr int64_t kTiledActBytes = 320;   // per (step, row)

__device__ __forceinline__ uint32_t tiled_bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Writes lane `sub` (0..3) of block bi of activation row `row`: 8 codes, and on lane 0 the
// block's d and s parts.  nsteps = ceil(nb32 / 8).
__device__ __forceinline__ void tiled_act_put(uint8_t *tiled, int64_t nsteps, int64_t n_rows, int64_t row, int64_t bi,
                                              int sub, uint32_t c0, uint32_t c1, uint32_t ds) {
    const int64_t slot = (bi >> 3) * n_rows + row;   // (step, row)
    const int blk = (int)(bi & 7);
    *(u32x2 *)(tiled + slot * 256 + 32 * blk + 8 * sub) = u32x2{c0, c1};
    if (sub == 0) {
        const size_t cells = (size_t)nsteps * (size_t)n_rows;
        ((float *)(tiled + cells * 256))[slot * 8 + blk] = h2f((uint16_t)(ds & 0xFFFF));
        const float s = h2f((uint16_t)(ds >> 16));
        const uint32_t t1 = tiled_bf16_bits(s);
        const float rest = s - __builtin_bit_cast(float, t1 << 16);   // exact: s has 11 significant bits
        ((uint32_t *)(tiled + cells * 288))[slot * 8 + blk] = t1 | (tiled_bf16_bits(rest) << 16);
    }
}

}  // namespace qmm
