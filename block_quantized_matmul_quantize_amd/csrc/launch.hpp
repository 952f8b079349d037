// Host-side launch functions implemented by the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qmm.h"

namespace qmm {

// Plan overrides (qmm_set_override), read once at the start of a call so that every decision of
// that call (workspace layout, regime, kernels) sees the same values; 0 = automatic throughout.
struct Ovr {
    int path = 0;        // 1 matrix-vector, 2 tiled
    int streamk = 0;     // 1 off, 2 on
    int tile_j = 0;      // 32, 64, 128
    int mv_steps = 0;    // register-streamed matrix-vector kernel: 256-value steps per wave (1, 2, 4)
    int mv_kernel = 0;   // 1 register-streamed, 2 LDS-staged, 3 dot4
    int fuse_cols = 0;   // most columns the LDS-staged kernel quantizes itself (1..8)
};

hipError_t launch_quantize_q8_1(const float *x, int64_t n_rows, int64_t k, uint8_t *y, hipStream_t s);

// Tiled-kernel activation layout (tiled_act.hpp): for each 256-value step kb and activation row r,
// the 8 blocks' codes (256 bytes), fp32 d (32 bytes) and s parts (32 bytes), each kind in a table
// of its own indexed by kb * n_rows + r.
inline size_t q8_1_tiled_bytes(int64_t n_rows, int64_t k) { return (size_t)((k / 32 + 7) / 8) * n_rows * 320; }
// fp32 rows -> tiled layout (and, if canon is not null, the canonical q8_1 blocks as well); the
// same launch sets the nzero words at zero to 0 (the tiled kernel's stream-K counters)
hipError_t launch_quantize_q8_1_tiled(const float *x, int64_t n_rows, int64_t k, uint8_t *tiled, uint8_t *canon,
                                      hipStream_t s, int32_t *zero = nullptr, int64_t nzero = 0);
// canonical q8_1 blocks -> tiled layout (zero / nzero as above)
hipError_t launch_relayout_q8_1_tiled(const uint8_t *xq, int64_t n_rows, int64_t k, uint8_t *tiled, hipStream_t s,
                                      int32_t *zero = nullptr, int64_t nzero = 0);
hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t v, hipStream_t s);

// Column map for the matrix-vector and tiled kernels.  Dense: column j reads activation row j
// and writes output row j.  Expert mode: columns are the expert's (token, slot) pairs taken from
// the device-side sorted list.
struct ColMap {
    // expert mode only (all null / zero for dense)
    const int32_t *sorted;     // [pairs] pair index (t*top_k + slot), grouped by expert
    const int32_t *bounds;     // [n_exp + 1] segment starts in `sorted`
    const int32_t *tile_start; // [n_exp + 1] prefix of tiled-kernel column tiles per expert
    const int32_t *small;      // [n_exp] experts handled by the matrix-vector kernel, then -1
    int32_t top_k;
    int32_t x_per_tok;
    int32_t n_exp;
    int64_t w_expert_stride;   // bytes between expert matrices
    int64_t act_rows;          // activation rows (n_tok * x_per_tok): row count of the tiled layout
    int64_t pairs;             // (token, slot) pairs of the call
};

// Matrix-vector kernel: n <= 8 columns (dense) or the small experts (expert mode, grid.y = n_exp).
hipError_t launch_mmvq(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n,
                       float *y, int32_t *dbg, const ColMap *cm, int64_t n_exp, const Ovr &o, hipStream_t s);

// Gate/up fusion, matrix-vector: y = silu(W_gate x) * (W_up x) for n <= 8 dense q8_1 columns (cm
// null) or the small experts (cm set, grid.y = n_exp); the LDS-staged kernel where both matrices
// meet its rules, else the register-streamed one.
int mmvq_glu_f32_choice(int type, const void *wg, const void *wu, int64_t rows, int64_t k, const float *x, int64_t n,
                        const Ovr &o);
hipError_t launch_mmvq_glu(int type, const uint8_t *wg, const uint8_t *wu, int64_t rows, int64_t k, const uint8_t *xq,
                           int64_t n, float *y, const ColMap *cm, int64_t n_exp, const Ovr &o, hipStream_t s);

// The same on the dot4 kernel for 1..3 dense fp32 columns (quantized inside); Q4_K and Q8_0 under
// mmvq_dot4_supported's alignment rules for both matrices.
hipError_t launch_mmvq_dot4_glu_f32(int type, const uint8_t *wg, const uint8_t *wu, int64_t rows, int64_t k,
                                    const float *x, int64_t n, float *y, hipStream_t s);

// And on the LDS-staged kernel (mmvq_stream_supported's rules for both matrices): dense fp32
// (x_fp32, quantized inside) or q8_1 columns, or the small experts (cm set, q8_1).
hipError_t launch_mmvq_stream_glu(int type, const uint8_t *wg, const uint8_t *wu, int64_t rows, int64_t k,
                                  const void *x, bool x_fp32, int64_t n, float *y, const ColMap *cm, int64_t n_exp,
                                  hipStream_t s);

// fp32-input matrix-vector product with the q8_1 quantization done inside the dot4 or the
// LDS-staged kernel (no separate quantize launch): dense calls either kernel would take.
// Kernel launch_mmvq takes for q8_1 input: 3 dot4, 2 LDS-staged MFMA, 1 register-streamed, 0 none
// (a forced kernel that cannot serve the call); host logic only.
int mmvq_kernel_choice(int type, const void *w, int64_t rows, int64_t k, const void *xq, int64_t n, const ColMap *cm,
                       const Ovr &o);
// Kernel launch_mmvq_fused takes for fp32 input: 3 dot4, 2 LDS-staged MFMA, 0 not fused.
int mmvq_fused_choice(int type, const void *w, int64_t rows, int64_t k, const float *x, int64_t n, const Ovr &o);
// Launches the kernel mmvq_fused_choice names (`choice`, non-zero).
hipError_t launch_mmvq_fused(int choice, int type, const uint8_t *w, int64_t rows, int64_t k, const float *x, int64_t n,
                             float *y, hipStream_t s);
hipError_t launch_mmvq_dot4_f32(int type, const uint8_t *w, int64_t rows, int64_t k, const float *x, int64_t n,
                                float *y, hipStream_t s);
hipError_t launch_mmvq_stream_f32(int type, const uint8_t *w, int64_t rows, int64_t k, const float *x, int64_t n,
                                  float *y, hipStream_t s);

// LDS-streamed matrix-vector kernel (mmvq_stream.hip): 16-byte aligned weights, activations and
// rows, K a multiple of 256.
bool mmvq_stream_supported(int type, const void *w, int64_t k, const void *xq, const ColMap *cm);
hipError_t launch_mmvq_stream(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n,
                              float *y, int32_t *dbg, const ColMap *cm, int64_t n_exp, hipStream_t s);
// dot4 matrix-vector kernel (mmvq_dot4.hip) for 1..mmvq_dot4_max_cols() dense columns: Q4_K and
// Q8_0, K a multiple of 256.
int device_cus();   // compute units of the current device, looked up once per device (api.cpp)
int mmvq_dot4_max_cols();
bool mmvq_dot4_supported(int type, const void *w, int64_t k, const void *xq, const ColMap *cm);
hipError_t launch_mmvq_dot4(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n,
                            float *y, int32_t *dbg, const ColMap *cm, int64_t n_exp, int max_cols, hipStream_t s);

// Tiled int8-MFMA kernel plan.
struct MmqLaunch {
    int tile_j;          // 32, 64 or 128
    int64_t ntiles;      // row tiles x column tiles (dense)
    int64_t n_ct;        // column tiles
    int64_t k_iters;     // K steps of 256 values
    int64_t units;       // workgroups (== ntiles unless stream-K)
    bool stream_k;
    float *partials;     // [units][2][128*tile_j] when stream_k
    int32_t *counters;   // [ntiles] split-tile arrival counters when stream_k, zero at launch
    bool packed = false; // w in the panel layout (repack.hip), k % 256 == 0
};
hipError_t launch_mmq(int type, const uint8_t *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n,
                      float *y, int32_t *dbg, const MmqLaunch &plan, hipStream_t s);
// Gate/up fusion: y[n][rows] = silu(W_gate x) * (W_up x), tiles of 64 outputs, no stream-K.
hipError_t launch_mmq_glu(int type, const uint8_t *wg, const uint8_t *wu, int64_t rows, int64_t k, const uint8_t *xq,
                          int64_t n, float *y, int tile_j, hipStream_t s);
// Expert mode: grid over (row tiles, max column tiles); experts with > 8 columns.  w_up not null:
// gate/up fusion, w the gate matrices.
hipError_t launch_mmq_id(int type, const uint8_t *w, const uint8_t *w_up, int64_t rows, int64_t k,
                         const uint8_t *xq, float *y, const ColMap &cm, int tile_j, int64_t max_col_tiles,
                         hipStream_t s);

// Expert grouping: counts, bounds, stable sorted pair list, column-tile prefix, small-expert list.
hipError_t launch_moe_group(const int32_t *ids, int64_t pairs, int32_t n_exp, int32_t tile_j,
                            int32_t small_max, int32_t *sorted, int32_t *bounds, int32_t *tile_start,
                            int32_t *small, int32_t *invalid, hipStream_t s);
// Grouping + activation quantization (tiled and canonical layouts) in one launch, for n_exp up to
// the per-wave grouping's limit (moe_prologue_fused); cus: compute units of the device.
bool moe_prologue_fused(int32_t n_exp);
hipError_t launch_moe_prologue(const int32_t *ids, int64_t pairs, int32_t n_exp, int32_t tile_j, int32_t small_max,
                               int32_t *sorted, int32_t *bounds, int32_t *tile_start, int32_t *small, int32_t *invalid,
                               const float *x, int64_t n_rows, int64_t k, uint8_t *tiled, uint8_t *canon,
                               int32_t cus, hipStream_t s);

// Panel layout (repack.hip): bytes of the layout for a [rows][k] matrix (-1: type or shape not
// supported), and the one-time repack of the original blocks w into wp (16-byte aligned).
int64_t panel_bytes(int type, int64_t rows, int64_t k);
hipError_t launch_repack_panels(int type, const uint8_t *w, int64_t rows, int64_t k, uint8_t *wp, hipStream_t s);
// Dense products reading panel-layout weights: n <= 8 fp32 columns (the LDS-staged kernel, which
// quantizes x itself; x 16-byte aligned), and the tiled kernel (plan.packed set).
hipError_t launch_mmvq_stream_panel_f32(int type, const uint8_t *wp, int64_t rows, int64_t k, const float *x, int64_t n,
                                        float *y, hipStream_t s);

// fp16-activation mode (f16act.hip)
hipError_t launch_f16act_encode(const float *x, int64_t n, int64_t k, uint16_t *y16, int32_t *e, float *bsum,
                                hipStream_t s);
hipError_t launch_mmvq_f16act(int type, const uint8_t *w, int64_t rows, int64_t k, const uint16_t *y16,
                              const int32_t *e, const float *bsum, int64_t n, float *out, hipStream_t s);

// Dense fp32-input product with a workspace sized exactly to its plan (api.cpp), for the
// allocation-free entry point (noalloc.hip).  o: one reading of the overrides for the whole call.
Ovr load_overrides();
// Sets the calling thread's qmm_last_error message and returns st.
qmm_status report(qmm_status st, const char *msg);
// qmm_matmul's argument checks; *need = the workspace bytes the call's plan uses (0 for n == 0).
qmm_status matmul_exact_check(int type, const void *w, int64_t rows, int64_t k, const float *x, int64_t n,
                              const float *y, const Ovr &o, size_t *need);
// The product itself, with ws holding at least matmul_exact_check's bytes.
qmm_status matmul_exact_run(int type, const void *w, int64_t rows, int64_t k, const float *x, int64_t n, float *y,
                            uint8_t *ws, const Ovr &o, hipStream_t s);

}  // namespace qmm
