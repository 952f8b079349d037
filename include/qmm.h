/*
 * qmm.h -- C ABI of libqmm: GGUF block-quantized weights (Q4_K, Q5_K, Q6_K, Q8_0, Q4_0, Q3_K,
 * IQ4_XS) times fp32 activations quantized to q8_1, on AMD Instinct MI355X (gfx950).
 *
 * Sources (the web pages this library implements):
 *  [MMQ]   "llama.cpp source walkthrough (15): quantized GEMM -- MMQ" (pinghaoyang.com.cn)
 *  [GP100] "Patch 0007: an fp16 matrix-vector path for GP100"
 *  [QMM]   "QTensor and QMatMul" (candle-core 0.11.0 documentation)
 *
 * Conventions shared by every entry point
 *  - Pointers named w, x, xq, y, ids, ws, d_out are DEVICE pointers owned by the caller.  The
 *    library never frees them and keeps no reference after the call returns.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL means the default stream).
 *    Arguments are validated on the host before anything is launched; a non-zero status means
 *    nothing was launched, except QMM_ERR_HIP (a launch failed part-way).
 *  - Weights are a row-major [rows][k] matrix stored as raw GGUF blocks: each row is k/QK blocks
 *    back to back, rows back to back ([QMM] "QTensor": the last dimension must be a multiple of
 *    the block size and a block never spans rows).  QK = 256 for Q4_K/Q6_K, 32 for Q8_0.  Block
 *    bytes: Q4_K 144 {fp16 d, fp16 dmin, 12 B packed 6-bit scales/mins, 128 B nibbles};
 *    Q6_K 210 {128 B ql, 64 B qh, 16 int8 scales, fp16 d}; Q8_0 34 {fp16 d, 32 int8}; Q5_K 176 and
 *    Q4_0 18 as GGUF's.  Q3_K 110 {32 B hmask, 64 B qs, 12 B of 6-bit scales, fp16 d} and IQ4_XS
 *    136 {fp16 d, 16-bit scales_h, 4 B scales_l, 128 B of 4-bit codebook indices} ([GP100] "How"
 *    step 3 names both, Q3_K's -4 code offset and IQ4_XS's codebook; the layouts and the codebook
 *    are GGUF's).  Only 2-byte alignment of w is required.
 *  - Activations x are fp32 row-major [n][k] (token-major, [QMM] "QMatMul": input [..., k]),
 *    16-byte aligned (the kernels read 8 values per lane as two 16-byte loads); QMM_ERR_ARG
 *    otherwise.  Outputs y are fp32 row-major [n][rows] (output [..., n]), 4-byte aligned.
 *  - q8_1 blocks (36 B): {fp16 d, fp16 s, int8 q[32]}, one per 32 activation values; [MMQ]
 *    introduction and "dp4a path Q4_K" section (the activation half2 (d, s), s = d * sum(q)).
 *    Quantization: amax = max|x|; d32 = amax/127 (fp32); q = round-half-away(x / d32);
 *    d = fp16(d32); s = fp16(d32 * sum(q)); an all-zero block gives d = s = q = 0.
 *  - Result ([MMQ] "dp4a path Q4_K", "Q6_K dot", "write-back"): per 32-value block b an exact
 *    integer dot D_b of weight codes and q8_1 codes, then fp32 scale fixups:
 *      Q4_K  y += d*sc_b*d_b*D_b - dmin*m_b*s_b
 *      Q6_K  y += d*d_b*(sc_{2b}*D_{2b} + sc_{2b+1}*D_{2b+1})   (16-value sub-blocks)
 *      Q8_0  y += dw_b*d_b*D_b
 *      Q3_K  as Q6_K with sc = 6-bit scale - 32 and codes q - 4 (q 3-bit)
 *      IQ4_XS y += d*(ls_b - 32)*d_b*D_b, D_b over the codebook values of the indices
 *    summed in fp32 in an order that depends on the chosen kernel (several fp32 results are
 *    correct; see qmm_set_override).  For a fixed plan the result is bitwise reproducible.
 *  - Errors: a status code; qmm_last_error() returns a message for the calling thread.
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QMM_OK = 0,
    QMM_ERR_ARG = -1,        /* null pointer, negative size, bad x_per_tok, ... */
    QMM_ERR_TYPE = -2,       /* weight type not supported */
    QMM_ERR_SHAPE = -3,      /* k not a multiple of the block size, or too large */
    QMM_ERR_WORKSPACE = -4,  /* workspace pointer null or smaller than the *_workspace size */
    QMM_ERR_HIP = -5         /* a HIP call failed (message in qmm_last_error) */
} qmm_status;

typedef enum {
    QMM_Q4_0 = 2, QMM_Q8_0 = 8, QMM_Q3_K = 11, QMM_Q4_K = 12, QMM_Q5_K = 13, QMM_Q6_K = 14, QMM_IQ4_XS = 23
} qmm_type; /* GGUF type ids */

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *qmm_last_error(void);

/* Library version string. */
const char *qmm_version(void);

/* ---------------------------------------------------------------------------------------------
 * a1: activation quantization ([MMQ] introduction; "dp4a path Q4_K": s = d * sum(q)).
 * x: fp32 [n_rows][k], k % 32 == 0, 16-byte aligned.  y: n_rows * (k/32) q8_1 blocks of 36 bytes, row-major,
 * 4-byte aligned.  n_rows == 0 is a no-op.
 * ------------------------------------------------------------------------------------------- */
qmm_status qmm_quantize_q8_1(const float *x, int64_t n_rows, int64_t k, void *y, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Dense product Y[n][rows] = W[rows][k] . X[n][k]^T with q8_1 activations.
 * Regimes ([MMQ] "shape criteria" and the MMVQ-vs-MMQ table): n <= 8 uses the matrix-vector
 * kernel (weights streamed once, all columns per pass); n > 8 uses the tiled int8-MFMA GEMM with
 * a tile-width selector and a stream-K split when the tiles underfill the GPU ([MMQ] "J runtime
 * selection", "tile efficiency", "stream-K", "fixup").
 *
 * qmm_matmul_workspace: bytes of device workspace qmm_matmul needs (256-byte aligned pointer
 *   expected).  A size of 0 means no workspace is needed (ws may be NULL); invalid arguments also
 *   give 0, and the call itself then reports the error.
 * qmm_matmul: quantizes x to q8_1 into the workspace, then multiplies.
 * qmm_matmul_q8_1: the same product from already-quantized activations xq (n * k/32 q8_1
 *   blocks, as written by qmm_quantize_q8_1), so one quantization can serve several weights
 *   ([GP100] "How": the activation-conversion cache).  Uses qmm_matmul_q8_1_workspace bytes.
 * n == 0 is a no-op.  rows >= 1, k >= QK, k % QK == 0, k <= 1<<20.
 * ------------------------------------------------------------------------------------------- */
size_t qmm_matmul_workspace(int type, int64_t rows, int64_t k, int64_t n);
qmm_status qmm_matmul(int type, const void *w, int64_t rows, int64_t k, const float *x, int64_t n,
                      float *y, void *ws, size_t ws_bytes, void *stream);
size_t qmm_matmul_q8_1_workspace(int type, int64_t rows, int64_t k, int64_t n);
qmm_status qmm_matmul_q8_1(int type, const void *w, int64_t rows, int64_t k, const void *xq,
                           int64_t n, float *y, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Allocation-free dense product, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The same product, plan,
 * kernels and argument checks as qmm_matmul, but the workspace is a buffer the library owns: a
 * static device array of QMM_NOALLOC_SCRATCH_BYTES on each GPU the library runs on (held until the
 * process ends), of which a call uses exactly what its plan needs.  The call itself allocates
 * nothing; its first call with a given device current looks up that device's buffer address.
 * A call whose plan needs more than QMM_NOALLOC_SCRATCH_BYTES returns QMM_ERR_WORKSPACE before
 * anything is launched (e.g. 4096 x 14336 Q6_K at 512 columns needs ~42 MB and fits; 65536
 * columns of k = 14336 do not).  Calls share their GPU's buffer: calls that overlap on one GPU
 * (different streams, different threads without ordering) race and must be serialised by the
 * caller, e.g. by issuing them on one stream.  No part of the buffer needs clearing between calls.
 * ------------------------------------------------------------------------------------------- */
#define QMM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
qmm_status qmm_matmul_noalloc(int type, const void *w, int64_t rows, int64_t k, const float *x, int64_t n,
                              float *y, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Panel layout: a one-time weight repack ([QMM] "Q4K 8-column repack": the blocks of adjacent
 * rows are interleaved once, on first use, into a layout the product reads faster, and the
 * original blocks are kept, so the weights then take twice the memory).  Here the caller repacks
 * explicitly and owns both buffers; the library keeps no state.
 *
 * Layout (k % 256 == 0): G = ceil(rows/16) row groups, S = k/256 steps, B = bytes of 256 values
 * of a row in the original layout (Q4_K 144, Q5_K 176, Q6_K 210, Q8_0 272, Q4_0 144), P = 16*B.
 * Panel (g, s) -- rows 16g..16g+15, values 256s..256s+255 -- is the P bytes at (g*S + s)*P.  In a
 * panel, slab j is the 256 bytes at 256*j, holding one 16-byte piece per row (row i at 16*i):
 *   Q4_K  slabs 0-7: qs[16j, +16);    slab 8: the header {d, dmin, scales[12]}
 *   Q5_K  slabs 0-1: qh[16j, +16);    slabs 2-9: qs[16(j-2), +16);   slab 10: the header
 *   Q6_K  slabs 0-7: ql[16j, +16);    slabs 8-11: qh[16(j-8), +16);  slab 12: scales[16];
 *         then 32 bytes: the fp16 d of row i at 3328 + 2i
 *   Q8_0  slab j (0-15): qs[16(j%2), +16) of block j/2 of the step; slab 16: the 8 fp16 d
 *         (block b at byte 2b of the row's piece)
 *   Q4_0  slab j (0-7): qs[16] (nibbles) of block j;  slab 8: the 8 fp16 d as for Q8_0
 * Rows of the last group past `rows` are zero.  Bytes are copied unchanged, so the values, and the
 * products below, are those of the original blocks; the total is the original size plus the
 * padding rows.  Each panel is contiguous and 16-byte aligned, so a kernel fetches it with
 * coalesced 16-byte loads and parks it in LDS as it is (no per-call byte shuffling of the 210- and
 * 34-byte blocks), and a slab read in the int8 MFMA operand layout is 256 consecutive LDS bytes.
 *
 * qmm_repack_bytes: bytes of the panel layout of a [rows][k] matrix of `type`; 0 for an
 *   unsupported type or shape (k not a positive multiple of 256, rows < 1, k > 1<<20).
 * qmm_repack: w (original blocks, 2-byte aligned) -> wp (device, 16-byte aligned, at least
 *   qmm_repack_bytes bytes; QMM_ERR_ARG if smaller).  Asynchronous on `stream`; w is only read.
 * qmm_matmul_packed: the dense product of qmm_matmul with wp in the panel layout.  n <= 8 runs the
 *   LDS-staged matrix-vector kernel, which quantizes x itself (no workspace); more columns run the
 *   tiled kernel with qmm_matmul's plan (J, stream-K) and the qmm_matmul_packed_workspace bytes
 *   (256-byte aligned).  x fp32 [n][k], 16-byte aligned; y fp32 [n][rows].  Results equal
 *   qmm_matmul's on the original blocks up to fp32 summation order (the same kernels' arithmetic).
 *   QMM_ERR_SHAPE for k % 256 != 0; QMM_ERR_TYPE for an unsupported type.
 * ------------------------------------------------------------------------------------------- */
uint64_t qmm_repack_bytes(int type, int64_t rows, int64_t k);
qmm_status qmm_repack(int type, const void *w, int64_t rows, int64_t k, void *wp, uint64_t wp_bytes,
                      void *stream);
size_t qmm_matmul_packed_workspace(int type, int64_t rows, int64_t k, int64_t n);
qmm_status qmm_matmul_packed(int type, const void *wp, int64_t rows, int64_t k, const float *x, int64_t n,
                             float *y, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Expert-indexed product (MoE mul_mat_id; [MMQ] "MoE dispatch", "expert bounds", "MoE skew").
 * w: n_exp weight matrices [rows][k] back to back (ggml [k, rows, n_exp]).
 * ids: int32 [n_tok][top_k] expert ids (ggml [n_expert_used, n_tokens]).
 * x: fp32 [n_tok][x_per_tok][k]; x_per_tok == 1 (one row shared by every slot, gate/up) or
 *    x_per_tok == top_k (one row per slot, down projection).
 * y: fp32 [n_tok][top_k][rows]: row (t, j) = W[ids[t][j]] . x[t][j or 0], written back in the
 *    original (token, slot) order.
 * Grouping by expert, per-expert column counts, tile enumeration and the per-expert choice of
 * matrix-vector vs tiled kernel all happen on the device; nothing is read back to the host.
 * An id outside [0, n_exp) is skipped: its output row is left untouched and a counter in the
 * workspace is incremented (qmm_matmul_id_invalid_count reads it after the stream completes).
 * ------------------------------------------------------------------------------------------- */
size_t qmm_matmul_id_workspace(int type, int64_t n_exp, int64_t rows, int64_t k, int64_t n_tok,
                               int64_t top_k, int64_t x_per_tok);
qmm_status qmm_matmul_id(int type, const void *w, int64_t n_exp, int64_t rows, int64_t k,
                         const float *x, int64_t x_per_tok, const int32_t *ids, int64_t n_tok,
                         int64_t top_k, float *y, void *ws, size_t ws_bytes, void *stream);
/* Host pointer out receives the invalid-id count of the last qmm_matmul_id that used `ws`
 * (synchronizes `stream` first). */
qmm_status qmm_matmul_id_invalid_count(const void *ws, int64_t *out, void *stream);
/* Test hook (host logic only, no GPU call): where the expert grouping of a qmm_matmul_id call of
 * this shape lives in its workspace, so a test can check it ([MMQ] "expert bounds").  out[6]:
 * byte offsets of sorted (int32 [pairs]: pair indices t*top_k+slot grouped by expert; inside an
 * expert's segment the order is not fixed up to 2304 experts -- slots come from LDS atomics --
 * and ascending beyond; no output depends on it), bounds (int32 [n_exp+1]: segment starts,
 * bounds[n_exp] = valid pairs),
 * tile_start (int32 [n_exp+1]: prefix of tiled-kernel column tiles), small (int32 [n_exp]:
 * experts with 1..small_max columns in ascending order, then -1), then the column-tile width
 * and small_max the call uses.  Returns QMM_ERR_ARG for a bad shape. */
qmm_status qmm_matmul_id_grouping_layout(int type, int64_t n_exp, int64_t k, int64_t n_tok,
                                         int64_t top_k, int64_t x_per_tok, int64_t *out);

/* ---------------------------------------------------------------------------------------------
 * fp16-activation matrix-vector mode ([GP100] "How", step 1, and the accuracy paragraph under its
 * results table): an alternative numeric definition for 1..8 columns in which the activations
 * are not quantized to 8 bits but rounded once to fp16 after a power-of-two prescale per 32
 * values: e = the largest integer with max|x| * 2^e < 2^15 over the block (0 for an all-zero
 * block), y = fp16(x * 2^e) (round to nearest even), and the block sum of the y kept in fp32.
 * The product is W . (y * 2^-e) with fp32 accumulation.
 *
 * qmm_encode_f16act: x fp32 [n][k] (k % 32 == 0, 4-byte aligned) -> y16 fp16 bit patterns [n][k]
 *   (2-byte aligned), e int32 [n][k/32], bsum fp32 [n][k/32] (4-byte aligned), all device memory
 *   owned by the caller.  n == 0 is a no-op.
 * qmm_matmul_f16act_workspace: bytes of device workspace (256-byte aligned) for n columns of k.
 * qmm_matmul_f16act: Y[n][rows] = W[rows][k] . X[n][k]^T in this mode; types Q4_0, Q8_0, Q4_K,
 *   Q5_K, Q6_K; 0 <= n <= 8 (more columns: QMM_ERR_ARG; n == 0 is a no-op); k a multiple of the
 *   type's block (256 for the K types), k <= 1<<20; Q4_K / Q5_K weights 16-byte aligned, the
 *   others 2-byte aligned; x and y 4-byte aligned.  Asynchronous on stream.
 * ------------------------------------------------------------------------------------------- */
qmm_status qmm_encode_f16act(const float *x, int64_t n, int64_t k, void *y16, int32_t *e, float *bsum,
                             void *stream);
size_t qmm_matmul_f16act_workspace(int64_t k, int64_t n);
qmm_status qmm_matmul_f16act(int type, const void *w, int64_t rows, int64_t k, const float *x, int64_t n,
                             float *y, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Gate/up products fused with SwiGLU ([MMQ] the fusion passage after "MoE dispatch": the gate and
 * up products of one input are computed together and the GLU is applied at write-back; SwiGLU
 * read as silu(g) * u, silu(g) = g / (1 + exp(-g))).
 * qmm_matmul_glu: y[n][rows] = silu(W_gate . x) * (W_up . x) elementwise; w_gate and w_up are two
 *   [rows][k] matrices of the same type (2-byte aligned), x fp32 [n][k] (16-byte aligned).  n <= 8:
 *   the matrix-vector kernel with 8 gate and 8 up rows per workgroup; otherwise the tiled kernel
 *   with tiles of 64 outputs whose 128 weight rows alternate in groups of 8 between gate and up
 *   (no stream-K: the two products of an output must meet in one workgroup).  Workspace:
 *   qmm_matmul_glu_workspace bytes, 256-byte aligned.
 * qmm_matmul_id_glu: the expert form; w_gate and w_up hold n_exp matrices each (as qmm_matmul_id),
 *   x fp32 [n_tok][k] (one row per token, shared by its slots), y fp32 [n_tok][top_k][rows].
 *   Grouping, small-expert dispatch, invalid-id handling and the workspace counter as
 *   qmm_matmul_id; workspace qmm_matmul_id_glu_workspace bytes.
 * The same shape rules and errors as the unfused calls; a null w_up is QMM_ERR_ARG.
 * ------------------------------------------------------------------------------------------- */
size_t qmm_matmul_glu_workspace(int type, int64_t rows, int64_t k, int64_t n);
qmm_status qmm_matmul_glu(int type, const void *w_gate, const void *w_up, int64_t rows, int64_t k,
                          const float *x, int64_t n, float *y, void *ws, size_t ws_bytes, void *stream);
size_t qmm_matmul_id_glu_workspace(int type, int64_t n_exp, int64_t rows, int64_t k, int64_t n_tok,
                                   int64_t top_k);
qmm_status qmm_matmul_id_glu(int type, const void *w_gate, const void *w_up, int64_t n_exp, int64_t rows,
                             int64_t k, const float *x, const int32_t *ids, int64_t n_tok, int64_t top_k,
                             float *y, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Test hook: the integer sub-block dots from the production kernels ([MMQ] "write-back": the
 * integer part is exact).  path: 1 = matrix-vector kernel, 2 = tiled MFMA kernel.  The call runs
 * the plan a qmm_matmul_q8_1 of this shape takes under the current overrides, with the path
 * forced: the same kernel, activation layout, LDS layout, MFMAs and accumulator seeding
 * (stream-K split included on the tiled path), and only where a kernel folds an integer dot into
 * its fp32 result does it store that integer to d_out instead (y is not written).
 * d_out: int32 [n][rows][per] (device, 4-byte aligned) with
 *   per = k/32 for Q4_K, Q5_K, Q8_0, Q4_0 (D_b),
 *   per = k/32 for IQ4_XS (D_b over the codebook values),
 *   Q6_K and Q3_K path 1: per = k/16 (D per 16-value sub-block),
 *   Q6_K and Q3_K path 2: per = k/32, the scale-folded integer sc_{2b}*D_{2b} + sc_{2b+1}*D_{2b+1}
 *   (Q3_K: sc = 6-bit scale - 32).
 * xq: n * k/32 q8_1 blocks (4-byte aligned).  Path 1 requires n <= 8.
 * qmm_debug_subdots_workspace: bytes of device workspace (256-byte aligned) the call needs; 0
 *   means none (ws may be NULL), also for invalid arguments.
 * ------------------------------------------------------------------------------------------- */
size_t qmm_debug_subdots_workspace(int type, int64_t rows, int64_t k, int64_t n, int path);
qmm_status qmm_debug_subdots(int type, const void *w, int64_t rows, int64_t k, const void *xq,
                             int64_t n, int path, int32_t *d_out, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Which matrix-vector kernel a dense call would launch ([MMQ] "shape criteria": n <= 8 takes the
 * matrix-vector regime), under the current overrides; host logic only, nothing is launched and
 * no GPU is needed.  x_fp32 = 1 asks about qmm_matmul with fp32 activations x, 0 about
 * qmm_matmul_q8_1 with q8_1 activations x; only the alignment of w and x, and the sizes, are looked
 * at (one to three columns of 8192 or more rows take the dot4 kernel -- Q8_0: one column from
 * 8192 rows, two or three from 12288 -- fewer rows the LDS-staged one; Q3_K and IQ4_XS take dot4
 * for one to three columns at any row count; Q6_K, which has no dot4 form, the LDS-staged one).
 * *out: 0 the call takes the tiled path (n > 8 or forced), 1 register-streamed, 2 LDS-staged
 * MFMA, 3 dot4; plus 16 when that kernel quantizes the fp32 activations itself (one launch, no
 * quantize kernel).  Errors: QMM_ERR_TYPE / QMM_ERR_SHAPE as for qmm_matmul, QMM_ERR_ARG for a
 * null out or an fp32 x that is not 16-byte aligned.
 * ------------------------------------------------------------------------------------------- */
qmm_status qmm_matvec_kernel(int type, const void *w, int64_t rows, int64_t k, const void *x, int64_t n,
                             int32_t x_fp32, int32_t *out);

/* ---------------------------------------------------------------------------------------------
 * Plan overrides for tests and tuning (process-wide; 0 = automatic).  Every other entry point
 * reads the overrides once when it starts, so a concurrent change never splits one call's
 * workspace layout from its plan; this is the only entry point that writes process-wide state.
 *   QMM_OVR_PATH:     1 force matrix-vector (only when n <= 8), 2 force tiled MFMA.
 *   QMM_OVR_STREAMK:  1 force off, 2 force on (tiled path).
 *   QMM_OVR_TILE_J:   tile width in columns (32, 64 or 128).
 *   QMM_OVR_MV_STEPS: 256-value steps per wave in the register-streamed matrix-vector kernel
 *                     (1, 2 or 4).
 *   QMM_OVR_MV_KERNEL: matrix-vector kernel: 1 register-streamed (any input), 2 LDS-staged
 *                     MFMA only (Q4_0, Q8_0, Q4_K, Q5_K, Q6_K), 3 dot4 only (up to 3 columns;
 *                     Q4_0, Q8_0, Q3_K, Q4_K, Q5_K, IQ4_XS); calls the forced kernel cannot serve
 *                     fail with QMM_ERR_HIP.  The automatic choice takes the dot4 kernel for one
 *                     column of 8192 or more rows (Q3_K, IQ4_XS: up to three columns at any
 *                     rows), else the LDS-staged kernel, when K is a multiple of 256 and the
 *                     weights are aligned (Q4_K, Q5_K, Q6_K: 16 bytes, rows too; Q8_0, Q4_0: 4;
 *                     Q3_K, IQ4_XS: 2) and q8_1 activations 4-byte aligned; otherwise the
 *                     register-streamed kernel.
 *   QMM_OVR_FUSE_COLS: qmm_matmul only: most columns (1..8) for which the LDS-staged kernel
 *                     quantizes the fp32 activations itself instead of a separate quantize
 *                     launch (automatic: 8).
 * Returns QMM_ERR_ARG for an unknown key or value.
 * ------------------------------------------------------------------------------------------- */
enum { QMM_OVR_PATH = 1, QMM_OVR_STREAMK = 2, QMM_OVR_TILE_J = 3, QMM_OVR_MV_STEPS = 4, QMM_OVR_MV_KERNEL = 5,
       QMM_OVR_FUSE_COLS = 6 };
qmm_status qmm_set_override(int key, int value);

/* ---------------------------------------------------------------------------------------------
 * Host-side planner, exposed so its arithmetic can be tested without a GPU.
 * ([MMQ] "J runtime selection": smallest J with the fewest column tiles -- except that 33-64
 * columns take one 128-column tile for Q6_K / Q3_K / Q8_0 and two 32-column tiles otherwise, the
 * 64-column tile measuring slowest there (plain and fused gate/up calls); "tile efficiency":
 * eff = floor(100 * ntiles / (nsm * ceil(ntiles / nsm))); "when not to use stream-K" and
 * "stream-K": nwork = ntiles * ceil(k_iters), units = min(nsm * occupancy, nwork), and unit u
 * owns the flattened (tile, k-iteration) range [u*W/units, (u+1)*W/units).)
 * ------------------------------------------------------------------------------------------- */
typedef struct {
    int32_t regime;          /* 1 matrix-vector, 2 tiled */
    int32_t tile_i;          /* rows per tile */
    int32_t tile_j;          /* columns per tile */
    int64_t ntiles;          /* output tiles */
    int32_t efficiency_pct;  /* tile efficiency on nsm compute units */
    int32_t stream_k;        /* 1 if the stream-K split is used */
    int64_t k_iters;         /* K steps per tile (one super-block of 256 values per step) */
    int64_t units;           /* stream-K work units launched (== ntiles without stream-K) */
    int32_t fixup;           /* 1 if some tiles are split across units (the last unit to finish
                                such a tile adds the units' partials in unit order) */
    uint64_t ws_bytes;       /* workspace qmm_matmul needs under this plan (from the same reading
                                of the overrides as the rest of the plan) */
} qmm_plan;

qmm_status qmm_plan_dense(int type, int64_t rows, int64_t k, int64_t n, int32_t nsm, qmm_plan *out);
/* Tile efficiency percentage for ntiles tiles on nsm units. */
int32_t qmm_tile_efficiency(int64_t ntiles, int32_t nsm);
/* Column tile width minimising ceil(ncols / J) over the candidate widths (ties -> smaller J). */
int32_t qmm_select_tile_j(int64_t ncols);
/* Stream-K partition: first flattened work item of unit u, aligned down to a tile boundary's
 * K step; returns the start index in [0, nwork].  The tiled kernel applies it to the tiles left
 * over after whole rounds of one tile per unit (ntiles - floor(ntiles/units)*units of them). */
int64_t qmm_streamk_unit_start(int64_t u, int64_t units, int64_t ntiles, int64_t k_iters);

#ifdef __cplusplus
}
#endif
#endif /* QMM_H */
