// C ABI of libqmm: argument validation, workspace layout, the host planner and the launches.
// Declarations and the contract of every entry point are in include/qmm.h.
#include "../../include/qmm.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "launch.hpp"

namespace qmm {

namespace {
int g_nsm_cache[64];
std::mutex g_nsm_mu;
}  // namespace

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lk(g_nsm_mu);
    if (g_nsm_cache[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        g_nsm_cache[dev] = v;
    }
    return g_nsm_cache[dev];
}

}  // namespace qmm

using qmm::device_cus;

namespace {

thread_local std::string g_err;

qmm_status fail(qmm_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
qmm_status fail(qmm_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

qmm_status hip_fail(hipError_t e, const char *what) {
    return fail(QMM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// qmm_set_override's values (the only process-wide state an entry point depends on besides the
// device-property cache); each call reads them once, into a qmm::Ovr.
std::atomic<int> g_ovr_path{0}, g_ovr_streamk{0}, g_ovr_tile_j{0}, g_ovr_mv_steps{0}, g_ovr_mv_kernel{0},
    g_ovr_fuse_cols{0};

qmm::Ovr load_ovr() {
    qmm::Ovr o;
    o.path = g_ovr_path.load();
    o.streamk = g_ovr_streamk.load();
    o.tile_j = g_ovr_tile_j.load();
    o.mv_steps = g_ovr_mv_steps.load();
    o.mv_kernel = g_ovr_mv_kernel.load();
    o.fuse_cols = g_ovr_fuse_cols.load();
    return o;
}

constexpr int64_t kMaxK = 1 << 20;
constexpr int64_t kMvMaxK = 32768;     // matrix-vector kernel stages k/32 scales in LDS
constexpr int kTI = 128;
constexpr int kSmallMax = 8;           // experts with <= 8 columns use the matrix-vector kernel

int block_values(int type) {
    switch (type) {
        case QMM_Q4_K: case QMM_Q5_K: case QMM_Q6_K: case QMM_Q3_K: case QMM_IQ4_XS: return 256;
        case QMM_Q8_0: case QMM_Q4_0: return 32;
        default: return 0;
    }
}
int block_bytes(int type) {
    switch (type) {
        case QMM_Q4_K: return 144;
        case QMM_Q5_K: return 176;
        case QMM_Q6_K: return 210;
        case QMM_Q8_0: return 34;
        case QMM_Q4_0: return 18;
        case QMM_Q3_K: return 110;
        case QMM_IQ4_XS: return 136;
        default: return 0;
    }
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

qmm_status check_common(int type, int64_t rows, int64_t k, int64_t n) {
    const int qk = block_values(type);
    if (qk == 0)
        return fail(QMM_ERR_TYPE, "unsupported weight type %d (supported: Q4_0=2, Q8_0=8, Q3_K=11, Q4_K=12, Q5_K=13, "
                    "Q6_K=14, IQ4_XS=23)", type);
    if (rows <= 0) return fail(QMM_ERR_ARG, "rows must be >= 1 (got %lld)", (long long)rows);
    if (n < 0) return fail(QMM_ERR_ARG, "n must be >= 0 (got %lld)", (long long)n);
    if (k <= 0 || k % qk != 0) return fail(QMM_ERR_SHAPE, "k=%lld is not a positive multiple of the block size %d", (long long)k, qk);
    if (k > kMaxK) return fail(QMM_ERR_SHAPE, "k=%lld exceeds the supported maximum %lld", (long long)k, (long long)kMaxK);
    if (rows > (1ll << 31) || n > (1ll << 31)) return fail(QMM_ERR_SHAPE, "rows/n too large");
    return QMM_OK;
}

// Shared-memory footprint of the tiled kernel, for its occupancy estimate.
// LDS bytes of one tiled-kernel workgroup (the Smem layout in mmq.hip): weight tile, fp32 row
// scales (and Q4_K mins), activation codes, fp32 (d, s).
int mmq_smem(int type, int J) {
    const bool k45 = type == QMM_Q4_K || type == QMM_Q5_K;
    const int wt = k45 ? kTI * 144 + (type == QMM_Q5_K ? kTI * 32 : 0)   // packed qs (+ Q5_K qh)
                       : (type == QMM_Q6_K || type == QMM_Q3_K ? 2 * kTI * 272 : kTI * 272);
    const int wm = k45 ? kTI * 48 + 8 * J * 4 : 0;   // bf16 pieces of the mins and of s
    const int one = wt + 8 * kTI * 4 + wm + J * 272 + 8 * (J + 4) * 8;
    return k45 && J == 128 ? 2 * one : one;   // Q4_K / Q5_K 8-wave tiles: two step buffers
}

// Tiled-kernel workgroups resident per compute unit: the kernels keep about 200 registers per
// lane, so two waves per SIMD (8 per CU): two 4-wave groups for J <= 64, one 8-wave group for
// J = 128; fewer if LDS runs out.
int mmq_resident(int type, int J) {
    const int by_waves = J == 128 ? 1 : 2;
    const int by_lds = (160 * 1024) / mmq_smem(type, J);
    return std::max(1, std::min(by_waves, by_lds));
}

}  // namespace

extern "C" {

const char *qmm_last_error(void) { return g_err.c_str(); }
const char *qmm_version(void) { return "qmm 0.1 (gfx950)"; }

int32_t qmm_tile_efficiency(int64_t ntiles, int32_t nsm) {
    if (ntiles <= 0 || nsm <= 0) return 0;
    const int64_t waves = (ntiles + nsm - 1) / nsm;
    return (int32_t)(100 * ntiles / (nsm * waves));
}

int32_t qmm_select_tile_j(int64_t ncols) {
    static const int32_t cand[] = {32, 64, 128};
    int32_t best = cand[0];
    int64_t best_tiles = INT64_MAX;
    for (int32_t J : cand) {
        const int64_t t = (ncols + J - 1) / J;
        if (t < best_tiles) { best_tiles = t; best = J; }
        if (best_tiles <= 1) break;
    }
    return best;
}

int64_t qmm_streamk_unit_start(int64_t u, int64_t units, int64_t ntiles, int64_t k_iters) {
    if (units <= 0 || u < 0) return 0;
    if (u > units) u = units;
    const int64_t W = ntiles * k_iters;
    return (u * W) / units;
}

qmm_status qmm_set_override(int key, int value) {
    switch (key) {
        case QMM_OVR_PATH:
            if (value < 0 || value > 2) return fail(QMM_ERR_ARG, "path override must be 0, 1 or 2");
            g_ovr_path = value; return QMM_OK;
        case QMM_OVR_STREAMK:
            if (value < 0 || value > 2) return fail(QMM_ERR_ARG, "stream-K override must be 0, 1 or 2");
            g_ovr_streamk = value; return QMM_OK;
        case QMM_OVR_TILE_J:
            if (value != 0 && value != 32 && value != 64 && value != 128)
                return fail(QMM_ERR_ARG, "tile width override must be 0, 32, 64 or 128");
            g_ovr_tile_j = value; return QMM_OK;
        case QMM_OVR_MV_STEPS:
            if (value != 0 && value != 1 && value != 2 && value != 4)
                return fail(QMM_ERR_ARG, "steps-per-wave override must be 0, 1, 2 or 4");
            g_ovr_mv_steps = value; return QMM_OK;
        case QMM_OVR_MV_KERNEL:
            if (value < 0 || value > 3) return fail(QMM_ERR_ARG, "matrix-vector kernel override must be 0..3");
            g_ovr_mv_kernel = value; return QMM_OK;
        case QMM_OVR_FUSE_COLS:
            if (value < 0 || value > 8) return fail(QMM_ERR_ARG, "fused-quantize column override must be 0..8");
            g_ovr_fuse_cols = value; return QMM_OK;
        default:
            return fail(QMM_ERR_ARG, "unknown override key %d", key);
    }
}

}  // extern "C"

namespace {

// Tile width of a dense tiled call, plain or fused gate/up: the fewest column tiles
// (qmm_select_tile_j), except where that is one 64-column tile (33-64 columns), measured the
// slowest of the three widths there (14336 x 4096 at 40-64 columns): Q6_K and Q3_K, whose planes
// are unpacked by half the threads in the 4-wave tiles, and Q8_0 take one 128-column tile (Q6_K /
// Q3_K 14-20 % faster, 40 % in the fused form; Q8_0 1-2 %), the other types two 32-column tiles
// (5-12 % faster).
int dense_tile_j(int type, int64_t n) {
    const int32_t J = qmm_select_tile_j(n);
    if (J != 64) return J;
    return type == QMM_Q6_K || type == QMM_Q3_K || type == QMM_Q8_0 ? 128 : 32;
}

// The planner under a given override snapshot (arguments already checked).
qmm_plan plan_dense_impl(int type, int64_t rows, int64_t k, int64_t n, int32_t nsm, const qmm::Ovr &o) {
    qmm_plan p{};
    const bool mv = o.path == 2 ? false : (n <= 8 && k <= kMvMaxK);
    p.k_iters = (k + 255) / 256;
    if (mv) {
        p.regime = 1;
        p.tile_i = 16;
        p.tile_j = 8;
        p.ntiles = (rows + 15) / 16;
        p.efficiency_pct = qmm_tile_efficiency(p.ntiles, nsm);
        p.units = p.ntiles;
        return p;
    }
    p.regime = 2;
    p.tile_i = kTI;
    p.tile_j = o.tile_j ? o.tile_j : dense_tile_j(type, n);
    const int64_t n_ct = (n + p.tile_j - 1) / p.tile_j;
    p.ntiles = ((rows + kTI - 1) / kTI) * n_ct;
    const int occ = mmq_resident(type, p.tile_j);
    const int32_t slots = nsm * occ;
    p.efficiency_pct = qmm_tile_efficiency(p.ntiles, slots);
    // stream-K pays a partial-tile round trip through memory and the last unit's sum: the MMQ
    // page's "when not to use stream-K" threshold, tile efficiency below 90 % (measured here: at
    // 87.5 % the split remainder is ~3 % faster, at 50 % 1.7x, at 100 % the plan takes no split)
    bool use_sk = p.efficiency_pct < 90 && p.k_iters > 1;
    if (o.streamk == 1) use_sk = false;
    if (o.streamk == 2) use_sk = p.k_iters > 1 || p.ntiles > 1;
    if (p.ntiles == 0) use_sk = false;   // n == 0: nothing to split (and no unit to divide by)
    p.stream_k = use_sk ? 1 : 0;
    const int64_t nwork = p.ntiles * p.k_iters;
    p.units = use_sk ? std::min<int64_t>(slots, nwork) : p.ntiles;
    p.fixup = use_sk && (p.ntiles % p.units != 0) ? 1 : 0;
    return p;
}

qmm_status check_plan_args(int type, int64_t rows, int64_t k, int64_t n, const qmm::Ovr &o) {
    qmm_status st = check_common(type, rows, k, n);
    if (st) return st;
    if (o.path == 1 && !(n <= 8 && k <= kMvMaxK))
        return fail(QMM_ERR_ARG, "matrix-vector path forced but n=%lld > 8 or k > %lld", (long long)n, (long long)kMvMaxK);
    return QMM_OK;
}

struct DenseWs {
    size_t xq_off, tiled_off, part_off, cnt_off, total;
    int64_t cnt_n;   // stream-K split-tile counters at cnt_off (zeroed by the activation launch)
};
DenseWs dense_layout(int type, int64_t rows, int64_t k, int64_t n, bool with_xq, const qmm::Ovr &o);

}  // namespace

extern "C" {

qmm_status qmm_plan_dense(int type, int64_t rows, int64_t k, int64_t n, int32_t nsm, qmm_plan *out) {
    const qmm::Ovr o = load_ovr();
    qmm_status st = check_plan_args(type, rows, k, n, o);
    if (st) return st;
    if (!out || nsm <= 0) return fail(QMM_ERR_ARG, "null plan pointer or nsm <= 0");
    out[0] = plan_dense_impl(type, rows, k, n, nsm, o);
    out[0].ws_bytes = dense_layout(type, rows, k, n, true, o).total;
    return QMM_OK;
}

// ----------------------------------------------------------------------------------------------
// Dense product
// ----------------------------------------------------------------------------------------------
namespace {

// Workspace of a dense call: canonical q8_1 blocks for fp32 input on the matrix-vector path (used
// only where the kernel does not quantize itself), the tiled-kernel activation layout and the
// stream-K partial slots on the tiled path.
DenseWs dense_layout(int type, int64_t rows, int64_t k, int64_t n, bool with_xq, const qmm::Ovr &o) {
    DenseWs L{};
    const int64_t nb = k / 32;
    const bool tiled = n > 8 || k > kMvMaxK || o.path == 2;   // as plan_dense_impl decides
    size_t off = 0;
    L.xq_off = off;
    if (with_xq && !tiled) off = align_up(off + (size_t)(n * nb * 36), 256);
    L.tiled_off = off;
    if (tiled) off = align_up(off + qmm::q8_1_tiled_bytes(n, k), 256);
    L.part_off = off;
    L.cnt_off = off;
    if (tiled) {
        // stream-K partial slots: at most (compute units x 2 resident) units x 2 slots x 128 x 128,
        // then one counter per tile of the most tiles any tile width gives
        const int64_t nsm = device_cus();
        const int64_t ntiles_max = ((rows + kTI - 1) / kTI) * ((n + 31) / 32);
        const int64_t units = std::min<int64_t>(2 * nsm, ntiles_max * ((k + 255) / 256));
        off = align_up(off + (size_t)(units * 2 * kTI * 128 * 4), 256);
        L.cnt_off = off;
        L.cnt_n = ntiles_max;
        off = align_up(off + (size_t)ntiles_max * 4, 256);
    }
    L.total = off;
    return L;
}

// The workspace a qmm_matmul of this shape uses under plan p exactly (qmm_matmul's own layout
// reserves stream-K slots for any plan, so that one size serves every override): the q8_1 copy on
// the matrix-vector path, the tiled activations and p's stream-K slots on the tiled path.
DenseWs dense_layout_exact(int64_t k, int64_t n, const qmm_plan &p) {
    DenseWs L{};
    size_t off = 0;
    L.xq_off = off;
    if (p.regime == 1) off = align_up(off + (size_t)(n * (k / 32) * 36), 256);
    L.tiled_off = off;
    if (p.regime == 2) off = align_up(off + qmm::q8_1_tiled_bytes(n, k), 256);
    L.part_off = off;
    L.cnt_off = off;
    if (p.regime == 2 && p.stream_k) {
        off = align_up(off + (size_t)p.units * 2 * kTI * p.tile_j * 4, 256);
        L.cnt_off = off;
        L.cnt_n = p.ntiles;
        off = align_up(off + (size_t)p.ntiles * 4, 256);
    }
    L.total = off;
    return L;
}

// xq: canonical q8_1 blocks, or (x_tiled) activations already in the tiled layout.  The plan,
// the workspace layout L and the kernel choices all come from the one override snapshot o.  dbg
// set: the integer-dot export of the planned kernel (the tiled kernel in its production plan,
// stream-K included, with only its epilogue changed; y is not written).
qmm_status run_dense(int type, const void *w, int64_t rows, int64_t k, const uint8_t *xq, int64_t n, float *y,
                     uint8_t *ws, const DenseWs &L, int32_t *dbg, const qmm::Ovr &o, hipStream_t s,
                     bool x_tiled = false, bool packed = false) {
    hipError_t e;
    const qmm_plan p = plan_dense_impl(type, rows, k, n, device_cus(), o);
    const bool tiled_ws = L.tiled_off != L.part_off;   // the layout reserved the tiled copy
    if (p.regime == 1) {
        if (x_tiled || packed) return fail(QMM_ERR_ARG, "internal: tiled activations or panel weights on the matrix-vector path");
        e = qmm::launch_mmvq(type, (const uint8_t *)w, rows, k, xq, n, y, dbg, nullptr, 0, o, s);
        if (e != hipSuccess) return hip_fail(e, "matrix-vector kernel launch");
        return QMM_OK;
    }
    if (!tiled_ws) return fail(QMM_ERR_ARG, "internal: workspace layout without the tiled activations");
    qmm::MmqLaunch ml{};
    ml.tile_j = p.tile_j;
    ml.ntiles = p.ntiles;
    ml.n_ct = (n + p.tile_j - 1) / p.tile_j;
    ml.k_iters = p.k_iters;
    ml.units = p.units;
    ml.stream_k = p.stream_k != 0;
    ml.partials = (float *)(ws + L.part_off);
    ml.counters = (int32_t *)(ws + L.cnt_off);
    ml.packed = packed;
    if (ml.stream_k && ((size_t)(L.part_off + (size_t)ml.units * 2 * kTI * p.tile_j * 4) > L.cnt_off ||
                        L.cnt_n < p.ntiles))
        return fail(QMM_ERR_WORKSPACE, "internal: stream-K partials or counters exceed the workspace");
    const uint8_t *xa = xq;
    if (!x_tiled) {
        e = qmm::launch_relayout_q8_1_tiled(xq, n, k, ws + L.tiled_off, s, (int32_t *)(ws + L.cnt_off), L.cnt_n);
        if (e != hipSuccess) return hip_fail(e, "relayout launch");
        xa = ws + L.tiled_off;
    }
    e = qmm::launch_mmq(type, (const uint8_t *)w, rows, k, xa, n, y, dbg, ml, s);
    if (e != hipSuccess) return hip_fail(e, "tiled kernel launch");
    return QMM_OK;
}

qmm_status check_ptrs_dense(const void *w, const void *x, const float *y, int64_t n) {
    if (n == 0) return QMM_OK;
    if (!w || !x || !y) return fail(QMM_ERR_ARG, "null w, x or y");
    if (((uintptr_t)w) & 1) return fail(QMM_ERR_ARG, "w must be 2-byte aligned");
    if (((uintptr_t)y) & 3) return fail(QMM_ERR_ARG, "y must be 4-byte aligned");
    return QMM_OK;
}

// fp32-input dense product once the arguments are checked; wsb holds at least L.total bytes.
qmm_status dense_f32(int type, const void *w, int64_t rows, int64_t k, const float *x, int64_t n, float *y,
                     uint8_t *wsb, const DenseWs &L, const qmm::Ovr &o, hipStream_t s) {
    const qmm_plan p = plan_dense_impl(type, rows, k, n, device_cus(), o);
    if (p.regime == 1) {
        const int fc = qmm::mmvq_fused_choice(type, w, rows, k, x, n, o);
        if (fc) {
            // few columns: the dot4 or LDS-staged kernel quantizes the activations itself (the same
            // q8_1 bytes as the quantize kernel below), one launch instead of two
            hipError_t e = qmm::launch_mmvq_fused(fc, type, (const uint8_t *)w, rows, k, x, n, y, s);
            if (e != hipSuccess) return hip_fail(e, "fused matrix-vector kernel launch");
            return QMM_OK;
        }
        hipError_t e = qmm::launch_quantize_q8_1(x, n, k, wsb + L.xq_off, s);
        if (e != hipSuccess) return hip_fail(e, "quantize launch");
        return run_dense(type, w, rows, k, wsb + L.xq_off, n, y, wsb, L, nullptr, o, s);
    }
    // tiled path: quantize straight into the tiled kernel's layout (and zero the stream-K counters)
    hipError_t e = qmm::launch_quantize_q8_1_tiled(x, n, k, wsb + L.tiled_off, nullptr, s, (int32_t *)(wsb + L.cnt_off),
                                                   L.cnt_n);
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    return run_dense(type, w, rows, k, wsb + L.tiled_off, n, y, wsb, L, nullptr, o, s, true);
}

}  // namespace

qmm_status qmm_quantize_q8_1(const float *x, int64_t n_rows, int64_t k, void *y, void *stream) {
    if (n_rows < 0) return fail(QMM_ERR_ARG, "n_rows must be >= 0");
    if (k <= 0 || k % 32 != 0) return fail(QMM_ERR_SHAPE, "k=%lld is not a positive multiple of 32", (long long)k);
    if (k > kMaxK) return fail(QMM_ERR_SHAPE, "k too large");
    if (n_rows == 0) return QMM_OK;
    if (!x || !y) return fail(QMM_ERR_ARG, "null x or y");
    if (((uintptr_t)x) & 15) return fail(QMM_ERR_ARG, "x must be 16-byte aligned");
    if (((uintptr_t)y) & 3) return fail(QMM_ERR_ARG, "y must be 4-byte aligned");
    hipError_t e = qmm::launch_quantize_q8_1(x, n_rows, k, (uint8_t *)y, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    return QMM_OK;
}

static size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

qmm_status qmm_encode_f16act(const float *x, int64_t n, int64_t k, void *y16, int32_t *e, float *bsum,
                             void *stream) {
    if (n < 0) return fail(QMM_ERR_ARG, "n must be >= 0");
    if (k <= 0 || k % 32 != 0) return fail(QMM_ERR_SHAPE, "k=%lld is not a positive multiple of 32", (long long)k);
    if (k > kMaxK) return fail(QMM_ERR_SHAPE, "k too large");
    if ((n * k + 255) / 256 >= ((int64_t)1 << 31)) return fail(QMM_ERR_SHAPE, "n * k too large");
    if (n == 0) return QMM_OK;
    if (!x || !y16 || !e || !bsum) return fail(QMM_ERR_ARG, "null pointer");
    if ((((uintptr_t)x) & 3) || (((uintptr_t)y16) & 1) || (((uintptr_t)e) & 3) || (((uintptr_t)bsum) & 3))
        return fail(QMM_ERR_ARG, "x, e, bsum must be 4-byte and y16 2-byte aligned");
    hipError_t h = qmm::launch_f16act_encode(x, n, k, (uint16_t *)y16, e, bsum, (hipStream_t)stream);
    if (h != hipSuccess) return hip_fail(h, "f16act encode launch");
    return QMM_OK;
}

size_t qmm_matmul_f16act_workspace(int64_t k, int64_t n) {
    if (k <= 0 || k % 32 != 0 || k > kMaxK || n < 0 || n > 8) return 0;
    return up256((size_t)(n * k) * 2) + 2 * up256((size_t)(n * (k / 32)) * 4);
}

qmm_status qmm_matmul_f16act(int type, const void *w, int64_t rows, int64_t k, const float *x, int64_t n, float *y,
                             void *ws, size_t ws_bytes, void *stream) {
    if (type != QMM_Q4_0 && type != QMM_Q8_0 && type != QMM_Q4_K && type != QMM_Q5_K && type != QMM_Q6_K)
        return fail(QMM_ERR_TYPE, "type %d: the fp16-activation mode serves Q4_0=2, Q8_0=8, Q4_K=12, Q5_K=13, Q6_K=14",
                    type);
    if (rows < 1) return fail(QMM_ERR_ARG, "rows must be >= 1");
    if (n < 0 || n > 8) return fail(QMM_ERR_ARG, "the fp16-activation mode takes 0..8 columns (n=%lld)", (long long)n);
    const int64_t qk = (type == QMM_Q4_0 || type == QMM_Q8_0) ? 32 : 256;
    if (k <= 0 || k % qk != 0) return fail(QMM_ERR_SHAPE, "k=%lld is not a positive multiple of %lld", (long long)k,
                                           (long long)qk);
    if (k > kMaxK) return fail(QMM_ERR_SHAPE, "k too large");
    if (rows >= ((int64_t)1 << 33)) return fail(QMM_ERR_SHAPE, "rows too large");
    if (n == 0) return QMM_OK;
    if (!w || !x || !y) return fail(QMM_ERR_ARG, "null w, x or y");
    const bool k45 = type == QMM_Q4_K || type == QMM_Q5_K;
    if (((uintptr_t)w) & (k45 ? 15 : 1)) return fail(QMM_ERR_ARG, k45 ? "w must be 16-byte aligned" : "w must be 2-byte aligned");
    if ((((uintptr_t)x) & 3) || (((uintptr_t)y) & 3)) return fail(QMM_ERR_ARG, "x and y must be 4-byte aligned");
    const size_t need = qmm_matmul_f16act_workspace(k, n);
    if (!ws || ws_bytes < need) return fail(QMM_ERR_WORKSPACE, "workspace needs %zu bytes", need);
    if (((uintptr_t)ws) & 255) return fail(QMM_ERR_ARG, "workspace must be 256-byte aligned");
    uint8_t *base = (uint8_t *)ws;
    uint16_t *y16 = (uint16_t *)base;
    int32_t *e = (int32_t *)(base + up256((size_t)(n * k) * 2));
    float *bsum = (float *)(base + up256((size_t)(n * k) * 2) + up256((size_t)(n * (k / 32)) * 4));
    hipStream_t s = (hipStream_t)stream;
    hipError_t h = qmm::launch_f16act_encode(x, n, k, y16, e, bsum, s);
    if (h != hipSuccess) return hip_fail(h, "f16act encode launch");
    h = qmm::launch_mmvq_f16act(type, (const uint8_t *)w, rows, k, y16, e, bsum, n, y, s);
    if (h != hipSuccess) return hip_fail(h, "f16act matrix-vector launch");
    return QMM_OK;
}

size_t qmm_matmul_workspace(int type, int64_t rows, int64_t k, int64_t n) {
    if (check_common(type, rows, k, n)) return 0;
    return dense_layout(type, rows, k, n, true, load_ovr()).total;
}

size_t qmm_matmul_q8_1_workspace(int type, int64_t rows, int64_t k, int64_t n) {
    if (check_common(type, rows, k, n)) return 0;
    return dense_layout(type, rows, k, n, false, load_ovr()).total;
}

qmm_status qmm_matmul(int type, const void *w, int64_t rows, int64_t k, const float *x, int64_t n, float *y,
                      void *ws, size_t ws_bytes, void *stream) {
    const qmm::Ovr o = load_ovr();
    qmm_status st = check_plan_args(type, rows, k, n, o);
    if (st) return st;
    if ((st = check_ptrs_dense(w, x, y, n))) return st;
    if (n == 0) return QMM_OK;
    if (((uintptr_t)x) & 15) return fail(QMM_ERR_ARG, "x must be 16-byte aligned");
    const DenseWs L = dense_layout(type, rows, k, n, true, o);
    if (L.total > 0 && (!ws || ws_bytes < L.total))
        return fail(QMM_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, L.total);
    if (((uintptr_t)ws) & 255) return fail(QMM_ERR_ARG, "workspace must be 256-byte aligned");
    return dense_f32(type, w, rows, k, x, n, y, (uint8_t *)ws, L, o, (hipStream_t)stream);
}

qmm_status qmm_matvec_kernel(int type, const void *w, int64_t rows, int64_t k, const void *x, int64_t n,
                             int32_t x_fp32, int32_t *out) {
    const qmm::Ovr o = load_ovr();
    qmm_status st = check_common(type, rows, k, n);
    if (st) return st;
    if (!out) return fail(QMM_ERR_ARG, "null out");
    if (n < 1 || n > 8 || k > kMvMaxK || o.path == 2) {
        *out = 0;
        return QMM_OK;
    }
    if (x_fp32) {
        if (((uintptr_t)x) & 15) return fail(QMM_ERR_ARG, "x must be 16-byte aligned");
        const int f = qmm::mmvq_fused_choice(type, w, rows, k, (const float *)x, n, o);
        if (f) {
            *out = f + 16;
            return QMM_OK;
        }
        x = (const void *)(uintptr_t)256;   // the q8_1 copy sits at the 256-byte aligned workspace start
    }
    *out = qmm::mmvq_kernel_choice(type, w, rows, k, x, n, nullptr, o);
    return QMM_OK;
}

qmm_status qmm_matmul_q8_1(int type, const void *w, int64_t rows, int64_t k, const void *xq, int64_t n, float *y,
                           void *ws, size_t ws_bytes, void *stream) {
    const qmm::Ovr o = load_ovr();
    qmm_status st = check_plan_args(type, rows, k, n, o);
    if (st) return st;
    if ((st = check_ptrs_dense(w, xq, y, n))) return st;
    if (n == 0) return QMM_OK;
    if (((uintptr_t)xq) & 3) return fail(QMM_ERR_ARG, "xq must be 4-byte aligned");
    const DenseWs L = dense_layout(type, rows, k, n, false, o);
    if (L.total > 0 && (!ws || ws_bytes < L.total))
        return fail(QMM_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, L.total);
    if (((uintptr_t)ws) & 255) return fail(QMM_ERR_ARG, "workspace must be 256-byte aligned");
    return run_dense(type, w, rows, k, (const uint8_t *)xq, n, y, (uint8_t *)ws, L, nullptr, o, (hipStream_t)stream);
}

// ----------------------------------------------------------------------------------------------
// Panel layout: one-time weight repack and the dense product that reads it
// ----------------------------------------------------------------------------------------------
namespace {

bool panel_type(int type) {
    return type == QMM_Q4_K || type == QMM_Q5_K || type == QMM_Q6_K || type == QMM_Q8_0 || type == QMM_Q4_0;
}

qmm_status check_panel_shape(int type, int64_t rows, int64_t k) {
    if (!panel_type(type))
        return fail(QMM_ERR_TYPE, "unsupported weight type %d (supported: Q4_0=2, Q8_0=8, Q4_K=12, Q5_K=13, Q6_K=14)", type);
    if (rows <= 0) return fail(QMM_ERR_ARG, "rows must be >= 1 (got %lld)", (long long)rows);
    if (k <= 0 || k % 256 != 0)
        return fail(QMM_ERR_SHAPE, "the panel layout needs k a positive multiple of 256 (got %lld)", (long long)k);
    if (k > kMaxK) return fail(QMM_ERR_SHAPE, "k=%lld exceeds the supported maximum %lld", (long long)k, (long long)kMaxK);
    if (rows > (1ll << 31)) return fail(QMM_ERR_SHAPE, "rows too large");
    return QMM_OK;
}

}  // namespace

uint64_t qmm_repack_bytes(int type, int64_t rows, int64_t k) {
    if (!panel_type(type) || rows <= 0 || rows > (1ll << 31) || k <= 0 || k % 256 != 0 || k > kMaxK) return 0;
    return (uint64_t)qmm::panel_bytes(type, rows, k);
}

qmm_status qmm_repack(int type, const void *w, int64_t rows, int64_t k, void *wp, uint64_t wp_bytes, void *stream) {
    qmm_status st = check_panel_shape(type, rows, k);
    if (st) return st;
    if (!w || !wp) return fail(QMM_ERR_ARG, "null w or wp");
    if (((uintptr_t)w) & 1) return fail(QMM_ERR_ARG, "w must be 2-byte aligned");
    if (((uintptr_t)wp) & 15) return fail(QMM_ERR_ARG, "wp must be 16-byte aligned");
    const uint64_t need = (uint64_t)qmm::panel_bytes(type, rows, k);
    if (wp_bytes < need)
        return fail(QMM_ERR_ARG, "wp holds %llu bytes, the panel layout needs %llu", (unsigned long long)wp_bytes,
                    (unsigned long long)need);
    hipError_t e = qmm::launch_repack_panels(type, (const uint8_t *)w, rows, k, (uint8_t *)wp, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "repack launch");
    return QMM_OK;
}

size_t qmm_matmul_packed_workspace(int type, int64_t rows, int64_t k, int64_t n) {
    if (check_common(type, rows, k, n) || k % 256 != 0 || !panel_type(type)) return 0;
    return dense_layout(type, rows, k, n, false, load_ovr()).total;
}

qmm_status qmm_matmul_packed(int type, const void *wp, int64_t rows, int64_t k, const float *x, int64_t n, float *y,
                             void *ws, size_t ws_bytes, void *stream) {
    const qmm::Ovr o = load_ovr();
    qmm_status st = check_panel_shape(type, rows, k);
    if (st) return st;
    if ((st = check_plan_args(type, rows, k, n, o))) return st;
    if ((st = check_ptrs_dense(wp, x, y, n))) return st;
    if (n == 0) return QMM_OK;
    if (((uintptr_t)wp) & 15) return fail(QMM_ERR_ARG, "wp must be 16-byte aligned");
    if (((uintptr_t)x) & 15) return fail(QMM_ERR_ARG, "x must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const qmm_plan p = plan_dense_impl(type, rows, k, n, device_cus(), o);
    if (p.regime == 1) {
        // few columns: the LDS-staged kernel quantizes x itself and parks each panel as it is
        hipError_t e = qmm::launch_mmvq_stream_panel_f32(type, (const uint8_t *)wp, rows, k, x, n, y, s);
        if (e != hipSuccess) return hip_fail(e, "panel matrix-vector kernel launch");
        return QMM_OK;
    }
    const DenseWs L = dense_layout(type, rows, k, n, false, o);
    if (L.total > 0 && (!ws || ws_bytes < L.total))
        return fail(QMM_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, L.total);
    if (((uintptr_t)ws) & 255) return fail(QMM_ERR_ARG, "workspace must be 256-byte aligned");
    uint8_t *wsb = (uint8_t *)ws;
    hipError_t e = qmm::launch_quantize_q8_1_tiled(x, n, k, wsb + L.tiled_off, nullptr, s, (int32_t *)(wsb + L.cnt_off),
                                                   L.cnt_n);
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    return run_dense(type, wp, rows, k, wsb + L.tiled_off, n, y, wsb, L, nullptr, o, s, true, true);
}

// ----------------------------------------------------------------------------------------------
// Dense gate/up fusion
// ----------------------------------------------------------------------------------------------
namespace {

bool glu_matvec(int64_t n, int64_t k, const qmm::Ovr &o) { return n <= 8 && k <= kMvMaxK && o.path != 2; }

size_t glu_ws(int64_t k, int64_t n, const qmm::Ovr &o) {
    return glu_matvec(n, k, o) ? align_up((size_t)(n * (k / 32) * 36), 256)
                               : align_up(qmm::q8_1_tiled_bytes(n, k), 256);
}

}  // namespace

size_t qmm_matmul_glu_workspace(int type, int64_t rows, int64_t k, int64_t n) {
    if (check_common(type, rows, k, n)) return 0;
    return glu_ws(k, n, load_ovr());
}

qmm_status qmm_matmul_glu(int type, const void *w_gate, const void *w_up, int64_t rows, int64_t k, const float *x,
                          int64_t n, float *y, void *ws, size_t ws_bytes, void *stream) {
    const qmm::Ovr o = load_ovr();
    qmm_status st = check_common(type, rows, k, n);
    if (st) return st;
    if ((st = check_ptrs_dense(w_gate, x, y, n))) return st;
    if (n == 0) return QMM_OK;
    if (!w_up) return fail(QMM_ERR_ARG, "null w_up");
    if (((uintptr_t)w_up) & 1) return fail(QMM_ERR_ARG, "w must be 2-byte aligned");
    if (((uintptr_t)x) & 15) return fail(QMM_ERR_ARG, "x must be 16-byte aligned");
    const size_t need = glu_ws(k, n, o);
    if (!ws || ws_bytes < need)
        return fail(QMM_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, need);
    if (((uintptr_t)ws) & 255) return fail(QMM_ERR_ARG, "workspace must be 256-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    uint8_t *wsb = (uint8_t *)ws;
    const uint8_t *wg = (const uint8_t *)w_gate, *wu = (const uint8_t *)w_up;
    hipError_t e;
    if (glu_matvec(n, k, o)) {
        // the dot4 or LDS-staged kernel quantizing x itself (one launch), as for one matrix
        const int kc = qmm::mmvq_glu_f32_choice(type, wg, wu, rows, k, x, n, o);
        if (kc == 3 || kc == 2) {
            e = kc == 3 ? qmm::launch_mmvq_dot4_glu_f32(type, wg, wu, rows, k, x, n, y, s)
                        : qmm::launch_mmvq_stream_glu(type, wg, wu, rows, k, x, true, n, y, nullptr, 0, s);
            if (e != hipSuccess) return hip_fail(e, "fused matrix-vector kernel launch");
            return QMM_OK;
        }
        e = qmm::launch_quantize_q8_1(x, n, k, wsb, s);
        if (e != hipSuccess) return hip_fail(e, "quantize launch");
        e = qmm::launch_mmvq_glu(type, wg, wu, rows, k, wsb, n, y, nullptr, 0, o, s);
        if (e != hipSuccess) return hip_fail(e, "fused matrix-vector kernel launch");
        return QMM_OK;
    }
    e = qmm::launch_quantize_q8_1_tiled(x, n, k, wsb, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "quantize launch");
    const int tile_j = o.tile_j ? o.tile_j : dense_tile_j(type, n);
    e = qmm::launch_mmq_glu(type, wg, wu, rows, k, wsb, n, y, tile_j, s);
    if (e != hipSuccess) return hip_fail(e, "fused tiled kernel launch");
    return QMM_OK;
}

size_t qmm_debug_subdots_workspace(int type, int64_t rows, int64_t k, int64_t n, int path) {
    if (check_common(type, rows, k, n) || (path != 1 && path != 2)) return 0;
    qmm::Ovr o = load_ovr();
    o.path = path;
    return dense_layout(type, rows, k, n, false, o).total;
}

qmm_status qmm_debug_subdots(int type, const void *w, int64_t rows, int64_t k, const void *xq, int64_t n, int path,
                             int32_t *d_out, void *ws, size_t ws_bytes, void *stream) {
    qmm_status st = check_common(type, rows, k, n);
    if (st) return st;
    if (path != 1 && path != 2) return fail(QMM_ERR_ARG, "path must be 1 (matrix-vector) or 2 (tiled)");
    if (path == 1 && (n > 8 || k > kMvMaxK)) return fail(QMM_ERR_ARG, "matrix-vector debug export needs n <= 8");
    if (n == 0) return QMM_OK;
    if (!w || !xq || !d_out) return fail(QMM_ERR_ARG, "null pointer");
    if ((((uintptr_t)w) & 1) || (((uintptr_t)xq) & 3) || (((uintptr_t)d_out) & 3))
        return fail(QMM_ERR_ARG, "w must be 2-byte, xq and d_out 4-byte aligned");
    // the plan a production call of this shape would take under the current overrides, with
    // the path forced
    qmm::Ovr o = load_ovr();
    o.path = path;
    const DenseWs L = dense_layout(type, rows, k, n, false, o);
    if (L.total > 0 && (!ws || ws_bytes < L.total))
        return fail(QMM_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, L.total);
    if (((uintptr_t)ws) & 255) return fail(QMM_ERR_ARG, "workspace must be 256-byte aligned");
    return run_dense(type, w, rows, k, (const uint8_t *)xq, n, nullptr, (uint8_t *)ws, L, d_out, o,
                     (hipStream_t)stream);
}

// ----------------------------------------------------------------------------------------------
// Expert-indexed product
// ----------------------------------------------------------------------------------------------
namespace {

struct IdWs {
    size_t invalid_off, xq_off, tiled_off, sorted_off, bounds_off, tstart_off, small_off, total;
};

IdWs id_layout(int64_t n_exp, int64_t k, int64_t n_tok, int64_t top_k, int64_t x_per_tok) {
    IdWs L{};
    const int64_t nb = k / 32;
    const int64_t nx = n_tok * x_per_tok;
    const int64_t pairs = n_tok * top_k;
    size_t off = 0;
    L.invalid_off = off; off = align_up(off + 4, 256);   // first, so the count is found from ws alone
    L.xq_off = off; off = align_up(off + (size_t)(nx * nb * 36), 256);           // small experts
    L.tiled_off = off; off = align_up(off + qmm::q8_1_tiled_bytes(nx, k), 256);   // tiled experts
    L.sorted_off = off; off = align_up(off + (size_t)(std::max<int64_t>(pairs, 1) * 4), 256);
    L.bounds_off = off; off = align_up(off + (size_t)((n_exp + 1) * 4), 256);
    L.tstart_off = off; off = align_up(off + (size_t)((n_exp + 1) * 4), 256);
    L.small_off = off; off = align_up(off + (size_t)(n_exp * 4), 256);
    L.total = off;
    return L;
}

int id_tile_j(int type, int64_t pairs, int64_t n_exp, const qmm::Ovr &o) {
    if (o.tile_j) return o.tile_j;
    // The MMQ page's "MoE skew": per-expert column counts are skewed, so the tile width follows
    // the columns of a typical expert, not the call's total: a quarter of the mean (on the Zipf
    // MoE shapes the median expert has 0.7x the mean with 8 experts, 0.4x with 128, and the last
    // tile of every expert is partly empty), then the smallest tile that covers it.  Measured on
    // 8 experts and on 128 experts, both with 128 columns on average (Q4_K): 32-column tiles 3-5 %
    // faster than 64 and 128.  Q6_K (and Q3_K, parked the same way) keeps 128: its 4-wave tiles
    // hold the unpacked planes and run one workgroup per CU (32 columns: 2x slower).
    if (type == QMM_Q6_K || type == QMM_Q3_K) return 128;
    const int64_t mean = pairs / (n_exp > 0 ? n_exp : 1);
    const int64_t typical = mean / 4;
    return typical > 64 ? 128 : (typical > 32 ? 64 : 32);
}

}  // namespace

size_t qmm_matmul_id_workspace(int type, int64_t n_exp, int64_t rows, int64_t k, int64_t n_tok, int64_t top_k,
                               int64_t x_per_tok) {
    if (check_common(type, rows, k, n_tok)) return 0;
    if (n_exp <= 0 || top_k <= 0 || (x_per_tok != 1 && x_per_tok != top_k)) return 0;
    return id_layout(n_exp, k, n_tok, top_k, x_per_tok).total;
}

namespace {

// Expert-indexed product; w_up not null: gate/up fusion (w the gate matrices, x_per_tok == 1).
qmm_status run_id(int type, const void *w, const void *w_up, int64_t n_exp, int64_t rows, int64_t k, const float *x,
                  int64_t x_per_tok, const int32_t *ids, int64_t n_tok, int64_t top_k, float *y, void *ws,
                  size_t ws_bytes, void *stream) {
    const qmm::Ovr o = load_ovr();
    qmm_status st = check_common(type, rows, k, n_tok);
    if (st) return st;
    if (n_exp <= 0 || n_exp > 32768) return fail(QMM_ERR_ARG, "n_exp must be in [1, 32768]");
    if (top_k <= 0) return fail(QMM_ERR_ARG, "top_k must be >= 1");
    if (x_per_tok != 1 && x_per_tok != top_k) return fail(QMM_ERR_ARG, "x_per_tok must be 1 or top_k");
    if (n_tok * top_k > (1ll << 30)) return fail(QMM_ERR_SHAPE, "too many (token, slot) pairs");
    const IdWs L = id_layout(n_exp, k, n_tok, top_k, x_per_tok);
    if (L.total > 0 && (!ws || ws_bytes < L.total))
        return fail(QMM_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, L.total);
    if (((uintptr_t)ws) & 255) return fail(QMM_ERR_ARG, "workspace must be 256-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    uint8_t *wsb = (uint8_t *)ws;
    int32_t *invalid = (int32_t *)(wsb + L.invalid_off);
    if (n_tok == 0) {
        hipError_t e = qmm::launch_fill_u32((uint32_t *)invalid, 1, 0u, s);
        return e == hipSuccess ? QMM_OK : hip_fail(e, "fill launch");
    }
    if (!w || !x || !ids || !y) return fail(QMM_ERR_ARG, "null w, x, ids or y");
    if (((uintptr_t)w) & 1 || ((uintptr_t)w_up) & 1) return fail(QMM_ERR_ARG, "w must be 2-byte aligned");
    if (((uintptr_t)x) & 15) return fail(QMM_ERR_ARG, "x must be 16-byte aligned");
    if (((uintptr_t)y) & 3 || ((uintptr_t)ids) & 3) return fail(QMM_ERR_ARG, "y and ids must be 4-byte aligned");

    const int64_t nx = n_tok * x_per_tok;
    const int64_t pairs = n_tok * top_k;
    uint8_t *xq = wsb + L.xq_off, *xt = wsb + L.tiled_off;
    const int tile_j = id_tile_j(type, pairs, n_exp, o);
    qmm::ColMap cm{};
    cm.sorted = (const int32_t *)(wsb + L.sorted_off);
    cm.bounds = (const int32_t *)(wsb + L.bounds_off);
    cm.tile_start = (const int32_t *)(wsb + L.tstart_off);
    cm.small = (const int32_t *)(wsb + L.small_off);
    cm.top_k = (int32_t)top_k;
    cm.x_per_tok = (int32_t)x_per_tok;
    cm.n_exp = (int32_t)n_exp;
    cm.w_expert_stride = rows * (k / block_values(type)) * block_bytes(type);
    cm.act_rows = nx;
    cm.pairs = pairs;
    const int small_max = k <= kMvMaxK ? kSmallMax : 0;
    hipError_t e;
    if (qmm::moe_prologue_fused((int32_t)n_exp)) {
        // grouping and the activations' quantization (both layouts) in one launch
        e = qmm::launch_moe_prologue(ids, pairs, (int32_t)n_exp, tile_j, small_max, (int32_t *)cm.sorted,
                                     (int32_t *)cm.bounds, (int32_t *)cm.tile_start, (int32_t *)cm.small, invalid, x,
                                     nx, k, xt, xq, device_cus(), s);
        if (e != hipSuccess) return hip_fail(e, "grouping and quantize launch");
    } else {
        e = qmm::launch_quantize_q8_1_tiled(x, nx, k, xt, xq, s);   // both layouts, one launch
        if (e != hipSuccess) return hip_fail(e, "quantize launch");
        e = qmm::launch_moe_group(ids, pairs, (int32_t)n_exp, tile_j, small_max, (int32_t *)cm.sorted,
                                  (int32_t *)cm.bounds, (int32_t *)cm.tile_start, (int32_t *)cm.small, invalid, s);
        if (e != hipSuccess) return hip_fail(e, "grouping launch");
    }
    // experts with <= 8 columns: matrix-vector kernel, one workgroup row per listed expert
    if (k <= kMvMaxK) {
        e = w_up ? qmm::launch_mmvq_glu(type, (const uint8_t *)w, (const uint8_t *)w_up, rows, k, xq, 0, y, &cm, n_exp, o, s)
                 : qmm::launch_mmvq(type, (const uint8_t *)w, rows, k, xq, 0, y, nullptr, &cm, n_exp, o, s);
        if (e != hipSuccess) return hip_fail(e, "expert matrix-vector launch");
    }
    // the rest: tiled kernel over the device-built column-tile list
    const int64_t mmq_experts = std::min<int64_t>(n_exp, pairs / (small_max + 1));
    const int64_t max_ct = (pairs + tile_j - 1) / tile_j + mmq_experts;
    e = qmm::launch_mmq_id(type, (const uint8_t *)w, (const uint8_t *)w_up, rows, k, xt, y, cm, tile_j, max_ct, s);
    if (e != hipSuccess) return hip_fail(e, "expert tiled launch");
    return QMM_OK;
}

}  // namespace

qmm_status qmm_matmul_id(int type, const void *w, int64_t n_exp, int64_t rows, int64_t k, const float *x,
                         int64_t x_per_tok, const int32_t *ids, int64_t n_tok, int64_t top_k, float *y, void *ws,
                         size_t ws_bytes, void *stream) {
    return run_id(type, w, nullptr, n_exp, rows, k, x, x_per_tok, ids, n_tok, top_k, y, ws, ws_bytes, stream);
}

size_t qmm_matmul_id_glu_workspace(int type, int64_t n_exp, int64_t rows, int64_t k, int64_t n_tok, int64_t top_k) {
    return qmm_matmul_id_workspace(type, n_exp, rows, k, n_tok, top_k, 1);
}

qmm_status qmm_matmul_id_glu(int type, const void *w_gate, const void *w_up, int64_t n_exp, int64_t rows, int64_t k,
                             const float *x, const int32_t *ids, int64_t n_tok, int64_t top_k, float *y, void *ws,
                             size_t ws_bytes, void *stream) {
    if (n_tok > 0 && !w_up) return fail(QMM_ERR_ARG, "null w_up");
    return run_id(type, w_gate, w_up, n_exp, rows, k, x, 1, ids, n_tok, top_k, y, ws, ws_bytes, stream);
}

qmm_status qmm_matmul_id_grouping_layout(int type, int64_t n_exp, int64_t k, int64_t n_tok, int64_t top_k,
                                         int64_t x_per_tok, int64_t *out) {
    if (!out) return fail(QMM_ERR_ARG, "null out");
    if (n_exp <= 0 || n_exp > 32768 || top_k <= 0 || n_tok < 0 || k <= 0 || (x_per_tok != 1 && x_per_tok != top_k))
        return fail(QMM_ERR_ARG, "bad expert-product shape");
    const IdWs L = id_layout(n_exp, k, n_tok, top_k, x_per_tok);
    out[0] = (int64_t)L.sorted_off;
    out[1] = (int64_t)L.bounds_off;
    out[2] = (int64_t)L.tstart_off;
    out[3] = (int64_t)L.small_off;
    out[4] = id_tile_j(type, n_tok * top_k, n_exp, load_ovr());
    out[5] = k <= kMvMaxK ? kSmallMax : 0;
    return QMM_OK;
}

qmm_status qmm_matmul_id_invalid_count(const void *ws, int64_t *out, void *stream) {
    if (!ws || !out) return fail(QMM_ERR_ARG, "null ws or out");
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "stream synchronize");
    int32_t v = 0;
    e = hipMemcpy(&v, ws, sizeof v, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "copy of the invalid-id count");
    *out = v;
    return QMM_OK;
}

}  // extern "C"

// ----------------------------------------------------------------------------------------------
// Hooks for the allocation-free dense entry point (noalloc.hip), which owns its scratch memory.
// ----------------------------------------------------------------------------------------------
namespace qmm {

Ovr load_overrides() { return load_ovr(); }

qmm_status report(qmm_status st, const char *msg) { return fail(st, "%s", msg); }

qmm_status matmul_exact_check(int type, const void *w, int64_t rows, int64_t k, const float *x, int64_t n,
                              const float *y, const Ovr &o, size_t *need) {
    qmm_status st = check_plan_args(type, rows, k, n, o);
    if (st) return st;
    if ((st = check_ptrs_dense(w, x, y, n))) return st;
    *need = 0;
    if (n == 0) return QMM_OK;
    if (((uintptr_t)x) & 15) return fail(QMM_ERR_ARG, "x must be 16-byte aligned");
    *need = dense_layout_exact(k, n, plan_dense_impl(type, rows, k, n, device_cus(), o)).total;
    return QMM_OK;
}

qmm_status matmul_exact_run(int type, const void *w, int64_t rows, int64_t k, const float *x, int64_t n, float *y,
                            uint8_t *ws, const Ovr &o, hipStream_t s) {
    const DenseWs L = dense_layout_exact(k, n, plan_dense_impl(type, rows, k, n, device_cus(), o));
    return dense_f32(type, w, rows, k, x, n, y, ws, L, o, s);
}

}  // namespace qmm
