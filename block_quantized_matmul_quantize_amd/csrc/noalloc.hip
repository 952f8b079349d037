// Allocation-free dense entry point: qmm_matmul with its workspace in a device buffer the library
// owns, for callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// `scratch` below is a file-scope device array: the code object loader gives every GPU the library
// runs on its own copy, held until the process ends.  In host code its name is only a host-side
// stand-in, never a device address; the device address of the current GPU's copy is looked up once
// per device with hipGetSymbolAddress and kept in scratch_base[], and only that address is handed
// to kernels.  The calls share the copy of their GPU, so two calls that overlap on one GPU race
// (callers serialise them, e.g. on one stream).  Nothing in it has to start at zero: every byte a
// call reads (q8_1 activations, stream-K partial slots and counters) is written earlier in that
// same call (the counters by the activation quantization launch).
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace {

constexpr size_t kScratchBytes = QMM_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
uint8_t *scratch_base[kMaxDevices];   // device address of `scratch` on each device, once looked up

// Device address of the current device's copy of `scratch` (looked up on the first call made
// with that device current).
qmm_status scratch_for_current_device(uint8_t **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return qmm::report(QMM_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return qmm::report(QMM_ERR_HIP, "device index out of range");
    std::lock_guard<std::mutex> lk(scratch_mu);
    if (!scratch_base[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return qmm::report(QMM_ERR_HIP, "hipGetSymbolAddress(scratch) failed");
        if (((uintptr_t)p) & 255) return qmm::report(QMM_ERR_HIP, "scratch is not 256-byte aligned");
        scratch_base[dev] = (uint8_t *)p;
    }
    *out = scratch_base[dev];
    return QMM_OK;
}

}  // namespace

extern "C" qmm_status qmm_matmul_noalloc(int type, const void *w, int64_t rows, int64_t k, const float *x, int64_t n,
                                         float *y, void *stream) {
    const qmm::Ovr o = qmm::load_overrides();
    size_t need = 0;
    qmm_status st = qmm::matmul_exact_check(type, w, rows, k, x, n, y, o, &need);
    if (st) return st;
    if (n == 0) return QMM_OK;
    if (need > kScratchBytes) {
        char msg[256];
        snprintf(msg, sizeof msg,
                 "this call needs %zu bytes of workspace; the allocation-free entry point holds %zu "
                 "(use qmm_matmul with a caller-provided workspace)",
                 need, kScratchBytes);
        return qmm::report(QMM_ERR_WORKSPACE, msg);
    }
    uint8_t *base = nullptr;
    if ((st = scratch_for_current_device(&base))) return st;
    return qmm::matmul_exact_run(type, w, rows, k, x, n, y, base, o, (hipStream_t)stream);
}
