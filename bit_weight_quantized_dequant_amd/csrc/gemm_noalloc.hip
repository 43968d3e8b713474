// gemm_noalloc.hip -- qmm_gemm without a caller-supplied workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// qmm_gemm quantizes the activations into a workspace (int8 codes in MFMA fragment order,
// then the fp32 block scales at a 256-byte aligned offset, both padded to whole 128-token
// tiles) and contracts against it.  Here that workspace is
// a file-scope device array of QMV_NOALLOC_SCRATCH_BYTES.  Every GPU the library runs on
// holds its own copy until the process ends.  Host code never passes the array's name to
// a kernel (on the host it is only a stand-in symbol): the device address of each GPU's
// copy is looked up once per device with hipGetSymbolAddress, with that device current,
// and kept; the kernels take that address as their workspace argument.
//
// Every call on one GPU shares that GPU's array.  Calls that overlap on one GPU (other
// streams, other host threads) race on it; the caller orders them.  Nothing in the array
// has to start at zero: the quantizer writes every xq and xs value the contraction reads.
#include <mutex>

#include "qmv_internal.h"

namespace qmv {
namespace {

__device__ __align__(256) static uint8_t scratch[QMV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// The device address of the current device's copy of `scratch` (looked up on the device's
// first call), or nullptr when the lookup fails.
void *scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace
}  // namespace qmv

using namespace qmv;

extern "C" int qmm_gemm_noalloc(const qmv_weights *w, int32_t m, const float *x, float *y, void *stream) {
    // host-only checks first, so that a bad call fails before any HIP call
    const int64_t need = qmm_workspace_bytes(w, m);
    if (need < 0) return (int)need;
    const int rc = qmv_validate(w, 1, QMV_F32);
    if (rc) return rc;
    if (!x || !y) return QMV_ERR_NULL;
    if (((uintptr_t)x & 15u) || ((uintptr_t)y & 15u)) return QMV_ERR_ALIGN;
    if (need > QMV_NOALLOC_SCRATCH_BYTES) return QMV_ERR_LIMIT;
    void *ws = scratch_ptr();
    if (!ws) {
        (void)hipGetLastError();
        return QMV_ERR_HIP;
    }
    return qmm_gemm(w, m, x, y, ws, need, stream);
}
