// api.cpp -- the C ABI of libqmv: host-side validation, size queries, dispatch and
// path labels.  Validation is pure host code (no HIP call, no dereference of device
// pointers) so every error path can be exercised without a GPU.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>

#include "qmv_internal.h"

namespace qmv {

namespace {
thread_local char g_last_path[160] = "";

bool debug_on() {
    static const bool on = [] {
        const char *e = std::getenv("QMV_DEBUG");
        return e && std::strcmp(e, "0") != 0 && e[0] != '\0';
    }();
    return on;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int block_of(int32_t fmt) {
    switch (fmt) {
    case QMV_Q4_0: return 32;
    case QMV_Q6_K: return 256;
    case QMV_CB4: return 128;
    case QMV_AQ2X8: return 8;
    case QMV_CB8: return 1;  // one index byte per weight: no block structure
    case QMV_AQ3X8: return 8;
    }
    return 0;
}
// Registered pre-expanded q6_K planes, keyed by the codes pointer of the weights they
// were built from; the entry also holds the geometry and the other planes, so that a
// descriptor reusing the pointer with another layout does not pick up a stale plane.
struct PlaneEntry {
    const void *codes_hi, *scales, *super;
    int64_t n, k;
    const int8_t *plane;
};
std::mutex g_plane_mu;
std::unordered_map<const void *, PlaneEntry> g_planes;

bool exp_opted_out() {
    const char *e = std::getenv("QMV_Q6K_EXP");
    return e && std::strcmp(e, "0") == 0;
}

// The plane to use for w and the suffix its label carries.
const int8_t *plane_of(const qmv_weights *w, const char **suffix) {
    std::lock_guard<std::mutex> lock(g_plane_mu);
    auto it = g_planes.find(w->codes);
    if (it != g_planes.end()) {
        const PlaneEntry &e = it->second;
        if (e.n == w->n && e.k == w->k && e.codes_hi == w->codes_hi && e.scales == w->scales &&
            e.super == w->super) {
            *suffix = ".plane";
            return e.plane;
        }
        *suffix = "(fallback!)";  // recorded for this pointer, but not for this layout
        return nullptr;
    }
    *suffix = exp_opted_out() ? "(exp=off)" : "";
    return nullptr;
}

// Runs a GEMM launcher with the plane lookup and records the decorated label.
template <class F>
int gemm_with_plane(const char *call, const qmv_weights *w, int m, F &&launch) {
    const char *suffix = "";
    const int8_t *plane = plane_of(w, &suffix);
    const char *path = launch(plane);
    if (!path) return QMV_ERR_LIMIT;
    const std::string label = std::string(path) + suffix;
    return finish_launch(call, w, m, label.c_str());
}
}  // namespace

const DeviceInfo &device_info() {
    static DeviceInfo info = [] {
        DeviceInfo d{65536, 256};
        int dev = 0;
        if (hipGetDevice(&dev) == hipSuccess) {
            int v = 0;
            if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0)
                d.lds_per_block = v;
            if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
                d.num_cus = v;
        }
        return d;
    }();
    return info;
}

// Read on every call (unlike QMV_DEBUG) so a test can switch variants in one process.
const char *forced_path() {
    const char *e = std::getenv("QMV_FORCE_PATH");
    return e ? e : "";
}

int finish_launch(const char *call, const qmv_weights *w, int m, const char *path) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        std::fprintf(stderr, "qmv: %s launch failed: %s\n", call, hipGetErrorString(e));
        return QMV_ERR_HIP;
    }
    std::snprintf(g_last_path, sizeof g_last_path, "%s", path);
    if (debug_on())
        std::fprintf(stderr, "qmv: %s fmt=%d n=%lld k=%lld m=%d path=%s\n", call, w ? w->fmt : 0,
                     w ? (long long)w->n : 0LL, w ? (long long)w->k : 0LL, m, path);
    return QMV_OK;
}

}  // namespace qmv

using namespace qmv;

extern "C" {

int64_t qmv_plane_bytes(int32_t fmt, int64_t n, int64_t k, int32_t plane) {
    const int blk = block_of(fmt);
    if (!blk) return QMV_ERR_FORMAT;
    if (n <= 0 || k <= 0 || k % blk) return QMV_ERR_SHAPE;
    switch (fmt) {
    case QMV_Q4_0:
        if (plane == QMV_PLANE_CODES) return n * k / 2;
        if (plane == QMV_PLANE_SCALES) return n * (k / 32) * 2;
        break;
    case QMV_Q6_K:
        if (plane == QMV_PLANE_CODES) return n * k / 2;
        if (plane == QMV_PLANE_CODES_HI) return n * k / 4;
        if (plane == QMV_PLANE_SCALES) return n * (k / 16);
        if (plane == QMV_PLANE_SUPER) return n * (k / 256) * 2;
        break;
    case QMV_CB4:
        if (plane == QMV_PLANE_CODES) return n * k / 2;
        if (plane == QMV_PLANE_CODEBOOK) return n * (k / 128) * 32;
        break;
    case QMV_AQ2X8:
    case QMV_AQ3X8: {
        const int nc = fmt == QMV_AQ3X8 ? 3 : 2;
        if (plane == QMV_PLANE_CODES) return n * (k / 8) * nc;
        if (plane == QMV_PLANE_SCALES) return n * 2;
        if (plane == QMV_PLANE_CODEBOOK) return nc * 256 * 8 * 2;
        break;
    }
    case QMV_CB8:
        if (plane == QMV_PLANE_CODES) return n * k;
        if (plane == QMV_PLANE_CODEBOOK) return n * 256 * 2;
        break;
    }
    if (plane < 0 || plane > QMV_PLANE_CODEBOOK) return QMV_ERR_SHAPE;
    return 0;
}

int64_t qmv_weight_bytes(int32_t fmt, int64_t n, int64_t k) {
    int64_t total = 0;
    for (int p = 0; p <= QMV_PLANE_CODEBOOK; p++) {
        const int64_t b = qmv_plane_bytes(fmt, n, k, p);
        if (b < 0) return b;
        total += b;
    }
    return total;
}

int qmv_validate(const qmv_weights *w, int32_t m, int32_t xt) {
    if (!w) return QMV_ERR_NULL;
    const int blk = block_of(w->fmt);
    if (!blk) return QMV_ERR_FORMAT;
    if (w->n <= 0 || w->k <= 0 || w->k % blk) return QMV_ERR_SHAPE;
    // the 8-bit codebook kernels stream 64 index bytes per lane step; the format has no block
    if (w->fmt == QMV_CB8 && w->k % 64) return QMV_ERR_SHAPE;
    if (xt != QMV_F32 && xt != QMV_BF16) return QMV_ERR_DTYPE;
    if (m < 1 || m > QMV_MAX_BATCH) return QMV_ERR_BATCH;
    const void *need[5] = {w->codes, nullptr, nullptr, nullptr, nullptr};
    switch (w->fmt) {
    case QMV_Q4_0: need[1] = w->scales; break;
    case QMV_Q6_K: need[1] = w->codes_hi; need[2] = w->scales; need[3] = w->super; break;
    case QMV_CB4: need[1] = w->codebook; break;
    case QMV_AQ2X8:
    case QMV_AQ3X8: need[1] = w->scales; need[2] = w->codebook; break;
    case QMV_CB8: need[1] = w->codebook; break;
    }
    const int nneed = w->fmt == QMV_Q6_K ? 4 : (w->fmt == QMV_AQ2X8 || w->fmt == QMV_AQ3X8 ? 3 : 2);
    for (int i = 0; i < nneed; i++)
        if (!need[i]) return QMV_ERR_NULL;
    for (int i = 0; i < nneed; i++)
        if (!aligned16(need[i])) return QMV_ERR_ALIGN;
    if (w->n > INT32_MAX || w->k > INT32_MAX) return QMV_ERR_LIMIT;
    return QMV_OK;
}

int qmv_gemv(const qmv_weights *w, int32_t m, const void *x, int32_t xt, float *y, void *stream) {
    int rc = qmv_validate(w, m, xt);
    if (rc) return rc;
    if (!x || !y) return QMV_ERR_NULL;
    if (!aligned16(x) || !aligned16(y)) return QMV_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    const char *path = nullptr;
    switch (w->fmt) {
    case QMV_Q4_0: path = launch_gemv_q4_0(w, m, x, xt, y, s); break;
    case QMV_Q6_K: path = launch_gemv_q6k(w, m, x, xt, y, s); break;
    case QMV_CB4: path = launch_gemv_cb4(w, m, x, xt, y, s); break;
    case QMV_AQ2X8:
    case QMV_AQ3X8: path = launch_gemv_aq(w, m, x, xt, y, s); break;
    case QMV_CB8: path = launch_gemv_cb8(w, m, x, xt, y, s); break;
    }
    if (!path) return QMV_ERR_LIMIT;
    return finish_launch("qmv_gemv", w, m, path);
}

int64_t qmv_gemv_workspace_bytes(const qmv_weights *w, int32_t m) {
    if (!w) return QMV_ERR_NULL;
    const int blk = block_of(w->fmt);
    if (!blk) return QMV_ERR_FORMAT;
    if (w->n <= 0 || w->k <= 0 || w->k % blk) return QMV_ERR_SHAPE;
    if (m < 1 || m > QMV_MAX_BATCH) return QMV_ERR_BATCH;
    if (w->n > INT32_MAX || w->k > INT32_MAX) return 0;
    return aq_lut_workspace_bytes(w, m);
}

int qmv_gemv_ws(const qmv_weights *w, int32_t m, const void *x, int32_t xt, float *y, void *ws, int64_t ws_bytes,
                void *stream) {
    int rc = qmv_validate(w, m, xt);
    if (rc) return rc;
    const int64_t need = qmv_gemv_workspace_bytes(w, m);
    if (need < 0) return (int)need;
    if (need == 0) return qmv_gemv(w, m, x, xt, y, stream);
    if (!x || !y) return QMV_ERR_NULL;
    if (!aligned16(x) || !aligned16(y)) return QMV_ERR_ALIGN;
    if (!ws || ws_bytes < need) return QMV_ERR_WORKSPACE;
    if (!aligned16(ws)) return QMV_ERR_ALIGN;
    const char *path = launch_gemv_aq_lut(w, x, xt, y, ws, (hipStream_t)stream);
    if (!path) return QMV_ERR_LIMIT;
    return finish_launch("qmv_gemv_ws", w, m, path);
}

int qmv_gemv_q8(const qmv_weights *w, int32_t m, const int8_t *xq, const float *xs, float *y, void *stream) {
    int rc = qmv_validate(w, m, QMV_F32);
    if (rc) return rc;
    if (w->fmt != QMV_Q4_0 && w->fmt != QMV_Q6_K) return QMV_ERR_FORMAT;
    if (!xq || !xs || !y) return QMV_ERR_NULL;
    if (!aligned16(xq) || !aligned16(xs) || !aligned16(y)) return QMV_ERR_ALIGN;
    const char *path = w->fmt == QMV_Q4_0 ? launch_gemv_q4_0_q8(w, m, xq, xs, y, (hipStream_t)stream)
                                          : launch_gemv_q6k_q8(w, m, xq, xs, y, (hipStream_t)stream);
    if (!path) return QMV_ERR_LIMIT;
    return finish_launch("qmv_gemv_q8", w, m, path);
}

int qmv_dequant(const qmv_weights *w, float *out, void *stream) {
    int rc = qmv_validate(w, 1, QMV_F32);
    if (rc) return rc;
    if (!out) return QMV_ERR_NULL;
    if (!aligned16(out)) return QMV_ERR_ALIGN;
    const char *path = launch_dequant(w, out, (hipStream_t)stream);
    if (!path) return QMV_ERR_LIMIT;
    return finish_launch("qmv_dequant", w, 1, path);
}

int qmm_quant_act(const float *x, int32_t m, int64_t k, int8_t *xq, float *xs, void *stream) {
    if (!x || !xq || !xs) return QMV_ERR_NULL;
    if (m < 1) return QMV_ERR_BATCH;
    if (k <= 0 || k % 32) return QMV_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(xs)) return QMV_ERR_ALIGN;
    const char *path = launch_quant_act(x, m, k, xq, xs, (hipStream_t)stream);
    if (!path) return QMV_ERR_LIMIT;
    return finish_launch("qmm_quant_act", nullptr, m, path);
}

int qmv_read_ceiling(const void *p, int64_t bytes, uint32_t *sink, void *stream) {
    if (!p || !sink) return QMV_ERR_NULL;
    if (bytes <= 0 || bytes % 16) return QMV_ERR_SHAPE;
    if (!aligned16(p) || ((uintptr_t)sink & 3u)) return QMV_ERR_ALIGN;
    const char *path = launch_read_ceiling(p, bytes, sink, (hipStream_t)stream);
    if (!path) return QMV_ERR_LIMIT;
    return finish_launch("qmv_read_ceiling", nullptr, 1, path);
}

int64_t qmm_workspace_bytes(const qmv_weights *w, int32_t m) {
    if (!w) return QMV_ERR_NULL;
    if (w->fmt != QMV_Q6_K) return QMV_ERR_FORMAT;
    if (w->n <= 0 || w->k <= 0 || w->k % 256) return QMV_ERR_SHAPE;
    if (m < 1) return QMV_ERR_BATCH;
    // the GEMM's activation layout for mp = m rounded up to 128 tokens: xq int8 in MFMA
    // fragment order (mp * k bytes), then xs fp32 [k/32][mp] at a 256-byte aligned offset
    const int64_t mp = gemm_tokens(m);
    return (mp * w->k + 255) / 256 * 256 + mp * (w->k / 32) * 4;
}

// The quantized activations' place in a qmm_gemm workspace.
static void ws_parts(const qmv_weights *w, int32_t m, void *ws, int8_t **xq, float **xs) {
    const int64_t mp = gemm_tokens(m);
    *xq = (int8_t *)ws;
    *xs = (float *)((char *)ws + (mp * w->k + 255) / 256 * 256);
}

static int check_gemm(const qmv_weights *w, int32_t m) {
    int rc = qmv_validate(w, 1, QMV_F32);
    if (rc) return rc;
    if (w->fmt != QMV_Q6_K) return QMV_ERR_FORMAT;
    if (m < 1) return QMV_ERR_BATCH;
    return QMV_OK;
}

int qmm_gemm_q8(const qmv_weights *w, int32_t m, const int8_t *xq, const float *xs, float *y,
                void *stream) {
    int rc = check_gemm(w, m);
    if (rc) return rc;
    if (!xq || !xs || !y) return QMV_ERR_NULL;
    if (!aligned16(xq) || !aligned16(xs) || !aligned16(y)) return QMV_ERR_ALIGN;
    return gemm_with_plane("qmm_gemm_q8", w, m, [&](const int8_t *plane) {
        return launch_gemm_q6k(w, m, plane, xq, xs, y, nullptr, (hipStream_t)stream, false);
    });
}

int qmm_gemm_ws(const qmv_weights *w, int32_t m, const void *ws, int64_t ws_bytes, float *y, void *stream) {
    int rc = check_gemm(w, m);
    if (rc) return rc;
    if (!y) return QMV_ERR_NULL;
    const int64_t need = qmm_workspace_bytes(w, m);
    if (!ws || ws_bytes < need) return QMV_ERR_WORKSPACE;
    if (!aligned16(y) || ((uintptr_t)ws & 255u)) return QMV_ERR_ALIGN;
    int8_t *xq;
    float *xs;
    ws_parts(w, m, (void *)ws, &xq, &xs);
    return gemm_with_plane("qmm_gemm_ws", w, m, [&](const int8_t *plane) {
        return launch_gemm_q6k(w, m, plane, xq, xs, y, nullptr, (hipStream_t)stream, true);
    });
}

int qmm_partials(const qmv_weights *w, int32_t m, const int8_t *xq, int32_t *i32, void *stream) {
    int rc = check_gemm(w, m);
    if (rc) return rc;
    if (!xq || !i32) return QMV_ERR_NULL;
    if (!aligned16(xq) || !aligned16(i32)) return QMV_ERR_ALIGN;
    return gemm_with_plane("qmm_partials", w, m, [&](const int8_t *plane) {
        return launch_gemm_q6k(w, m, plane, xq, nullptr, nullptr, i32, (hipStream_t)stream);
    });
}

int qmm_gemm(const qmv_weights *w, int32_t m, const float *x, float *y, void *ws, int64_t ws_bytes,
             void *stream) {
    int rc = check_gemm(w, m);
    if (rc) return rc;
    if (!x || !y) return QMV_ERR_NULL;
    const int64_t need = qmm_workspace_bytes(w, m);
    if (!ws || ws_bytes < need) return QMV_ERR_WORKSPACE;
    if (!aligned16(x) || !aligned16(y) || ((uintptr_t)ws & 255u)) return QMV_ERR_ALIGN;
    int8_t *xq;
    float *xs;
    ws_parts(w, m, ws, &xq, &xs);
    const char *p1 = launch_quant_act(x, m, w->k, xq, xs, (hipStream_t)stream, (int)gemm_tokens(m));
    if (!p1) return QMV_ERR_LIMIT;
    rc = finish_launch("qmm_quant_act", w, m, p1);
    if (rc) return rc;
    return gemm_with_plane("qmm_gemm", w, m, [&](const int8_t *plane) {
        return launch_gemm_q6k(w, m, plane, xq, xs, y, nullptr, (hipStream_t)stream, true);
    });
}

int64_t qmm_plane_bytes(const qmv_weights *w) {
    int rc = qmv_validate(w, 1, QMV_F32);
    if (rc) return rc;
    if (w->fmt != QMV_Q6_K) return QMV_ERR_FORMAT;
    return gemm_plane_bytes(w->n, w->k);
}

int qmm_register_plane(const qmv_weights *w, void *plane, int64_t plane_bytes, void *stream) {
    const int64_t need = qmm_plane_bytes(w);
    if (need < 0) return (int)need;
    if (!plane) return QMV_ERR_NULL;
    if (plane_bytes < need) return QMV_ERR_WORKSPACE;
    if ((uintptr_t)plane & 255u) return QMV_ERR_ALIGN;
    if (exp_opted_out()) {  // explicit opt-out: nothing built, nothing recorded
        std::snprintf(g_last_path, sizeof g_last_path, "plane.q6k(exp=off)");
        return QMV_OK;
    }
    const char *path = launch_expand_q6k(w, (int8_t *)plane, (hipStream_t)stream);
    if (!path) return QMV_ERR_LIMIT;
    const int rc = finish_launch("qmm_register_plane", w, 1, path);
    if (rc) return rc;
    std::lock_guard<std::mutex> lock(g_plane_mu);
    g_planes[w->codes] = PlaneEntry{w->codes_hi, w->scales, w->super, w->n, w->k, (const int8_t *)plane};
    return QMV_OK;
}

int qmm_unregister_plane(const qmv_weights *w) {
    if (!w) return QMV_ERR_NULL;
    std::lock_guard<std::mutex> lock(g_plane_mu);
    g_planes.erase(w->codes);
    return QMV_OK;
}

int qmv_moe_ffn(const qmv_weights *gate, const qmv_weights *up, const qmv_weights *down,
                int32_t n_experts, const int32_t *ids, int32_t n_ids, const void *x, int32_t xt,
                float *h, float *y, void *stream) {
    int rc;
    if ((rc = qmv_validate(gate, 1, xt)) || (rc = qmv_validate(up, 1, xt)) ||
        (rc = qmv_validate(down, 1, QMV_F32)))
        return rc;
    if (gate->fmt != QMV_CB4 || up->fmt != QMV_CB4 || down->fmt != QMV_CB4) return QMV_ERR_FORMAT;
    if (gate->n != up->n || gate->k != up->k || down->k != gate->n || down->n != gate->k)
        return QMV_ERR_SHAPE;
    if (n_experts < 1) return QMV_ERR_SHAPE;
    if (n_ids < 1 || n_ids > 64) return QMV_ERR_BATCH;
    if (!ids || !x || !h || !y) return QMV_ERR_NULL;
    if (!aligned16(x) || !aligned16(h) || !aligned16(y) || ((uintptr_t)ids & 3u)) return QMV_ERR_ALIGN;
    const char *path = launch_moe_cb4(gate, up, down, n_experts, ids, n_ids, x, xt, h, y,
                                      (hipStream_t)stream);
    if (!path) return QMV_ERR_LIMIT;
    return finish_launch("qmv_moe_ffn", gate, n_ids, path);
}

const char *qmv_last_path(void) { return g_last_path; }

const char *qmv_strerror(int code) {
    switch (code) {
    case QMV_OK: return "ok";
    case QMV_ERR_NULL: return "a required pointer is NULL";
    case QMV_ERR_SHAPE: return "bad shape: n, k must be positive and k a multiple of the format's block";
    case QMV_ERR_FORMAT: return "unknown or unsupported weight format";
    case QMV_ERR_DTYPE: return "unknown activation dtype";
    case QMV_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QMV_ERR_BATCH: return "batch size out of range";
    case QMV_ERR_WORKSPACE: return "workspace missing or too small";
    case QMV_ERR_HIP: return "HIP launch failed";
    case QMV_ERR_LIMIT: return "size beyond the kernels' supported limit";
    }
    return "unknown status";
}

const char *qmv_version(void) { return "qmv 0.1 gfx950"; }

}  // extern "C"
