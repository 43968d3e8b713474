// qmv_internal.h -- host-side declarations shared by the libqmv translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qmv.h"

namespace qmv {

// Device facts read once per process (thread-safe static init).
struct DeviceInfo {
    int lds_per_block;  // bytes of LDS one workgroup may use
    int num_cus;
};
const DeviceInfo &device_info();

// Records the label of the launched variant (thread-local) and prints it when
// QMV_DEBUG=1.  Returns QMV_OK or QMV_ERR_HIP after checking hipGetLastError.
int finish_launch(const char *call, const qmv_weights *w, int m, const char *path);

// Optional forced variant for tests (QMV_FORCE_PATH); empty string when unset.
const char *forced_path();

// Kernel launchers.  Arguments are already validated; each returns the label of the
// variant it launched, or nullptr when the shape is outside what it supports.
const char *launch_gemv_q4_0(const qmv_weights *w, int m, const void *x, int xt, float *y,
                             hipStream_t s);
// q4_0 over per-32 int8 activations (xq int8 [m][k], xs fp32 [m][k/32]).
const char *launch_gemv_q4_0_q8(const qmv_weights *w, int m, const int8_t *xq, const float *xs, float *y,
                                hipStream_t s);
// q6_K over per-32 int8 activations (the same arithmetic as the q6_K contraction).
const char *launch_gemv_q6k_q8(const qmv_weights *w, int m, const int8_t *xq, const float *xs, float *y,
                               hipStream_t s);
const char *launch_gemv_q6k(const qmv_weights *w, int m, const void *x, int xt, float *y,
                            hipStream_t s);
const char *launch_gemv_cb4(const qmv_weights *w, int m, const void *x, int xt, float *y,
                            hipStream_t s);
const char *launch_gemv_aq(const qmv_weights *w, int m, const void *x, int xt, float *y,
                           hipStream_t s);
// Additive formats at batch 1 through per-slice lookup tables (split k, workspace ws as
// qmv_gemv_ws describes).  aq_lut_workspace_bytes: its workspace size, 0 when (w, m) has no
// such kernel.
int64_t aq_lut_workspace_bytes(const qmv_weights *w, int m);
const char *launch_gemv_aq_lut(const qmv_weights *w, const void *x, int xt, float *y, void *ws, hipStream_t s);
const char *launch_gemv_cb8(const qmv_weights *w, int m, const void *x, int xt, float *y,
                            hipStream_t s);
const char *launch_dequant(const qmv_weights *w, float *out, hipStream_t s);
// The stream-read ceiling: reads `bytes` (a multiple of 16) from p and nothing else.
const char *launch_read_ceiling(const void *p, int64_t bytes, uint32_t *sink, hipStream_t s);
// mp > 0: the prefill GEMM's operand layout (xq in MFMA fragment order, xs [k/32][mp]);
// else row-major xq [m][k], xs [m][k/32].
const char *launch_quant_act(const float *x, int m, int64_t k, int8_t *xq, float *xs, hipStream_t s, int mp = 0);
// Tokens of the prefill GEMM's activation layout: m rounded up to its 128-token tile.
inline int64_t gemm_tokens(int64_t m) { return (m + 127) / 128 * 128; }
// plane: the registered pre-expanded plane of w (h and l bytes in MFMA fragment order, see
// qmm_plane_bytes), or nullptr for the in-kernel expansion of the codes.
// frag: xq / xs are in the GEMM's operand layout (launch_quant_act with mp); else row-major.
const char *launch_gemm_q6k(const qmv_weights *w, int m, const int8_t *plane, const int8_t *xq, const float *xs,
                            float *y, int32_t *partials, hipStream_t s, bool frag = false);
const char *launch_expand_q6k(const qmv_weights *w, int8_t *plane, hipStream_t s);
// Bytes of the pre-expanded q6_K plane of an n x k matrix (32-row groups in MFMA fragment
// order, h and l bytes).
int64_t gemm_plane_bytes(int64_t n, int64_t k);
const char *launch_moe_cb4(const qmv_weights *gate, const qmv_weights *up, const qmv_weights *down,
                           int n_experts, const int32_t *ids, int n_ids, const void *x, int xt,
                           float *h, float *y, hipStream_t s);

}  // namespace qmv
