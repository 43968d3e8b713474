// pending.cpp -- launchers for variants that are not built yet: each reports
// "unsupported" so the C ABI returns QMV_ERR_LIMIT instead of launching anything.
#include "qmv_internal.h"

namespace qmv {
const char *launch_gemv_q6k(const qmv_weights *, int, const void *, int, float *, hipStream_t) { return nullptr; }
const char *launch_gemv_cb4(const qmv_weights *, int, const void *, int, float *, hipStream_t) { return nullptr; }
const char *launch_gemv_aq(const qmv_weights *, int, const void *, int, float *, hipStream_t) { return nullptr; }
const char *launch_dequant(const qmv_weights *, float *, hipStream_t) { return nullptr; }
const char *launch_quant_act(const float *, int, int64_t, int8_t *, float *, hipStream_t) { return nullptr; }
const char *launch_gemm_q6k(const qmv_weights *, int, const int8_t *, const float *, float *, int32_t *,
                            hipStream_t) { return nullptr; }
const char *launch_moe_ffn(const qmv_weights *, const qmv_weights *, const qmv_weights *, int,
                           const int32_t *, int, const void *, int, float *, float *, hipStream_t) {
    return nullptr;
}
}  // namespace qmv
