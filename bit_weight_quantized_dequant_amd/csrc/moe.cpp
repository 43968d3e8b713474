// Format dispatch of the routed-expert FFN: an unsupported format combination reports
// "unsupported" (nullptr) so the C ABI returns QMV_ERR_LIMIT instead of launching.
#include "qmv_internal.h"

namespace qmv {

const char *launch_moe_ffn(const qmv_weights *gate, const qmv_weights *up, const qmv_weights *down,
                           int n_experts, const int32_t *ids, int n_ids, const void *x, int xt, float *h,
                           float *y, hipStream_t s) {
    if (gate->fmt == QMV_CB4 && up->fmt == QMV_CB4 && down->fmt == QMV_CB4)
        return launch_moe_cb4(gate, up, down, n_experts, ids, n_ids, x, xt, h, y, s);
    return nullptr;
}
}  // namespace qmv
