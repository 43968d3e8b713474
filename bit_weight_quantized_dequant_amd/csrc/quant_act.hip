// quant_act.hip -- per-32 int8 activation quantizer for the q6_K prefill GEMM.
//
// For each row and each 32-element block: amax = max |x|, xs = amax / 127 and
// xq = clamp(round-half-away-from-zero(x / xs), -127, 127), all in IEEE binary32
// (the divisions compile to hipcc's correctly rounded fp32 divide; roundf rounds
// halves away from zero), so the result is bit-identical to any correct binary32
// evaluation of the same formula.  An all-zero block gives xs = 0 and xq = 0.
// Eight lanes hold one block (four elements each); its maximum is combined with DPP.
// Two output layouts: row-major (xq [m][k], xs [m][k/32]) and the prefill GEMM's operand
// layout (FRAG): xq in int8 MFMA fragment order, [token group m/32][block k/32][64 lanes]
// [16 bytes], lane l holding token 32 g + l % 32 and k 32 c + 16 (l / 32) .. + 15; xs
// block-major, [k/32][mp] (mp = m rounded up to the GEMM's 128-token tile).
#include "device_common.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int TB = 256;

template <int CTRL>
QMV_DEV float dpp_max_step(float v) {
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false)));
}

QMV_DEV int8_t q1(float v, float xs) {
    float r = roundf(v / xs);
    r = fminf(fmaxf(r, -127.f), 127.f);
    return (int8_t)(int)r;
}

// Thread c handles elements 4c .. 4c+3 of the flattened [m][k] array (k % 32 == 0, so a
// block never straddles rows); the grid covers whole groups of eight threads.
template <bool FRAG>
__global__ void __launch_bounds__(TB) quant_act_kernel(const float *__restrict__ x, int8_t *__restrict__ xq,
                                                       float *__restrict__ xs, int64_t nchunks, int k, int mp) {
    const int64_t c = (int64_t)blockIdx.x * TB + threadIdx.x;
    const bool ok = c < nchunks;
    const float4 v = ok ? ((const float4 *)x)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = dpp_max_step<0xB1>(a);   // quad_perm [1,0,3,2]
    a = dpp_max_step<0x4E>(a);   // quad_perm [2,3,0,1]
    a = dpp_max_step<0x141>(a);  // row_half_mirror: max over the 8 lanes of the block
    if (!ok) return;
    const float scale = a / 127.0f;
    uint32_t packed = 0;
    if (a != 0.0f) {
        packed = (uint32_t)(uint8_t)q1(v.x, scale) | ((uint32_t)(uint8_t)q1(v.y, scale) << 8) |
                 ((uint32_t)(uint8_t)q1(v.z, scale) << 16) | ((uint32_t)(uint8_t)q1(v.w, scale) << 24);
    }
    if constexpr (FRAG) {
        const int64_t e = 4 * c, row = e / k;
        const int kk = (int)(e - row * k), blk = kk >> 5, o = kk & 31;
        const int64_t chunk = (row >> 5) * (k >> 5) + blk;
        const int lane = (int)(row & 31) + 32 * (o >> 4);
        *(uint32_t *)(xq + chunk * 1024 + 16 * lane + (o & 15)) = packed;
        if ((c & 7) == 0) xs[(int64_t)blk * mp + row] = scale;
    } else {
        ((uint32_t *)xq)[c] = packed;
        if ((c & 7) == 0) xs[c >> 3] = scale;
    }
}

}  // namespace

const char *launch_quant_act(const float *x, int m, int64_t k, int8_t *xq, float *xs, hipStream_t s, int mp) {
    const int64_t nchunks = (int64_t)m * k / 4;
    const int64_t grid = (nchunks + TB - 1) / TB;
    if (grid > INT32_MAX || k > INT32_MAX) return nullptr;
    if (mp > 0) {
        hipLaunchKernelGGL(quant_act_kernel<true>, dim3((unsigned)grid), dim3(TB), 0, s, x, xq, xs, nchunks, (int)k, mp);
        return "quant_act.dpp8.gemm-layout";
    }
    hipLaunchKernelGGL(quant_act_kernel<false>, dim3((unsigned)grid), dim3(TB), 0, s, x, xq, xs, nchunks, (int)k, 0);
    return "quant_act.dpp8";
}

}  // namespace qmv
