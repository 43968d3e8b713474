// dequant.hip -- dense fp32 dequantization of every format (the unpack stage alone).
//
// One thread per group of weights that one 128-bit code load covers.  q4_0, q6_K and
// 4-bit-codebook weights are exactly representable in fp32 (q4_0: an fp16 scale times a
// 4-bit integer; q6_K: fp16 d times an int8 sub-scale times a 6-bit integer, at most
// 11 + 7 + 6 significant bits; the codebook: fp16 entries), so those outputs are exact.
// The additive code sums two fp16 codebook entries and multiplies by the row scale in
// fp32 (two roundings).  Layouts: see include/qmv.h.
#include "device_common.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int TB = 256;

__global__ void __launch_bounds__(TB) dq_q4_0(const uint8_t *__restrict__ qs, const uint16_t *__restrict__ dsc,
                                              float *__restrict__ out, int64_t nblocks) {
    const int64_t i = (int64_t)blockIdx.x * TB + threadIdx.x;
    if (i >= nblocks) return;
    const uint4 q = *(const uint4 *)(qs + i * 16);
    const float d = h2f(dsc[i]);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float4 *o = (float4 *)(out + i * 32);
#pragma unroll
    for (int j = 0; j < 4; j++) {
        o[j] = make_float4(d * (float)((int)(w[j] & 15) - 8), d * (float)((int)((w[j] >> 8) & 15) - 8),
                           d * (float)((int)((w[j] >> 16) & 15) - 8), d * (float)((int)((w[j] >> 24) & 15) - 8));
        o[4 + j] = make_float4(d * (float)((int)((w[j] >> 4) & 15) - 8), d * (float)((int)((w[j] >> 12) & 15) - 8),
                               d * (float)((int)((w[j] >> 20) & 15) - 8), d * (float)((int)((w[j] >> 28) & 15) - 8));
    }
}

// One thread per 64-weight unit (half h, offset 16*odd) of a q6_K super-block.
__global__ void __launch_bounds__(TB) dq_q6k(const uint8_t *__restrict__ ql, const uint8_t *__restrict__ qh,
                                             const int8_t *__restrict__ sc, const uint16_t *__restrict__ dsup,
                                             float *__restrict__ out, int64_t nunits) {
    const int64_t i = (int64_t)blockIdx.x * TB + threadIdx.x;
    if (i >= nunits) return;
    const int64_t sb = i >> 2;
    const int h = (int)((i >> 1) & 1), odd = (int)(i & 1);
    const uint8_t *a = ql + sb * 128 + 64 * h + 16 * odd;
    const uint8_t *hb = qh + sb * 64 + 32 * h + 16 * odd;
    const float d = h2f(dsup[sb]);
    float *o = out + sb * 256 + 128 * h + 16 * odd;
#pragma unroll
    for (int t = 0; t < 4; t++) {
        const float s = d * (float)sc[sb * 16 + 8 * h + 2 * t + odd];
        for (int j = 0; j < 16; j++) {
            const int lo = (a[j + 32 * (t & 1)] >> (4 * (t >> 1))) & 15;
            const int hi = (hb[j] >> (2 * t)) & 3;
            o[32 * t + j] = s * (float)((lo | (hi << 4)) - 32);
        }
    }
}

// One thread per 32 weights (16 index bytes).
__global__ void __launch_bounds__(TB) dq_cb4(const uint8_t *__restrict__ idx, const uint16_t *__restrict__ cb,
                                             float *__restrict__ out, int64_t nchunks) {
    const int64_t i = (int64_t)blockIdx.x * TB + threadIdx.x;
    if (i >= nchunks) return;
    const uint4 q = *(const uint4 *)(idx + i * 16);
    const uint16_t *tab = cb + (i >> 2) * 16;  // 4 chunks of 32 weights per 128-weight group
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float *o = out + i * 32;
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
        for (int e = 0; e < 8; e++) o[8 * j + e] = h2f(tab[(w[j] >> (4 * e)) & 15]);
}

// One thread per 8-weight group of an NC-codebook additive code: s * ((C1 + C2) + C3).
template <int NC>
__global__ void __launch_bounds__(TB) dq_aq(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ cbk,
                                            const uint16_t *__restrict__ srow, float *__restrict__ out,
                                            int64_t ngroups, int64_t groups_per_row) {
    const int64_t i = (int64_t)blockIdx.x * TB + threadIdx.x;
    if (i >= ngroups) return;
    const float s = h2f(srow[i / groups_per_row]);
    float *o = out + i * 8;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        float v = h2f(cbk[codes[NC * i] * 8 + j]);
#pragma unroll
        for (int b = 1; b < NC; b++) v += h2f(cbk[2048 * b + codes[NC * i + b] * 8 + j]);
        o[j] = s * v;
    }
}

// One thread per 16 weights (16 index bytes) of the 8-bit codebook format.
__global__ void __launch_bounds__(TB) dq_cb8(const uint8_t *__restrict__ idx, const uint16_t *__restrict__ cb,
                                             float *__restrict__ out, int64_t nchunks, int64_t chunks_per_row) {
    const int64_t i = (int64_t)blockIdx.x * TB + threadIdx.x;
    if (i >= nchunks) return;
    const uint4 q = *(const uint4 *)(idx + i * 16);
    const uint16_t *tab = cb + (i / chunks_per_row) * 256;
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float *o = out + i * 16;
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
        for (int e = 0; e < 4; e++) o[4 * j + e] = h2f(tab[(w[j] >> (8 * e)) & 255]);
}

int grid_of(int64_t n) { return (int)((n + TB - 1) / TB); }

}  // namespace

const char *launch_dequant(const qmv_weights *w, float *out, hipStream_t s) {
    const int64_t n = w->n, k = w->k;
    if (n * k / 8 > (int64_t)INT32_MAX * TB) return nullptr;
    switch (w->fmt) {
    case QMV_Q4_0:
        hipLaunchKernelGGL(dq_q4_0, dim3(grid_of(n * k / 32)), dim3(TB), 0, s, (const uint8_t *)w->codes,
                           (const uint16_t *)w->scales, out, n * k / 32);
        return "dequant.q4_0";
    case QMV_Q6_K:
        hipLaunchKernelGGL(dq_q6k, dim3(grid_of(n * k / 64)), dim3(TB), 0, s, (const uint8_t *)w->codes,
                           (const uint8_t *)w->codes_hi, (const int8_t *)w->scales, (const uint16_t *)w->super,
                           out, n * k / 64);
        return "dequant.q6_K";
    case QMV_CB4:
        hipLaunchKernelGGL(dq_cb4, dim3(grid_of(n * k / 32)), dim3(TB), 0, s, (const uint8_t *)w->codes,
                           (const uint16_t *)w->codebook, out, n * k / 32);
        return "dequant.cb4";
    case QMV_AQ2X8:
        hipLaunchKernelGGL(dq_aq<2>, dim3(grid_of(n * k / 8)), dim3(TB), 0, s, (const uint8_t *)w->codes,
                           (const uint16_t *)w->codebook, (const uint16_t *)w->scales, out, n * k / 8, k / 8);
        return "dequant.aq2x8";
    case QMV_AQ3X8:
        hipLaunchKernelGGL(dq_aq<3>, dim3(grid_of(n * k / 8)), dim3(TB), 0, s, (const uint8_t *)w->codes,
                           (const uint16_t *)w->codebook, (const uint16_t *)w->scales, out, n * k / 8, k / 8);
        return "dequant.aq3x8";
    case QMV_CB8:
        hipLaunchKernelGGL(dq_cb8, dim3(grid_of(n * k / 16)), dim3(TB), 0, s, (const uint8_t *)w->codes,
                           (const uint16_t *)w->codebook, out, n * k / 16, k / 16);
        return "dequant.cb8";
    }
    return nullptr;
}

}  // namespace qmv
