// gemv_q4_0.hip -- q4_0 decode GEMV for gfx950.
//
// y[m][n] = sum_k d[n][k/32] * (q[n][k] - 8) * x[m][k]   (q4_0: 32 weights per block,
// 16 code bytes + an fp16 scale; "LLMs on the Xiaomi TV Box", §11.5 E18 gives its
// 4.5 bits per weight).  The GEMV streams weight bytes, so its roofline is HBM
// bandwidth (quantprobe LAWS.md, Law 4); L-15 says the unpack instructions are the
// tax on top, so the unpack here is a handful of SWAR ops per 8 weights:
//
//   * Each lane owns whole blocks: one 128-bit load of 16 code bytes + one fp16 scale.
//   * Activations for the workgroup are staged once into LDS as fp32, 32 per block
//     (row stride 36 floats so that eight lanes reading eight blocks with ds_read_b128
//     touch disjoint banks), together with each block's sum sum_k x[k].
//   * The offset is folded per block: sum (q-8) x = sum q x - 8 sum x.
//   * A dword of codes is split by masks 0x000F000F / 0x00F000F0 into pairs of binary16
//     subnormals whose bit patterns are the codes (value q * 2^-24, or q * 2^-20 for the
//     high nibble of a byte); v_fma_mix_f32 consumes a binary16 half directly, so each
//     weight costs one FMA plus 5/8 of a bitwise op, and the products are exact.
//   * The 64 lane partials of a row are summed across the wavefront.
#include <cstring>

#include "device_common.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int WG = 512;  // threads per workgroup: 8 waves
constexpr int WAVES = WG / 64;
constexpr int XS = 36;   // floats per staged 32-activation block

// Stage x [M][k] into LDS: block (m, b) at sx[(m*nblk + b)*XS], its sum at ssum[m*nblk + b].
template <int M, int XT>
__device__ void stage_x32(const void *x, int k, float *sx, float *ssum) {
    const int nblk = k >> 5;
    for (int i = threadIdx.x; i < M * nblk; i += WG) {
        const int m = i / nblk, b = i - m * nblk;
        float v[32];
#pragma unroll
        for (int j = 0; j < 4; j++) ld_act8<XT>(x, (int64_t)m * k + b * 32 + 8 * j, v + 8 * j);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 32; e++) s += v[e];
        float4 *dst = (float4 *)(sx + i * XS);
#pragma unroll
        for (int j = 0; j < 8; j++) dst[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
        ssum[i] = s;
    }
}

// sum_{i<32} q_i * x_i for one block (codes q in 4 dwords, staged x at xb), exact products.
QMV_DEV float dot_q4_mix(uint4 q, const float *xb) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float4 xl = *(const float4 *)(xb + 4 * i);       // weights 4i .. 4i+3
        const float4 xh = *(const float4 *)(xb + 16 + 4 * i);  // weights 16+4i .. 16+4i+3
        const uint32_t w8 = w[i] >> 8;
        const uint32_t t0 = w[i] & 0x000F000Fu;  // byte 0 / byte 2, low nibbles   (x 2^-24)
        const uint32_t t1 = w[i] & 0x00F000F0u;  // byte 0 / byte 2, high nibbles  (x 2^-20)
        const uint32_t t2 = w8 & 0x000F000Fu;    // byte 1 / byte 3, low nibbles
        const uint32_t t3 = w8 & 0x00F000F0u;    // byte 1 / byte 3, high nibbles
        a0 = fmaf(lo_h(t0), xl.x, a0);
        a0 = fmaf(hi_h(t0), xl.z, a0);
        b0 = fmaf(lo_h(t2), xl.y, b0);
        b0 = fmaf(hi_h(t2), xl.w, b0);
        a1 = fmaf(lo_h(t1), xh.x, a1);
        a1 = fmaf(hi_h(t1), xh.z, a1);
        b1 = fmaf(lo_h(t3), xh.y, b1);
        b1 = fmaf(hi_h(t3), xh.w, b1);
    }
    return (a0 + b0) * 16777216.0f + (a1 + b1) * 1048576.0f;
}

// Same sum with byte-to-float conversions (v_cvt_f32_ubyte*), kept as a reference variant.
QMV_DEV float dot_q4_cvt(uint4 q, const float *xb) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float4 xl = *(const float4 *)(xb + 4 * i);
        const float4 xh = *(const float4 *)(xb + 16 + 4 * i);
        const uint32_t lo = w[i] & 0x0F0F0F0Fu, hi = (w[i] >> 4) & 0x0F0F0F0Fu;
        a = fmaf((float)(lo & 0xFFu), xl.x, a);
        a = fmaf((float)((lo >> 8) & 0xFFu), xl.y, a);
        a = fmaf((float)((lo >> 16) & 0xFFu), xl.z, a);
        a = fmaf((float)(lo >> 24), xl.w, a);
        b = fmaf((float)(hi & 0xFFu), xh.x, b);
        b = fmaf((float)((hi >> 8) & 0xFFu), xh.y, b);
        b = fmaf((float)((hi >> 16) & 0xFFu), xh.z, b);
        b = fmaf((float)(hi >> 24), xh.w, b);
    }
    return a + b;
}

// One wave computes rows row0 .. row0+rpw-1; lane l owns blocks l, l+64, ... of each row.
template <int M, int BPL, int XT, bool MIX>
__global__ void __launch_bounds__(WG) gemv_q4_0_kernel(const uint8_t *__restrict__ qs,
                                                       const uint16_t *__restrict__ dsc,
                                                       const void *__restrict__ x,
                                                       float *__restrict__ y, int n, int k, int rpw) {
    extern __shared__ float lds[];
    const int nblk = k >> 5;
    float *sx = lds;
    float *ssum = lds + M * nblk * XS;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * WAVES + wave) * rpw;

    uint4 q[BPL];
    uint16_t dd[BPL];
    auto load = [&](int row) {
        const uint4 *qr = (const uint4 *)(qs + (int64_t)row * (k >> 1));
        const uint16_t *dr = dsc + (int64_t)row * nblk;
#pragma unroll
        for (int u = 0; u < BPL; u++) {
            const int b = lane + 64 * u;
            if (b < nblk) {
                q[u] = ld_stream16(qr + b);
                dd[u] = dr[b];
            } else {
                q[u] = make_uint4(0, 0, 0, 0);
                dd[u] = 0;
            }
        }
    };
    if (row0 < n) load(row0);
    stage_x32<M, XT>(x, k, sx, ssum);
    __syncthreads();

    for (int r = 0; r < rpw; r++) {
        const int row = row0 + r;
        if (row >= n) break;
        uint4 cq[BPL];
        uint16_t cd[BPL];
#pragma unroll
        for (int u = 0; u < BPL; u++) { cq[u] = q[u]; cd[u] = dd[u]; }
        if (r + 1 < rpw && row + 1 < n) load(row + 1);
        float acc[M];
#pragma unroll
        for (int m = 0; m < M; m++) acc[m] = 0.f;
#pragma unroll
        for (int u = 0; u < BPL; u++) {
            const int b = lane + 64 * u;
            if (b < nblk) {
                const float d = h2f(cd[u]);
#pragma unroll
                for (int m = 0; m < M; m++) {
                    const float *xb = sx + (m * nblk + b) * XS;
                    const float s = MIX ? dot_q4_mix(cq[u], xb) : dot_q4_cvt(cq[u], xb);
                    acc[m] = fmaf(d, s - 8.f * ssum[m * nblk + b], acc[m]);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float t = wave_sum(acc[m]);
            if (lane == 0) y[(int64_t)m * n + row] = t;
        }
    }
}

template <int M, int BPL, int XT, bool MIX>
void launch(const qmv_weights *w, const void *x, float *y, int rpw, hipStream_t s) {
    const int n = (int)w->n, k = (int)w->k, nblk = k >> 5;
    const size_t lds = (size_t)M * nblk * (XS + 1) * sizeof(float);
    const int grid = (n + WAVES * rpw - 1) / (WAVES * rpw);
    hipLaunchKernelGGL((gemv_q4_0_kernel<M, BPL, XT, MIX>), dim3(grid), dim3(WG), lds, s,
                       (const uint8_t *)w->codes, (const uint16_t *)w->scales, x, y, n, k, rpw);
}

template <int M, int XT, bool MIX>
bool dispatch_bpl(int bpl, const qmv_weights *w, const void *x, float *y, int rpw, hipStream_t s) {
    switch (bpl) {
    case 1: launch<M, 1, XT, MIX>(w, x, y, rpw, s); return true;
    case 2: launch<M, 2, XT, MIX>(w, x, y, rpw, s); return true;
    case 3: launch<M, 3, XT, MIX>(w, x, y, rpw, s); return true;
    case 4: launch<M, 4, XT, MIX>(w, x, y, rpw, s); return true;
    case 5: launch<M, 5, XT, MIX>(w, x, y, rpw, s); return true;
    case 6: launch<M, 6, XT, MIX>(w, x, y, rpw, s); return true;
    case 7: launch<M, 7, XT, MIX>(w, x, y, rpw, s); return true;
    case 8: launch<M, 8, XT, MIX>(w, x, y, rpw, s); return true;
    }
    return false;
}

template <int XT, bool MIX>
bool dispatch_m(int m, int bpl, const qmv_weights *w, const void *x, float *y, int rpw, hipStream_t s) {
    switch (m) {
    case 1: return dispatch_bpl<1, XT, MIX>(bpl, w, x, y, rpw, s);
    case 2: return dispatch_bpl<2, XT, MIX>(bpl, w, x, y, rpw, s);
    case 3: return dispatch_bpl<3, XT, MIX>(bpl, w, x, y, rpw, s);
    case 4: return dispatch_bpl<4, XT, MIX>(bpl, w, x, y, rpw, s);
    case 5: return dispatch_bpl<5, XT, MIX>(bpl, w, x, y, rpw, s);
    case 6: return dispatch_bpl<6, XT, MIX>(bpl, w, x, y, rpw, s);
    case 7: return dispatch_bpl<7, XT, MIX>(bpl, w, x, y, rpw, s);
    case 8: return dispatch_bpl<8, XT, MIX>(bpl, w, x, y, rpw, s);
    }
    return false;
}

}  // namespace

const char *launch_gemv_q4_0(const qmv_weights *w, int m, const void *x, int xt, float *y,
                             hipStream_t s) {
    const int64_t n = w->n, k = w->k, nblk = k / 32;
    const int bpl = (int)((nblk + 63) / 64);
    if (bpl > 8 || (int64_t)m * k > 16384 || n > INT32_MAX) return nullptr;
    const size_t lds = (size_t)m * nblk * (XS + 1) * sizeof(float);
    if ((int64_t)lds > device_info().lds_per_block) return nullptr;
    // Rows per wave: keep at least ~2 workgroups per CU before giving a wave more rows.
    const int64_t target_waves = (int64_t)device_info().num_cus * 2 * WAVES;
    int rpw = (int)(n / target_waves);
    rpw = rpw < 1 ? 1 : (rpw > 4 ? 4 : rpw);
    const bool mix = strcmp(forced_path(), "q4_0.cvt") != 0;
    bool ok;
    if (xt == QMV_F32)
        ok = mix ? dispatch_m<0, true>(m, bpl, w, x, y, rpw, s) : dispatch_m<0, false>(m, bpl, w, x, y, rpw, s);
    else
        ok = mix ? dispatch_m<1, true>(m, bpl, w, x, y, rpw, s) : dispatch_m<1, false>(m, bpl, w, x, y, rpw, s);
    if (!ok) return nullptr;
    return mix ? "q4_0.lds-x.fma-mix" : "q4_0.lds-x.cvt-ubyte";
}

}  // namespace qmv
