// gemv_q6k.hip -- q6_K decode GEMV for gfx950.
//
// Weight e of a 256-weight super-block is d * sc[e/16] * (q - 32) with the 6-bit q
// built from a low nibble of ql and a 2-bit field of qh ("57 · r54 —
// MINFER_MMQ_Q6K_EXP", §2.1 recombination; §2.3: a pure integer transform).  The
// GEMV streams 210 bytes per 256 weights from HBM (quantprobe LAWS.md, Law 4).
//
// Work unit of one lane: a quarter super-block of 64 weights = half h (0/1) and
// lane offset l0 (0/16).  Its bytes are two 16-byte runs of ql (ql[64h+l0..] and
// ql[64h+32+l0..]) and one 16-byte run of qh (qh[32h+l0..]), i.e. three aligned
// 128-bit loads; the low and high nibbles of those ql bytes and the four 2-bit
// fields of each qh byte give four runs t = 0..3 of 16 consecutive weights,
// e = 128h + 32t + l0 + j, each under one sub-scale sc[8h + 2t + l0/16].
//
// Activations are staged once per workgroup into LDS in that same unit order
// (64 floats per unit, 4 floats of padding so eight lanes reading eight
// consecutive units with ds_read_b128 hit disjoint banks), before the weight loads
// are issued.  Centering is exact: each 6-bit code is OR-ed under the binary16
// exponent of 1024 and one packed half subtract gives q - 32 exactly; v_fma_mix_f32
// multiplies it by the fp32 activation exactly.  Per run the kernel applies its
// sub-scale, and d once per unit.
#include "device_common.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int WG = 512;
constexpr int WAVES = WG / 64;
constexpr int US = 68;  // floats per staged 64-activation unit

// Stage x [M][k] into LDS in unit order: unit u of row m at sx[(m*nu + u)*US], with
// run t (16 floats) at +16t.  Threads move coalesced 16-byte chunks.
template <int M, int XT>
__device__ void stage_units(const void *x, int k, float *sx) {
    const int nu = k >> 6, nq = k >> 2;
    const int total = M * nq;
    for (int c = threadIdx.x; c < total; c += WG) {
        const int m = c / nq, e = (c - m * nq) * 4;
        const int sb = e >> 8, h = (e >> 7) & 1, t = (e >> 5) & 3, odd = (e >> 4) & 1;
        const int u = m * nu + 4 * sb + 2 * h + odd;
        *(float4 *)(sx + u * US + 16 * t + (e & 15)) = ld_act4<XT>(x, (int64_t)c * 4);
    }
}

// sum_j (q_j - 32) x_j over the four bytes (values 0..63) of dword q and x[0..3], exact products.
QMV_DEV float dot4_c32(uint32_t q, float4 xv, float acc) {
    const qmv_h2 off = {(_Float16)-1056.f, (_Float16)-1056.f};
    const qmv_h2 e0 = as_h2(and_or(q, 0x00FF00FFu, 0x64006400u)) + off;       // bytes 0 and 2
    const qmv_h2 e1 = as_h2(and_or(q >> 8, 0x00FF00FFu, 0x64006400u)) + off;  // bytes 1 and 3
    acc = fmaf((float)e0.x, xv.x, acc);
    acc = fmaf((float)e0.y, xv.z, acc);
    acc = fmaf((float)e1.x, xv.y, acc);
    acc = fmaf((float)e1.y, xv.w, acc);
    return acc;
}

struct Unit {
    uint4 a, b, h;   // ql run (t=0 low / t=2 high), ql run (t=1 low / t=3 high), qh run
    uint32_t sc4;    // the unit's four sub-scales, byte t = sc[8h + 2t + odd]
    uint16_t d;
};

// sum over the unit's 64 weights of (q - 32) * sc * x, times d.
QMV_DEV float unit_dot(const Unit &w, const float *xu) {
    const uint32_t A[4] = {w.a.x, w.a.y, w.a.z, w.a.w};
    const uint32_t B[4] = {w.b.x, w.b.y, w.b.z, w.b.w};
    const uint32_t H[4] = {w.h.x, w.h.y, w.h.z, w.h.w};
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t q0 = and_or(H[i] << 4, 0x30303030u, A[i] & 0x0F0F0F0Fu);
        const uint32_t q1 = and_or(H[i] << 2, 0x30303030u, B[i] & 0x0F0F0F0Fu);
        const uint32_t q2 = and_or(H[i], 0x30303030u, (A[i] >> 4) & 0x0F0F0F0Fu);
        const uint32_t q3 = and_or(H[i] >> 2, 0x30303030u, (B[i] >> 4) & 0x0F0F0F0Fu);
        s0 = dot4_c32(q0, *(const float4 *)(xu + 4 * i), s0);
        s1 = dot4_c32(q1, *(const float4 *)(xu + 16 + 4 * i), s1);
        s2 = dot4_c32(q2, *(const float4 *)(xu + 32 + 4 * i), s2);
        s3 = dot4_c32(q3, *(const float4 *)(xu + 48 + 4 * i), s3);
    }
    const float sc0 = (float)(int8_t)(w.sc4 & 0xFF), sc1 = (float)(int8_t)((w.sc4 >> 8) & 0xFF);
    const float sc2 = (float)(int8_t)((w.sc4 >> 16) & 0xFF), sc3 = (float)(int8_t)(w.sc4 >> 24);
    float r = sc0 * s0;
    r = fmaf(sc1, s1, r);
    r = fmaf(sc2, s2, r);
    r = fmaf(sc3, s3, r);
    return h2f(w.d) * r;
}

// Lane l of a wave: when G > 1 the wave covers G rows, lane l taking unit l % U of row
// l / U (U = 64 / G units per row); when G == 1 it covers one row, lane l taking units
// l, l+64, ... (UPL of them).  Activations are staged before the weight loads are issued
// (vector loads return in order).
template <int M, int UPL, int XT>
__global__ void __launch_bounds__(WG) gemv_q6k_kernel(const uint8_t *__restrict__ ql,
                                                      const uint8_t *__restrict__ qh,
                                                      const int8_t *__restrict__ scp,
                                                      const uint16_t *__restrict__ dp,
                                                      const void *__restrict__ x,
                                                      float *__restrict__ y, int n, int k, int G) {
    extern __shared__ float lds[];
    const int nu = k >> 6, nsb = k >> 8;
    float *sx = lds;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int U = G > 1 ? 64 / G : nu;
    const int sub = G > 1 ? lane / U : 0;
    const int ul = G > 1 ? lane % U : lane;
    const int row = (blockIdx.x * WAVES + wave) * G + sub;

    stage_units<M, XT>(x, k, sx);

    Unit wv[UPL];
#pragma unroll
    for (int j = 0; j < UPL; j++) {
        const int u = ul + 64 * j;
        if (row < n && u < nu) {
            const int sb = u >> 2, h = (u >> 1) & 1, odd = u & 1;
            const uint8_t *qlr = ql + (int64_t)row * (k >> 1) + sb * 128 + 64 * h + 16 * odd;
            const uint8_t *qhr = qh + (int64_t)row * (k >> 2) + sb * 64 + 32 * h + 16 * odd;
            wv[j].a = ld_stream16(qlr);
            wv[j].b = ld_stream16(qlr + 32);
            wv[j].h = ld_stream16(qhr);
            const uint4 s16 = *(const uint4 *)(scp + (int64_t)row * (k >> 4) + sb * 16);
            // sub-scales 8h + odd + {0, 2, 4, 6}: bytes odd and odd+2 of dwords 2h and 2h+1
            const uint32_t lo = h ? s16.z : s16.x, hi = h ? s16.w : s16.y;
            const uint32_t a0 = (lo >> (8 * odd)) & 0xFF, a1 = (lo >> (8 * odd + 16)) & 0xFF;
            const uint32_t a2 = (hi >> (8 * odd)) & 0xFF, a3 = (hi >> (8 * odd + 16)) & 0xFF;
            wv[j].sc4 = a0 | (a1 << 8) | (a2 << 16) | (a3 << 24);
            wv[j].d = dp[(int64_t)row * nsb + sb];
        } else {
            wv[j].a = wv[j].b = wv[j].h = make_uint4(0, 0, 0, 0);
            wv[j].sc4 = 0;
            wv[j].d = 0;
        }
    }
    __syncthreads();

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; m++) acc[m] = 0.f;
#pragma unroll
    for (int j = 0; j < UPL; j++) {
        const int u = ul + 64 * j;
        if (u < nu) {
#pragma unroll
            for (int m = 0; m < M; m++)
                acc[m] += unit_dot(wv[j], sx + (m * nu + u) * US);
        }
    }
#pragma unroll
    for (int m = 0; m < M; m++) {
        const float t = G == 1 ? wave_sum(acc[m]) : group_sum(acc[m], U);
        if (ul == 0 && row < n) y[(int64_t)m * n + row] = t;
    }
}

template <int M, int UPL, int XT>
void launch(const qmv_weights *w, const void *x, float *y, int G, hipStream_t s) {
    const int n = (int)w->n, k = (int)w->k, nu = k >> 6;
    const size_t lds = (size_t)M * nu * US * sizeof(float);
    const int rows_per_wg = WAVES * G;
    const int grid = (n + rows_per_wg - 1) / rows_per_wg;
    hipLaunchKernelGGL((gemv_q6k_kernel<M, UPL, XT>), dim3(grid), dim3(WG), lds, s,
                       (const uint8_t *)w->codes, (const uint8_t *)w->codes_hi, (const int8_t *)w->scales,
                       (const uint16_t *)w->super, x, y, n, k, G);
}

template <int M, int XT>
bool dispatch_upl(int upl, const qmv_weights *w, const void *x, float *y, int G, hipStream_t s) {
    switch (upl) {
    case 1: launch<M, 1, XT>(w, x, y, G, s); return true;
    case 2: launch<M, 2, XT>(w, x, y, G, s); return true;
    case 3: launch<M, 3, XT>(w, x, y, G, s); return true;
    case 4: launch<M, 4, XT>(w, x, y, G, s); return true;
    }
    return false;
}

template <int XT>
bool dispatch_m(int m, int upl, const qmv_weights *w, const void *x, float *y, int G, hipStream_t s) {
    switch (m) {
    case 1: return dispatch_upl<1, XT>(upl, w, x, y, G, s);
    case 2: return dispatch_upl<2, XT>(upl, w, x, y, G, s);
    case 3: return dispatch_upl<3, XT>(upl, w, x, y, G, s);
    case 4: return dispatch_upl<4, XT>(upl, w, x, y, G, s);
    case 5: return dispatch_upl<5, XT>(upl, w, x, y, G, s);
    case 6: return dispatch_upl<6, XT>(upl, w, x, y, G, s);
    case 7: return dispatch_upl<7, XT>(upl, w, x, y, G, s);
    case 8: return dispatch_upl<8, XT>(upl, w, x, y, G, s);
    }
    return false;
}

}  // namespace

const char *launch_gemv_q6k(const qmv_weights *w, int m, const void *x, int xt, float *y, hipStream_t s) {
    const int64_t n = w->n, k = w->k, nu = k / 64;
    if ((int64_t)m * k > 16384 || n > INT32_MAX) return nullptr;
    const size_t lds = (size_t)m * nu * US * sizeof(float);
    if ((int64_t)lds > device_info().lds_per_block) return nullptr;
    // G rows at a time when a row has fewer than 64 units and 64 is a multiple of them.
    int G = 1;
    if (nu < 64 && 64 % nu == 0) G = (int)(64 / nu);
    const int upl = G > 1 ? 1 : (int)((nu + 63) / 64);
    if (upl > 4) return nullptr;
    const bool ok = xt == QMV_F32 ? dispatch_m<0>(m, upl, w, x, y, G, s)
                                  : dispatch_m<1>(m, upl, w, x, y, G, s);
    if (!ok) return nullptr;
    return G > 1 ? "q6_K.lds-x.fma-mix.rowgroup" : "q6_K.lds-x.fma-mix";
}

}  // namespace qmv
