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
// Activations are staged per workgroup into LDS in that same unit order (64 floats
// per unit, 4 floats of padding so eight lanes reading eight consecutive units with
// ds_read_b128 hit disjoint banks), 64 units (4096 activations) of K at a time.  Centering is exact: each 6-bit code is OR-ed under the binary16
// exponent of 1024 and one packed half subtract gives q - 32 exactly; v_fma_mix_f32
// multiplies it by the fp32 activation exactly.  Per run the kernel applies its
// sub-scale, and d once per unit.
#include <cstring>

#include "device_common.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int US = 68;    // floats per staged 64-activation unit

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

// Raw bytes of one unit (quarter super-block), as loaded.
struct Unit {
    uint4 a, b, h;   // ql run (t=0 low / t=2 high), ql run (t=1 low / t=3 high), qh run
    uint4 s16;       // the super-block's 16 sub-scales
    uint16_t d;
};

QMV_DEV void load_unit(Unit &w, const uint8_t *ql, const uint8_t *qh, const int8_t *scp, const uint16_t *dp,
                       int row, int k, int u) {
    const int sb = u >> 2, h = (u >> 1) & 1, odd = u & 1;
    const uint8_t *qlr = ql + (int64_t)row * (k >> 1) + sb * 128 + 64 * h + 16 * odd;
    w.a = ld_stream16(qlr);
    w.b = ld_stream16(qlr + 32);
    w.h = ld_stream16(qh + (int64_t)row * (k >> 2) + sb * 64 + 32 * h + 16 * odd);
    w.s16 = *(const uint4 *)(scp + (int64_t)row * (k >> 4) + sb * 16);
    w.d = dp[(int64_t)row * (k >> 8) + sb];
}

// sum over unit u's 64 weights of (q - 32) * sc * x, times d.  The sub-scales are picked
// from the raw super-block bytes here, where they are used, not next to the load.
QMV_DEV float unit_dot(const Unit &w, int u, const float *xu) {
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
    // sub-scales 8h + odd + {0, 2, 4, 6}: bytes odd and odd+2 of dwords 2h and 2h+1
    const int h = (u >> 1) & 1, odd = u & 1;
    const uint32_t lo = h ? w.s16.z : w.s16.x, hi = h ? w.s16.w : w.s16.y;
    const float sc0 = (float)(int8_t)(lo >> (8 * odd)), sc1 = (float)(int8_t)(lo >> (8 * odd + 16));
    const float sc2 = (float)(int8_t)(hi >> (8 * odd)), sc3 = (float)(int8_t)(hi >> (8 * odd + 16));
    float r = sc0 * s0;
    r = fmaf(sc1, s1, r);
    r = fmaf(sc2, s2, r);
    r = fmaf(sc3, s3, r);
    return h2f(w.d) * r;
}

// The unit's sum for every batch row at once (batch 3 and up): each dword of codes is
// centred and converted to exact fp32 once and then applied with v_fmac_f32 to every
// row (unit_dot per row would repeat the unpack M times and convert inside each
// v_fma_mix_f32).  r[m] = d * sum over the unit of (q - 32) * sc * x[m], x[m] at
// xu + m * xstride.
template <int M>
QMV_DEV void unit_dot_rows(const Unit &w, int u, const float *xu, int xstride, float (&r)[M]) {
    const uint32_t A[4] = {w.a.x, w.a.y, w.a.z, w.a.w};
    const uint32_t B[4] = {w.b.x, w.b.y, w.b.z, w.b.w};
    const uint32_t H[4] = {w.h.x, w.h.y, w.h.z, w.h.w};
    const qmv_h2 off = {(_Float16)-1056.f, (_Float16)-1056.f};
    float s[4][M];
#pragma unroll
    for (int t = 0; t < 4; t++)
#pragma unroll
        for (int m = 0; m < M; m++) s[t][m] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t q[4];
        q[0] = and_or(H[i] << 4, 0x30303030u, A[i] & 0x0F0F0F0Fu);
        q[1] = and_or(H[i] << 2, 0x30303030u, B[i] & 0x0F0F0F0Fu);
        q[2] = and_or(H[i], 0x30303030u, (A[i] >> 4) & 0x0F0F0F0Fu);
        q[3] = and_or(H[i] >> 2, 0x30303030u, (B[i] >> 4) & 0x0F0F0F0Fu);
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const qmv_h2 e0 = as_h2(and_or(q[t], 0x00FF00FFu, 0x64006400u)) + off;       // bytes 0 and 2
            const qmv_h2 e1 = as_h2(and_or(q[t] >> 8, 0x00FF00FFu, 0x64006400u)) + off;  // bytes 1 and 3
            float c0 = (float)e0.x, c1 = (float)e1.x, c2 = (float)e0.y, c3 = (float)e1.y;
            // converted here, once, rather than folded into a v_fma_mix_f32 per row
            asm volatile("" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3));
#pragma unroll
            for (int m = 0; m < M; m++) {
                const float4 xv = *(const float4 *)(xu + m * xstride + 16 * t + 4 * i);
                float a = s[t][m];
                a = fmaf(c0, xv.x, a);
                a = fmaf(c1, xv.y, a);
                a = fmaf(c2, xv.z, a);
                s[t][m] = fmaf(c3, xv.w, a);
            }
            // the sums are formed here: otherwise the FMAs sink to the end of the unit and
            // every activation read of the unit is hoisted and held (spills from batch 3)
#pragma unroll
            for (int m = 0; m < M; m++) asm volatile("" : "+v"(s[t][m]));
        }
    }
    const int h = (u >> 1) & 1, odd = u & 1;
    const uint32_t lo = h ? w.s16.z : w.s16.x, hi = h ? w.s16.w : w.s16.y;
    const float sc0 = (float)(int8_t)(lo >> (8 * odd)), sc1 = (float)(int8_t)(lo >> (8 * odd + 16));
    const float sc2 = (float)(int8_t)(hi >> (8 * odd)), sc3 = (float)(int8_t)(hi >> (8 * odd + 16));
    const float d = h2f(w.d);
#pragma unroll
    for (int m = 0; m < M; m++) {
        float v = sc0 * s[0][m];
        v = fmaf(sc1, s[1][m], v);
        v = fmaf(sc2, s[2][m], v);
        v = fmaf(sc3, s[3][m], v);
        r[m] = d * v;
    }
}

// Lane l of a wave: when G > 1 the wave covers G rows, lane l taking unit l % U of row
// l / U (U = 64 / G units per row, the whole row in one chunk); when G == 1 it covers one
// row and K is walked in chunks of 64 units, lane l taking unit l of each chunk.  Per
// chunk: the activation loads, then the next chunk's unit loads (the current chunk's were
// issued during the previous one), then the LDS writes, a barrier, the dots.  No branch
// sits around a load (row and unit indices are clamped); activations of chunk row m, unit
// slot j sit at sx[(m * 64 + j) * US], run t at +16 t.
template <int M, int XT, int WGT, int CU>
__global__ void __launch_bounds__(WGT, M == 4 ? 4 : 2) gemv_q6k_kernel(const uint8_t *__restrict__ ql,
                                                      const uint8_t *__restrict__ qh,
                                                      const int8_t *__restrict__ scp,
                                                      const uint16_t *__restrict__ dp,
                                                      const void *__restrict__ x,
                                                      float *__restrict__ y, int n, int k, int G) {
    extern __shared__ float lds[];
    constexpr int WAVES_ = WGT / 64;
    constexpr int XPT = M * (CU * 16) / WGT;  // 16-byte activation pieces per thread per chunk
    const int nu = k >> 6;
    float *sx = lds;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int U = 64 / G;                     // units of a row per chunk (CU when nch > 1)
    const int nch = (nu + U - 1) / U;
    const int sub = lane / U, ul = lane % U;
    const int row = (blockIdx.x * WAVES_ + wave) * G + sub;
    const int rowc = row < n ? row : n - 1;
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; m++) acc[m] = 0.f;
    // One chunk: its activation loads, then the next chunk's unit into `fill` (clamped to
    // the row's last unit past the end), then the LDS writes and the dots with `use`.  Two
    // register sets alternate, so no copy waits on the loads just issued.
    auto step = [&](int c, const Unit &use, Unit &fill) {
        const int k0 = c * CU * 64;
        const int kq = min(CU * 64, k - k0) >> 2;  // 16-byte pieces of this chunk, per row
        float4 xv[XPT];
#pragma unroll
        for (int j = 0; j < XPT; j++) {
            const int p = threadIdx.x + j * WGT, m = p / (CU * 16), e = p % (CU * 16);
            xv[j] = ld_act4<XT>(x, (int64_t)m * k + k0 + 4 * (e < kq ? e : kq - 1));
        }
        const int un = (c + 1) * CU + ul;
        load_unit(fill, ql, qh, scp, dp, rowc, k, un < nu ? un : nu - 1);
        __builtin_amdgcn_sched_barrier(0);  // every load is issued before the LDS writes wait
        if (c) lds_barrier();  // the previous chunk's activations are consumed
#pragma unroll
        for (int j = 0; j < XPT; j++) {
            const int p = threadIdx.x + j * WGT, m = p / (CU * 16), e = 4 * (p % (CU * 16));
            const int slot = 4 * (e >> 8) + 2 * ((e >> 7) & 1) + ((e >> 4) & 1);
            *(float4 *)(sx + (m * CU + slot) * US + 16 * ((e >> 5) & 3) + (e & 15)) = xv[j];
        }
        lds_barrier();
        const int u = c * CU + ul;
        const int uc = u < nu ? u : nu - 1;
        if constexpr (M >= 3) {
            float r[M];
            unit_dot_rows<M>(use, uc, sx + (uc - c * CU) * US, CU * US, r);
#pragma unroll
            for (int m = 0; m < M; m++) acc[m] = u < nu ? acc[m] + r[m] : acc[m];
        } else {
#pragma unroll
            for (int m = 0; m < M; m++) {
                const float v = acc[m] + unit_dot(use, uc, sx + (m * CU + (uc - c * CU)) * US);
                acc[m] = u < nu ? v : acc[m];
            }
        }
    };
    Unit w0, w1;
    load_unit(w0, ql, qh, scp, dp, rowc, k, ul < nu ? ul : nu - 1);
    for (int c = 0; c < nch; c += 2) {
        step(c, w0, w1);
        if (c + 1 < nch) step(c + 1, w1, w0);
    }
#pragma unroll
    for (int m = 0; m < M; m++) {
        const float t = G == 1 ? wave_sum(acc[m]) : group_sum(acc[m], U);
        if (ul == 0 && row < n) y[(int64_t)m * n + row] = t;
    }
}

constexpr size_t lds_bytes(int m, int cu) { return (size_t)m * cu * US * sizeof(float); }

// WGT threads per workgroup, CU units staged per chunk: <512, 64> (one row per wave, or G
// short rows), or <256, 32> (two rows per wave, each lane one unit of a 32-unit chunk):
// from batch 5 up the staged activations of a 64-unit chunk (m x 17 KB) leave room for one
// 512-thread workgroup per CU, which then waits on its loads with nothing to overlap; the
// half chunk lets two 256-thread workgroups share a CU.
template <int M, int XT, int WGT, int CU>
void launch(const qmv_weights *w, const void *x, float *y, int G, hipStream_t s) {
    const int n = (int)w->n, k = (int)w->k;
    const int rows_per_wg = WGT / 64 * G;
    const int grid = (n + rows_per_wg - 1) / rows_per_wg;
    hipLaunchKernelGGL((gemv_q6k_kernel<M, XT, WGT, CU>), dim3(grid), dim3(WGT), lds_bytes(M, CU), s,
                       (const uint8_t *)w->codes, (const uint8_t *)w->codes_hi, (const int8_t *)w->scales,
                       (const uint16_t *)w->super, x, y, n, k, G);
}

template <int XT>
bool dispatch_m(int m, bool half, const qmv_weights *w, const void *x, float *y, int G, hipStream_t s) {
    if (half) {
        switch (m) {
        case 5: launch<5, XT, 256, 32>(w, x, y, G, s); return true;
        case 6: launch<6, XT, 256, 32>(w, x, y, G, s); return true;
        case 7: launch<7, XT, 256, 32>(w, x, y, G, s); return true;
        case 8: launch<8, XT, 256, 32>(w, x, y, G, s); return true;
        }
        return false;
    }
    switch (m) {
    case 1: launch<1, XT, 512, 64>(w, x, y, G, s); return true;
    case 2: launch<2, XT, 512, 64>(w, x, y, G, s); return true;
    case 3: launch<3, XT, 512, 64>(w, x, y, G, s); return true;
    case 4: launch<4, XT, 512, 64>(w, x, y, G, s); return true;
    case 5: launch<5, XT, 512, 64>(w, x, y, G, s); return true;
    case 6: launch<6, XT, 512, 64>(w, x, y, G, s); return true;
    case 7: launch<7, XT, 512, 64>(w, x, y, G, s); return true;
    case 8: launch<8, XT, 512, 64>(w, x, y, G, s); return true;
    }
    return false;
}

}  // namespace

const char *launch_gemv_q6k(const qmv_weights *w, int m, const void *x, int xt, float *y, hipStream_t s) {
    const int64_t n = w->n, k = w->k, nu = k / 64;
    if (n > INT32_MAX || k > INT32_MAX / 8) return nullptr;
    // batch 5 and up: 256-thread workgroups over 32-unit chunks (test override "q6_K.wg512":
    // the 512-thread form)
    const bool half = m >= 5 && std::strcmp(forced_path(), "q6_K.wg512") != 0;
    if ((int64_t)lds_bytes(m, half ? 32 : 64) > device_info().lds_per_block) return nullptr;
    // G rows at a time when a row has fewer than 64 units and 64 is a multiple of them; at
    // least two (32 units of a row per chunk) in the 256-thread form.
    int G = 1;
    if (nu < 64 && 64 % nu == 0) G = (int)(64 / nu);
    if (half && G < 2) G = 2;
    const bool ok = xt == QMV_F32 ? dispatch_m<0>(m, half, w, x, y, G, s) : dispatch_m<1>(m, half, w, x, y, G, s);
    if (!ok) return nullptr;
    if (half) return "q6_K.lds-x.fmac.wg256";
    const char *path[2][2] = {{"q6_K.lds-x.fma-mix", "q6_K.lds-x.fma-mix.rowgroup"},
                              {"q6_K.lds-x.fmac", "q6_K.lds-x.fmac.rowgroup"}};
    return path[m >= 3][G > 1];
}

}  // namespace qmv
