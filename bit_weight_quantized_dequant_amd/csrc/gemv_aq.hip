// gemv_aq.hip -- 2-bit two-codebook additive GEMV (batch 1..8) for gfx950.
//
// Format ("Chasing x100", "The kernel is ready": a 2-bit additive-code GEMV checked
// against a bit-faithful CPU reference): each group of 8 consecutive weights of a row
// stores two 8-bit codes (c1, c2); the group's weights are C1[c1] + C2[c2] (two
// per-matrix tables of 256 x 8 fp16 entries), times a per-row fp16 scale s[n].
//
// Kernel:
//   * both tables (8 KiB) are copied into LDS once per workgroup;
//   * K is processed in chunks of 4096 activations; each chunk of x is staged into LDS
//     as fp32 (64 floats per lane unit + 4 of padding, so ds_read_b128 over
//     consecutive lanes does not collide) before the chunk's code loads are issued;
//   * lane l owns 16 code bytes (8 groups, 64 weights) of the chunk: one 128-bit load;
//   * per group two ds_read_b128 fetch C1[c1] and C2[c2]; v_fma_mix_f32 forms each
//     weight as fl32(C1 + C2) (fp16 halves times 1.0 plus fp16 half), so an exactly
//     cancelling pair gives 0 and the rounding is relative to |w|; the weight is then
//     applied to every batch row with an fp32 FMA (decoded once for all rows);
//   * the 64 lane partials are summed with DPP and scaled by s[n].
#include "device_common.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int WG = 512;
constexpr int WAVES = WG / 64;
constexpr int KC = 4096;   // activations per chunk: 64 lanes x 64 weights
constexpr int XU = 68;     // floats per staged 64-activation lane unit

template <int M, int XT>
__device__ void stage_chunk(const void *x, int k, int k0, int kc, float *sx) {
    const int q = kc >> 2, total = M * q;
    for (int c = threadIdx.x; c < total; c += WG) {
        const int m = c / q, e = (c - m * q) * 4;
        *(float4 *)(sx + (m * 64 + (e >> 6)) * XU + (e & 63)) = ld_act4<XT>(x, (int64_t)m * k + k0 + e);
    }
}

// The lane's code bytes for `ng` groups at p: one 128-bit load when all 8 groups are
// present and p is 16-byte aligned (k % 64 == 0), else byte loads (ragged rows / tails).
QMV_DEV uint4 load_codes(const uint8_t *p, int ng) {
    if (ng == 8 && ((uintptr_t)p & 15) == 0) return ld_stream16(p);
    uint32_t v[4] = {0, 0, 0, 0};
    for (int i = 0; i < 2 * ng; i++) v[i >> 2] |= (uint32_t)p[i] << (8 * (i & 3));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int M, int XT>
__global__ void __launch_bounds__(WG) gemv_aq_kernel(const uint8_t *__restrict__ codes,
                                                     const uint16_t *__restrict__ cbk,
                                                     const uint16_t *__restrict__ srow,
                                                     const void *__restrict__ x, float *__restrict__ y,
                                                     int n, int k) {
    extern __shared__ float lds[];
    uint32_t *tab = (uint32_t *)lds;  // C1 then C2: 2 x 256 entries x 4 dwords
    float *sx = lds + 2048;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * WAVES + wave;
    const uint32_t tab_addr = (uint32_t)(uintptr_t)tab;

    for (int i = threadIdx.x; i < 512; i += WG) ((uint4 *)tab)[i] = ((const uint4 *)cbk)[i];

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; m++) acc[m] = 0.f;
    const uint8_t *crow = codes + (int64_t)row * (k >> 2);

    for (int k0 = 0; k0 < k; k0 += KC) {
        const int kc = min(KC, k - k0);
        if (k0) __syncthreads();  // previous chunk fully consumed
        stage_chunk<M, XT>(x, k, k0, kc, sx);
        const int e0 = lane * 64;  // first weight of this lane's unit within the chunk
        const bool mine = row < n && e0 < kc;
        const int ng = mine ? min(8, (kc - e0) >> 3) : 0;
        const uint4 cq = mine ? load_codes(crow + ((k0 + e0) >> 2), ng) : make_uint4(0, 0, 0, 0);
        __syncthreads();
        if (mine) {
            const uint32_t cw[4] = {cq.x, cq.y, cq.z, cq.w};
#pragma unroll
            for (int g = 0; g < 8; g++) {
                if (g < ng) {
                    const uint32_t word = cw[g >> 1];
                    const uint32_t c1 = (word >> (16 * (g & 1))) & 0xFF, c2 = (word >> (16 * (g & 1) + 8)) & 0xFF;
                    const uint4 a = lds_ld16(tab_addr + (c1 << 4));
                    const uint4 b = lds_ld16(tab_addr + 4096 + (c2 << 4));
                    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
                    float wv[8];
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        wv[2 * j] = fmaf(lo_h(av[j]), 1.0f, lo_h(bv[j]));
                        wv[2 * j + 1] = fmaf(hi_h(av[j]), 1.0f, hi_h(bv[j]));
                    }
#pragma unroll
                    for (int m = 0; m < M; m++) {
                        const float *xg = sx + (m * 64 + lane) * XU + 8 * g;
                        const float4 x0 = *(const float4 *)xg, x1 = *(const float4 *)(xg + 4);
                        float t = acc[m];
                        t = fmaf(wv[0], x0.x, t);
                        t = fmaf(wv[1], x0.y, t);
                        t = fmaf(wv[2], x0.z, t);
                        t = fmaf(wv[3], x0.w, t);
                        t = fmaf(wv[4], x1.x, t);
                        t = fmaf(wv[5], x1.y, t);
                        t = fmaf(wv[6], x1.z, t);
                        t = fmaf(wv[7], x1.w, t);
                        acc[m] = t;
                    }
                }
            }
        }
    }
    const float s = row < n ? h2f(srow[row]) : 0.f;
#pragma unroll
    for (int m = 0; m < M; m++) {
        const float t = wave_sum(acc[m]);
        if (lane == 0 && row < n) y[(int64_t)m * n + row] = s * t;
    }
}

template <int M, int XT>
void launch(const qmv_weights *w, const void *x, float *y, hipStream_t s) {
    const int n = (int)w->n, k = (int)w->k;
    const size_t lds = 2048 * 4 + (size_t)M * 64 * XU * 4;
    hipLaunchKernelGGL((gemv_aq_kernel<M, XT>), dim3((n + WAVES - 1) / WAVES), dim3(WG), lds, s,
                       (const uint8_t *)w->codes, (const uint16_t *)w->codebook, (const uint16_t *)w->scales,
                       x, y, n, k);
}

template <int XT>
bool dispatch_m(int m, const qmv_weights *w, const void *x, float *y, hipStream_t s) {
    switch (m) {
    case 1: launch<1, XT>(w, x, y, s); return true;
    case 2: launch<2, XT>(w, x, y, s); return true;
    case 3: launch<3, XT>(w, x, y, s); return true;
    case 4: launch<4, XT>(w, x, y, s); return true;
    case 5: launch<5, XT>(w, x, y, s); return true;
    case 6: launch<6, XT>(w, x, y, s); return true;
    case 7: launch<7, XT>(w, x, y, s); return true;
    case 8: launch<8, XT>(w, x, y, s); return true;
    }
    return false;
}

}  // namespace

const char *launch_gemv_aq(const qmv_weights *w, int m, const void *x, int xt, float *y, hipStream_t s) {
    if (w->n > INT32_MAX || w->k > INT32_MAX / 8) return nullptr;
    const size_t lds = 2048 * 4 + (size_t)m * 64 * XU * 4;
    if ((int64_t)lds > device_info().lds_per_block) return nullptr;
    const bool ok = xt == QMV_F32 ? dispatch_m<0>(m, w, x, y, s) : dispatch_m<1>(m, w, x, y, s);
    return ok ? "aq2x8.lds-codebook.fma-mix" : nullptr;
}

}  // namespace qmv
