// gemv_aq.hip -- additive-code GEMVs (batch 1..8) for gfx950: the 2-bit code (two
// codebooks) and the 3-bit code (three codebooks).
//
// Format ("Chasing x100", "The kernel is ready": 2-bit and 3-bit additive-code GEMVs
// checked against a bit-faithful CPU reference): each group of 8 consecutive weights of
// a row stores NC 8-bit codes (c1, .., cNC), one byte each; the group's weights are
// C1[c1] + .. + CNC[cNC] (NC per-matrix tables of 256 x 8 fp16 entries), times a per-row
// fp16 scale s[n].
//
// Kernel (k % 64 == 0, the streaming skeleton of gemv_stream.h):
//   * the NC tables (4 KiB each) are copied into LDS once per workgroup;
//   * lane l owns unit l of each 4096-weight step: 8 groups, NC * 8 code bytes (one
//     128-bit load for NC = 2, three 64-bit loads for NC = 3), prefetched a step ahead;
//   * per group, NC ds_read_b128 fetch the table rows; v_fma_mix_f32 forms each weight
//     in fp32 as fl32(C1 + C2) (+ C3): exact when the entries are below 1/4 in
//     magnitude (the sum then fits 24 bits), else rounded relative to the partial sum;
//     an exactly cancelling pair gives 0.  The weight is applied to every batch row with
//     an fp32 FMA (decoded once for all rows);
//   * the 64 lane partials are summed with DPP and scaled by s[n];
//   * batches run two rows per wave (four at batch 8 on tall matrices): each activation
//     read from LDS serves all of them.
// Rows whose length is not a multiple of 64 take a plain kernel (byte loads, one K chunk
// staged at a time).
#include <cstring>

#include "device_common.h"
#include "gemv_stream.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

using stream::WG;
using stream::WAVES;
using stream::XU;

// fl32(h + g) for halves h of a and g of b (HI selects the high halves), and fl32(h + f) for a
// half h of a and an fp32 f: one v_fma_mix_f32 each (h * 1.0 + g, a single rounding).
// Written as fmaf((float)h, 1.0f, (float)g) the compiler folds the multiply and emits two
// conversions and an add instead.
template <int HI>
QMV_DEV float sum_hh(uint32_t a, uint32_t b) {
    float r;
    if (HI) asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(a), "v"(b));
    else asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,1]" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
template <int HI>
QMV_DEV float sum_hf(uint32_t a, float f) {
    float r;
    if (HI) asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(a), "v"(f));
    else asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(a), "v"(f));
    return r;
}

// Table rows of codebook b at LDS byte address tab + b * 4096 + 16 * code.  R rows per wave:
// lane l owns unit l of each of the R rows, and each activation read serves all of them.
template <int NC, int RR, int L = 64>
struct AqPolicy {
    static constexpr int R = RR;  // rows per lane group
    static constexpr int XB = stream::xbuf_of(L);  // floats between batch rows' staged steps
    struct Codes {
        uint32_t w[R][2 * NC];  // row r: byte NC * g + b = code b of group g
    };
    const uint8_t *crow[R];  // the rows' codes
    uint32_t tab;            // LDS byte address of the tables

    __device__ __forceinline__ void load(Codes &c, int unit) const {
#pragma unroll
        for (int r = 0; r < R; r++) {
            const uint8_t *p = crow[r] + (int64_t)unit * (8 * NC);
            if (NC == 2) {
                const uint4 v = ld_stream16(p);
                c.w[r][0] = v.x; c.w[r][1] = v.y; c.w[r][2] = v.z; c.w[r][3] = v.w;
            } else {
#pragma unroll
                for (int i = 0; i < NC; i++) {
                    const u32x2 v = __builtin_nontemporal_load((const u32x2 *)(p + 8 * i));
                    c.w[r][2 * i] = v.x;
                    c.w[r][2 * i + 1] = v.y;
                }
            }
        }
    }

    template <int M>
    __device__ __forceinline__ void dot(const Codes &c, const float *xu, float (&s)[R * M]) const {
#pragma unroll
        for (int g = 0; g < 8; g++) {
            float wv[R][8];
#pragma unroll
            for (int r = 0; r < R; r++) {
                uint32_t row[NC];
#pragma unroll
                for (int b = 0; b < NC; b++) {
                    const int bi = NC * g + b;
                    row[b] = tab + b * 4096 + (((c.w[r][bi >> 2] >> (8 * (bi & 3))) & 0xFFu) << 4);
                }
                const uint4 a = lds_ld16(row[0]), b = lds_ld16(row[1]);
                const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    wv[r][2 * j] = sum_hh<0>(av[j], bv[j]);
                    wv[r][2 * j + 1] = sum_hh<1>(av[j], bv[j]);
                }
                if (NC == 3) {
                    const uint4 t = lds_ld16(row[NC - 1]);
                    const uint32_t tv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        wv[r][2 * j] = sum_hf<0>(tv[j], wv[r][2 * j]);
                        wv[r][2 * j + 1] = sum_hf<1>(tv[j], wv[r][2 * j + 1]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < M; m++) {
                const float *xg = xu + m * XB + 8 * g;
                const float4 x0 = *(const float4 *)xg, x1 = *(const float4 *)(xg + 4);
#pragma unroll
                for (int r = 0; r < R; r++) {
                    float t = s[r * M + m];
                    t = fmaf(wv[r][0], x0.x, t);
                    t = fmaf(wv[r][1], x0.y, t);
                    t = fmaf(wv[r][2], x0.z, t);
                    t = fmaf(wv[r][3], x0.w, t);
                    t = fmaf(wv[r][4], x1.x, t);
                    t = fmaf(wv[r][5], x1.y, t);
                    t = fmaf(wv[r][6], x1.z, t);
                    t = fmaf(wv[r][7], x1.w, t);
                    s[r * M + m] = t;
                }
            }
        }
    }
};

// LDS layout: the activation buffers (xfloats floats), then the NC tables.  L lanes per
// row group: 64 (one group of R rows per wave, 512-thread workgroups, 4096-weight steps)
// or 32 (two groups per wave, 256-thread workgroups, 2048-weight steps: half the staged
// activations, so two workgroups share a CU from batch 5 up).
template <int NC, int M, int R, int XT, int L = 64>
__global__ void __launch_bounds__(stream::wg_of(L)) aq_stream_kernel(const uint8_t *__restrict__ codes,
                                                                     const uint16_t *__restrict__ cbk,
                                                                     const uint16_t *__restrict__ srow,
                                                                     const void *__restrict__ x,
                                                                     float *__restrict__ y, int n, int k,
                                                                     int xfloats) {
    extern __shared__ float4 lds4[];
    constexpr int WG_ = stream::wg_of(L), WAVES_ = WG_ / 64, G = 64 / L;
    float *sx = (float *)lds4;
    uint4 *tab = (uint4 *)(sx + xfloats);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane / L, ul = lane % L;
    const int row0 = ((blockIdx.x * WAVES_ + wave) * G + sub) * R;  // this group's rows: row0 .. row0 + R - 1

    // NC * 256 table rows of 16 bytes; threads past the end rewrite the last row
    const uint4 *src = (const uint4 *)cbk;
#pragma unroll
    for (int i = 0; i < (NC * 256 + WG_ - 1) / WG_; i++) {
        const int e = threadIdx.x + i * WG_;
        const int ec = e < NC * 256 ? e : NC * 256 - 1;
        tab[ec] = src[ec];
    }

    AqPolicy<NC, R, L> pol;
    pol.tab = (uint32_t)(uintptr_t)tab;
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int rowc = row0 + r < n ? row0 + r : n - 1;
        pol.crow[r] = codes + (int64_t)rowc * (k >> 3) * NC;
    }
    float acc[R * M];
#pragma unroll
    for (int m = 0; m < R * M; m++) acc[m] = 0.f;
    stream::walk_row<AqPolicy<NC, R, L>, M, XT, L>(pol, x, k, sx, acc);

#pragma unroll
    for (int r = 0; r < R; r++) {
        const int row = row0 + r;
        const float s = h2f(srow[row < n ? row : n - 1]);
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float t = L == 64 ? wave_sum(acc[r * M + m]) : group_sum(acc[r * M + m], L);
            if (ul == 0 && row < n) y[(int64_t)m * n + row] = s * t;
        }
    }
}

// ---- rows whose length is not a multiple of 64: one K chunk of 4096 staged at a time,
// code bytes read one by one.
constexpr int KC = 4096;

template <int M, int XT>
__device__ void stage_chunk(const void *x, int k, int k0, int kc, float *sx) {
    const int q = kc >> 2, total = M * q;
    for (int c = threadIdx.x; c < total; c += WG) {
        const int m = c / q, e = (c - m * q) * 4;
        *(float4 *)(sx + (m * 64 + (e >> 6)) * XU + (e & 63)) = ld_act4<XT>(x, (int64_t)m * k + k0 + e);
    }
}

template <int NC, int M, int XT>
__global__ void __launch_bounds__(WG) aq_ragged_kernel(const uint8_t *__restrict__ codes,
                                                       const uint16_t *__restrict__ cbk,
                                                       const uint16_t *__restrict__ srow,
                                                       const void *__restrict__ x, float *__restrict__ y,
                                                       int n, int k) {
    extern __shared__ float lds[];
    uint4 *tab = (uint4 *)lds;  // NC tables of 256 rows
    float *sx = lds + NC * 1024;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * WAVES + wave;
    const uint32_t tab_addr = (uint32_t)(uintptr_t)tab;

    for (int i = threadIdx.x; i < NC * 256; i += WG) tab[i] = ((const uint4 *)cbk)[i];

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; m++) acc[m] = 0.f;
    const uint8_t *crow = codes + (int64_t)row * (k >> 3) * NC;

    for (int k0 = 0; k0 < k; k0 += KC) {
        const int kc = min(KC, k - k0);
        if (k0) lds_barrier();  // previous chunk fully consumed
        stage_chunk<M, XT>(x, k, k0, kc, sx);
        lds_barrier();
        const int e0 = lane * 64;  // first weight of this lane's unit within the chunk
        if (row < n && e0 < kc) {
            const int ng = min(8, (kc - e0) >> 3);
            const uint8_t *cp = crow + (int64_t)((k0 + e0) >> 3) * NC;
            for (int g = 0; g < ng; g++) {
                float wv[8];
                const uint4 a = lds_ld16(tab_addr + (cp[NC * g] << 4));
                const uint4 b = lds_ld16(tab_addr + 4096 + (cp[NC * g + 1] << 4));
                const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    wv[2 * j] = sum_hh<0>(av[j], bv[j]);
                    wv[2 * j + 1] = sum_hh<1>(av[j], bv[j]);
                }
                if (NC == 3) {
                    const uint4 t = lds_ld16(tab_addr + 8192 + (cp[NC * g + NC - 1] << 4));
                    const uint32_t tv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        wv[2 * j] = sum_hf<0>(tv[j], wv[2 * j]);
                        wv[2 * j + 1] = sum_hf<1>(tv[j], wv[2 * j + 1]);
                    }
                }
#pragma unroll
                for (int m = 0; m < M; m++) {
                    const float *xg = sx + (m * 64 + lane) * XU + 8 * g;
#pragma unroll
                    for (int j = 0; j < 8; j++) acc[m] = fmaf(wv[j], xg[j], acc[m]);
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

size_t stream_lds(int nc, int m, int64_t k, int l = 64) { return stream::x_lds_bytes(m, k, l) + (size_t)nc * 4096; }
size_t ragged_lds(int nc, int m) { return (size_t)nc * 4096 + (size_t)m * 64 * XU * 4; }

template <int NC, int M, int R, int XT, int L = 64>
void launch_stream(const qmv_weights *w, const void *x, float *y, hipStream_t s) {
    const int n = (int)w->n, k = (int)w->k;
    constexpr int ROWS = stream::wg_of(L) / L * R;  // rows per workgroup: 8 R
    hipLaunchKernelGGL((aq_stream_kernel<NC, M, R, XT, L>), dim3((n + ROWS - 1) / ROWS), dim3(stream::wg_of(L)),
                       stream_lds(NC, M, k, L), s, (const uint8_t *)w->codes, (const uint16_t *)w->codebook,
                       (const uint16_t *)w->scales, x, y, n, k, (int)(stream::x_lds_bytes(M, k, L) / 4));
}

// The half-step form at batch 5-7, two rows per lane group, on matrices with rows for two
// of its 16-row workgroups per CU (14336x4096, 2-bit / 3-bit: batch 5 25.9 -> 23.4 /
// 31.3 -> 28.6 us, batch 7 32.2 -> 29.5 / 37.2 -> 34.4 us); at batch 8 four rows per wave
// in the full-step form stay faster (29.1 against 32.7 us).  Test overrides "aq.half" (any
// size and batch from 5) and "aq.wg512" (never).
bool stream_half(int m, int64_t n) {
    const char *fp = forced_path();
    if (m < 5 || strcmp(fp, "aq.wg512") == 0 || strcmp(fp, "aq.r1") == 0 || strcmp(fp, "aq.r2") == 0 ||
        strcmp(fp, "aq.r4") == 0)
        return false;
    return strcmp(fp, "aq.half") == 0 || (m < 8 && n >= 32 * (int64_t)device_info().num_cus);
}

// Rows per wave of the streaming kernel: two for batches (each activation read from LDS
// serves both rows, which the batch's LDS traffic needs) when there are rows for at least one
// such workgroup per CU, else one; four at batch 8 with rows for one such workgroup per CU
// (14336x4096: 34.7 -> 28.9 us for the 2-bit code, 39.2 -> 33.3 for the 3-bit one; at batch 4
// and on 4096-row matrices the halved occupancy loses); test overrides "aq.r1" / "aq.r2" /
// "aq.r4" force any of them.
int stream_rows(int m, int64_t n) {
    const char *fp = forced_path();
    if (strcmp(fp, "aq.r1") == 0) return 1;
    if (strcmp(fp, "aq.r2") == 0) return 2;
    if (strcmp(fp, "aq.r4") == 0) return 4;
    const int64_t cus = device_info().num_cus;
    if (m >= 8 && n >= 4 * WAVES * cus) return 4;
    return m > 1 && n >= 2 * WAVES * cus ? 2 : 1;
}

template <int NC, int M, int XT>
void launch(const qmv_weights *w, const void *x, float *y, hipStream_t s) {
    const int n = (int)w->n, k = (int)w->k;
    const dim3 grid((n + WAVES - 1) / WAVES);
    if (k % 64 == 0) {
        const int r = stream_rows(M, n);
        if constexpr (M >= 5) {
            if (stream_half(M, n)) {
                launch_stream<NC, M, 2, XT, 32>(w, x, y, s);
                return;
            }
        }
        if (r == 4) launch_stream<NC, M, 4, XT>(w, x, y, s);
        else if (r == 2) launch_stream<NC, M, 2, XT>(w, x, y, s);
        else launch_stream<NC, M, 1, XT>(w, x, y, s);
    } else {
        hipLaunchKernelGGL((aq_ragged_kernel<NC, M, XT>), grid, dim3(WG), ragged_lds(NC, M), s,
                           (const uint8_t *)w->codes, (const uint16_t *)w->codebook,
                           (const uint16_t *)w->scales, x, y, n, k);
    }
}

template <int NC, int XT>
bool dispatch_m(int m, const qmv_weights *w, const void *x, float *y, hipStream_t s) {
    switch (m) {
    case 1: launch<NC, 1, XT>(w, x, y, s); return true;
    case 2: launch<NC, 2, XT>(w, x, y, s); return true;
    case 3: launch<NC, 3, XT>(w, x, y, s); return true;
    case 4: launch<NC, 4, XT>(w, x, y, s); return true;
    case 5: launch<NC, 5, XT>(w, x, y, s); return true;
    case 6: launch<NC, 6, XT>(w, x, y, s); return true;
    case 7: launch<NC, 7, XT>(w, x, y, s); return true;
    case 8: launch<NC, 8, XT>(w, x, y, s); return true;
    }
    return false;
}

}  // namespace

const char *launch_gemv_aq(const qmv_weights *w, int m, const void *x, int xt, float *y, hipStream_t s) {
    if (w->n > INT32_MAX || w->k > INT32_MAX / 8) return nullptr;
    const int nc = w->fmt == QMV_AQ3X8 ? 3 : 2;
    const bool str = w->k % 64 == 0;
    const bool half = str && stream_half(m, w->n);
    const size_t lds = !str ? ragged_lds(nc, m) : stream_lds(nc, m, w->k, half ? 32 : 64);
    if ((int64_t)lds > device_info().lds_per_block) return nullptr;
    bool ok;
    if (nc == 2)
        ok = xt == QMV_F32 ? dispatch_m<2, 0>(m, w, x, y, s) : dispatch_m<2, 1>(m, w, x, y, s);
    else
        ok = xt == QMV_F32 ? dispatch_m<3, 0>(m, w, x, y, s) : dispatch_m<3, 1>(m, w, x, y, s);
    if (!ok) return nullptr;
    if (!str) return nc == 2 ? "aq2x8.ragged.lds-codebook.fma-mix" : "aq3x8.ragged.lds-codebook.fma-mix";
    if (half)
        return nc == 2 ? "aq2x8.stream.lds-codebook.fma-mix.2row.half-step" : "aq3x8.stream.lds-codebook.fma-mix.2row.half-step";
    if (stream_rows(m, w->n) == 4)
        return nc == 2 ? "aq2x8.stream.lds-codebook.fma-mix.4row" : "aq3x8.stream.lds-codebook.fma-mix.4row";
    if (stream_rows(m, w->n) == 2)
        return nc == 2 ? "aq2x8.stream.lds-codebook.fma-mix.2row" : "aq3x8.stream.lds-codebook.fma-mix.2row";
    return nc == 2 ? "aq2x8.stream.lds-codebook.fma-mix" : "aq3x8.stream.lds-codebook.fma-mix";
}

}  // namespace qmv
