// gemv_cb8.hip -- 8-bit codebook GEMV (batch 1..8) for gfx950.
//
// Format ("Chasing x100", quality table: the 8-bit codebook has K=256 entries and is the
// precision lifted onto the shared experts and the output head): one index byte per
// weight, in k order, into a 256-entry fp16 codebook of the weight's output row
// (reading: one codebook per row; a codebook per 128-weight group, as the 4-bit format
// has, would cost 32 bits per weight in codebook bytes alone).
//
// Kernel (the streaming skeleton of gemv_stream.h; the format takes k % 64 == 0):
//   * each wave copies its row's codebook (512 bytes, one 8-byte load per lane) into its
//     own LDS slice, so one ds_read_u16 returns the fp16 weight for an index;
//   * lane l owns unit l of each 4096-weight step: 64 index bytes, four 128-bit loads,
//     prefetched a step ahead;
//   * per dword of 4 indices: two masks form 2 * index in the two 16-bit halves of two
//     registers (even and odd bytes), one SDWA add per weight selects the half and adds
//     the slice address, one ds_read_u16 fetches the weight; v_fma_mix_f32 multiplies
//     the fp16 weight by the fp32 activation (exact product); each looked-up weight is
//     used for every batch row;
//   * the 64 lane partials are summed with DPP.
#include "device_common.h"
#include "gemv_stream.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

using stream::WG;
using stream::WAVES;
using stream::XU;

// base + 16-bit half H of v, in one v_add_u32 with an SDWA word select on the second source.
template <int H>
QMV_DEV uint32_t add_half(uint32_t base, uint32_t v) {
    uint32_t r;
    if (H == 0) asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_0" : "=v"(r) : "v"(base), "v"(v));
    if (H == 1) asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1" : "=v"(r) : "v"(base), "v"(v));
    return r;
}

QMV_DEV float lds_h(uint32_t a) {
    return h2f(*(const __attribute__((address_space(3))) uint16_t *)(uintptr_t)a);
}

struct Cb8Policy {
    static constexpr int R = 1;  // rows per wave
    struct Codes {
        uint4 q[4];  // index bytes 0..63 of the unit
    };
    const uint8_t *irow;  // this row's indices
    uint32_t tb;          // LDS byte address of this wave's codebook

    __device__ __forceinline__ void load(Codes &c, int unit) const {
        const uint8_t *p = irow + (int64_t)unit * 64;
#pragma unroll
        for (int i = 0; i < 4; i++) c.q[i] = ld_stream16(p + 16 * i);
    }

    template <int M>
    __device__ __forceinline__ void dot(const Codes &c, const float *xu, float (&s)[M]) const {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const uint4 q4 = c.q[i >> 2];
            const uint32_t w = (i & 3) == 0 ? q4.x : (i & 3) == 1 ? q4.y : (i & 3) == 2 ? q4.z : q4.w;
            const uint32_t ev = (w << 1) & 0x01FE01FEu;  // 2 * index of bytes 0 and 2
            const uint32_t od = (w >> 7) & 0x01FE01FEu;  // 2 * index of bytes 1 and 3
            const float v0 = lds_h(add_half<0>(tb, ev)), v1 = lds_h(add_half<0>(tb, od));
            const float v2 = lds_h(add_half<1>(tb, ev)), v3 = lds_h(add_half<1>(tb, od));
#pragma unroll
            for (int m = 0; m < M; m++) {
                const float4 xv = *(const float4 *)(xu + m * stream::XBUF + 4 * i);
                float t = s[m];
                t = fmaf(v0, xv.x, t);
                t = fmaf(v1, xv.y, t);
                t = fmaf(v2, xv.z, t);
                s[m] = fmaf(v3, xv.w, t);
            }
        }
    }
};

// LDS layout: the activation buffers (xfloats floats), then one 512-byte codebook per wave.
template <int M, int XT>
__global__ void __launch_bounds__(WG) cb8_stream_kernel(const uint8_t *__restrict__ idx,
                                                        const uint16_t *__restrict__ cb,
                                                        const void *__restrict__ x, float *__restrict__ y,
                                                        int n, int k, int xfloats) {
    extern __shared__ float4 lds4[];
    float *sx = (float *)lds4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint16_t *tab = (uint16_t *)(sx + xfloats) + wave * 256;
    const int row = blockIdx.x * WAVES + wave;
    const int rowc = row < n ? row : n - 1;

    const u32x2 e = __builtin_nontemporal_load((const u32x2 *)(cb + (int64_t)rowc * 256 + 4 * lane));
    *(uint2 *)(tab + 4 * lane) = make_uint2(e.x, e.y);  // visible after the walk's first barrier

    Cb8Policy pol{idx + (int64_t)rowc * k, (uint32_t)(uintptr_t)tab};
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; m++) acc[m] = 0.f;
    stream::walk_row<Cb8Policy, M, XT>(pol, x, k, sx, acc);
#pragma unroll
    for (int m = 0; m < M; m++) {
        const float t = wave_sum(acc[m]);
        if (lane == 0 && row < n) y[(int64_t)m * n + row] = t;
    }
}

size_t lds_of(int m, int64_t k) { return stream::x_lds_bytes(m, k) + (size_t)WAVES * 512; }

template <int M, int XT>
void launch(const qmv_weights *w, const void *x, float *y, hipStream_t s) {
    const int n = (int)w->n, k = (int)w->k;
    hipLaunchKernelGGL((cb8_stream_kernel<M, XT>), dim3((n + WAVES - 1) / WAVES), dim3(WG), lds_of(M, k), s,
                       (const uint8_t *)w->codes, (const uint16_t *)w->codebook, x, y, n, k,
                       (int)(stream::x_lds_bytes(M, k) / 4));
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

const char *launch_gemv_cb8(const qmv_weights *w, int m, const void *x, int xt, float *y, hipStream_t s) {
    if (w->n > INT32_MAX || w->k > INT32_MAX / 8 || w->k % 64) return nullptr;
    if ((int64_t)lds_of(m, w->k) > device_info().lds_per_block) return nullptr;
    const bool ok = xt == QMV_F32 ? dispatch_m<0>(m, w, x, y, s) : dispatch_m<1>(m, w, x, y, s);
    return ok ? "cb8.stream.lds-table.fma-mix" : nullptr;
}

}  // namespace qmv
