// gemv_cb8.hip -- 8-bit codebook GEMV (batch 1..8) for gfx950.
//
// Format ("Chasing x100", quality table: the 8-bit codebook has K=256 entries and is the
// precision lifted onto the shared experts and the output head): one index byte per
// weight, in k order, into a 256-entry fp16 codebook of the weight's output row
// (reading: one codebook per row; a codebook per 128-weight group, as the 4-bit format
// has, would cost 32 bits per weight in codebook bytes alone).
//
// Kernel (the streaming skeleton of gemv_stream.h; the format takes k % 64 == 0):
//   * each wave copies its row's codebook (256 fp16 entries, one 8-byte load per lane)
//     into its own LDS slice; at batch 3 and from batch 5 up it expands the entries to
//     exact fp32 there, so one ds_read_b32 returns the weight of an index as fp32 and no
//     conversion is left in the dot (otherwise ds_read_u16 and v_fma_mix_f32);
//   * lane l owns unit l of each 4096-weight step: 64 index bytes, four 128-bit loads,
//     prefetched a step ahead;
//   * per dword of 4 indices: two masks form 4 * index (fp32 slice) or 2 * index (fp16)
//     in the two 16-bit halves of two registers (even and odd bytes), one SDWA add per
//     weight selects the half and adds the slice address, one LDS read fetches the
//     weight; each looked-up weight feeds one FMA per batch row (exact product, fp32
//     sum); on the fp32 path the reads of the next dword are in flight during the FMAs
//     of this one, and each row keeps two partial sums (even and odd dwords);
//   * the 64 lane partials are summed with DPP.
#include <cstring>

#include "device_common.h"
#include "gemv_stream.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

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

QMV_DEV float lds_f(uint32_t a) { return *(const __attribute__((address_space(3))) float *)(uintptr_t)a; }

// The fp32-slice path (expanded codebook, v_fmac_f32, pipelined reads) at batch 3 and from
// batch 5 up.  At batch 4 it needs 138 VGPRs, which costs rows of at most 4096 weights
// their second workgroup per CU (7168x2048: 14.2 -> 17.6 us) and spills when capped at
// 128, so batch 4 keeps the fp16 path like batch 1 and 2 (measured on one device in turn:
// batch 3 10.6/13.4 -> 10.3/11.8 us, batch 8 16.2/30.5 -> 14.9/28.0 us at 2048x7168 and
// 7168x2048).
constexpr bool f32_tab(int m) { return m == 3 || m >= 5; }

template <int L>
struct Cb8Policy {
    static constexpr int R = 1;  // rows per lane group
    static constexpr int XB = stream::xbuf_of(L);  // floats between batch rows' staged steps
    struct Codes {
        uint4 q[4];  // index bytes 0..63 of the unit
    };
    const uint8_t *irow;  // this row's indices
    uint32_t tb;          // LDS byte address of this wave's codebook slice

    __device__ __forceinline__ void load(Codes &c, int unit) const {
        const uint8_t *p = irow + (int64_t)unit * 64;
#pragma unroll
        for (int i = 0; i < 4; i++) c.q[i] = ld_stream16(p + 16 * i);
    }

    // The 4 weights of dword i; the slice holds fp32 (4 * index) or fp16 (2 * index).
    template <int M>
    __device__ __forceinline__ void lookup(const Codes &c, int i, float (&v)[4]) const {
        const uint4 q4 = c.q[i >> 2];
        const uint32_t w = (i & 3) == 0 ? q4.x : (i & 3) == 1 ? q4.y : (i & 3) == 2 ? q4.z : q4.w;
        if constexpr (f32_tab(M)) {
            const uint32_t ev = (w << 2) & 0x03FC03FCu;  // 4 * index of bytes 0 and 2
            const uint32_t od = (w >> 6) & 0x03FC03FCu;  // 4 * index of bytes 1 and 3
            v[0] = lds_f(add_half<0>(tb, ev));
            v[1] = lds_f(add_half<0>(tb, od));
            v[2] = lds_f(add_half<1>(tb, ev));
            v[3] = lds_f(add_half<1>(tb, od));
        } else {
            const uint32_t ev = (w << 1) & 0x01FE01FEu;  // 2 * index of bytes 0 and 2
            const uint32_t od = (w >> 7) & 0x01FE01FEu;  // 2 * index of bytes 1 and 3
            v[0] = lds_h(add_half<0>(tb, ev));
            v[1] = lds_h(add_half<0>(tb, od));
            v[2] = lds_h(add_half<1>(tb, ev));
            v[3] = lds_h(add_half<1>(tb, od));
        }
    }

    // The 4 weights of dword i and the activations of every batch row for them.
    template <int M>
    __device__ __forceinline__ void fetch(const Codes &c, const float *xu, int i, float (&v)[4], float4 (&xv)[M]) const {
        lookup<M>(c, i, v);
#pragma unroll
        for (int m = 0; m < M; m++) xv[m] = *(const float4 *)(xu + m * XB + 4 * i);
    }

    template <int M>
    __device__ __forceinline__ static void fma4(const float (&v)[4], const float4 (&xv)[M], float (&t)[M]) {
#pragma unroll
        for (int m = 0; m < M; m++) {
            float a = t[m];
            a = fmaf(v[0], xv[m].x, a);
            a = fmaf(v[1], xv[m].y, a);
            a = fmaf(v[2], xv[m].z, a);
            t[m] = fmaf(v[3], xv[m].w, a);
        }
    }

    // Pins the sums here: without it the FMAs sink to the end of the unit and every
    // looked-up weight and activation of the unit stays live.
    template <int M>
    __device__ __forceinline__ static void pin(float (&t)[M]) {
#pragma unroll
        for (int m = 0; m < M; m++) asm volatile("" : "+v"(t[m]));
    }

    // fp16 path: straight-line code, left to the scheduler, each batch row's activations
    // read next to its FMAs (the fp16 weight is converted inside v_fma_mix_f32).  fp32
    // path: the reads of dword i + 1 are issued before the FMAs of dword i and nothing
    // else is hoisted (left alone, the scheduler hoisted every activation read of the
    // unit: 256 VGPRs at batch 4, spills at batch 8), two partial sums per batch row.
    template <int M>
    __device__ __forceinline__ void dot(const Codes &c, const float *xu, float (&s)[M]) const {
        float v[2][4];
        float4 xv[2][M];
        if constexpr (!f32_tab(M)) {
#pragma unroll
            for (int i = 0; i < 16; i++) {
                lookup<M>(c, i, v[0]);
#pragma unroll
                for (int m = 0; m < M; m++) {
                    const float4 x4 = *(const float4 *)(xu + m * XB + 4 * i);
                    float a = s[m];
                    a = fmaf(v[0][0], x4.x, a);
                    a = fmaf(v[0][1], x4.y, a);
                    a = fmaf(v[0][2], x4.z, a);
                    s[m] = fmaf(v[0][3], x4.w, a);
                }
            }
        } else {
            float t[2][M];
#pragma unroll
            for (int m = 0; m < M; m++) t[0][m] = s[m], t[1][m] = 0.f;
            fetch<M>(c, xu, 0, v[0], xv[0]);
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                fetch<M>(c, xu, i + 1, v[1], xv[1]);
                __builtin_amdgcn_sched_barrier(0);
                fma4<M>(v[0], xv[0], t[0]);
                pin<M>(t[0]);
                __builtin_amdgcn_sched_barrier(0);
                if (i + 2 < 16) fetch<M>(c, xu, i + 2, v[0], xv[0]);
                __builtin_amdgcn_sched_barrier(0);
                fma4<M>(v[1], xv[1], t[1]);
                pin<M>(t[1]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int m = 0; m < M; m++) s[m] = t[0][m] + t[1][m];
        }
    }
};

constexpr int tab_bytes(int m) { return f32_tab(m) ? 1024 : 512; }

// L lanes per row: 64 (one row per wave, 512-thread workgroups, 4096-weight steps) or 32
// (two rows per wave, 256-thread workgroups, 2048-weight steps).  From batch 5 up the
// activations of a 4096-weight step (m x 17 KB, one buffer) leave room for one 512-thread
// workgroup per CU, which then waits on its loads with nothing to overlap; the half step
// lets two workgroups share a CU.
// LDS layout: the activation buffers (xfloats floats), then one codebook slice per row:
// 512 B of fp16 (an fp32 slice would cost batch 1 a workgroup per CU) or 1 KB of fp32.
template <int M, int XT, int L>
__global__ void __launch_bounds__(stream::wg_of(L)) cb8_stream_kernel(const uint8_t *__restrict__ idx,
                                                                      const uint16_t *__restrict__ cb,
                                                                      const void *__restrict__ x,
                                                                      float *__restrict__ y, int n, int k,
                                                                      int xfloats) {
    extern __shared__ float4 lds4[];
    constexpr int G = 64 / L;  // rows per wave
    constexpr int WAVES_ = stream::wg_of(L) / 64;
    constexpr int TB = tab_bytes(M);
    float *sx = (float *)lds4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane / L, ul = lane % L;
    char *tab = (char *)(sx + xfloats) + (wave * G + sub) * TB;
    const int row = (blockIdx.x * WAVES_ + wave) * G + sub;
    const int rowc = row < n ? row : n - 1;

    // the row's 256 entries over its L lanes; visible after the walk's first barrier
    const uint16_t *cbr = cb + (int64_t)rowc * 256;
#pragma unroll
    for (int h = 0; h < G; h++) {
        const int j = 4 * (ul + L * h);  // first of this lane's four entries
        const u32x2 e = __builtin_nontemporal_load((const u32x2 *)(cbr + j));
        if constexpr (TB == 1024)
            *(float4 *)(tab + 4 * j) = make_float4(lo_h(e.x), hi_h(e.x), lo_h(e.y), hi_h(e.y));
        else
            *(uint2 *)(tab + 2 * j) = make_uint2(e.x, e.y);
    }

    Cb8Policy<L> pol{idx + (int64_t)rowc * k, (uint32_t)(uintptr_t)tab};
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; m++) acc[m] = 0.f;
    stream::walk_row<Cb8Policy<L>, M, XT, L>(pol, x, k, sx, acc);
#pragma unroll
    for (int m = 0; m < M; m++) {
        const float t = L == 64 ? wave_sum(acc[m]) : group_sum(acc[m], L);
        if (ul == 0 && row < n) y[(int64_t)m * n + row] = t;
    }
}

size_t lds_of(int m, int64_t k, int l) {
    return stream::x_lds_bytes(m, k, l) + (size_t)(stream::wg_of(l) / l) * tab_bytes(m);
}

template <int M, int XT, int L>
void launch(const qmv_weights *w, const void *x, float *y, hipStream_t s) {
    const int n = (int)w->n, k = (int)w->k;
    constexpr int ROWS = stream::wg_of(L) / L;  // rows per workgroup: 8
    hipLaunchKernelGGL((cb8_stream_kernel<M, XT, L>), dim3((n + ROWS - 1) / ROWS), dim3(stream::wg_of(L)),
                       lds_of(M, k, L), s, (const uint8_t *)w->codes, (const uint16_t *)w->codebook, x, y, n, k,
                       (int)(stream::x_lds_bytes(M, k, L) / 4));
}

template <int XT>
bool dispatch_m(int m, bool half, const qmv_weights *w, const void *x, float *y, hipStream_t s) {
    if (half) {
        switch (m) {
        case 5: launch<5, XT, 32>(w, x, y, s); return true;
        case 6: launch<6, XT, 32>(w, x, y, s); return true;
        case 7: launch<7, XT, 32>(w, x, y, s); return true;
        case 8: launch<8, XT, 32>(w, x, y, s); return true;
        }
        return false;
    }
    switch (m) {
    case 1: launch<1, XT, 64>(w, x, y, s); return true;
    case 2: launch<2, XT, 64>(w, x, y, s); return true;
    case 3: launch<3, XT, 64>(w, x, y, s); return true;
    case 4: launch<4, XT, 64>(w, x, y, s); return true;
    case 5: launch<5, XT, 64>(w, x, y, s); return true;
    case 6: launch<6, XT, 64>(w, x, y, s); return true;
    case 7: launch<7, XT, 64>(w, x, y, s); return true;
    case 8: launch<8, XT, 64>(w, x, y, s); return true;
    }
    return false;
}

}  // namespace

const char *launch_gemv_cb8(const qmv_weights *w, int m, const void *x, int xt, float *y, hipStream_t s) {
    if (w->n > INT32_MAX || w->k > INT32_MAX / 8 || w->k % 64) return nullptr;
    // Batch 5 and up on matrices of at least 16 rows per CU (two 8-row workgroups per CU):
    // the half-step form.  With fewer rows it would leave one 4-wave workgroup per CU
    // (2048x7168 at batch 5: 11.6 -> 13.2 us; 7168x2048: 21.1 -> 11.2 us).  Test overrides
    // "cb8.half" and "cb8.wg512" force either form from batch 5 up.
    const char *fp = forced_path();
    const bool half = m >= 5 && std::strcmp(fp, "cb8.wg512") != 0 &&
                      (w->n >= 16 * (int64_t)device_info().num_cus || std::strcmp(fp, "cb8.half") == 0);
    if ((int64_t)lds_of(m, w->k, half ? 32 : 64) > device_info().lds_per_block) return nullptr;
    const bool ok = xt == QMV_F32 ? dispatch_m<0>(m, half, w, x, y, s) : dispatch_m<1>(m, half, w, x, y, s);
    if (!ok) return nullptr;
    if (half) return "cb8.stream.lds-f32-table.fmac.half-step";
    return f32_tab(m) ? "cb8.stream.lds-f32-table.fmac" : "cb8.stream.lds-table.fma-mix";
}

}  // namespace qmv
