// gemv_cb4.hip -- 4-bit codebook GEMV and the routed-expert FFN built on it (gfx950).
//
// Format ("Chasing x100": a 4-bit codebook format with K=16 entries, decoded by a fused
// GEMV; the routed experts of a mixture dominate the bytes per token): every 128
// consecutive weights of a row share one 16-entry fp16 codebook, and each weight is a
// 4-bit index into it.  Index byte i holds indices 2i (bits 0-3) and 2i+1 (bits 4-7).
//
// The page's CPU kernel decodes with one byte-shuffle per 32 weights; on gfx950 the
// table lookup is an LDS gather instead:
//   * the workgroup stages the activations once into LDS as fp32 (blocks of 32 with a
//     4-float pad, so lanes reading consecutive blocks with ds_read_b128 do not collide);
//   * each wave copies its row's codebooks into its own LDS slice (coalesced 16-byte
//     loads), so one ds_read_u16 returns the fp16 weight for an index;
//   * v_fma_mix_f32 multiplies that fp16 value by the fp32 activation (exact product),
//     so the only rounding is the fp32 accumulation;
//   * lane l owns the 32-weight chunks l, l+64, ... of the row (16 index bytes = one
//     128-bit load); the 64 partials are summed with DPP.
// The same kernel runs three jobs: a plain GEMV (one row per wave), the fused gate/up
// stage of the expert FFN (a wave computes row r of G_e and of U_e and writes
// SiLU(g) * u), and the down stage (y_e = D_e h_e), with the expert id read on the
// device and its planes found at e * plane_bytes from expert 0's.
#include <cstring>

#include "device_common.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int WG = 512;
constexpr int WAVES = WG / 64;
constexpr int XS = 36;

enum { JOB_GEMV = 0, JOB_GATEUP = 1, JOB_DOWN = 2, JOB_DOWN2 = 3 };  // DOWN2: two rows per wave

struct Cb4Args {
    const uint8_t *idx0, *idx1;  // index planes (expert 0): first matrix, second (gate/up: up)
    const uint16_t *cb0, *cb1;   // codebook planes
    int64_t idx_stride, cb_stride;  // bytes / entries between experts
    const void *x;               // activations: [M][k] (GEMV, GATEUP) or h [n_ids][k] (DOWN)
    float *y;                    // GEMV: [M][n]; GATEUP: h [n_ids][n]; DOWN: y [n_ids][n]
    const int32_t *ids;
    int n, k, n_experts;
};

// Activation chunks (16 bytes each) a thread stages, and the LDS floats of the padded
// x image: XPT * WG chunk slots in blocks of 8 (36 floats per block).
constexpr int xpt_of(int m, int cpl) { return (m * cpl * 512 + WG - 1) / WG; }
constexpr int x_floats(int m, int cpl) { return xpt_of(m, cpl) * WG / 8 * XS; }

// base + byte `B` of v, in one v_add_u32 with an SDWA byte select on the second source.
template <int B>
QMV_DEV uint32_t add_byte(uint32_t base, uint32_t v) {
    uint32_t r;
    if (B == 0) asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(base), "v"(v));
    if (B == 1) asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(base), "v"(v));
    if (B == 2) asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(base), "v"(v));
    if (B == 3) asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(base), "v"(v));
    return r;
}

// fp16 LDS word at byte address a, as float.
QMV_DEV float lds_h(uint32_t a) {
    return h2f(*(const __attribute__((address_space(3))) uint16_t *)(uintptr_t)a);
}

// sum over one 32-weight chunk: cb[idx] * x, with the chunk's table at LDS byte address tb.
// The byte offsets 2*idx of a dword's eight indices are formed with two masks (even and
// odd nibbles, one per byte lane); each lookup is then one SDWA add and one ds_read_u16.
QMV_DEV float chunk_dot(uint4 q, uint32_t tb, const float *xb) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const float4 x0 = *(const float4 *)(xb + 8 * j), x1 = *(const float4 *)(xb + 8 * j + 4);
        const uint32_t ev = (w[j] << 1) & 0x1E1E1E1Eu;  // 2 * index of weights 0, 2, 4, 6
        const uint32_t od = (w[j] >> 3) & 0x1E1E1E1Eu;  // 2 * index of weights 1, 3, 5, 7
        a = fmaf(lds_h(add_byte<0>(tb, ev)), x0.x, a);
        b = fmaf(lds_h(add_byte<0>(tb, od)), x0.y, b);
        a = fmaf(lds_h(add_byte<1>(tb, ev)), x0.z, a);
        b = fmaf(lds_h(add_byte<1>(tb, od)), x0.w, b);
        a = fmaf(lds_h(add_byte<2>(tb, ev)), x1.x, a);
        b = fmaf(lds_h(add_byte<2>(tb, od)), x1.y, b);
        a = fmaf(lds_h(add_byte<3>(tb, ev)), x1.z, a);
        b = fmaf(lds_h(add_byte<3>(tb, od)), x1.w, b);
    }
    return a + b;
}

// One row's index chunks (lane l: chunks l, l+64, ...) and its codebooks (16 B pieces
// lane, lane+64, ...; two pieces per 128-weight group), loaded with clamped indices so
// that no branch sits around a load (a branch would make the compiler wait for the load
// on the spot).
template <int CPL>
struct RowData {
    uint4 q[CPL];
    uint4 t[(CPL + 1) / 2];
};

// Codebooks first: the barrier before the dots waits for them (vector loads complete in
// issue order), while the index chunks may still be arriving.
template <int CPL>
QMV_DEV void load_tables(RowData<CPL> &r, const uint16_t *cb_row, int nchunk, int lane) {
    const int npieces = nchunk >> 1;  // 16-byte codebook pieces of the row
#pragma unroll
    for (int u = 0; u < (CPL + 1) / 2; u++) {
        const int i = lane + 64 * u;
        r.t[u] = ld_stream16(cb_row + 8 * (int64_t)(i < npieces ? i : npieces - 1));
    }
}

template <int CPL>
QMV_DEV void load_codes(RowData<CPL> &r, const uint8_t *idx_row, int nchunk, int lane) {
#pragma unroll
    for (int u = 0; u < CPL; u++) {
        const int c = lane + 64 * u;
        r.q[u] = ld_stream16(idx_row + 16 * (int64_t)(c < nchunk ? c : nchunk - 1));
    }
}

template <int CPL>
QMV_DEV void store_tables(const RowData<CPL> &r, uint16_t *tab, int nchunk, int lane) {
    const int npieces = nchunk >> 1;
#pragma unroll
    for (int u = 0; u < (CPL + 1) / 2; u++) {
        const int i = lane + 64 * u;
        // a lane past the end rewrites the last piece with the same bytes
        ((uint4 *)tab)[i < npieces ? i : npieces - 1] = r.t[u];
    }
}

template <int CPL>
QMV_DEV float row_dot(const RowData<CPL> &r, const uint16_t *tab, const float *sx, int nchunk, int lane) {
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < CPL; u++) {
        const int c = lane + 64 * u;
        const int cc = c < nchunk ? c : nchunk - 1;
        const float v = acc + chunk_dot(r.q[u], (uint32_t)(uintptr_t)(tab + (cc >> 2) * 16), sx + cc * XS);
        acc = c < nchunk ? v : acc;
    }
    return acc;
}

// GEMV job: grid.x over row blocks; one row per wave.
// GATEUP job: grid.x over row blocks, grid.y = expert slot j; x is the token's activations.
// DOWN job: grid.x over row blocks, grid.y = expert slot j; x is h (fp32) [n_ids][k].
// Order of work: expert id and activation loads, then (once the id is known) every code
// and codebook load of the wave's row(s), then the LDS writes, one barrier, the dots.
// Rows past n and invalid expert ids read clamped (in-bounds) addresses; their outputs are
// not written (rows) or are NaN (ids).
template <int JOB, int M, int CPL, int XT>
__global__ void __launch_bounds__(WG) cb4_kernel(Cb4Args a) {
    extern __shared__ float4 lds4[];
    constexpr int XPT = xpt_of(M, CPL);
    constexpr bool DOWN = JOB == JOB_DOWN || JOB == JOB_DOWN2;
    constexpr int XT_ = DOWN ? 0 : XT;
    const int k = a.k, ngroups = k >> 7, nchunk = k >> 5;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = (blockIdx.x * WAVES + wave) * (JOB == JOB_DOWN2 ? 2 : 1);
    const int rowc = row < a.n ? row : a.n - 1;
    const int rowc1 = row + 1 < a.n ? row + 1 : a.n - 1;  // DOWN2: the wave's second row
    constexpr int NT = JOB == JOB_GATEUP || JOB == JOB_DOWN2 ? 2 : 1;  // tables (rows) per wave
    float *sx = (float *)lds4;
    uint16_t *tabs = (uint16_t *)(sx + x_floats(M, CPL));
    uint16_t *tab0 = tabs + wave * NT * ngroups * 16;
    uint16_t *tab1 = tab0 + ngroups * 16;

    int32_t id = 0;
    if (JOB != JOB_GEMV) id = a.ids[blockIdx.y];
    const void *x = DOWN ? (const void *)((const float *)a.x + (int64_t)blockIdx.y * k) : a.x;
    const int total = M * (k >> 2);
    float4 xv[XPT];
#pragma unroll
    for (int j = 0; j < XPT; j++) {
        const int c = threadIdx.x + j * WG;
        xv[j] = ld_act4<XT_>(x, (int64_t)(c < total ? c : total - 1) * 4);
    }

    const bool ok_expert = JOB == JOB_GEMV || (id >= 0 && id < a.n_experts);
    const int64_t e = ok_expert ? id : 0;
    RowData<CPL> r0, r1;
    load_tables<CPL>(r0, a.cb0 + e * a.cb_stride + (int64_t)rowc * ngroups * 16, nchunk, lane);
    if (JOB == JOB_GATEUP) load_tables<CPL>(r1, a.cb1 + e * a.cb_stride + (int64_t)rowc * ngroups * 16, nchunk, lane);
    if (JOB == JOB_DOWN2) load_tables<CPL>(r1, a.cb0 + e * a.cb_stride + (int64_t)rowc1 * ngroups * 16, nchunk, lane);
    load_codes<CPL>(r0, a.idx0 + e * a.idx_stride + (int64_t)rowc * (k >> 1), nchunk, lane);
    if (JOB == JOB_GATEUP) load_codes<CPL>(r1, a.idx1 + e * a.idx_stride + (int64_t)rowc * (k >> 1), nchunk, lane);
    if (JOB == JOB_DOWN2) load_codes<CPL>(r1, a.idx0 + e * a.idx_stride + (int64_t)rowc1 * (k >> 1), nchunk, lane);
    __builtin_amdgcn_sched_barrier(0);  // every load is issued before the LDS writes wait

    float4 *dst = lds4 + (threadIdx.x >> 3) * (XS / 4) + (threadIdx.x & 7);
#pragma unroll
    for (int j = 0; j < XPT; j++) dst[j * (WG / 8) * (XS / 4)] = xv[j];
    store_tables<CPL>(r0, tab0, nchunk, lane);
    if (NT == 2) store_tables<CPL>(r1, tab1, nchunk, lane);
    lds_barrier();

    if (JOB == JOB_GEMV) {
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float t = wave_sum(row_dot<CPL>(r0, tab0, sx + m * nchunk * XS, nchunk, lane));
            if (lane == 0 && row < a.n) a.y[(int64_t)m * a.n + row] = t;
        }
        return;
    }
    float *out = a.y + (int64_t)blockIdx.y * a.n;
    if (JOB == JOB_GATEUP) {
        const float g = wave_sum(row_dot<CPL>(r0, tab0, sx, nchunk, lane));
        const float u = wave_sum(row_dot<CPL>(r1, tab1, sx, nchunk, lane));
        if (lane == 0 && row < a.n) out[row] = ok_expert ? g / (1.f + expf(-g)) * u : __builtin_nanf("");
    } else if (JOB == JOB_DOWN2) {
        const float t0 = wave_sum(row_dot<CPL>(r0, tab0, sx, nchunk, lane));
        const float t1 = wave_sum(row_dot<CPL>(r1, tab1, sx, nchunk, lane));
        if (lane == 0 && row < a.n) out[row] = ok_expert ? t0 : __builtin_nanf("");
        if (lane == 0 && row + 1 < a.n) out[row + 1] = ok_expert ? t1 : __builtin_nanf("");
    } else {
        const float t = wave_sum(row_dot<CPL>(r0, tab0, sx, nchunk, lane));
        if (lane == 0 && row < a.n) out[row] = ok_expert ? t : __builtin_nanf("");
    }
}

template <int JOB, int M, int CPL, int XT>
void launch(const Cb4Args &a, int slots, hipStream_t s) {
    constexpr int NT = JOB == JOB_GATEUP || JOB == JOB_DOWN2 ? 2 : 1;
    constexpr int RPW = JOB == JOB_DOWN2 ? 2 : 1;  // matrix rows per wave
    const size_t lds = (size_t)x_floats(M, CPL) * 4 + (size_t)WAVES * NT * (a.k >> 7) * 32;
    const int waves = (a.n + RPW - 1) / RPW;
    hipLaunchKernelGGL((cb4_kernel<JOB, M, CPL, XT>), dim3((waves + WAVES - 1) / WAVES, slots), dim3(WG), lds, s, a);
}

template <int JOB, int M, int XT>
bool dispatch_cpl(int cpl, const Cb4Args &a, int slots, hipStream_t s) {
    switch (cpl) {
    case 1: launch<JOB, M, 1, XT>(a, slots, s); return true;
    case 2: launch<JOB, M, 2, XT>(a, slots, s); return true;
    case 3: launch<JOB, M, 3, XT>(a, slots, s); return true;
    case 4: launch<JOB, M, 4, XT>(a, slots, s); return true;
    case 5: launch<JOB, M, 5, XT>(a, slots, s); return true;
    case 6: launch<JOB, M, 6, XT>(a, slots, s); return true;
    case 7: launch<JOB, M, 7, XT>(a, slots, s); return true;
    case 8: launch<JOB, M, 8, XT>(a, slots, s); return true;
    }
    return false;
}

template <int XT>
bool dispatch_m(int m, int cpl, const Cb4Args &a, hipStream_t s) {
    switch (m) {
    case 1: return dispatch_cpl<JOB_GEMV, 1, XT>(cpl, a, 1, s);
    case 2: return dispatch_cpl<JOB_GEMV, 2, XT>(cpl, a, 1, s);
    case 3: return dispatch_cpl<JOB_GEMV, 3, XT>(cpl, a, 1, s);
    case 4: return dispatch_cpl<JOB_GEMV, 4, XT>(cpl, a, 1, s);
    case 5: return dispatch_cpl<JOB_GEMV, 5, XT>(cpl, a, 1, s);
    case 6: return dispatch_cpl<JOB_GEMV, 6, XT>(cpl, a, 1, s);
    case 7: return dispatch_cpl<JOB_GEMV, 7, XT>(cpl, a, 1, s);
    case 8: return dispatch_cpl<JOB_GEMV, 8, XT>(cpl, a, 1, s);
    }
    return false;
}

// ---- K-chunked GEMV, for batches whose activations exceed one workgroup's LDS and for
// rows longer than 16384.  K is walked 2048 weights at a time: per step a lane holds one
// 32-weight index chunk (16 bytes) and four codebook entries (8 bytes; the wave's 64 lanes
// together hold the step's 16 codebooks), the next step's are loaded while this one is
// computed (two register sets alternate), and each looked-up weight is used for all M
// activation rows.  One row per wave.  The wave's codebook slice holds the step's entries
// expanded to exact fp32 (1 KB), so a lookup is one ds_read_b32 of 4 * index and the
// products are plain v_fmac_f32 (no conversion per batch row, none of the dependency
// stalls of back-to-back v_fma_mix_f32).
constexpr int KCB = 2048;
constexpr int RXS = 64 * XS;  // floats of one activation row's staged step

struct StepData {
    uint4 q;  // index chunk
    uint2 t;  // codebook entries 4 lane .. 4 lane + 3 of the step (fp16)
};

// Step c's bytes for this lane, with clamped (in-bounds) indices past the row's end.
QMV_DEV void load_step(StepData &d, const uint8_t *idx_row, const uint16_t *cb_row, int c, int nchunk, int lane) {
    const int ci = c * 64 + lane;
    d.q = ld_stream16(idx_row + 16 * (int64_t)(ci < nchunk ? ci : nchunk - 1));
    const int ne = (nchunk >> 2) * 16, ei = c * 256 + 4 * lane;
    const u32x2 v = __builtin_nontemporal_load((const u32x2 *)(cb_row + (ei < ne ? ei : ne - 4)));
    d.t = make_uint2(v.x, v.y);
}

QMV_DEV float lds_f(uint32_t a) { return *(const __attribute__((address_space(3))) float *)(uintptr_t)a; }

// s[m] += sum over one 32-weight chunk of cb[idx] * x[m]; activation row m at xb + m RXS,
// the chunk's fp32 codebook at LDS byte address tb.
template <int M>
QMV_DEV void chunk_dot_m(uint4 q, uint32_t tb, const float *xb, float (&s)[M]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t ev = (w[j] << 2) & 0x3C3C3C3Cu;  // 4 * index of weights 0, 2, 4, 6
        const uint32_t od = (w[j] >> 2) & 0x3C3C3C3Cu;  // 4 * index of weights 1, 3, 5, 7
        const float v[8] = {lds_f(add_byte<0>(tb, ev)), lds_f(add_byte<0>(tb, od)),
                            lds_f(add_byte<1>(tb, ev)), lds_f(add_byte<1>(tb, od)),
                            lds_f(add_byte<2>(tb, ev)), lds_f(add_byte<2>(tb, od)),
                            lds_f(add_byte<3>(tb, ev)), lds_f(add_byte<3>(tb, od))};
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float4 x0 = *(const float4 *)(xb + m * RXS + 8 * j);
            const float4 x1 = *(const float4 *)(xb + m * RXS + 8 * j + 4);
            float a = s[m];
            a = fmaf(v[0], x0.x, a);
            a = fmaf(v[1], x0.y, a);
            a = fmaf(v[2], x0.z, a);
            a = fmaf(v[3], x0.w, a);
            a = fmaf(v[4], x1.x, a);
            a = fmaf(v[5], x1.y, a);
            a = fmaf(v[6], x1.z, a);
            s[m] = fmaf(v[7], x1.w, a);
        }
        // the sums are formed here: otherwise the FMAs can sink to the chunk's end with
        // every activation read of the chunk held live
#pragma unroll
        for (int m = 0; m < M; m++) asm volatile("" : "+v"(s[m]));
    }
}

// Per step: the activation loads (thread t loads piece t of each batch row), the next
// step's weight loads, the LDS writes (activations in padded 32-float blocks; the wave's
// codebook slice), a barrier, the dots.
template <int M, int XT>
__global__ void __launch_bounds__(WG) cb4_chunked_kernel(const uint8_t *__restrict__ idx,
                                                         const uint16_t *__restrict__ cb,
                                                         const void *__restrict__ x,
                                                         float *__restrict__ y, int n, int k) {
    extern __shared__ float4 lds4[];
    float *sx = (float *)lds4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float *tab = sx + M * RXS + wave * 256;
    const int nchunk = k >> 5, nst = (nchunk + 63) / 64;
    const int row = blockIdx.x * WAVES + wave;
    const int rowc = row < n ? row : n - 1;
    const uint8_t *idx_row = idx + (int64_t)rowc * (k >> 1);
    const uint16_t *cb_row = cb + (int64_t)rowc * (k >> 7) * 16;
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; m++) acc[m] = 0.f;
    auto step = [&](int c, const StepData &use, StepData &fill) {
        const int k0 = c * KCB;
        const int kq = min(KCB, k - k0) >> 2;  // 16-byte pieces of this step, per row
        const int t = threadIdx.x < kq ? threadIdx.x : kq - 1;
        float4 xv[M];
#pragma unroll
        for (int m = 0; m < M; m++) xv[m] = ld_act4<XT>(x, (int64_t)m * k + k0 + 4 * t);
        load_step(fill, idx_row, cb_row, c + 1, nchunk, lane);
        __builtin_amdgcn_sched_barrier(0);  // every load is issued before the LDS writes wait
        if (c) lds_barrier();  // the previous step's activations and tables are consumed
#pragma unroll
        for (int m = 0; m < M; m++)
            *(float4 *)(sx + m * RXS + (threadIdx.x >> 3) * XS + (threadIdx.x & 7) * 4) = xv[m];
        *(float4 *)(tab + 4 * lane) = make_float4(lo_h(use.t.x), hi_h(use.t.x), lo_h(use.t.y), hi_h(use.t.y));
        lds_barrier();
        const int ci = c * 64 + lane;
        const int lc = ci < nchunk ? lane : nchunk - 1 - c * 64;
        float s[M];
#pragma unroll
        for (int m = 0; m < M; m++) s[m] = 0.f;
        chunk_dot_m<M>(use.q, (uint32_t)(uintptr_t)(tab + (lc >> 2) * 16), sx + lc * XS, s);
        // the dots are computed here, not sunk into a branch over the valid lanes (which
        // would keep every activation read of the step live at once)
#pragma unroll
        for (int m = 0; m < M; m++) asm volatile("" : "+v"(s[m]));
#pragma unroll
        for (int m = 0; m < M; m++) acc[m] = ci < nchunk ? acc[m] + s[m] : acc[m];
    };
    StepData d0, d1;
    load_step(d0, idx_row, cb_row, 0, nchunk, lane);
    for (int c = 0; c < nst; c += 2) {
        step(c, d0, d1);
        if (c + 1 < nst) step(c + 1, d1, d0);
    }
#pragma unroll
    for (int m = 0; m < M; m++) {
        const float v = wave_sum(acc[m]);
        if (lane == 0 && row < n) y[(int64_t)m * n + row] = v;
    }
}

constexpr size_t chunked_lds(int m) { return (size_t)m * RXS * 4 + (size_t)WAVES * 256 * 4; }

template <int M, int XT>
void launch_chunked(const qmv_weights *w, const void *x, float *y, hipStream_t s) {
    const int n = (int)w->n, k = (int)w->k;
    hipLaunchKernelGGL((cb4_chunked_kernel<M, XT>), dim3((n + WAVES - 1) / WAVES), dim3(WG), chunked_lds(M), s,
                       (const uint8_t *)w->codes, (const uint16_t *)w->codebook, x, y, n, k);
}

template <int XT>
bool dispatch_chunked(int m, const qmv_weights *w, const void *x, float *y, hipStream_t s) {
    switch (m) {
    case 1: launch_chunked<1, XT>(w, x, y, s); return true;
    case 2: launch_chunked<2, XT>(w, x, y, s); return true;
    case 3: launch_chunked<3, XT>(w, x, y, s); return true;
    case 4: launch_chunked<4, XT>(w, x, y, s); return true;
    case 5: launch_chunked<5, XT>(w, x, y, s); return true;
    case 6: launch_chunked<6, XT>(w, x, y, s); return true;
    case 7: launch_chunked<7, XT>(w, x, y, s); return true;
    case 8: launch_chunked<8, XT>(w, x, y, s); return true;
    }
    return false;
}

size_t lds_need(int m, int64_t k, int nt) {
    const int cpl = (int)((k / 32 + 63) / 64);
    return (size_t)((m * cpl * 512 + WG - 1) / WG) * WG / 8 * XS * 4 + (size_t)WAVES * nt * (k >> 7) * 32;
}

}  // namespace

const char *launch_gemv_cb4(const qmv_weights *w, int m, const void *x, int xt, float *y, hipStream_t s) {
    const int64_t k = w->k, nchunk = k / 32;
    const int cpl = (int)((nchunk + 63) / 64);
    if (w->n > INT32_MAX || k > INT32_MAX / 8) return nullptr;
    // From batch 3 up the K-chunked kernel also where the one-shot kernel would fit: at
    // 7168x2048 it measured 8.7 / 9.6 / 13.7 us at batch 3 / 4 / 8 against 10.2 / 12.9 /
    // 22.7 (the one-shot kernel redoes each lookup per batch row); batch 2 is even and
    // batch 1 is faster one-shot.  Test override "cb4.chunked": the K-chunked kernel at
    // any size.
    const bool force_chunked = std::strcmp(forced_path(), "cb4.chunked") == 0;
    if (force_chunked || m >= 3 || cpl > 8 || (int64_t)m * k > 16384 ||
        (int64_t)lds_need(m, k, 1) > device_info().lds_per_block) {
        if ((int64_t)chunked_lds(m) > device_info().lds_per_block) return nullptr;
        const bool ok = xt == QMV_F32 ? dispatch_chunked<0>(m, w, x, y, s) : dispatch_chunked<1>(m, w, x, y, s);
        return ok ? "cb4.lds-f32-table-chunked.fmac" : nullptr;
    }
    Cb4Args a{(const uint8_t *)w->codes, nullptr, (const uint16_t *)w->codebook, nullptr, 0, 0, x, y, nullptr,
              (int)w->n, (int)k, 1};
    const bool ok = xt == QMV_F32 ? dispatch_m<0>(m, cpl, a, s) : dispatch_m<1>(m, cpl, a, s);
    return ok ? "cb4.lds-table.fma-mix" : nullptr;
}

// Routed-expert FFN over CB4 experts: gate/up/SiLU*mul, then down.
const char *launch_moe_cb4(const qmv_weights *gate, const qmv_weights *up, const qmv_weights *down,
                           int n_experts, const int32_t *ids, int n_ids, const void *x, int xt, float *h,
                           float *y, hipStream_t s) {
    const int64_t dm = gate->k, dff = gate->n;
    const int cpl1 = (int)((dm / 32 + 63) / 64), cpl2 = (int)((dff / 32 + 63) / 64);
    if (cpl1 > 8 || cpl2 > 8 || dm > 16384 || dff > 16384) return nullptr;
    if ((int64_t)lds_need(1, dm, 2) > device_info().lds_per_block ||
        (int64_t)lds_need(1, dff, 2) > device_info().lds_per_block)
        return nullptr;
    const int64_t idx_gu = dff * dm / 2, cb_gu = dff * (dm / 128) * 16;
    Cb4Args a1{(const uint8_t *)gate->codes, (const uint8_t *)up->codes, (const uint16_t *)gate->codebook,
               (const uint16_t *)up->codebook, idx_gu, cb_gu, x, h, ids, (int)dff, (int)dm, n_experts};
    const bool ok1 = xt == QMV_F32 ? dispatch_cpl<JOB_GATEUP, 1, 0>(cpl1, a1, n_ids, s)
                                   : dispatch_cpl<JOB_GATEUP, 1, 1>(cpl1, a1, n_ids, s);
    if (!ok1) return nullptr;
    const int64_t idx_d = dm * dff / 2, cb_d = dm * (dff / 128) * 16;
    Cb4Args a2{(const uint8_t *)down->codes, nullptr, (const uint16_t *)down->codebook, nullptr, idx_d, cb_d,
               h, y, ids, (int)dm, (int)dff, n_experts};
    const bool two = strcmp(forced_path(), "moe.down1") != 0;  // test override: one row per wave
    if (!(two ? dispatch_cpl<JOB_DOWN2, 1, 0>(cpl2, a2, n_ids, s) : dispatch_cpl<JOB_DOWN, 1, 0>(cpl2, a2, n_ids, s)))
        return nullptr;
    return two ? "moe.cb4.gateup-silu+down2" : "moe.cb4.gateup-silu+down";
}

}  // namespace qmv
