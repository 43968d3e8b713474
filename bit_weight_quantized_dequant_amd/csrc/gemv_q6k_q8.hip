// gemv_q6k_q8.hip -- q6_K decode GEMV over per-32 int8 activations, for gfx950.
//
// y[m][n] = sum_s d[n][s] * sum_{c in s} xs[m][c] * I[m][n][c], where
// I[m][n][c] = sum over the two 16-weight sub-blocks b of activation block c of
//              sc[n][b] * sum_{j in b} (q[n][j] - 32) * xq[m][j]          (exact integers)
// with xq / xs from the per-32 activation quantizer: the arithmetic of the q6_K prefill
// contraction ("57 · r54 — MINFER_MMQ_Q6K_EXP", §2.1: the 6-bit values recombined from
// ql and qh and centred by 32; §2.3: an integer transform), here at decode batch sizes
// with integer dot products instead of matrix cores (quantprobe LAWS.md, Law 4's
// per-format amendment: L-15, integer dot products recover most of the unpack cost, and
// L-16, the metadata is applied at the coarsest granularity the format allows).
//
// Work unit of one lane: a quarter super-block of 64 weights, half h and offset l0 = 16 odd
// (three 128-bit loads: ql[64h + l0 ..], ql[64h + 32 + l0 ..], qh[32h + l0 ..], plus the
// half's eight sub-scales and d).  Its four runs t = 0..3 of 16 weights (k = 128h + 32t +
// l0 + j) each lie under one sub-scale sc[8h + 2t + odd]:
//   * run t's codes, four per dword: the low (t < 2) or high (t >= 2) nibbles of the ql
//     run, OR-ed with (qh >> 2t) << 4 masked to bits 4-5 -- bytes 0..63, valid int8;
//   * four v_dot4c_i32_i8 per run, the chain started at -32 * (sum of the run's 16
//     activations), staged once per workgroup, so it ends at sum (q - 32) * xq exactly;
//   * the sub-scale multiplies in int32 (|value| < 2^24, so the conversion is exact), xs
//     multiplies the converted run sum, d multiplies the unit's sum once.
// The codes of a unit are unpacked once for all m batch rows.
//
// Activations are staged per workgroup in LDS as 16-byte runs (one per 16 activations, the
// batch rows of a run adjacent) and (xs of the run's 32-block, -32 * run sum) pairs.  Load order as in the q4_0 kernels:
// activation loads, then every weight load of the wave's row, then the LDS writes and one
// barrier; indices clamped, threads past the end write a junk slot.
#include "device_common.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int NP_MAX = 4;  // units per lane: k <= 64 * 64 * 4 = 16384

// 16-activation runs a workgroup stages (every unit a lane may own, all batch rows) plus a
// junk slot; 24 bytes each (16 activation bytes, xs, correction).
constexpr int q6q8_slots(int m, int np) { return m * np * 256 + 1; }
constexpr size_t q6q8_lds_bytes(int m, int np) { return (size_t)q6q8_slots(m, np) * 24; }

// Raw bytes of one unit (quarter super-block), as loaded.
struct Q6Unit {
    uint4 a, b, h;  // ql run (t = 0 low / t = 2 high nibbles), ql run (t = 1 / t = 3), qh run
    uint2 s8;       // the half's eight sub-scales
    uint16_t d;
};

QMV_DEV void q6_load(Q6Unit &w, const uint8_t *qlr, const uint8_t *qhr, const int8_t *scr, const uint16_t *dr,
                     int u) {
    const int sb = u >> 2, h = (u >> 1) & 1, odd = u & 1;
    const uint8_t *a = qlr + sb * 128 + 64 * h + 16 * odd;
    w.a = ld_stream16(a);
    w.b = ld_stream16(a + 32);
    w.h = ld_stream16(qhr + sb * 64 + 32 * h + 16 * odd);
    w.s8 = *(const uint2 *)(scr + sb * 16 + 8 * h);
    w.d = dr[sb];
}

// Adds unit u (clamped to uc) of the row to acc[m] for every batch row (nothing when u is
// past the row end).
template <int M>
QMV_DEV void q6_unit(const Q6Unit &w, int u, int uc, int nq, const uint4 *xr16, const float2 *meta,
                     float (&acc)[M]) {
    const int sb = uc >> 2, h = (uc >> 1) & 1, odd = uc & 1;
    // the unit's codes: run t, dword i = weights 128h + 32t + l0 + 4i .. + 3
    const uint32_t A[4] = {w.a.x, w.a.y, w.a.z, w.a.w};
    const uint32_t B[4] = {w.b.x, w.b.y, w.b.z, w.b.w};
    const uint32_t H[4] = {w.h.x, w.h.y, w.h.z, w.h.w};
    uint32_t q[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        q[0][i] = (A[i] & 0x0F0F0F0Fu) | ((H[i] << 4) & 0x30303030u);
        q[1][i] = (B[i] & 0x0F0F0F0Fu) | ((H[i] << 2) & 0x30303030u);
        q[2][i] = ((A[i] >> 4) & 0x0F0F0F0Fu) | (H[i] & 0x30303030u);
        q[3][i] = ((B[i] >> 4) & 0x0F0F0F0Fu) | ((H[i] >> 2) & 0x30303030u);
    }
    // sub-scale of run t: byte 2t + odd of the half's eight
    int sc[4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
        const uint32_t word = t < 2 ? w.s8.x : w.s8.y;
        sc[t] = (int)(int8_t)(uint8_t)(word >> (8 * (2 * (t & 1) + odd)));
    }
    const float d = h2f(w.d);
    const int run0 = sb * 16 + 8 * h + odd;  // run index of t = 0 (t adds 2)
#pragma unroll
    for (int m = 0; m < M; m++) {
        float f = 0.f;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int slot = (run0 + 2 * t) * M + m;
            const uint4 xv4 = xr16[slot];
            const float2 mt = meta[slot];
            int s = __float_as_int(mt.y);
            s = __builtin_amdgcn_sdot4((int)q[t][0], (int)xv4.x, s, false);
            s = __builtin_amdgcn_sdot4((int)q[t][1], (int)xv4.y, s, false);
            s = __builtin_amdgcn_sdot4((int)q[t][2], (int)xv4.z, s, false);
            s = __builtin_amdgcn_sdot4((int)q[t][3], (int)xv4.w, s, false);
            f = fmaf((float)__mul24(s, sc[t]), mt.x, f);
        }
        const float v = fmaf(d, f, acc[m]);
        acc[m] = u < nq ? v : acc[m];
    }
}

// ROLL: units walked in a rolled loop with the next unit's loads in flight during this
// one's dots (two units' bytes live); otherwise every unit of the lane is loaded up front
// (at most 8 batch-row x unit products: beyond that the unrolled form spills).
template <int WG, int M, int NP>
__global__ void __launch_bounds__(WG, 512 / WG) gemv_q6k_q8_kernel(const uint8_t *__restrict__ ql,
                                                                 const uint8_t *__restrict__ qh,
                                                                 const int8_t *__restrict__ scp,
                                                                 const uint16_t *__restrict__ dp,
                                                                 const int8_t *__restrict__ xq,
                                                                 const float *__restrict__ xs,
                                                                 float *__restrict__ y, int n, int k) {
    extern __shared__ uint4 lds4[];
    constexpr int WAVES = WG / 64;
    constexpr int SLOTS = q6q8_slots(M, NP);
    constexpr int XPT = (M * NP * 256 + WG - 1) / WG;  // runs each thread stages
    constexpr bool ROLL = M * NP > 8;
    constexpr int NU = ROLL ? 1 : NP;                  // units held in registers before the barrier
    const int nrun = k >> 4, nq = k >> 6;            // 16-activation runs and units per row
    const int total = M * nrun;
    uint4 *xr16 = lds4;                               // [SLOTS] activation bytes of each run, [run][m]
    float2 *meta = (float2 *)(lds4 + SLOTS);          // [SLOTS] (xs, -32 * run sum as int bits)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = blockIdx.x * WAVES + wave;
    const int rowc = row < n ? row : n - 1;

    // slot s holds run s / M of batch row s % M (batch rows adjacent, so that every run and
    // batch row of a unit is a constant offset from one address)
    uint4 xv[XPT];
    float sv[XPT];
#pragma unroll
    for (int j = 0; j < XPT; j++) {
        int c = threadIdx.x + j * WG;
        c = c < total ? c : total - 1;
        const int m = c % M, r = c / M;
        xv[j] = *(const uint4 *)(xq + (int64_t)m * k + 16 * r);
        sv[j] = xs[(int64_t)m * (k >> 5) + (r >> 1)];
    }
    __builtin_amdgcn_sched_barrier(0);  // the activation loads are issued before the weights'

    const uint8_t *qlr = ql + (int64_t)rowc * (k >> 1);
    const uint8_t *qhr = qh + (int64_t)rowc * (k >> 2);
    const int8_t *scr = scp + (int64_t)rowc * (k >> 4);
    const uint16_t *dr = dp + (int64_t)rowc * (k >> 8);
    Q6Unit w[NU];
#pragma unroll
    for (int p = 0; p < NU; p++) {
        const int u = lane + 64 * p;
        q6_load(w[p], qlr, qhr, scr, dr, u < nq ? u : nq - 1);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load is issued before the LDS writes wait on x

#pragma unroll
    for (int j = 0; j < XPT; j++) {
        const int c = threadIdx.x + j * WG;
        const int slot = c < total ? c : SLOTS - 1;
        int sum = __builtin_amdgcn_sdot4((int)xv[j].x, 0x01010101, 0, false);
        sum = __builtin_amdgcn_sdot4((int)xv[j].y, 0x01010101, sum, false);
        sum = __builtin_amdgcn_sdot4((int)xv[j].z, 0x01010101, sum, false);
        sum = __builtin_amdgcn_sdot4((int)xv[j].w, 0x01010101, sum, false);
        xr16[slot] = xv[j];
        meta[slot] = make_float2(sv[j], __int_as_float(-32 * sum));
    }
    lds_barrier();

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; m++) acc[m] = 0.f;
    if constexpr (ROLL) {
        Q6Unit cur = w[0];
#pragma unroll 1
        for (int p = 0; p < NP; p++) {
            const int u = lane + 64 * p, un = u + 64;
            Q6Unit nxt;
            q6_load(nxt, qlr, qhr, scr, dr, un < nq ? un : nq - 1);  // past the end: re-read, unused
            q6_unit<M>(cur, u, u < nq ? u : nq - 1, nq, xr16, meta, acc);
            cur = nxt;
        }
    } else {
#pragma unroll
        for (int p = 0; p < NP; p++) {
            const int u = lane + 64 * p;
            q6_unit<M>(w[p], u, u < nq ? u : nq - 1, nq, xr16, meta, acc);
            // keep the next unit's unpack and activation reads below this unit's dots
            if (NP > 1) __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int m = 0; m < M; m++) {
        const float t = wave_sum(acc[m]);
        if (lane == 0 && row < n) y[(int64_t)m * n + row] = t;
    }
}

// One row per wave; 256-thread workgroups when a row is one pass of 64 units (k <= 4096),
// 512 otherwise (as for the q4_0 kernels).
template <int M, int NP>
bool launch(const qmv_weights *w, const int8_t *xq, const float *xs, float *y, hipStream_t s) {
    const int n = (int)w->n, k = (int)w->k;
    constexpr int WG = NP <= 1 ? 256 : 512;
    constexpr int ROWS = WG / 64;
    hipLaunchKernelGGL((gemv_q6k_q8_kernel<WG, M, NP>), dim3((n + ROWS - 1) / ROWS), dim3(WG),
                       q6q8_lds_bytes(M, NP), s, (const uint8_t *)w->codes, (const uint8_t *)w->codes_hi,
                       (const int8_t *)w->scales, (const uint16_t *)w->super, xq, xs, y, n, k);
    return true;
}

template <int M>
bool dispatch_np(int np, const qmv_weights *w, const int8_t *xq, const float *xs, float *y, hipStream_t s) {
    switch (np) {
    case 1: return launch<M, 1>(w, xq, xs, y, s);
    case 2: return launch<M, 2>(w, xq, xs, y, s);
    case 3: return launch<M, 3>(w, xq, xs, y, s);
    case 4: return launch<M, 4>(w, xq, xs, y, s);
    }
    return false;
}

bool dispatch_m(int m, int np, const qmv_weights *w, const int8_t *xq, const float *xs, float *y, hipStream_t s) {
    switch (m) {
    case 1: return dispatch_np<1>(np, w, xq, xs, y, s);
    case 2: return dispatch_np<2>(np, w, xq, xs, y, s);
    case 3: return dispatch_np<3>(np, w, xq, xs, y, s);
    case 4: return dispatch_np<4>(np, w, xq, xs, y, s);
    case 5: return dispatch_np<5>(np, w, xq, xs, y, s);
    case 6: return dispatch_np<6>(np, w, xq, xs, y, s);
    case 7: return dispatch_np<7>(np, w, xq, xs, y, s);
    case 8: return dispatch_np<8>(np, w, xq, xs, y, s);
    }
    return false;
}

}  // namespace

const char *launch_gemv_q6k_q8(const qmv_weights *w, int m, const int8_t *xq, const float *xs, float *y,
                               hipStream_t s) {
    const int64_t n = w->n, k = w->k, nq = k / 64;
    const int np = (int)((nq + 63) / 64);
    if (n > INT32_MAX || np > NP_MAX) return nullptr;
    if ((int64_t)q6q8_lds_bytes(m, np) > device_info().lds_per_block) return nullptr;
    return dispatch_m(m, np, w, xq, xs, y, s) ? "q6_K.q8.lds-x.dot4" : nullptr;
}

}  // namespace qmv
