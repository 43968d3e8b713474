// gemm_q6k.hip -- q6_K prefill GEMM on int8 MFMA (gfx950, v_mfma_i32_32x32x32_i8).
//
// y[m][n] = sum_s d[n][s] * sum_{c in s} xs[m][c] * I32[m][n][c], where
// I32[m][n][c] = sum over the 32 weights k of activation block c of
//               sc[n][k/16] * (q[n][k] - 32) * xq[m][k]
// is computed exactly in int32 ("57 · r54 — MINFER_MMQ_Q6K_EXP", §2.1: the q6_K
// values are expanded into centred integers for an int8 contraction; §2.3: that
// expansion is an integer transform, so the partials are exact).
//
// Design for gfx950 (the page's NB-BT CUDA kernel stages raw or pre-expanded int8 B
// tiles with cp.async; here):
//   * Orientation: MFMA rows are weight rows n (operand A), columns are tokens m
//     (operand B = int8 activations), so each lane's column has one activation scale
//     xs[m][c] per block: the block epilogue is one convert and one FMA per value.
//   * The sub-scale is folded into the weights: w' = sc * (q - 32) lies in
//     [-3968, 4096] and is split exactly as w' = 64 h + l with l = w' & 63 in [0, 63]
//     and h = w' >> 6 in [-62, 64], two int8 planes.  Two MFMAs per 32-block give
//     C_H and C_L, and I32 = 64 C_H + C_L (one shift-add) is exact in int32.
//   * K advances in steps of 128 (half a super-block) through double-buffered LDS:
//     the raw codes and activation bytes of step s+1 are fetched into registers while
//     step s runs on the matrix cores, then expanded (6-bit code -> w' -> h, l on packed
//     16-bit lanes) into the other buffer; one barrier per step.  The expansion of a
//     64-row tile is reused by the tile's 128 token columns.
//   * fp32 partial sums per super-block are scaled by d once.
// Tile: 256 threads = 4 waves in a 2 (n) x 2 (m) grid; wave tile 32 n x 64 m = two
// 32x32 MFMA tiles sharing the A fragments.
//
// MFMA operand layout used (32x32x32 i8): lane l supplies row (or column) l % 32 and
// the 16 consecutive k of group l / 32; the accumulator's value v of lane l is
// C[8 (v / 4) + 4 (l / 32) + (v % 4)][l % 32].  A debug entry point writes the exact
// I32 partials from this same code path, which pins the layout against the oracle.
#include "device_common.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

constexpr int TB = 256;
constexpr int BN = 64;        // weight rows per workgroup tile
constexpr int BM = 128;       // token columns per workgroup tile
constexpr int RS = 128 + 16;  // LDS row stride (bytes) of the staged int8 planes (one K step)

// (q0, q1, q2, q3) bytes of Q -> 4 exact w' = sc * (q - 32), split into h bytes and l bytes.
QMV_DEV void expand4(uint32_t Q, uint32_t sc2, uint32_t &hb, uint32_t &lb) {
    const uint32_t lo = __builtin_amdgcn_perm(0u, Q, 0x0C010C00u);  // (q0, q1) as 16-bit lanes
    const uint32_t hi = __builtin_amdgcn_perm(0u, Q, 0x0C030C02u);  // (q2, q3)
    const s16x2 c32 = {32, 32};
    const s16x2 wlo = (__builtin_bit_cast(s16x2, lo) - c32) * __builtin_bit_cast(s16x2, sc2);
    const s16x2 whi = (__builtin_bit_cast(s16x2, hi) - c32) * __builtin_bit_cast(s16x2, sc2);
    const s16x2 hlo = wlo >> (s16x2){6, 6}, hhi = whi >> (s16x2){6, 6};
    const uint32_t llo = __builtin_bit_cast(uint32_t, wlo) & 0x003F003Fu;
    const uint32_t lhi = __builtin_bit_cast(uint32_t, whi) & 0x003F003Fu;
    hb = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hhi), __builtin_bit_cast(uint32_t, hlo), 0x06040200u);
    lb = __builtin_amdgcn_perm(lhi, llo, 0x06040200u);
}

// Raw inputs of one K step (128 weights per row) held in registers between the
// prefetch and the expansion: this thread's 32 weights of one row and 64 activation bytes.
struct StepRaw {
    uint4 ql, qh, b[4];
    uint32_t sca, scb;  // the two sub-scale bytes of this thread's runs, as loaded
    uint32_t d;         // fp16 bits of this thread's row's super-block scale, as loaded
    float4 xs4[2];  // activation scales of the step's four blocks, for the lane's two columns
};

template <bool PARTIALS>
__global__ void __launch_bounds__(TB, 2) gemm_q6k_kernel(const uint8_t *__restrict__ ql, const uint8_t *__restrict__ qh,
                                                         const int8_t *__restrict__ scp, const uint16_t *__restrict__ dp,
                                                         const int8_t *__restrict__ xq, const float *__restrict__ xs,
                                                         float *__restrict__ y, int32_t *__restrict__ part,
                                                         int M, int N, int K) {
    __shared__ __attribute__((aligned(16))) uint8_t sH[2][BN * RS];
    __shared__ __attribute__((aligned(16))) uint8_t sL[2][BN * RS];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BM * RS];
    __shared__ __attribute__((aligned(16))) float sD[2][BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int nsteps = K >> 7, nblk = K >> 5;
    const int li = lane & 31, lg = lane >> 5;

    // expansion role: row er of the tile, lane offset eo (0/16), run pair tp ({0,2} or {1,3})
    const int er = tid >> 2, eo = tid & 1, tp = (tid >> 1) & 1;
    const int erow = n0 + er;
    const bool evalid = erow < N;

    auto fetch = [&](int st, StepRaw &r) {
        const int sb = st >> 1, h = st & 1;
        if (evalid) {
            r.ql = ld_stream16(ql + (int64_t)erow * (K >> 1) + sb * 128 + 64 * h + 32 * tp + 16 * eo);
            r.qh = ld_stream16(qh + (int64_t)erow * (K >> 2) + sb * 64 + 32 * h + 16 * eo);
            // raw bytes only: any arithmetic on them here would make the compiler wait
            // for these loads now instead of at the expansion (loads return in order)
            const uint8_t *scr = (const uint8_t *)scp + (int64_t)erow * (K >> 4) + sb * 16 + 8 * h + 2 * tp + eo;
            r.sca = scr[0];
            r.scb = scr[4];
            r.d = dp[(int64_t)erow * (K >> 8) + sb];
        } else {
            r.ql = r.qh = make_uint4(0, 0, 0, 0);
            r.sca = r.scb = 0;
            r.d = 0;
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int c = tid + i * TB, rr = c >> 3, o = (c & 7) * 16;
            const int m = m0 + rr;
            r.b[i] = m < M ? *(const uint4 *)(xq + (int64_t)m * K + st * 128 + o) : make_uint4(0, 0, 0, 0);
        }
        if (!PARTIALS) {
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const int m = m0 + 64 * wm + 32 * t + li;
                const float4 a = *(const float4 *)(xs + (int64_t)min(m, M - 1) * nblk + st * 4);
                r.xs4[t] = m < M ? a : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    };

    auto store = [&](int st, const StepRaw &r, int buf) {
        const uint32_t a4[4] = {r.ql.x, r.ql.y, r.ql.z, r.ql.w};
        const uint32_t h4[4] = {r.qh.x, r.qh.y, r.qh.z, r.qh.w};
#pragma unroll
        for (int half = 0; half < 2; half++) {  // run t = tp (low nibbles), t = tp + 2 (high nibbles)
            const int scv = (int)(int8_t)(half == 0 ? r.sca : r.scb);
            const uint32_t sc2 = ((uint32_t)scv & 0xFFFFu) | ((uint32_t)scv << 16);
            uint32_t hv[4], lv[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t qhs = h4[i] >> (2 * tp);
                const uint32_t q = half == 0 ? ((a4[i] & 0x0F0F0F0Fu) | ((qhs << 4) & 0x30303030u))
                                             : (((a4[i] >> 4) & 0x0F0F0F0Fu) | (qhs & 0x30303030u));
                expand4(q, sc2, hv[i], lv[i]);
            }
            const int kofs = 32 * (tp + 2 * half) + 16 * eo;
            *(uint4 *)(&sH[buf][er * RS + kofs]) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
            *(uint4 *)(&sL[buf][er * RS + kofs]) = make_uint4(lv[0], lv[1], lv[2], lv[3]);
        }
        if ((st & 1) == 0 && (tid & 3) == 0) sD[(st >> 1) & 1][er] = h2f((uint16_t)r.d);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int c = tid + i * TB, rr = c >> 3, o = (c & 7) * 16;
            *(uint4 *)(&sB[buf][rr * RS + o]) = r.b[i];
        }
    };

    float accf[2][16], Y[2][16];
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
        for (int v = 0; v < 16; v++) { Y[t][v] = 0.f; accf[t][v] = 0.f; }

    StepRaw raw;
    fetch(0, raw);
    store(0, raw, 0);
    __syncthreads();

    for (int st = 0; st < nsteps; st++) {
        const int buf = st & 1;
        // this step's activation scales were fetched with its codes (loads return in
        // order, so nothing issued after the prefetch below may be waited on here)
        float xsv[2][4];
#pragma unroll
        for (int t = 0; t < 2; t++) {
            xsv[t][0] = raw.xs4[t].x;
            xsv[t][1] = raw.xs4[t].y;
            xsv[t][2] = raw.xs4[t].z;
            xsv[t][3] = raw.xs4[t].w;
        }
        if (st + 1 < nsteps) fetch(st + 1, raw);  // in flight during this step's MFMAs

#pragma unroll
        for (int cb = 0; cb < 4; cb++) {
            const int ko = cb * 32 + 16 * lg;
            const v4i aH = __builtin_bit_cast(v4i, *(const uint4 *)(&sH[buf][(32 * wn + li) * RS + ko]));
            const v4i aL = __builtin_bit_cast(v4i, *(const uint4 *)(&sL[buf][(32 * wn + li) * RS + ko]));
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const int mc = 64 * wm + 32 * t + li;  // tile-local token column of this lane
                const v4i b = __builtin_bit_cast(v4i, *(const uint4 *)(&sB[buf][mc * RS + ko]));
                const v16i z = {};
                const v16i cH = __builtin_amdgcn_mfma_i32_32x32x32_i8(aH, b, z, 0, 0, 0);
                const v16i cL = __builtin_amdgcn_mfma_i32_32x32x32_i8(aL, b, z, 0, 0, 0);
                if (PARTIALS) {
                    const int m = m0 + mc, c = st * 4 + cb;
#pragma unroll
                    for (int v = 0; v < 16; v++) {
                        const int n = n0 + 32 * wn + 8 * (v >> 2) + 4 * lg + (v & 3);
                        if (m < M && n < N) part[((int64_t)m * N + n) * nblk + c] = (cH[v] << 6) + cL[v];
                    }
                } else {
#pragma unroll
                    for (int v = 0; v < 16; v++)
                        accf[t][v] = fmaf((float)((cH[v] << 6) + cL[v]), xsv[t][cb], accf[t][v]);
                }
            }
        }
        if (!PARTIALS && (st & 1)) {  // end of a super-block: apply d once
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const float4 dv = *(const float4 *)(&sD[(st >> 1) & 1][32 * wn + 8 * g + 4 * lg]);
                const float d4[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
                for (int t = 0; t < 2; t++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        Y[t][4 * g + e] = fmaf(d4[e], accf[t][4 * g + e], Y[t][4 * g + e]);
                        accf[t][4 * g + e] = 0.f;
                    }
            }
        }
        if (st + 1 < nsteps) store(st + 1, raw, buf ^ 1);
        __syncthreads();
    }
    if (PARTIALS) return;
#pragma unroll
    for (int t = 0; t < 2; t++) {
        const int m = m0 + 64 * wm + 32 * t + li;
        if (m >= M) continue;
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int n = n0 + 32 * wn + 8 * g + 4 * lg;
            float *dst = y + (int64_t)m * N + n;
            if (n + 3 < N && (N & 3) == 0) {
                *(float4 *)dst = make_float4(Y[t][4 * g], Y[t][4 * g + 1], Y[t][4 * g + 2], Y[t][4 * g + 3]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++)
                    if (n + e < N) dst[e] = Y[t][4 * g + e];
            }
        }
    }
}

}  // namespace

const char *launch_gemm_q6k(const qmv_weights *w, int m, const int8_t *xq, const float *xs, float *y,
                            int32_t *partials, hipStream_t s) {
    const int64_t n = w->n, k = w->k;
    if (n > INT32_MAX || k > INT32_MAX || (int64_t)m * k > INT32_MAX) return nullptr;
    const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM));
    if (partials) {
        hipLaunchKernelGGL(gemm_q6k_kernel<true>, grid, dim3(TB), 0, s, (const uint8_t *)w->codes,
                           (const uint8_t *)w->codes_hi, (const int8_t *)w->scales, (const uint16_t *)w->super, xq,
                           xs, y, partials, m, (int)n, (int)k);
        return "gemm.q6k.mfma-i8-32x32x32.hl-split.partials";
    }
    hipLaunchKernelGGL(gemm_q6k_kernel<false>, grid, dim3(TB), 0, s, (const uint8_t *)w->codes,
                       (const uint8_t *)w->codes_hi, (const int8_t *)w->scales, (const uint16_t *)w->super, xq, xs,
                       y, partials, m, (int)n, (int)k);
    return "gemm.q6k.mfma-i8-32x32x32.hl-split";
}

}  // namespace qmv
