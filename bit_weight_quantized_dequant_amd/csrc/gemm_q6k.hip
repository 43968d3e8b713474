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
//   * The expansion (6-bit code -> w' -> h, l) runs in-kernel on packed 16-bit lanes
//     into LDS once per workgroup tile of 64 weight rows x one 256-weight super-block,
//     and is reused by the tile's 128 token columns.
//   * Activations (xq int8, already quantized per 32) are staged into LDS per
//     super-block; fp32 partial sums per super-block are scaled by d once.
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
constexpr int RS = 256 + 16;  // LDS row stride (bytes) of the staged int8 planes

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

template <bool PARTIALS>
__global__ void __launch_bounds__(TB) gemm_q6k_kernel(const uint8_t *__restrict__ ql, const uint8_t *__restrict__ qh,
                                                      const int8_t *__restrict__ scp, const uint16_t *__restrict__ dp,
                                                      const int8_t *__restrict__ xq, const float *__restrict__ xs,
                                                      float *__restrict__ y, int32_t *__restrict__ part,
                                                      int M, int N, int K) {
    __shared__ __attribute__((aligned(16))) uint8_t sH[BN * RS];
    __shared__ __attribute__((aligned(16))) uint8_t sL[BN * RS];
    __shared__ __attribute__((aligned(16))) uint8_t sB[BM * RS];
    __shared__ __attribute__((aligned(16))) float sD[BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int nsb = K >> 8, nblk = K >> 5;
    const int li = lane & 31, lg = lane >> 5;

    float accf[2][16], Y[2][16];
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
        for (int v = 0; v < 16; v++) Y[t][v] = 0.f;

    // expansion role of this thread: weight row r of the tile, quarter unit u
    const int er = tid >> 2, eu = tid & 3, eh = eu >> 1, eo = eu & 1;
    const int erow = n0 + er;
    const bool evalid = erow < N;

    for (int sb = 0; sb < nsb; sb++) {
        // ---- stage activations: 128 rows x 256 int8 (16-byte chunks, 2048 of them)
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int c = tid + i * TB, r = c >> 4, o = (c & 15) * 16;
            const int m = m0 + r;
            const uint4 v = m < M ? *(const uint4 *)(xq + (int64_t)m * K + sb * 256 + o) : make_uint4(0, 0, 0, 0);
            *(uint4 *)(sB + r * RS + o) = v;
        }
        // ---- expand weights: 64 rows x 256 -> h, l planes
        {
            uint4 A = make_uint4(0, 0, 0, 0), Bq = A, H = A;
            uint32_t sc4 = 0;
            if (evalid) {
                const uint8_t *qlr = ql + (int64_t)erow * (K >> 1) + sb * 128 + 64 * eh + 16 * eo;
                const uint8_t *qhr = qh + (int64_t)erow * (K >> 2) + sb * 64 + 32 * eh + 16 * eo;
                A = ld_stream16(qlr);
                Bq = ld_stream16(qlr + 32);
                H = ld_stream16(qhr);
                const int8_t *scr = scp + (int64_t)erow * (K >> 4) + sb * 16 + 8 * eh + eo;
                sc4 = (uint32_t)(uint8_t)scr[0] | ((uint32_t)(uint8_t)scr[2] << 8) | ((uint32_t)(uint8_t)scr[4] << 16) |
                      ((uint32_t)(uint8_t)scr[6] << 24);
                if (eu == 0) sD[er] = h2f(dp[(int64_t)erow * nsb + sb]);
            } else if (eu == 0) {
                sD[er] = 0.f;
            }
            const uint32_t a4[4] = {A.x, A.y, A.z, A.w}, b4[4] = {Bq.x, Bq.y, Bq.z, Bq.w}, h4[4] = {H.x, H.y, H.z, H.w};
#pragma unroll
            for (int t = 0; t < 4; t++) {
                // sub-scale of run t as a 16-bit pair (sign-extended int8); all-zero codes
                // on invalid rows expand to w' = 0 because sc = 0
                const int scv = (int)(int8_t)((sc4 >> (8 * t)) & 0xFF);
                const uint32_t sc2 = ((uint32_t)scv & 0xFFFFu) | ((uint32_t)scv << 16);
                uint32_t hv[4], lv[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    uint32_t q;
                    if (t == 0) q = (a4[i] & 0x0F0F0F0Fu) | ((h4[i] << 4) & 0x30303030u);
                    else if (t == 1) q = (b4[i] & 0x0F0F0F0Fu) | ((h4[i] << 2) & 0x30303030u);
                    else if (t == 2) q = ((a4[i] >> 4) & 0x0F0F0F0Fu) | (h4[i] & 0x30303030u);
                    else q = ((b4[i] >> 4) & 0x0F0F0F0Fu) | ((h4[i] >> 2) & 0x30303030u);
                    expand4(q, sc2, hv[i], lv[i]);
                }
                const int kofs = 128 * eh + 32 * t + 16 * eo;
                *(uint4 *)(sH + er * RS + kofs) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
                *(uint4 *)(sL + er * RS + kofs) = make_uint4(lv[0], lv[1], lv[2], lv[3]);
            }
        }
        __syncthreads();

#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int v = 0; v < 16; v++) accf[t][v] = 0.f;
        // this super-block's eight activation scales of the lane's two token columns
        float xsv[2][8];
        if (!PARTIALS) {
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const int m = m0 + 64 * wm + 32 * t + li;
                const float4 *src = (const float4 *)(xs + (int64_t)min(m, M - 1) * nblk + sb * 8);
                const float4 a = src[0], b = src[1];
                const bool ok = m < M;
                xsv[t][0] = ok ? a.x : 0.f; xsv[t][1] = ok ? a.y : 0.f; xsv[t][2] = ok ? a.z : 0.f;
                xsv[t][3] = ok ? a.w : 0.f; xsv[t][4] = ok ? b.x : 0.f; xsv[t][5] = ok ? b.y : 0.f;
                xsv[t][6] = ok ? b.z : 0.f; xsv[t][7] = ok ? b.w : 0.f;
            }
        }

#pragma unroll
        for (int cb = 0; cb < 8; cb++) {
            const int ko = cb * 32 + 16 * lg;
            const v4i aH = __builtin_bit_cast(v4i, *(const uint4 *)(sH + (32 * wn + li) * RS + ko));
            const v4i aL = __builtin_bit_cast(v4i, *(const uint4 *)(sL + (32 * wn + li) * RS + ko));
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const int mc = 64 * wm + 32 * t + li;  // tile-local token column of this lane
                const v4i b = __builtin_bit_cast(v4i, *(const uint4 *)(sB + mc * RS + ko));
                const v16i z = {};
                const v16i cH = __builtin_amdgcn_mfma_i32_32x32x32_i8(aH, b, z, 0, 0, 0);
                const v16i cL = __builtin_amdgcn_mfma_i32_32x32x32_i8(aL, b, z, 0, 0, 0);
                if (PARTIALS) {
                    const int m = m0 + mc;
                    const int c = sb * 8 + cb;
#pragma unroll
                    for (int v = 0; v < 16; v++) {
                        const int n = n0 + 32 * wn + 8 * (v >> 2) + 4 * lg + (v & 3);
                        if (m < M && n < N) part[((int64_t)m * N + n) * nblk + c] = (cH[v] << 6) + cL[v];
                    }
                } else {
                    const float s = xsv[t][cb];
#pragma unroll
                    for (int v = 0; v < 16; v++) accf[t][v] = fmaf((float)((cH[v] << 6) + cL[v]), s, accf[t][v]);
                }
            }
        }
        if (!PARTIALS) {
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const float4 dv = *(const float4 *)(sD + 32 * wn + 8 * g + 4 * lg);
                const float d4[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
                for (int t = 0; t < 2; t++)
#pragma unroll
                    for (int e = 0; e < 4; e++) Y[t][4 * g + e] = fmaf(d4[e], accf[t][4 * g + e], Y[t][4 * g + e]);
            }
        }
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
