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
//     [-4064, 4096] and is split exactly as w' = 64 h + l with l = w' & 63 in [0, 63]
//     and h = w' >> 6 in [-64, 64], two int8 planes.  Two MFMAs per 32-block give
//     I32 = 64 C_H + C_L exactly in int32: the first gives C_H, which is shifted by 6 and
//     handed to the second as its accumulator input.
//   * K advances in steps of 64 (two activation blocks) through double-buffered LDS:
//     the raw codes and activation bytes of a later step are fetched into registers while
//     this step runs on the matrix cores, then expanded (6-bit code -> w' = sc (q - 32)
//     by one packed 16-bit multiply-add -> h, l bytes) into the other buffer; one barrier
//     per step.  Loads are unconditional (row and token indices clamped), so no branch
//     makes the compiler wait for them early.
//   * fp32 partial sums per super-block are scaled by d once.
// Tiles: 256 threads = 4 waves; 128 token columns per workgroup.  Wide matrices use
// 64-row tiles (waves 2 (n) x 2 (m), wave tile 32 n x 64 m = two 32x32 MFMA tiles sharing
// the A fragments; three workgroups per CU); narrow ones, which would leave CUs idle with
// 64-row tiles, use 32-row tiles (waves 1 x 4, wave tile 32 x 32) with loads two steps
// ahead.  The per-block epilogue (shift-add, convert, FMA on every 32x32 value) is the
// VALU cost that bounds this kernel, not the matrix cores.
//
// MFMA operand layout used (32x32x32 i8): lane l supplies row (or column) l % 32 and
// the 16 consecutive k of group l / 32; the accumulator's value v of lane l is
// C[8 (v / 4) + 4 (l / 32) + (v % 4)][l % 32].  A debug entry point writes the exact
// I32 partials from this same code path, which pins the layout against the oracle.
#include <cstring>
#include <type_traits>

#include "device_common.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

constexpr int TB = 256;       // 4 waves
constexpr int BM = 128;       // token columns per workgroup tile
constexpr int KS = 64;        // k per step: two 32-activation blocks
constexpr int RS = KS + 16;   // LDS row stride (bytes) of the staged int8 planes

// Tile geometry: WN wave rows of 32 weight rows each, 4 / WN wave columns; a wave covers
// 32 rows x TPW 32-token MFMA tiles (sharing its A fragments).
template <int WN>
struct Geo {
    static constexpr int BN = 32 * WN;                 // weight rows per workgroup
    static constexpr int WMC = 4 / WN;                 // wave columns
    static constexpr int TPW = BM / (32 * WMC);        // token tiles per wave
    static constexpr int TPR = TB / BN;                // expanding threads per row
    static constexpr int W = KS / TPR;                 // weights each thread expands per step
    static constexpr int LDS = 2 * (2 * BN + BM) * RS; // two buffers of sH, sL, sB
};

// Four 6-bit codes (bytes of q) of one sub-block -> w' = sc * (q - 32) in [-4064, 4096],
// split exactly as w' = 64 h + l (h = w' >> 6 in [-64, 64], l = w' & 63), packed as four h
// bytes and four l bytes.  (w' << 2) keeps h in the high byte of each 16-bit lane.
QMV_DEV void expand4(uint32_t q, uint32_t sc2, uint32_t c2, uint32_t &hb, uint32_t &lb) {
    const uint32_t q01 = __builtin_amdgcn_perm(0u, q, 0x0C010C00u);  // (q0, q1) as 16-bit lanes
    const uint32_t q23 = __builtin_amdgcn_perm(0u, q, 0x0C030C02u);
    const s16x2 w01 = __builtin_bit_cast(s16x2, q01) * __builtin_bit_cast(s16x2, sc2) + __builtin_bit_cast(s16x2, c2);
    const s16x2 w23 = __builtin_bit_cast(s16x2, q23) * __builtin_bit_cast(s16x2, sc2) + __builtin_bit_cast(s16x2, c2);
    const uint32_t t01 = __builtin_bit_cast(uint32_t, w01 << (s16x2){2, 2});
    const uint32_t t23 = __builtin_bit_cast(uint32_t, w23 << (s16x2){2, 2});
    hb = __builtin_amdgcn_perm(t23, t01, 0x07050301u);
    lb = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, w23), __builtin_bit_cast(uint32_t, w01), 0x06040200u) &
         0x3F3F3F3Fu;
}

template <int NW> struct RawA;
template <> struct RawA<16> { uint4 ql, qh; };
template <> struct RawA<8> { uint2 ql, qh; };
// The same thread's share of a step from the pre-expanded planes: its h and l bytes.
template <int NW> struct RawE;
template <> struct RawE<16> { uint4 h, l; };
template <> struct RawE<8> { uint2 h, l; };

// Step st = 4 s + j covers weights [64 j, 64 j + 64) of super-block s: half h = j >> 1,
// runs t = 2 (j & 1) + {0, 1}, each run 32 consecutive l.  Weight (h, t, l) has its low
// nibble in ql[64 h + 32 (t & 1) + l] (bits 4 (t >> 1)..) and its high bits in
// qh[32 h + l] (bits 2 t..); ql/qh bytes of a half serve both of its steps.  Tile byte
// 32 tt + l of the step is weight 64 st + 32 tt + l of the row: natural k order, which
// is also the order of the pre-expanded planes (EXP: the thread copies its h and l bytes
// instead of expanding codes).
template <int WN, bool PARTIALS, int PD, bool EXP>
__global__ void __launch_bounds__(TB, PD == 1 ? 3 : 2) gemm_q6k_kernel(const uint8_t *__restrict__ ql, const uint8_t *__restrict__ qh,
                                                         const int8_t *__restrict__ scp, const uint16_t *__restrict__ dp,
                                                         const int8_t *__restrict__ ph, const int8_t *__restrict__ pl,
                                                         const int8_t *__restrict__ xq, const float *__restrict__ xs,
                                                         float *__restrict__ y, int32_t *__restrict__ part,
                                                         int M, int N, int K) {
    using G = Geo<WN>;
    constexpr int BN = G::BN, TPW = G::TPW, NWT = G::W;
    using RA = std::conditional_t<EXP, RawE<NWT>, RawA<NWT>>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ float sD[2][BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % WN, wm = wave / WN;
    // Workgroups are dealt to the eight XCDs round-robin in dispatch order (x fastest).
    // Remap so that XCD x takes one contiguous run of row tiles with all their column
    // tiles: the column tiles that share a weight tile then share one L2.
    int n0, m0;
    {
        const int nrt = gridDim.x, nct = gridDim.y, ntiles = nrt * nct;
        const int b = blockIdx.x + nrt * blockIdx.y;
        const int xcd = b & 7, q = b >> 3, base = ntiles >> 3, rem = ntiles & 7;
        const int t = xcd * base + min(xcd, rem) + q;
        n0 = (t / nct) * BN;
        m0 = (t % nct) * BM;
    }
    const int nsteps = K / KS, nblk = K >> 5;
    const int li = lane & 31, lg = lane >> 5;

    // expansion role: row er, run tt of the step, first l of this thread's NWT weights
    const int er = tid / G::TPR, ep = tid % G::TPR;
    const int tt = (ep * NWT) >> 5, l0 = (ep * NWT) & 31;
    const int erow = min(n0 + er, N - 1);
    const uint8_t *qlr = ql + (int64_t)erow * (K >> 1) + 32 * tt + l0;
    const uint8_t *qhr = qh + (int64_t)erow * (K >> 2) + l0;
    const int8_t *scr = scp + (int64_t)erow * (K >> 4) + 2 * tt + (l0 >> 4);
    const uint16_t *dr = dp + (int64_t)erow * (K >> 8);
    const int8_t *phr = ph + (int64_t)erow * K + 32 * tt + l0;  // EXP: this thread's h, l bytes
    const int8_t *plr = pl + (int64_t)erow * K + 32 * tt + l0;
    // activation staging role: token bt, bytes [32 bo, 32 bo + 32) of the step
    const int bt = tid >> 1, bo = tid & 1;
    const int8_t *xr = xq + (int64_t)min(m0 + bt, M - 1) * K + 32 * bo;
    // epilogue: the lane's token of each tile
    int tok[TPW];
#pragma unroll
    for (int t = 0; t < TPW; t++) tok[t] = m0 + 32 * (wm * TPW + t) + li;

    uint8_t *const sbase = smem;
    auto sH = [&](int b) { return sbase + b * (2 * BN + BM) * RS; };
    auto sL = [&](int b) { return sbase + b * (2 * BN + BM) * RS + BN * RS; };
    auto sB = [&](int b) { return sbase + b * (2 * BN + BM) * RS + 2 * BN * RS; };

    // raw inputs of one step, held in registers from the prefetch to the expansion; with a
    // prefetch distance of 2 there are two sets, used by even and odd steps
    struct Raw {
        RA ra;
        int scb;
        uint32_t dbits;
        uint4 rb0, rb1;
        float2 xsv[TPW];
    };

    auto fetch = [&](int st, Raw &r) {
        auto &ra = r.ra;
        auto &scb = r.scb;
        auto &dbits = r.dbits;
        auto &rb0 = r.rb0;
        auto &rb1 = r.rb1;
        auto &xsv = r.xsv;
        const int s = st >> 2, j = st & 3, h = j >> 1;
        // Plain (cached) loads for the weights: every column tile of a row tile reads the
        // same weight bytes on the same XCD (see the tile order above), and with cached
        // loads the later ones hit in its L2 (nontemporal loads measured 2-10 % slower).
        if constexpr (EXP) {
            if constexpr (NWT == 16) {
                ra.h = *(const uint4 *)(phr + st * KS);
                ra.l = *(const uint4 *)(plr + st * KS);
            } else {
                ra.h = *(const uint2 *)(phr + st * KS);
                ra.l = *(const uint2 *)(plr + st * KS);
            }
        } else {
            if ((j & 1) == 0) {  // a new half: its ql/qh bytes
                if constexpr (NWT == 16) {
                    ra.ql = *(const uint4 *)(qlr + 128 * s + 64 * h);
                    ra.qh = *(const uint4 *)(qhr + 64 * s + 32 * h);
                } else {
                    ra.ql = *(const uint2 *)(qlr + 128 * s + 64 * h);
                    ra.qh = *(const uint2 *)(qhr + 64 * s + 32 * h);
                }
            }
            scb = scr[16 * s + 8 * h + 4 * (j & 1)];
        }
        if (j == 0) dbits = dr[s];
        rb0 = *(const uint4 *)(xr + st * KS);
        rb1 = *(const uint4 *)(xr + st * KS + 16);
        if (!PARTIALS) {
#pragma unroll
            for (int t = 0; t < TPW; t++)
                xsv[t] = *(const float2 *)(xs + (int64_t)min(tok[t], M - 1) * nblk + 2 * st);
        }
    };

    // Stage step st into LDS buffer buf: the weight tile (expanded from the codes, or copied
    // from the planes), the super-block's d once per super-block, the activation bytes.
    auto store = [&](int st, int buf, const Raw &r) {
        const RA ra = r.ra;
        const uint32_t dbits = r.dbits;
        const uint4 rb0 = r.rb0, rb1 = r.rb1;
        uint8_t *dh = sH(buf) + er * RS + 32 * tt + l0;
        uint8_t *dl = sL(buf) + er * RS + 32 * tt + l0;
        if constexpr (EXP) {
            if constexpr (NWT == 16) {
                *(uint4 *)dh = make_uint4(ra.h.x, ra.h.y, ra.h.z, ra.h.w);
                *(uint4 *)dl = make_uint4(ra.l.x, ra.l.y, ra.l.z, ra.l.w);
            } else {
                *(uint2 *)dh = make_uint2(ra.h.x, ra.h.y);
                *(uint2 *)dl = make_uint2(ra.l.x, ra.l.y);
            }
        } else {
            const int scb = r.scb;
            const int j = st & 3;
            const int sh = 2 * (2 * (j & 1) + tt);  // qh bit offset of run t
            const uint32_t sc16 = (uint32_t)scb & 0xFFFFu;
            const uint32_t sc2 = sc16 | (sc16 << 16);
            const uint32_t c16 = (uint32_t)(-32 * scb) & 0xFFFFu;
            const uint32_t c2 = c16 | (c16 << 16);
            constexpr int ND = NWT / 4;
            uint32_t qlw[ND], qhw[ND], hv[ND], lv[ND];
            if constexpr (NWT == 16) {
                qlw[0] = ra.ql.x; qlw[1] = ra.ql.y; qlw[2] = ra.ql.z; qlw[3] = ra.ql.w;
                qhw[0] = ra.qh.x; qhw[1] = ra.qh.y; qhw[2] = ra.qh.z; qhw[3] = ra.qh.w;
            } else {
                qlw[0] = ra.ql.x; qlw[1] = ra.ql.y;
                qhw[0] = ra.qh.x; qhw[1] = ra.qh.y;
            }
#pragma unroll
            for (int i = 0; i < ND; i++) {
                const uint32_t nib = ((j & 1) ? qlw[i] >> 4 : qlw[i]) & 0x0F0F0F0Fu;
                const uint32_t q = nib | (((qhw[i] >> sh) & 0x03030303u) << 4);
                expand4(q, sc2, c2, hv[i], lv[i]);
            }
            if constexpr (NWT == 16) {
                *(uint4 *)dh = make_uint4(hv[0], hv[1], hv[2], hv[3]);
                *(uint4 *)dl = make_uint4(lv[0], lv[1], lv[2], lv[3]);
            } else {
                *(uint2 *)dh = make_uint2(hv[0], hv[1]);
                *(uint2 *)dl = make_uint2(lv[0], lv[1]);
            }
        }
        if ((st & 3) == 0 && ep == 0) sD[(st >> 2) & 1][er] = h2f((uint16_t)dbits);
        uint8_t *db = sB(buf) + bt * RS + 32 * bo;
        *(uint4 *)db = rb0;
        *(uint4 *)(db + 16) = rb1;
    };

    float accf[TPW][16], Y[TPW][16];
#pragma unroll
    for (int t = 0; t < TPW; t++)
#pragma unroll
        for (int v = 0; v < 16; v++) { Y[t][v] = 0.f; accf[t][v] = 0.f; }

    // One step: compute st from LDS buffer st & 1 while the loads of a later step are in
    // flight, then expand step st + 1 into the other buffer.  With PD = 1 the loads of
    // st + 1 are issued at the top of st (one set of registers); with PD = 2 the loads of
    // st + 2 go into the set step st has just released (two sets, alternating by parity,
    // so the set is chosen at compile time).  The ql/qh bytes of a half are loaded by its
    // first step; its second step reuses them.
    auto step = [&](int st, Raw &cur, Raw &nxt) {
        const int buf = st & 1;
        float xsc[TPW][2];
#pragma unroll
        for (int t = 0; t < TPW; t++) { xsc[t][0] = cur.xsv[t].x; xsc[t][1] = cur.xsv[t].y; }
        // The prefetch is unconditional (past the end it re-reads the last step, unused): a
        // branch around it would make the compiler wait for these loads at the join, i.e.
        // before this step's MFMAs, costing a memory round trip per step.
        if (PD == 1) {
            fetch(st + 1 < nsteps ? st + 1 : nsteps - 1, cur);
        } else {
            if (!EXP && (st & 1) == 1) cur.ra = nxt.ra;  // st + 2 odd: same half as st + 1
            fetch(st + 2 < nsteps ? st + 2 : nsteps - 2 + (st & 1), cur);
        }

#pragma unroll
        for (int cb = 0; cb < 2; cb++) {
            const int ko = cb * 32 + 16 * lg;
            const v4i aH = __builtin_bit_cast(v4i, *(const uint4 *)(sH(buf) + (32 * wn + li) * RS + ko));
            const v4i aL = __builtin_bit_cast(v4i, *(const uint4 *)(sL(buf) + (32 * wn + li) * RS + ko));
#pragma unroll
            for (int t = 0; t < TPW; t++) {
                const int mc = 32 * (wm * TPW + t) + li;  // tile-local token column of this lane
                const v4i b = __builtin_bit_cast(v4i, *(const uint4 *)(sB(buf) + mc * RS + ko));
                // I32 = 64 C_H + C_L: C_H is shifted (one VOP2 shift per value) and handed to
                // the second MFMA as its accumulator input, which adds C_L exactly
                const v16i z = {};
                const v16i cH = __builtin_amdgcn_mfma_i32_32x32x32_i8(aH, b, z, 0, 0, 0);
                const v16i i32 = __builtin_amdgcn_mfma_i32_32x32x32_i8(aL, b, cH << 6, 0, 0, 0);
                if (PARTIALS) {
                    const int m = tok[t], c = st * 2 + cb;
#pragma unroll
                    for (int v = 0; v < 16; v++) {
                        const int n = n0 + 32 * wn + 8 * (v >> 2) + 4 * lg + (v & 3);
                        if (m < M && n < N) part[((int64_t)m * N + n) * nblk + c] = i32[v];
                    }
                } else {
#pragma unroll
                    for (int v = 0; v < 16; v++) accf[t][v] = fmaf((float)i32[v], xsc[t][cb], accf[t][v]);
                }
            }
        }
        if (!PARTIALS && (st & 3) == 3) {  // end of a super-block: apply d once
            const float *dcur = sD[(st >> 2) & 1];
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const float4 dv = *(const float4 *)(&dcur[32 * wn + 8 * g + 4 * lg]);
                const float d4[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
                for (int t = 0; t < TPW; t++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        Y[t][4 * g + e] = fmaf(d4[e], accf[t][4 * g + e], Y[t][4 * g + e]);
                        accf[t][4 * g + e] = 0.f;
                    }
            }
        }
        if (st + 1 < nsteps) store(st + 1, buf ^ 1, PD == 1 ? cur : nxt);
        __syncthreads();
    };

    Raw R0, R1;
    fetch(0, R0);
    if (PD == 2 && nsteps > 1) {
        fetch(1, R1);
        if (!EXP) R1.ra = R0.ra;  // step 1 is the second step of half 0
    }
    store(0, 0, R0);
    __syncthreads();
    if (PD == 1) {
        for (int st = 0; st < nsteps; st++) step(st, R0, R0);
    } else {
        for (int st = 0; st < nsteps; st += 2) {  // nsteps is a multiple of 4
            step(st, R0, R1);
            step(st + 1, R1, R0);
        }
    }
    if (PARTIALS) return;
#pragma unroll
    for (int t = 0; t < TPW; t++) {
        const int m = tok[t];
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

template <int WN, bool PARTIALS, int PD, bool EXP>
void launch_tiles(const qmv_weights *w, int m, const int8_t *plane, const int8_t *xq, const float *xs, float *y,
                  int32_t *partials, hipStream_t s) {
    using G = Geo<WN>;
    const int64_t n = w->n, k = w->k;
    const dim3 grid((unsigned)((n + G::BN - 1) / G::BN), (unsigned)((m + BM - 1) / BM));
    hipLaunchKernelGGL((gemm_q6k_kernel<WN, PARTIALS, PD, EXP>), grid, dim3(TB), G::LDS, s, (const uint8_t *)w->codes,
                       (const uint8_t *)w->codes_hi, (const int8_t *)w->scales, (const uint16_t *)w->super, plane,
                       plane ? plane + n * k : nullptr, xq, xs, y, partials, m, (int)n, (int)k);
}

template <bool EXP>
const char *launch_gemm(const qmv_weights *w, int m, const int8_t *plane, const int8_t *xq, const float *xs,
                        float *y, int32_t *partials, hipStream_t s) {
    const int64_t n = w->n;
    // 64-row tiles when they give at least two workgroups per CU (one, when copying
    // registered planes: 4096x11008 at M = 512 then runs 288-292 against 276-287 TOPS with
    // 32-row tiles, while the in-kernel expansion keeps 32-row tiles there, 256-266 against
    // 220-221), else 32-row tiles
    const int64_t tiles64 = ((n + 63) / 64) * ((m + BM - 1) / BM);
    const char *fp = forced_path();  // test-only overrides of the tile width and prefetch distance
    const bool wide = strcmp(fp, "gemm.w64") == 0 ? true : strcmp(fp, "gemm.w32") == 0 ? false
                                                      : tiles64 >= (EXP ? 1 : 2) * (int64_t)device_info().num_cus;
    if (partials) {
        if (wide) launch_tiles<2, true, 1, EXP>(w, m, plane, xq, xs, y, partials, s);
        else launch_tiles<1, true, 1, EXP>(w, m, plane, xq, xs, y, partials, s);
        return "gemm.q6k.mfma-i8-32x32x32.hl-split.partials";
    }
    // 64-row tiles that expand codes keep the loads of the next step in flight (their
    // register budget allows three workgroups per CU); 32-row tiles, and 64-row tiles that
    // copy registered planes (fewer registers per step), fetch two steps ahead
    const int pd = strcmp(fp, "gemm.pd1") == 0 ? 1 : strcmp(fp, "gemm.pd2") == 0 ? 2 : (wide && !EXP ? 1 : 2);
    if (wide) {
        if (pd == 1) launch_tiles<2, false, 1, EXP>(w, m, plane, xq, xs, y, partials, s);
        else launch_tiles<2, false, 2, EXP>(w, m, plane, xq, xs, y, partials, s);
    } else {
        if (pd == 1) launch_tiles<1, false, 1, EXP>(w, m, plane, xq, xs, y, partials, s);
        else launch_tiles<1, false, 2, EXP>(w, m, plane, xq, xs, y, partials, s);
    }
    return "gemm.q6k.mfma-i8-32x32x32.hl-split";
}

// Pre-expansion of a q6_K matrix into the planes the EXP kernels copy: for every weight,
// w' = sc * (q - 32) = 64 h + l with h = w' >> 6 (arithmetic) and l = w' & 63, stored
// as int8 H[n][k] then L[n][k].  One thread per 64-weight unit (half h, offset 16 odd)
// of a super-block, as in the dequantizer.
__global__ void __launch_bounds__(256) expand_q6k_planes(const uint8_t *__restrict__ ql, const uint8_t *__restrict__ qh,
                                                         const int8_t *__restrict__ sc, int8_t *__restrict__ H,
                                                         int8_t *__restrict__ L, int64_t nunits) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nunits) return;
    const int64_t sb = i >> 2;
    const int h = (int)((i >> 1) & 1), odd = (int)(i & 1);
    const uint8_t *a = ql + sb * 128 + 64 * h + 16 * odd;
    const uint8_t *hb = qh + sb * 64 + 32 * h + 16 * odd;
    const int64_t e0 = sb * 256 + 128 * h + 16 * odd;
#pragma unroll
    for (int t = 0; t < 4; t++) {
        const int s = sc[sb * 16 + 8 * h + 2 * t + odd];
        for (int j = 0; j < 16; j++) {
            const int q = ((a[j + 32 * (t & 1)] >> (4 * (t >> 1))) & 15) | (((hb[j] >> (2 * t)) & 3) << 4);
            const int wv = s * (q - 32);
            H[e0 + 32 * t + j] = (int8_t)(wv >> 6);
            L[e0 + 32 * t + j] = (int8_t)(wv & 63);
        }
    }
}

}  // namespace

const char *launch_gemm_q6k(const qmv_weights *w, int m, const int8_t *plane, const int8_t *xq, const float *xs,
                            float *y, int32_t *partials, hipStream_t s) {
    const int64_t n = w->n, k = w->k;
    if (n > INT32_MAX || k > INT32_MAX || (int64_t)m * k > INT32_MAX) return nullptr;
    return plane ? launch_gemm<true>(w, m, plane, xq, xs, y, partials, s)
                 : launch_gemm<false>(w, m, nullptr, xq, xs, y, partials, s);
}

const char *launch_expand_q6k(const qmv_weights *w, int8_t *plane, hipStream_t s) {
    const int64_t nunits = w->n * w->k / 64;
    if (nunits > (int64_t)INT32_MAX * 256) return nullptr;
    hipLaunchKernelGGL(expand_q6k_planes, dim3((unsigned)((nunits + 255) / 256)), dim3(256), 0, s,
                       (const uint8_t *)w->codes, (const uint8_t *)w->codes_hi, (const int8_t *)w->scales, plane,
                       plane + w->n * w->k, nunits);
    return "plane.q6k.expand";
}

}  // namespace qmv
