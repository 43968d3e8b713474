// gemv_q4_0_q8.hip -- q4_0 decode GEMV over per-32 int8 activations, for gfx950.
//
// y[m][n] = sum_b d[n][b] * xs[m][b] * I[m][n][b],  I = sum over block b of (q - 8) * xq,
// with xq / xs from the per-32 activation quantizer.  This is the integer-dot form of the
// decode GEMV: quantprobe LAWS.md (Law 4's per-format amendment, L-15) measures that on a
// standalone matvec the unpack instructions, not the bytes, set the speed, and that integer
// dot products over quantized activations recover most of that loss.  On gfx950 the dot
// product is v_dot4c_i32_i8 (four int8 products added to an int32 per instruction), so a
// block of 32 weights costs 8 dot instructions and 8 bit operations instead of 32 fused
// multiply-adds and 32 conversions:
//
//   * low nibbles (block elements 0..15): (w & 0x0F0F0F0F) are the codes q as int8 bytes;
//     the dot starts from -8 * (sum of those 16 activations), staged once per workgroup,
//     so the chain ends at sum (q - 8) * xq;
//   * high nibbles (elements 16..31): (w & 0xF0F0F0F0) ^ 0x80808080 is 16 * (q - 8) as
//     int8 bytes exactly (the top bit flip subtracts 128), so the chain ends at
//     16 * sum (q - 8) * xq;
//   * I16 = 16 * low + high = 16 * I is exact in int32; the block adds d * xs * I16 to the
//     fp32 row sum (one conversion, one multiply, one mixed fp16 x fp32 multiply-add), and
//     the row sum is scaled by 1/16 (exact) at the end.
//
// Activations of the workgroup are staged in LDS once, in three planes per (batch row,
// block): bytes 0..15, bytes 16..31 (each 16 B, so eight lanes reading eight consecutive
// blocks touch disjoint banks), and (xs, -8 * low sum); one thread stages a whole block.
// The loads follow the order of the fp32-activation kernel: activation loads first, then
// every code and scale load of the wave's row, then the LDS writes and one barrier.
// Indices are clamped and threads past the end write to a junk slot, so that no load sits
// behind a branch (the compiler would sink it there, behind the weight loads).
#include "device_common.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int BPL_MAX = 8;  // blocks per lane: k <= 64 * 32 * 8 = 16384

// (batch row, block) slots a workgroup stages: every block a lane may own, plus one junk
// slot that threads past the end write to (so that the staging has no branch).
constexpr int q8_slots(int m, int bpl) { return m * bpl * 64 + 1; }
// LDS bytes: two 16-byte planes and an 8-byte plane over the slots.
constexpr size_t q8_lds_bytes(int m, int bpl) { return (size_t)q8_slots(m, bpl) * 40; }
// Blocks (32 bytes of xq each) each thread stages.
constexpr int q8_blocks_per_thread(int wg, int m, int bpl) { return (m * bpl * 64 + wg - 1) / wg; }

// Adds block b (clamped to bc) of the row to acc[m] for every batch row (nothing when b is
// past the row end).
template <int M>
QMV_DEV void q4_block(uint4 w, uint16_t dbits, int b, int bc, int nblk, const uint4 *xlo, const uint4 *xhi,
                      const float2 *meta, float (&acc)[M]) {
    const float d = h2f(dbits);
#pragma unroll
    for (int m = 0; m < M; m++) {
        const uint4 lo = xlo[m * nblk + bc], hi = xhi[m * nblk + bc];
        const float2 mt = meta[m * nblk + bc];
        int a = __float_as_int(mt.y);
        a = __builtin_amdgcn_sdot4((int)(w.x & 0x0F0F0F0Fu), (int)lo.x, a, false);
        a = __builtin_amdgcn_sdot4((int)(w.y & 0x0F0F0F0Fu), (int)lo.y, a, false);
        a = __builtin_amdgcn_sdot4((int)(w.z & 0x0F0F0F0Fu), (int)lo.z, a, false);
        a = __builtin_amdgcn_sdot4((int)(w.w & 0x0F0F0F0Fu), (int)lo.w, a, false);
        int h = __builtin_amdgcn_sdot4((int)((w.x & 0xF0F0F0F0u) ^ 0x80808080u), (int)hi.x, 0, false);
        h = __builtin_amdgcn_sdot4((int)((w.y & 0xF0F0F0F0u) ^ 0x80808080u), (int)hi.y, h, false);
        h = __builtin_amdgcn_sdot4((int)((w.z & 0xF0F0F0F0u) ^ 0x80808080u), (int)hi.z, h, false);
        h = __builtin_amdgcn_sdot4((int)((w.w & 0xF0F0F0F0u) ^ 0x80808080u), (int)hi.w, h, false);
        const float t = (float)((a << 4) + h) * mt.x;
        const float v = fmaf(d, t, acc[m]);
        acc[m] = b < nblk ? v : acc[m];
    }
}

// One wave per weight row, all m batch rows; lane l owns blocks l, l + 64, ...
// ROLL (more than 8 batch-row x block products per lane): the blocks are walked in a rolled
// loop with the next block's loads in flight during this one's dots; unrolled, the compiler
// keeps every block's activation reads live and runs out of registers.  Otherwise every
// block of the lane is loaded up front.
template <int WG, int M, int BPL>
__global__ void __launch_bounds__(WG, 512 / WG) gemv_q4_0_q8_kernel(const uint8_t *__restrict__ qs,
                                                                  const uint16_t *__restrict__ dsc,
                                                                  const int8_t *__restrict__ xq,
                                                                  const float *__restrict__ xs,
                                                                  float *__restrict__ y, int n, int k) {
    extern __shared__ uint4 lds4[];
    constexpr int WAVES = WG / 64;
    constexpr int SLOTS = q8_slots(M, BPL);
    constexpr int XPT = q8_blocks_per_thread(WG, M, BPL);
    constexpr bool ROLL = M * BPL > 8;
    constexpr int NU = ROLL ? 1 : BPL;             // blocks held in registers before the barrier
    const int nblk = k >> 5;
    const int mb_total = M * nblk;                 // (batch row, block) pairs, m-major
    uint4 *xlo = lds4;                             // bytes 0..15 of each block
    uint4 *xhi = lds4 + SLOTS;                     // bytes 16..31
    float2 *meta = (float2 *)(lds4 + 2 * SLOTS);   // (xs, -8 * sum of bytes 0..15 as int bits)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = blockIdx.x * WAVES + wave;
    const int rowc = row < n ? row : n - 1;

    // thread t stages blocks t, t + WG, ...: 32 contiguous bytes of xq and one scale each
    uint4 xa[XPT], xb[XPT];
    float sv[XPT];
#pragma unroll
    for (int j = 0; j < XPT; j++) {
        int c = threadIdx.x + j * WG;
        c = c < mb_total ? c : mb_total - 1;
        xa[j] = *(const uint4 *)(xq + (int64_t)c * 32);
        xb[j] = *(const uint4 *)(xq + (int64_t)c * 32 + 16);
        sv[j] = xs[c];
    }
    __builtin_amdgcn_sched_barrier(0);  // the activation loads are issued before the weights'

    uint4 q[NU];
    uint16_t dd[NU];
    const uint4 *qrow = (const uint4 *)(qs + (int64_t)rowc * (k >> 1));
    const uint16_t *drow = dsc + (int64_t)rowc * nblk;
#pragma unroll
    for (int u = 0; u < NU; u++) {
        int b = lane + 64 * u;
        b = b < nblk ? b : nblk - 1;
        q[u] = ld_stream16(qrow + b);
        dd[u] = drow[b];
    }
    __builtin_amdgcn_sched_barrier(0);  // every load is issued before the LDS writes wait on x

#pragma unroll
    for (int j = 0; j < XPT; j++) {
        const int c = threadIdx.x + j * WG;
        const int slot = c < mb_total ? c : SLOTS - 1;
        int sum = __builtin_amdgcn_sdot4((int)xa[j].x, 0x01010101, 0, false);
        sum = __builtin_amdgcn_sdot4((int)xa[j].y, 0x01010101, sum, false);
        sum = __builtin_amdgcn_sdot4((int)xa[j].z, 0x01010101, sum, false);
        sum = __builtin_amdgcn_sdot4((int)xa[j].w, 0x01010101, sum, false);
        xlo[slot] = xa[j];
        xhi[slot] = xb[j];
        meta[slot] = make_float2(sv[j], __int_as_float(-8 * sum));
    }
    lds_barrier();

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; m++) acc[m] = 0.f;
    if constexpr (ROLL) {
        uint4 qc = q[0];
        uint16_t dc = dd[0];
#pragma unroll 1
        for (int u = 0; u < BPL; u++) {
            const int b = lane + 64 * u, bn = b + 64;
            const int bnc = bn < nblk ? bn : nblk - 1;  // past the end: re-read, unused
            const uint4 qn = ld_stream16(qrow + bnc);
            const uint16_t dn = drow[bnc];
            q4_block<M>(qc, dc, b, b < nblk ? b : nblk - 1, nblk, xlo, xhi, meta, acc);
            qc = qn;
            dc = dn;
        }
    } else {
#pragma unroll
        for (int u = 0; u < BPL; u++) {
            const int b = lane + 64 * u;
            q4_block<M>(q[u], dd[u], b, b < nblk ? b : nblk - 1, nblk, xlo, xhi, meta, acc);
        }
    }
#pragma unroll
    for (int m = 0; m < M; m++) {
        const float t = wave_sum(acc[m]) * 0.0625f;
        if (lane == 0 && row < n) y[(int64_t)m * n + row] = t;
    }
}

// 256-thread workgroups for rows of at most 4096 weights (more workgroups, each staging
// less), 512 for longer rows.  (Two rows per wave, each staged block read once for both,
// measured slower on every decode shape: half as many waves.)
template <int M, int BPL>
bool launch(const qmv_weights *w, const int8_t *xq, const float *xs, float *y, hipStream_t s) {
    const int n = (int)w->n, k = (int)w->k;
    constexpr int WG = BPL <= 2 ? 256 : 512;
    constexpr int ROWS = WG / 64;
    hipLaunchKernelGGL((gemv_q4_0_q8_kernel<WG, M, BPL>), dim3((n + ROWS - 1) / ROWS), dim3(WG),
                       q8_lds_bytes(M, BPL), s, (const uint8_t *)w->codes, (const uint16_t *)w->scales, xq, xs,
                       y, n, k);
    return true;
}

template <int M>
bool dispatch_bpl(int bpl, const qmv_weights *w, const int8_t *xq, const float *xs, float *y, hipStream_t s) {
    switch (bpl) {
    case 1: return launch<M, 1>(w, xq, xs, y, s);
    case 2: return launch<M, 2>(w, xq, xs, y, s);
    case 3: return launch<M, 3>(w, xq, xs, y, s);
    case 4: return launch<M, 4>(w, xq, xs, y, s);
    case 5: return launch<M, 5>(w, xq, xs, y, s);
    case 6: return launch<M, 6>(w, xq, xs, y, s);
    case 7: return launch<M, 7>(w, xq, xs, y, s);
    case 8: return launch<M, 8>(w, xq, xs, y, s);
    }
    return false;
}

bool dispatch_m(int m, int bpl, const qmv_weights *w, const int8_t *xq, const float *xs, float *y,
                hipStream_t s) {
    switch (m) {
    case 1: return dispatch_bpl<1>(bpl, w, xq, xs, y, s);
    case 2: return dispatch_bpl<2>(bpl, w, xq, xs, y, s);
    case 3: return dispatch_bpl<3>(bpl, w, xq, xs, y, s);
    case 4: return dispatch_bpl<4>(bpl, w, xq, xs, y, s);
    case 5: return dispatch_bpl<5>(bpl, w, xq, xs, y, s);
    case 6: return dispatch_bpl<6>(bpl, w, xq, xs, y, s);
    case 7: return dispatch_bpl<7>(bpl, w, xq, xs, y, s);
    case 8: return dispatch_bpl<8>(bpl, w, xq, xs, y, s);
    }
    return false;
}

}  // namespace

const char *launch_gemv_q4_0_q8(const qmv_weights *w, int m, const int8_t *xq, const float *xs, float *y,
                                hipStream_t s) {
    const int64_t n = w->n, k = w->k, nblk = k / 32;
    const int bpl = (int)((nblk + 63) / 64);
    if (n > INT32_MAX || bpl > BPL_MAX) return nullptr;
    if ((int64_t)q8_lds_bytes(m, bpl) > device_info().lds_per_block) return nullptr;
    return dispatch_m(m, bpl, w, xq, xs, y, s) ? "q4_0.q8.lds-x.dot4" : nullptr;
}

}  // namespace qmv
