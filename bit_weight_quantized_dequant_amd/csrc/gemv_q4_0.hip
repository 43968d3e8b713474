// gemv_q4_0.hip -- q4_0 decode GEMV for gfx950.
//
// y[m][n] = sum_k d[n][k/32] * (q[n][k] - 8) * x[m][k]   (q4_0: 32 weights per block,
// 16 code bytes + an fp16 scale; "LLMs on the Xiaomi TV Box", §11.5 E18 gives its
// 4.5 bits per weight).  The GEMV streams weight bytes, so its roofline is HBM
// bandwidth (quantprobe LAWS.md, Law 4); L-15 says the unpack instructions are the
// tax on top, so the unpack here is a handful of SWAR ops per 8 weights:
//
//   * Each lane owns whole blocks: one 128-bit load of 16 code bytes + one fp16 scale.
//   * Activations for the workgroup are staged once into LDS as fp32, 32 per block
//     (row stride 36 floats so that eight lanes reading eight blocks with ds_read_b128
//     touch disjoint banks).  They are staged before the weight loads are issued:
//     vector loads return in order, so staging after them would wait for every weight.
//   * Centering is exact: a nibble is OR-ed under the binary16 exponent of 1024 (bits
//     0-3) or of 256 with a quarter ulp (bits 4-7), and one packed half subtract turns
//     the pair into (q - 8) or 4 (q - 8), exactly.  v_fma_mix_f32 then multiplies the
//     binary16 half by the fp32 activation with an exact product, so a zero weight adds
//     exactly zero and the rounding error is relative to sum |w||x|.
//   * The 64 lane partials of a row are summed across the wavefront with DPP.
#include <cstring>

#include "device_common.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int XS = 36;   // floats per staged 32-activation block (32 + 4 of padding)
constexpr int XS4 = XS / 4;
constexpr int MAX_CHUNKS = 4096;  // 16-byte activation chunks one workgroup stages (m*k <= 16384)

// Activation chunks each thread stages: enough for m * k / 4 chunks at k <= 2048 * BPL.
constexpr int xchunks_per_thread(int wg, int m, int bpl) {
    return ((m * bpl * 512 < MAX_CHUNKS ? m * bpl * 512 : MAX_CHUNKS) + wg - 1) / wg;
}
// LDS bytes: every staged chunk slot (XPT * WG of them, 8 per padded 36-float block).
constexpr size_t lds_bytes(int wg, int m, int bpl) {
    return (size_t)xchunks_per_thread(wg, m, bpl) * wg / 8 * XS * sizeof(float);
}

// and_or with a volatile asm: kept in program order relative to the scheduling barriers,
// so the unpack of a later block is not hoisted next to this one (its halves would all be
// live at once).
QMV_DEV uint32_t and_or_ordered(uint32_t a, uint32_t mask, uint32_t bits) {
    uint32_t r;
    asm volatile("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(mask), "v"(bits));
    return r;
}

// sum_{i<32} (q_i - 8) * x_i for one block (codes in 4 dwords, activations in xb[0..31]).
// Each (q - 8) is an exact binary16 half; v_fma_mix_f32 multiplies it by the fp32
// activation inside a fused multiply-add, so the only roundings are those of the sums.
template <bool ORDERED = false>
QMV_DEV float dot_q4_mix(uint4 q, const float *xb) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    const qmv_h2 off_lo = {(_Float16)-1032.f, (_Float16)-1032.f};  // (1024 + q) - 1032 = q - 8
    const qmv_h2 off_hi = {(_Float16)-288.f, (_Float16)-288.f};    // (256 + 4q) - 288 = 4 (q - 8)
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t w8 = w[i] >> 8;
        auto ao = [](uint32_t a, uint32_t mk, uint32_t b) { return ORDERED ? and_or_ordered(a, mk, b) : and_or(a, mk, b); };
        const qmv_h2 t0 = as_h2(ao(w[i], 0x000F000Fu, 0x64006400u)) + off_lo;  // bytes 0, 2 low
        const qmv_h2 t1 = as_h2(ao(w[i], 0x00F000F0u, 0x5C005C00u)) + off_hi;  // bytes 0, 2 high
        const qmv_h2 t2 = as_h2(ao(w8, 0x000F000Fu, 0x64006400u)) + off_lo;    // bytes 1, 3 low
        const qmv_h2 t3 = as_h2(ao(w8, 0x00F000F0u, 0x5C005C00u)) + off_hi;    // bytes 1, 3 high
        a0 = fmaf((float)t0.x, xb[4 * i + 0], a0);
        a0 = fmaf((float)t0.y, xb[4 * i + 2], a0);
        b0 = fmaf((float)t2.x, xb[4 * i + 1], b0);
        b0 = fmaf((float)t2.y, xb[4 * i + 3], b0);
        a1 = fmaf((float)t1.x, xb[16 + 4 * i + 0], a1);
        a1 = fmaf((float)t1.y, xb[16 + 4 * i + 2], a1);
        b1 = fmaf((float)t3.x, xb[16 + 4 * i + 1], b1);
        b1 = fmaf((float)t3.y, xb[16 + 4 * i + 3], b1);
    }
    return (a0 + b0) + (a1 + b1) * 0.25f;
}

// The centred sums of two rows' blocks against the same 32 activations, interleaved per
// dword (each activation used by both rows as soon as it is read).
QMV_DEV void dot_q4_mix2(uint4 qa, uint4 qb, const float *xb, float &sa, float &sb) {
    const uint32_t wa[4] = {qa.x, qa.y, qa.z, qa.w}, wb[4] = {qb.x, qb.y, qb.z, qb.w};
    const qmv_h2 off_lo = {(_Float16)-1032.f, (_Float16)-1032.f};
    const qmv_h2 off_hi = {(_Float16)-288.f, (_Float16)-288.f};
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f, c0 = 0.f, c1 = 0.f, e0 = 0.f, e1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t va8 = wa[i] >> 8, vb8 = wb[i] >> 8;
        const qmv_h2 t0 = as_h2(and_or_ordered(wa[i], 0x000F000Fu, 0x64006400u)) + off_lo;
        const qmv_h2 t1 = as_h2(and_or_ordered(wa[i], 0x00F000F0u, 0x5C005C00u)) + off_hi;
        const qmv_h2 t2 = as_h2(and_or_ordered(va8, 0x000F000Fu, 0x64006400u)) + off_lo;
        const qmv_h2 t3 = as_h2(and_or_ordered(va8, 0x00F000F0u, 0x5C005C00u)) + off_hi;
        const qmv_h2 u0 = as_h2(and_or_ordered(wb[i], 0x000F000Fu, 0x64006400u)) + off_lo;
        const qmv_h2 u1 = as_h2(and_or_ordered(wb[i], 0x00F000F0u, 0x5C005C00u)) + off_hi;
        const qmv_h2 u2 = as_h2(and_or_ordered(vb8, 0x000F000Fu, 0x64006400u)) + off_lo;
        const qmv_h2 u3 = as_h2(and_or_ordered(vb8, 0x00F000F0u, 0x5C005C00u)) + off_hi;
        const float x0 = xb[4 * i], x1 = xb[4 * i + 1], x2 = xb[4 * i + 2], x3 = xb[4 * i + 3];
        const float y0 = xb[16 + 4 * i], y1 = xb[16 + 4 * i + 1], y2 = xb[16 + 4 * i + 2], y3 = xb[16 + 4 * i + 3];
        a0 = fmaf((float)t0.x, x0, a0);
        a0 = fmaf((float)t0.y, x2, a0);
        b0 = fmaf((float)t2.x, x1, b0);
        b0 = fmaf((float)t2.y, x3, b0);
        a1 = fmaf((float)t1.x, y0, a1);
        a1 = fmaf((float)t1.y, y2, a1);
        b1 = fmaf((float)t3.x, y1, b1);
        b1 = fmaf((float)t3.y, y3, b1);
        c0 = fmaf((float)u0.x, x0, c0);
        c0 = fmaf((float)u0.y, x2, c0);
        e0 = fmaf((float)u2.x, x1, e0);
        e0 = fmaf((float)u2.y, x3, e0);
        c1 = fmaf((float)u1.x, y0, c1);
        c1 = fmaf((float)u1.y, y2, c1);
        e1 = fmaf((float)u3.x, y1, e1);
        e1 = fmaf((float)u3.y, y3, e1);
    }
    sa = (a0 + b0) + (a1 + b1) * 0.25f;
    sb = (c0 + e0) + (c1 + e1) * 0.25f;
}

// Same centred sum with byte-to-float conversions (v_cvt_f32_ubyte*), a reference variant.
QMV_DEV float dot_q4_cvt(uint4 q, const float *xb) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t lo = w[i] & 0x0F0F0F0Fu, hi = (w[i] >> 4) & 0x0F0F0F0Fu;
        a = fmaf((float)(lo & 0xFFu) - 8.f, xb[4 * i + 0], a);
        a = fmaf((float)((lo >> 8) & 0xFFu) - 8.f, xb[4 * i + 1], a);
        a = fmaf((float)((lo >> 16) & 0xFFu) - 8.f, xb[4 * i + 2], a);
        a = fmaf((float)(lo >> 24) - 8.f, xb[4 * i + 3], a);
        b = fmaf((float)(hi & 0xFFu) - 8.f, xb[16 + 4 * i + 0], b);
        b = fmaf((float)((hi >> 8) & 0xFFu) - 8.f, xb[16 + 4 * i + 1], b);
        b = fmaf((float)((hi >> 16) & 0xFFu) - 8.f, xb[16 + 4 * i + 2], b);
        b = fmaf((float)(hi >> 24) - 8.f, xb[16 + 4 * i + 3], b);
    }
    return a + b;
}

// One wave computes one row for all m activation rows; lane l owns blocks l, l+64, ...
//   * The activation loads are issued first, then every weight load of the row (128-bit
//     codes + the fp16 scale per block), then x is written to LDS.  The code is free of
//     branches around loads: row and block indices are clamped (a lane past the row end
//     re-reads the last block and its sum is dropped by a select), and activation chunks
//     past the end are written to a junk slot after the staged blocks.  A branch around a
//     load would split the block and make the compiler wait for that load on the spot,
//     serialising the row into one memory round trip per block.
//   * Vector loads complete in issue order, so the LDS writes wait for x only, and block u
//     becomes usable as soon as loads 0..u have landed.
//   * The 64 lane partials of a row are summed across the wavefront with DPP.
template <int WG, int M, int BPL, int XT, bool MIX, int R>
__global__ void __launch_bounds__(WG, 512 / WG) gemv_q4_0_kernel(const uint8_t *__restrict__ qs,
                                                       const uint16_t *__restrict__ dsc,
                                                       const void *__restrict__ x,
                                                       float *__restrict__ y, int n, int k) {
    extern __shared__ float4 sx4[];
    constexpr int WAVES = WG / 64;
    constexpr int XPT = xchunks_per_thread(WG, M, BPL);
    const int nblk = k >> 5;
    const int total = M * (k >> 2);  // 16-byte activation chunks, m-major; 8 per block
    // the wave index is uniform: made scalar, the row bases live in SGPRs and each load takes
    // a 32-bit lane offset instead of a 64-bit address per lane
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row0 = (blockIdx.x * WAVES + wave) * R;  // this wave's rows: row0 .. row0 + R - 1

    float4 xv[XPT];
#pragma unroll
    for (int j = 0; j < XPT; j++) {
        const int c = threadIdx.x + j * WG;
        xv[j] = ld_act4<XT>(x, (int64_t)(c < total ? c : total - 1) * 4);
    }

    // block-major load order (block u of every row, then block u + 1), so that block u
    // can be computed as soon as its loads have landed
    uint4 q[BPL][R];
    uint16_t dd[BPL][R];
    const uint4 *qrow[R];
    const uint16_t *drow[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int rowc = row0 + r < n ? row0 + r : n - 1;
        qrow[r] = (const uint4 *)(qs + (int64_t)rowc * (k >> 1));
        drow[r] = dsc + (int64_t)rowc * nblk;
    }
#pragma unroll
    for (int u = 0; u < BPL; u++) {
        int b = lane + 64 * u;
        b = b < nblk ? b : nblk - 1;
#pragma unroll
        for (int r = 0; r < R; r++) {
            q[u][r] = ld_stream16(qrow[r] + b);
            dd[u][r] = drow[r][b];
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // every load is issued before the LDS writes wait on x

    // chunk c -> block c >> 3, slot c & 7; chunks past the end land in the padding blocks
    float4 *dst = sx4 + (threadIdx.x >> 3) * XS4 + (threadIdx.x & 7);
#pragma unroll
    for (int j = 0; j < XPT; j++) dst[j * (WG / 8) * XS4] = xv[j];
    lds_barrier();

    // each block's 32 activations are read from LDS once per batch row and used for all R rows
    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < M; m++) acc[r][m] = 0.f;
#pragma unroll
    for (int u = 0; u < BPL; u++) {
        const int b = lane + 64 * u;
        const int bc = b < nblk ? b : nblk - 1;
#pragma unroll
        for (int m = 0; m < M; m++) {
            float xb[32];
#pragma unroll
            for (int i = 0; i < 8; i++) *(float4 *)(xb + 4 * i) = sx4[(m * nblk + bc) * XS4 + i];
            float sr[R];
            if constexpr (R == 2 && MIX) {
                dot_q4_mix2(q[u][0], q[u][1], xb, sr[0], sr[1]);
            } else {
#pragma unroll
                for (int r = 0; r < R; r++) sr[r] = MIX ? dot_q4_mix(q[u][r], xb) : dot_q4_cvt(q[u][r], xb);
            }
#pragma unroll
            for (int r = 0; r < R; r++) {
                const float v = fmaf(h2f(dd[u][r]), sr[r], acc[r][m]);
                acc[r][m] = b < nblk ? v : acc[r][m];
            }
        }
        // keep the next block's activation reads below this block's dots: hoisted, every
        // block's 32 activations would be live at once
        if (R > 1) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float t = wave_sum(acc[r][m]);
            if (lane == 0 && row0 + r < n) y[(int64_t)m * n + row0 + r] = t;
        }
}

// Batches (m >= 2) and rows longer than 16384: K is walked in chunks of 2048 (64 blocks, one
// per lane).  The wave's block of chunk c + 1 is requested before the dots of chunk c, and
// each chunk's activations (m x 2048) are staged once per workgroup, with the same
// branch-free loads (clamped indices) as the one-shot kernel; each looked-up block serves
// all m batch rows.
constexpr int KC = 2048;

template <int WG, int M, int XT>
__global__ void __launch_bounds__(WG) gemv_q4_0_chunked_kernel(const uint8_t *__restrict__ qs,
                                                               const uint16_t *__restrict__ dsc,
                                                               const void *__restrict__ x,
                                                               float *__restrict__ y, int n, int k) {
    extern __shared__ float4 sx4[];
    constexpr int WAVES = WG / 64, NX = M * (KC / 4), XPT = (NX + WG - 1) / WG;  // NX: chunk's x pieces
    const int nblk = k >> 5, nch = (nblk + 63) >> 6;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = blockIdx.x * WAVES + wave;
    const int rowc = row < n ? row : n - 1;
    const uint4 *qr = (const uint4 *)(qs + (int64_t)rowc * (k >> 1));
    const uint16_t *dr = dsc + (int64_t)rowc * nblk;

    uint4 qc = ld_stream16(qr + (lane < nblk ? lane : nblk - 1));
    uint16_t dc = dr[lane < nblk ? lane : nblk - 1];
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; m++) acc[m] = 0.f;
    for (int c = 0; c < nch; c++) {
        const int k0 = c * KC;
        const int kq = min(KC, k - k0) >> 2;  // 16-byte activation chunks of this K chunk, per row
        float4 xv[XPT];
#pragma unroll
        for (int j = 0; j < XPT; j++) {
            const int cc = threadIdx.x + j * WG, e = cc & 511;
            const int m = (cc >> 9) < M ? cc >> 9 : M - 1;  // pieces past the batch re-read row M - 1
            xv[j] = ld_act4<XT>(x, (int64_t)m * k + k0 + 4 * (e < kq ? e : kq - 1));
        }
        int bn = (c + 1) * 64 + lane;  // next chunk's block (clamped on the last chunk)
        bn = bn < nblk ? bn : nblk - 1;
        const uint4 qn = ld_stream16(qr + bn);
        const uint16_t dn = dr[bn];
        __builtin_amdgcn_sched_barrier(0);
        if (c) lds_barrier();  // the previous chunk's activations are consumed
#pragma unroll
        for (int j = 0; j < XPT; j++) {
            const int cc = threadIdx.x + j * WG, m = cc >> 9, e = cc & 511;
            if (XPT * WG == NX || cc < NX) sx4[(m * 64 + (e >> 3)) * XS4 + (e & 7)] = xv[j];
        }
        lds_barrier();
        const int b = c * 64 + lane;
        const float d = h2f(dc);
        if constexpr (M <= 2) {
#pragma unroll
            for (int m = 0; m < M; m++) {
                float xb[32];
#pragma unroll
                for (int i = 0; i < 8; i++) *(float4 *)(xb + 4 * i) = sx4[(m * 64 + lane) * XS4 + i];
                const float v = fmaf(d, dot_q4_mix(qc, xb), acc[m]);
                acc[m] = b < nblk ? v : acc[m];
            }
        } else {
            // three or more batch rows: the block's 32 weights (q - 8) expanded once to fp32
            // (exact: a nibble under the binary16 exponent of 1024, one packed half subtract,
            // a conversion), then one fp32 FMA per weight and batch row, v_fmac_f32 instead of
            // v_fma_mix_f32: the same exact products in fewer cycles once the expansion is
            // shared by enough rows
            float wq[32];
            const uint32_t wv[4] = {qc.x, qc.y, qc.z, qc.w};
            const qmv_h2 off = {(_Float16)-1032.f, (_Float16)-1032.f};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t w = wv[i];
                const qmv_h2 l02 = as_h2(and_or(w, 0x000F000Fu, 0x64006400u)) + off;         // bytes 0, 2 low
                const qmv_h2 l13 = as_h2(and_or(w >> 8, 0x000F000Fu, 0x64006400u)) + off;    // bytes 1, 3 low
                const qmv_h2 h02 = as_h2(and_or(w >> 4, 0x000F000Fu, 0x64006400u)) + off;    // bytes 0, 2 high
                const qmv_h2 h13 = as_h2(and_or(w >> 12, 0x000F000Fu, 0x64006400u)) + off;   // bytes 1, 3 high
                wq[4 * i + 0] = (float)l02.x;
                wq[4 * i + 1] = (float)l13.x;
                wq[4 * i + 2] = (float)l02.y;
                wq[4 * i + 3] = (float)l13.y;
                wq[16 + 4 * i + 0] = (float)h02.x;
                wq[16 + 4 * i + 1] = (float)h13.x;
                wq[16 + 4 * i + 2] = (float)h02.y;
                wq[16 + 4 * i + 3] = (float)h13.y;
            }
            // materialise the fp32 weights: otherwise every use folds the conversion back
            // into a v_fma_mix_f32, once per batch row
#pragma unroll
            for (int i = 0; i < 32; i++) asm volatile("" : "+v"(wq[i]));
#pragma unroll
            for (int m = 0; m < M; m++) {
                float xb[32];
#pragma unroll
                for (int i = 0; i < 8; i++) *(float4 *)(xb + 4 * i) = sx4[(m * 64 + lane) * XS4 + i];
                float s0 = 0.f, s1 = 0.f;
#pragma unroll
                for (int i = 0; i < 32; i += 2) {
                    s0 = fmaf(wq[i], xb[i], s0);
                    s1 = fmaf(wq[i + 1], xb[i + 1], s1);
                }
                const float v = fmaf(d, s0 + s1, acc[m]);
                acc[m] = b < nblk ? v : acc[m];
            }
        }
        qc = qn;
        dc = dn;
    }
#pragma unroll
    for (int m = 0; m < M; m++) {
        const float t = wave_sum(acc[m]);
        if (lane == 0 && row < n) y[(int64_t)m * n + row] = t;
    }
}

// 512-thread workgroups: each chunk's activations are staged once for eight rows (with four
// rows per workgroup the batch-8 staging traffic outweighed the weights).
template <int XT>
bool launch_chunked(int m, const qmv_weights *w, const void *x, float *y, hipStream_t s) {
    constexpr int WG = 512;
    const int n = (int)w->n, k = (int)w->k;
    const dim3 grid((n + WG / 64 - 1) / (WG / 64));
    const size_t lds = (size_t)m * 64 * XS * sizeof(float);
#define QMV_Q4C(MM)                                                                                          \
    case MM:                                                                                                 \
        hipLaunchKernelGGL((gemv_q4_0_chunked_kernel<WG, MM, XT>), grid, dim3(WG), lds, s,                   \
                           (const uint8_t *)w->codes, (const uint16_t *)w->scales, x, y, n, k);             \
        return true;
    switch (m) { QMV_Q4C(1) QMV_Q4C(2) QMV_Q4C(3) QMV_Q4C(4) QMV_Q4C(5) QMV_Q4C(6) QMV_Q4C(7) QMV_Q4C(8) }
#undef QMV_Q4C
    return false;
}

// 256-thread workgroups for short rows (more workgroups, x staged by fewer waves each),
// 512 for long ones; R rows per wave.
template <int M, int BPL, int XT, bool MIX, int R>
bool launch(const qmv_weights *w, const void *x, float *y, hipStream_t s) {
    if constexpr (R > 1 && M * BPL > 4) {
        return false;  // not instantiated: the launcher takes one row per wave there
    } else {
        const int n = (int)w->n, k = (int)w->k;
        constexpr int WG = BPL <= 2 ? 256 : 512;
        constexpr int ROWS = WG / 64 * R;
        hipLaunchKernelGGL((gemv_q4_0_kernel<WG, M, BPL, XT, MIX, R>), dim3((n + ROWS - 1) / ROWS), dim3(WG),
                           lds_bytes(WG, M, BPL), s, (const uint8_t *)w->codes, (const uint16_t *)w->scales, x,
                           y, n, k);
        return true;
    }
}

template <int M, int XT, bool MIX, int R>
bool dispatch_bpl(int bpl, const qmv_weights *w, const void *x, float *y, hipStream_t s) {
    switch (bpl) {
    case 1: return launch<M, 1, XT, MIX, R>(w, x, y, s);
    case 2: return launch<M, 2, XT, MIX, R>(w, x, y, s);
    case 3: return launch<M, 3, XT, MIX, R>(w, x, y, s);
    case 4: return launch<M, 4, XT, MIX, R>(w, x, y, s);
    case 5: return launch<M, 5, XT, MIX, R>(w, x, y, s);
    case 6: return launch<M, 6, XT, MIX, R>(w, x, y, s);
    case 7: return launch<M, 7, XT, MIX, R>(w, x, y, s);
    case 8: return launch<M, 8, XT, MIX, R>(w, x, y, s);
    }
    return false;
}

}  // namespace

const char *launch_gemv_q4_0(const qmv_weights *w, int m, const void *x, int xt, float *y,
                             hipStream_t s) {
    const int64_t n = w->n, k = w->k, nblk = k / 32;
    const int bpl = (int)((nblk + 63) / 64);
    if (n > INT32_MAX || k > INT32_MAX / 8) return nullptr;
    const char *fp = forced_path();
    // Batches, and rows longer than 16384, go through the K-chunked kernel: for m >= 2 it beats
    // the one-shot kernels, which hold m rows' dots for every block of a lane in registers.
    if (bpl > 8 || m > 1 || strcmp(fp, "q4_0.chunked") == 0) {
        if ((int64_t)m * 64 * XS * (int64_t)sizeof(float) > device_info().lds_per_block) return nullptr;
        const bool ok = xt == QMV_F32 ? launch_chunked<0>(m, w, x, y, s) : launch_chunked<1>(m, w, x, y, s);
        if (!ok) return nullptr;
        return m >= 3 ? "q4_0.lds-x-chunked.fmac" : "q4_0.lds-x-chunked.fma-mix";
    }
    // batch 1: two rows per wave (each staged activation block read once for both) while both
    // rows' blocks fit in registers (bpl <= 4) and the matrix has at most 32 rows per CU; one
    // row per wave otherwise (11008 x 4096: 7.71 against 7.85 us; 4096 x 4096: 4.26 against
    // 4.21), on request (test override) and for the reference variant
    const bool cvt = strcmp(fp, "q4_0.cvt") == 0 && xt == QMV_F32;
    const bool r1 = cvt || strcmp(fp, "q4_0.r1") == 0 || bpl > 4 || n > 32 * (int64_t)device_info().num_cus;
    const size_t lds = bpl <= 2 ? lds_bytes(256, 1, bpl) : lds_bytes(512, 1, bpl);
    if ((int64_t)lds > device_info().lds_per_block) return nullptr;
    bool ok;
    if (cvt)
        ok = dispatch_bpl<1, 0, false, 1>(bpl, w, x, y, s);
    else if (r1)
        ok = xt == QMV_F32 ? dispatch_bpl<1, 0, true, 1>(bpl, w, x, y, s) : dispatch_bpl<1, 1, true, 1>(bpl, w, x, y, s);
    else
        ok = xt == QMV_F32 ? dispatch_bpl<1, 0, true, 2>(bpl, w, x, y, s) : dispatch_bpl<1, 1, true, 2>(bpl, w, x, y, s);
    if (!ok) return nullptr;
    return cvt ? "q4_0.lds-x.cvt-ubyte" : r1 ? "q4_0.lds-x.fma-mix" : "q4_0.lds-x.fma-mix.2row";
}

}  // namespace qmv
