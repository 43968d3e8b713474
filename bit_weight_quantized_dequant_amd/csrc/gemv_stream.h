// gemv_stream.h -- the K-streaming skeleton shared by the codebook GEMVs whose work unit
// is 64 consecutive weights of one row per lane (the additive codes and the 8-bit
// codebook).  gfx950, wave64, one output row per wave, eight waves per workgroup.
//
// A row is walked in steps of KC = 4096 weights (64 lanes x 64).  The activations of a
// step are staged into LDS as fp32 in unit order: unit u (weights 64u .. 64u+63 of the
// step) of batch row m at sx + (m * 64 + u) * XU, with XU = 68 floats (4 of padding, so
// that lanes reading consecutive units with ds_read_b128 fall on disjoint banks).
//
// Pipeline, per step c (every wave of the workgroup in lock step, one barrier per step):
//   1. issue the loads of step c+1 into registers: its activations (2M float4 per
//      thread) and this lane's code bytes (the policy's Codes);
//   2. compute step c from LDS buffer c & 1 with the codes loaded one step earlier;
//   3. write the prefetched activations into LDS buffer (c+1) & 1, then the barrier.
// So every load has a whole step of compute to arrive, and no branch sits around a
// load: indices are clamped to the row (a clamped unit is computed and dropped by a
// select), and the last step (nothing to prefetch) is a separate copy of the step.  With more than
// four batch rows two activation buffers do not fit in LDS; the single-buffer variant
// writes after a second barrier instead.
//
// A policy P provides (R = P::R rows per wave, 1 or more):
//   typename P::Codes                                  the lane's code bytes of one unit (R rows)
//   void load(Codes &c, int unit) const                issue the loads (unit clamped)
//   template <int M> void dot(const Codes &c, const float *xu, float (&s)[R * M]) const
//       s[r * M + m] += sum over unit's 64 weights of row r of w * x[m], x[m] at
//       xu + m * 64 * XU (each activation read once for the R rows)
#pragma once

#include <type_traits>

#include "device_common.h"

namespace qmv {
namespace stream {

constexpr int WG = 512;
constexpr int WAVES = WG / 64;
constexpr int KC = 4096;
constexpr int XU = 68;
constexpr int XBUF = 64 * XU;  // floats of one batch row's staged step

// The half-step form (L = 32 lanes per row, two rows per wave, 256-thread workgroups,
// 2048-weight steps) stages half as many activations per workgroup; L = 64 is the form
// described above.
constexpr int wg_of(int l) { return 8 * l; }
constexpr int kc_of(int l) { return 64 * l; }
constexpr int xbuf_of(int l) { return l * XU; }

// LDS floats of the activation buffers for batch m and a row of k weights.
constexpr int nbuf(int m) { return m <= 4 ? 2 : 1; }
inline size_t x_lds_bytes(int m, int64_t k, int l = 64) {
    const int bufs = k > kc_of(l) ? nbuf(m) : 1;
    return (size_t)bufs * m * xbuf_of(l) * sizeof(float);
}

// Thread t loads 16-byte pieces t and t + WG of each batch row's step (a step row is
// 1024 pieces; pieces past the row's end are clamped to its last piece).
template <int M, int XT, int L = 64>
QMV_DEV void load_x(float4 (&xv)[2 * M], const void *x, int k, int c) {
    const int k0 = c * kc_of(L);
    const int kq = min(kc_of(L), k - k0) >> 2;
#pragma unroll
    for (int j = 0; j < 2 * M; j++) {
        const int m = j >> 1, e = threadIdx.x + (j & 1) * wg_of(L);
        xv[j] = ld_act4<XT>(x, (int64_t)m * k + k0 + 4 * (e < kq ? e : kq - 1));
    }
}

// Piece e of a step row holds weights 4e .. 4e+3: unit e >> 4, offset 4 (e & 15).
template <int M, int L = 64>
QMV_DEV void store_x(const float4 (&xv)[2 * M], float *buf) {
#pragma unroll
    for (int j = 0; j < 2 * M; j++) {
        const int m = j >> 1, e = threadIdx.x + (j & 1) * wg_of(L);
        *(float4 *)(buf + m * xbuf_of(L) + (e >> 4) * XU + 4 * (e & 15)) = xv[j];
    }
}

// Walk the wave's row(s): acc[r * M + m] += sum over row r's k weights of w * x[m].  `sx` holds nbuf(M)
// activation buffers when k > KC, one otherwise; every thread of the workgroup calls
// this with the same k (the barriers are workgroup-wide).
template <class P, int M, int XT, int L = 64>
QMV_DEV void walk_row(const P &pol, const void *x, int k, float *sx, float (&acc)[P::R * M]) {
    constexpr int RM = P::R * M;
    constexpr bool TWO = nbuf(M) == 2;
    constexpr int XB = xbuf_of(L);
    const int lane = threadIdx.x & (L - 1);  // this lane's unit slot in a step of its row
    const int nunits = k >> 6, nst = (nunits + L - 1) / L;
    typename P::Codes c0, c1;
    float4 xv[2 * M];

    load_x<M, XT, L>(xv, x, k, 0);
    pol.load(c0, lane < nunits ? lane : nunits - 1);
    __builtin_amdgcn_sched_barrier(0);
    store_x<M, L>(xv, sx);
    lds_barrier();

    // One step; MORE = there is a next step to prefetch.  The choice is made outside the
    // step so that each step is straight-line code: a branch around the prefetch loads
    // would make the compiler wait for them at the join, before the dot.
    auto step = [&](auto more_tag, int c, const typename P::Codes &use, typename P::Codes &fill) {
        constexpr bool MORE = decltype(more_tag)::value;
        if (MORE) {
            load_x<M, XT, L>(xv, x, k, c + 1);
            const int un = (c + 1) * L + lane;
            pol.load(fill, un < nunits ? un : nunits - 1);
        }
        const float *buf = sx + (TWO ? (c & 1) * M * XB : 0);
        const int u = c * L + lane;
        const int uc = u < nunits ? lane : nunits - 1 - c * L;
        float s[RM];
#pragma unroll
        for (int m = 0; m < RM; m++) s[m] = 0.f;
        pol.template dot<M>(use, buf + uc * XU, s);
        // keep the dot here rather than sunk into a branch over the valid lanes
#pragma unroll
        for (int m = 0; m < RM; m++) asm volatile("" : "+v"(s[m]));
#pragma unroll
        for (int m = 0; m < RM; m++) acc[m] = u < nunits ? acc[m] + s[m] : acc[m];
        if (MORE) {
            if (!TWO) lds_barrier();  // every wave is done with the only buffer
            store_x<M, L>(xv, sx + (TWO ? ((c + 1) & 1) * M * XB : 0));
            lds_barrier();
        }
    };
    using Y = std::true_type;
    using N = std::false_type;
    int c = 0;
    for (; c + 2 < nst; c += 2) {
        step(Y{}, c, c0, c1);
        step(Y{}, c + 1, c1, c0);
    }
    if (c + 1 < nst) {
        step(Y{}, c, c0, c1);
        step(N{}, c + 1, c1, c0);
    } else {
        step(N{}, c, c0, c1);
    }
}

}  // namespace stream
}  // namespace qmv
