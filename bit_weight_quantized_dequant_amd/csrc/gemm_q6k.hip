// gemm_q6k.hip -- q6_K prefill GEMM on int8 MFMA (gfx950, v_mfma_i32_32x32x32_i8).
//
// y[m][n] = sum_s d[n][s] * sum_{c in s} xs[m][c] * I32[m][n][c], where
// I32[m][n][c] = sum over the 32 weights k of activation block c of
//               sc[n][k/16] * (q[n][k] - 32) * xq[m][k]
// is computed exactly in int32 ("57 · r54 — MINFER_MMQ_Q6K_EXP", §2.1: the q6_K
// values are expanded into centred integers for an int8 contraction; §2.3: that
// expansion is an integer transform, so the partials are exact).
//
// Design for gfx950 (the page's NB-BT CUDA kernel stages raw or pre-expanded int8 weight
// tiles with cp.async; here):
//   * Orientation: MFMA rows are weight rows n (operand A), columns are tokens m (operand
//     B = int8 activations), so each lane's column has one activation scale xs[m][c] per
//     block: the block epilogue is a shift, a convert and an FMA per value.
//   * The sub-scale is folded into the weights: w' = sc * (q - 32) lies in [-4064, 4096]
//     and is split exactly as w' = 64 h + l (l = w' & 63 in [0, 63], h = w' >> 6 in
//     [-64, 64]), two int8 operands.  Two MFMAs per 32-block give I32 = 64 C_H + C_L
//     exactly: C_H is shifted by 6 and handed to the second MFMA as its accumulator.
//   * Every operand tile sits in LDS in MFMA fragment order: a 32 x 32 int8 block is 64
//     lanes x 16 bytes, lane l holding row l % 32 and k 16 (l / 32) .. + 15.  Fragment
//     reads are then lane-linear ds_read_b128 (no bank conflicts), and so are the direct
//     global-to-LDS loads that fill them (global_load_lds_dwordx4: lane l's 16 bytes land
//     at the chunk base + 16 l), so activations and registered weight planes reach LDS
//     without passing through registers.
//   * K advances 64 per stage through a ring of four LDS stages (one per stage of a
//     super-block, so every slot address is an immediate): the loads of stage st + 3 are
//     issued right after the barrier of stage st and land while st .. st + 2 are computed.  Waits are explicit (s_waitcnt vmcnt on this stage's loads, then an
//     LDS-only barrier), so loads for later stages stay in flight across barriers.
//   * Each wave software-pipelines its 32-blocks: the previous block's epilogue (convert
//     and FMA, VALU) is interleaved with this block's MFMAs, so the matrix cores and the
//     VALU work on different blocks at the same time.
//   * fp32 sums per super-block are scaled by d once; the workgroup's d values are staged
//     in LDS once.
// Tiles: 64 weight rows x 128 tokens per workgroup.  Four waves (2 row groups x 2 token
// pairs), each 32 rows x 64 tokens (two MFMA tiles sharing the weight fragments).  When
// there are too few tiles to give every CU several workgroups, eight waves split K by the
// parity of the 32-block (KSPLIT = 2) and add their sums through LDS at the end, so a CU
// still holds two waves per SIMD.
// Weights come either from registered pre-expanded planes (EXP: the h and l bytes already in
// fragment order, loaded straight into LDS) or from the codes, expanded by the threads into
// the same LDS image.
//
// MFMA operand layout (32x32x32 i8): lane l supplies row (or column) l % 32 and the 16
// consecutive k of group l / 32; accumulator value v of lane l is
// C[8 (v / 4) + 4 (l / 32) + (v % 4)][l % 32].  A debug entry point writes the exact I32
// partials from this same code path, which pins the layout against the oracle.
#include <cstring>

#include "device_common.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BN = 64;     // weight rows per workgroup tile
constexpr int BM = 128;    // tokens per workgroup tile
constexpr int NSTAGE = 4;  // LDS ring depth: one slot per stage of a super-block
constexpr int MAXSB = 80;  // super-blocks (k / 256) whose d values fit the workgroup's table

// Four 6-bit codes (bytes of q) -> w' = sc * (q - 32) in [-4064, 4096], split exactly as
// w' = 64 h + l, packed as four h bytes and four l bytes.  (w' << 2) keeps h in the high byte
// of each 16-bit lane.
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

// s_waitcnt with only the vector-memory count set (expcnt and lgkmcnt left unlimited).
template <int N>
QMV_DEV void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Pins 16 VALU results at this point of the program: without it the compiler sinks a block's
// epilogue arithmetic towards its next use, behind later blocks' MFMAs, undoing the
// interleaving of one block's epilogue with the next block's matrix work.
QMV_DEV void pin16(float (&v)[16]) {
    asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),
                 "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15]));
}

// The ring's barrier: this wave's LDS operations complete (its reads of the stage about to
// be refilled, its expanded-weight writes), then s_barrier.  The direct loads of the stage
// are waited for separately (wait_vmcnt): a workgroup fence here would also wait for the
// loads already issued for later stages, since they write LDS too.  The empty asm
// statements keep the compiler from moving memory accesses across the barrier.
QMV_DEV void ring_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unlimited
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// 16 bytes per lane from global memory straight into LDS at chunk + 16 * lane.
QMV_DEV void dma16(const void *src, uint8_t *chunk) {
    __builtin_amdgcn_global_load_lds(src, (lds_void *)chunk, 16, 0, 0);
}
// 4 bytes per lane into LDS at chunk + 4 * lane.
QMV_DEV void dma4(const void *src, uint8_t *chunk) {
    __builtin_amdgcn_global_load_lds(src, (lds_void *)chunk, 4, 0, 0);
}

// Raw codes of one thread's share of a stage's weight tile (in-kernel expansion): NW
// consecutive weights of one row.
template <int NW> struct Raw;
template <> struct Raw<16> { uint4 ql, qh; int sc; };
template <> struct Raw<8> { uint2 ql, qh; int sc; };
template <> struct Raw<4> { uint32_t ql, qh; int sc; };

// Workgroup: 8 * KSPLIT waves.  Wave w computes MFMA tile (row group w & 1, token group
// (w >> 1) & 3) of the 64 x 128 workgroup tile, over the 32-blocks of its K part
// kh = w >> 3 (block b of a stage when b % KSPLIT == kh).  A stage holds KB 32-blocks.
template <int KSPLIT, int KB>
struct Lay {
    static constexpr int WAVES = 8 * KSPLIT, THREADS = 64 * WAVES;
    static constexpr int KS = 32 * KB;                        // k per stage
    static constexpr int A = 0;                               // [row group 2][block KB][h, l][64][16 B]
    static constexpr int B = A + 2 * KB * 2048;               // [token group 4][block KB][64][16 B]
    static constexpr int XS = B + 4 * KB * 1024;              // [block KB][128 tokens] fp32
    static constexpr int STAGE = XS + KB * 512;
    static constexpr int RING = NSTAGE * STAGE;
    static constexpr int NA = 4 * KB, NB = 4 * KB, NX = 2 * KB;  // direct-load jobs per stage
    static constexpr int NW = 16 * 2 * KB * 64 / THREADS;     // weights each thread expands
};

// FA: the activations are in the quantizer's GEMM layout (xq in fragment order, xs
// [k/32][tokens rounded up to 128]), so every activation chunk and a stage's scales are each
// one contiguous 1 KiB load; otherwise they are read from row-major xq [m][k], xs [m][k/32]
// (32 rows per activation chunk, 64 per scale load).
template <int KSPLIT, int KB, bool EXP, bool PARTIALS, bool FA>
__global__ void __launch_bounds__(512 * KSPLIT, 1)
gemm_q6k_kernel(const uint8_t *__restrict__ ql, const uint8_t *__restrict__ qh, const int8_t *__restrict__ scp,
                const uint16_t *__restrict__ dp, const int8_t *__restrict__ plane, const int8_t *__restrict__ xq,
                const float *__restrict__ xs, float *__restrict__ y, int32_t *__restrict__ part, int M, int N, int K) {
    using L = Lay<KSPLIT, KB>;
    constexpr int WAVES = L::WAVES, NW = L::NW, KS = L::KS;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches, scalar offsets
    const int rg = wave & 1, tg = (wave >> 1) & 3, kh = wave >> 3;
    const int li = lane & 31, lg = lane >> 5;
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
    const int nst = K / KS, nblk = K >> 5, nsb = K >> 8, G = (N + 31) >> 5;

    // ---- this wave's direct loads of a stage: D16 chunks of 16 bytes per lane (weight chunks
    // with EXP, then activation chunks; waves past their number repeat one, the same bytes to
    // the same LDS address) and, on the first NX waves, one word per lane of activation
    // scales (unless PARTIALS: each such load touches 64 rows, so they are not repeated).
    // Sources are for stage 0.
    constexpr int N16 = (EXP ? L::NA : 0) + L::NB;
    constexpr int D16 = (N16 + WAVES - 1) / WAVES;
    const bool has_x = !PARTIALS && wave < (FA ? 1 : L::NX);  // wave-uniform
    const int8_t *src16[D16];
    int lds16[D16], step16[D16];
#pragma unroll
    for (int i = 0; i < D16; i++) {
        const int j = (wave + i * WAVES) % N16;
        if (EXP && j < L::NA) {  // weight chunk [row group][block][h/l]
            const int r = j / (2 * KB), blk = (j >> 1) % KB, p = j & 1;
            const int g = min((n0 >> 5) + r, G - 1);
            src16[i] = plane + ((int64_t)g * nblk + blk) * 2048 + p * 1024 + 16 * lane;
            lds16[i] = L::A + j * 1024;
            step16[i] = KB * 2048;
        } else {  // activation chunk [token group][block]
            const int b = j - (EXP ? L::NA : 0), t = b / KB, blk = b % KB;
            if constexpr (FA) {
                src16[i] = xq + ((int64_t)((m0 >> 5) + t) * nblk + blk) * 1024 + 16 * lane;
                step16[i] = KB * 1024;
            } else {
                const int tk = min(m0 + 32 * t + li, M - 1);
                src16[i] = xq + (int64_t)tk * K + 32 * blk + 16 * lg;
                step16[i] = KS;
            }
            lds16[i] = L::B + b * 1024;
        }
    }
    // activation scales of a stage, [block KB][128 tokens]: with FA one 16-byte load per lane
    // on wave 0 (lane l: block l / 32, tokens 4 (l % 32) ..); else entries 64 jx + lane, one
    // word per lane, on waves jx < NX
    const int mp = (M + BM - 1) / BM * BM;
    const int8_t *srcx = nullptr;
    int ldsx = 0, stepx = 0;
    if constexpr (!PARTIALS) {
        if constexpr (FA) {
            srcx = (const int8_t *)(xs + (int64_t)(lane >> 5) * mp + m0 + 4 * (lane & 31));
            ldsx = L::XS;
            stepx = KB * mp * 4;
        } else {
            const int jx = wave % L::NX, e = 64 * jx + lane;
            srcx = (const int8_t *)(xs + (int64_t)min(m0 + (e & 127), M - 1) * nblk + (e >> 7));
            ldsx = L::XS + 256 * jx;
            stepx = KB * 4;
        }
    }
    auto dma = [&](int st, int buf) {
        uint8_t *s = smem + buf * L::STAGE;
#pragma unroll
        for (int i = 0; i < D16; i++) dma16(src16[i] + (int64_t)st * step16[i], s + lds16[i]);
        if (has_x) {
            if constexpr (FA) dma16(srcx + (int64_t)st * stepx, s + ldsx);
            else dma4(srcx + (int64_t)st * stepx, s + ldsx);
        }
    };

    // ---- in-kernel expansion role (no EXP): lane chunk eu of the stage's weight tile
    // ([row group][block] x 64 lanes), NW weights from sub-offset esub
    constexpr int TPC = 16 / NW;  // threads per lane chunk
    const int eu = tid / TPC, esub = NW * (tid % TPC);
    const int ea = eu >> 6, el = eu & 63;  // chunk [row group ea / KB][block ea % KB]
    const int erg = ea / KB, eblk = ea % KB;
    const int erow = min(n0 + 32 * erg + (el & 31), N - 1);
    const int ek = 16 * (el >> 5) + esub;  // k within the block
    auto load_raw = [&](int st, Raw<NW> &r) {
        const int kk = KS * st + 32 * eblk + ek;  // k of the first weight
        const int s = kk >> 8, e0 = kk & 255;
        const int h = e0 >> 7, t = (e0 >> 5) & 3, lo = e0 & 31;
        const uint8_t *a = ql + (int64_t)erow * (K >> 1) + 128 * s + 64 * h + 32 * (t & 1) + lo;
        const uint8_t *b = qh + (int64_t)erow * (K >> 2) + 64 * s + 32 * h + lo;
        if constexpr (NW == 16) {
            r.ql = *(const uint4 *)a;
            r.qh = *(const uint4 *)b;
        } else if constexpr (NW == 8) {
            r.ql = *(const uint2 *)a;
            r.qh = *(const uint2 *)b;
        } else {
            r.ql = *(const uint32_t *)a;
            r.qh = *(const uint32_t *)b;
        }
        r.sc = scp[(int64_t)erow * (K >> 4) + 16 * s + (e0 >> 4)];
    };
    auto expand = [&](int st, const Raw<NW> &r, int buf) {
        const int e0 = (KS * st + 32 * eblk + ek) & 255, t = (e0 >> 5) & 3;
        const int sh = 4 * (t >> 1), hs = 2 * t;
        const uint32_t sc16 = (uint32_t)r.sc & 0xFFFFu, c16 = (uint32_t)(-32 * r.sc) & 0xFFFFu;
        const uint32_t sc2 = sc16 | (sc16 << 16), c2 = c16 | (c16 << 16);
        constexpr int ND = NW / 4;
        uint32_t qlw[ND], qhw[ND], hv[ND], lv[ND];
        if constexpr (NW == 16) {
            qlw[0] = r.ql.x; qlw[1] = r.ql.y; qlw[2] = r.ql.z; qlw[3] = r.ql.w;
            qhw[0] = r.qh.x; qhw[1] = r.qh.y; qhw[2] = r.qh.z; qhw[3] = r.qh.w;
        } else if constexpr (NW == 8) {
            qlw[0] = r.ql.x; qlw[1] = r.ql.y;
            qhw[0] = r.qh.x; qhw[1] = r.qh.y;
        } else {
            qlw[0] = r.ql;
            qhw[0] = r.qh;
        }
#pragma unroll
        for (int i = 0; i < ND; i++) {
            const uint32_t q = ((qlw[i] >> sh) & 0x0F0F0F0Fu) | (((qhw[i] >> hs) & 0x03030303u) << 4);
            expand4(q, sc2, c2, hv[i], lv[i]);
        }
        uint8_t *dst = smem + buf * L::STAGE + L::A + ea * 2048 + 16 * el + esub;
        if constexpr (NW == 16) {
            *(uint4 *)dst = make_uint4(hv[0], hv[1], hv[2], hv[3]);
            *(uint4 *)(dst + 1024) = make_uint4(lv[0], lv[1], lv[2], lv[3]);
        } else if constexpr (NW == 8) {
            *(uint2 *)dst = make_uint2(hv[0], hv[1]);
            *(uint2 *)(dst + 1024) = make_uint2(lv[0], lv[1]);
        } else {
            *(uint32_t *)dst = hv[0];
            *(uint32_t *)(dst + 1024) = lv[0];
        }
    };

    // ---- the workgroup's d values, [super-block][64 rows] fp16, staged once (an array of its
    // own: its reads need not wait for the direct loads into the ring)
    __shared__ __attribute__((aligned(16))) uint16_t sd[MAXSB * BN];
    for (int i = tid; i < BN * nsb; i += L::THREADS) {
        const int r = i / nsb, s = i - r * nsb;
        sd[s * BN + r] = dp[(int64_t)min(n0 + r, N - 1) * nsb + s];
    }

    // ---- the pipelined contraction: this wave's one 32 x 32 tile.  Two blocks are in flight:
    // at the wave's block j it reads j's fragments, issues the L product of block j - 1 (whose
    // H product was issued a stage earlier), forms the epilogue of block j - 2 (whose L product
    // was issued a stage earlier), and issues the H product of block j.  Every matrix result
    // is read one barrier interval after it was issued.
    float acc[16], Y[16];
    v16i Hs = {};       // H product of block j - 1
    v16i I2 = {};       // I32 of block j - 2
    v4i aLp = {}, bp = {};
    float x1 = 0.f, x2 = 0.f;  // activation scales of blocks j - 1 and j - 2
#pragma unroll
    for (int v = 0; v < 16; v++) { acc[v] = 0.f; Y[v] = 0.f; }
    const int tok = m0 + 32 * tg + li;

    // epilogue of block c: `first` when it starts a super-block (acc = ...); dsb >= 0 when
    // it ends super-block dsb (then Y += d acc)
    auto finish = [&](const v16i &I, float xv, bool first, int c, int dsb) {
        if constexpr (PARTIALS) {
            if (c < 0) return;
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int n = n0 + 32 * rg + 8 * (v >> 2) + 4 * lg + (v & 3);
                if (tok < M && n < N) part[((int64_t)tok * N + n) * nblk + c] = I[v];
            }
        } else {
#pragma unroll
            for (int v = 0; v < 16; v++) acc[v] = first ? (float)I[v] * xv : fmaf((float)I[v], xv, acc[v]);
            pin16(acc);
            if (dsb >= 0) {
                // the wave's 16 d values (rows 32 rg + 8 q + 4 lg + e).  Read in one asm block
                // that also waits for them: compiled LDS reads here would be made to wait for
                // every direct load in flight (the compiler cannot tell the table apart from
                // the ring they fill)
                const uint32_t da = (uint32_t)(uintptr_t)(sd + dsb * BN + 32 * rg + 4 * lg);
                uint2 d4[4];
                asm volatile(
                    "ds_read_b64 %0, %4\n\t"
                    "ds_read_b64 %1, %4 offset:16\n\t"
                    "ds_read_b64 %2, %4 offset:32\n\t"
                    "ds_read_b64 %3, %4 offset:48\n\t"
                    "s_waitcnt lgkmcnt(0)"
                    : "=&v"(d4[0]), "=&v"(d4[1]), "=&v"(d4[2]), "=&v"(d4[3])
                    : "v"(da)
                    : "memory");
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const uint2 dd = d4[q];
                    Y[4 * q + 0] = fmaf(h2f((uint16_t)dd.x), acc[4 * q + 0], Y[4 * q + 0]);
                    Y[4 * q + 1] = fmaf(h2f((uint16_t)(dd.x >> 16)), acc[4 * q + 1], Y[4 * q + 1]);
                    Y[4 * q + 2] = fmaf(h2f((uint16_t)dd.y), acc[4 * q + 2], Y[4 * q + 2]);
                    Y[4 * q + 3] = fmaf(h2f((uint16_t)(dd.y >> 16)), acc[4 * q + 3], Y[4 * q + 3]);
                }
                pin16(Y);
            }
        }
    };

    // the wave's block j (its q-th of super-block S; global block c) in ring slot buf.  Block
    // j - 2 is the first of its super-block when q == 2 and the last when q == 1.
    constexpr int BPS = 8 / KSPLIT;  // the wave's blocks per super-block
    auto block = [&](int buf, int blk, int q, int S, int c) {
        const uint8_t *s = smem + buf * L::STAGE;
        const v4i aH = *(const v4i *)(s + L::A + ((rg * KB + blk) * 2 + 0) * 1024 + 16 * lane);
        const v4i aL = *(const v4i *)(s + L::A + ((rg * KB + blk) * 2 + 1) * 1024 + 16 * lane);
        const v4i b = *(const v4i *)(s + L::B + (tg * KB + blk) * 1024 + 16 * lane);
        const float x = *(const float *)(s + L::XS + (blk * 128 + 32 * tg + li) * 4);
        __builtin_amdgcn_sched_barrier(0);
        const v16i I1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(aLp, bp, Hs << 6, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        finish(I2, x2, q == 2, c - 2 * KSPLIT, q == 1 ? max(S - 1, 0) : (BPS == 2 && q == 0 ? max(S - 1, 0) : -1));
        __builtin_amdgcn_sched_barrier(0);
        const v16i z = {};
        Hs = __builtin_amdgcn_mfma_i32_32x32x32_i8(aH, b, z, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        I2 = I1;
        x2 = x1;
        x1 = x;
        aLp = aL;
        bp = b;
    };

    Raw<NW> raw[2];
    dma(0, 0);
    dma(min(1, nst - 1), 1);
    dma(min(2, nst - 1), 2);
    if constexpr (!EXP) {
        load_raw(0, raw[0]);
        load_raw(min(1, nst - 1), raw[1]);
        expand(0, raw[0], 0);
    }

    // this wave's blocks of a stage: b = kh, kh + KSPLIT, ... < KB; a super-block is SPS stages
    constexpr int SPS = 256 / KS, JPS = KB / KSPLIT;
    static_assert(SPS == NSTAGE, "one ring slot per stage of a super-block");
    static_assert(BPS == JPS * SPS && BPS >= 3, "blocks per super-block");
    for (int S = 0; S < nsb; S++) {
#pragma unroll
        for (int sp = 0; sp < SPS; sp++) {
            const int st = SPS * S + sp, buf = sp;  // slot: compile-time
            // this wave's direct loads of stage st have landed (those of st + 1 and st + 2, issued
            // after them, may still be in flight)
            if (has_x) wait_vmcnt<2 * (D16 + 1)>();
            else wait_vmcnt<2 * D16>();
            ring_barrier();  // ... and every wave's, with the expanded weights of st
            {
                dma(min(st + 3, nst - 1), (sp + 3) % NSTAGE);  // the slot stage st - 1 used
                if constexpr (!EXP) load_raw(min(st + 2, nst - 1), raw[sp & 1]);
            }
#pragma unroll
            for (int j = 0; j < JPS; j++) {
                const int blk = kh + KSPLIT * j;
                block(buf, blk, JPS * sp + j, S, KB * st + blk);
            }
            if constexpr (!EXP) {
                if (st + 1 < nst) expand(st + 1, raw[(sp + 1) & 1], (sp + 1) % NSTAGE);
            }
        }
    }
    // drain: the last block's L product, then the epilogues of the last two blocks
    {
        const int clast = KB * (nst - 1) + kh + KSPLIT * (JPS - 1);
        const v16i I1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(aLp, bp, Hs << 6, 0, 0, 0);
        finish(I2, x2, false, clast - KSPLIT, -1);
        finish(I1, x1, false, clast, nsb - 1);
    }
    wait_vmcnt<0>();  // the clamped prefetches of the last stages still write the ring
    if constexpr (PARTIALS) return;

    if constexpr (KSPLIT == 2) {
        // the two K parts of each tile are added through LDS (fixed order: kh 0 + kh 1)
        lds_barrier();
        float4 *red = (float4 *)smem + ((wave & 7) * 4) * 64 + lane;
        if (kh == 1) {
#pragma unroll
            for (int q = 0; q < 4; q++) red[q * 64] = make_float4(Y[4 * q], Y[4 * q + 1], Y[4 * q + 2], Y[4 * q + 3]);
        }
        lds_barrier();
        if (kh == 1) return;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const float4 o = red[q * 64];
            Y[4 * q] += o.x;
            Y[4 * q + 1] += o.y;
            Y[4 * q + 2] += o.z;
            Y[4 * q + 3] += o.w;
        }
    }
    if (tok >= M) return;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const int n = n0 + 32 * rg + 8 * q + 4 * lg;
        float *dst = y + (int64_t)tok * N + n;
        if (n + 3 < N && (N & 3) == 0) {
            *(float4 *)dst = make_float4(Y[4 * q], Y[4 * q + 1], Y[4 * q + 2], Y[4 * q + 3]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; e++)
                if (n + e < N) dst[e] = Y[4 * q + e];
        }
    }
}

template <int KSPLIT, int KB>
constexpr size_t gemm_lds(int64_t) { return Lay<KSPLIT, KB>::RING; }  // dynamic part (the ring)

template <int KSPLIT, int KB, bool EXP, bool PARTIALS, bool FA>
void launch_tiles(const qmv_weights *w, int m, const int8_t *plane, const int8_t *xq, const float *xs, float *y,
                  int32_t *partials, hipStream_t s) {
    using L = Lay<KSPLIT, KB>;
    const int64_t n = w->n, k = w->k;
    const dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM));
    const size_t lds = gemm_lds<KSPLIT, KB>(k);
    hipLaunchKernelGGL((gemm_q6k_kernel<KSPLIT, KB, EXP, PARTIALS, FA>), grid, dim3(L::THREADS), lds, s,
                       (const uint8_t *)w->codes, (const uint8_t *)w->codes_hi, (const int8_t *)w->scales,
                       (const uint16_t *)w->super, plane, xq, xs, y, partials, m, (int)n, (int)k);
}

template <bool EXP, bool FA>
const char *launch_gemm(const qmv_weights *w, int m, const int8_t *plane, const int8_t *xq, const float *xs,
                        float *y, int32_t *partials, hipStream_t s) {
    if (partials) {
        launch_tiles<1, 2, EXP, true, false>(w, m, plane, xq, xs, y, partials, s);
        return "gemm.q6k.mfma-i8-32x32x32.hl-split.partials";
    }
    // Eight-wave workgroups over all of K when there are tiles for two per CU; else 16-wave
    // workgroups whose two halves take alternate 32-blocks.  The choice never depends on EXP
    // or on the activation layout, so every form sums in the same order (byte-identical
    // outputs).  Test overrides: "gemm.ks1", "gemm.ks2".
    const int64_t tiles = ((w->n + BN - 1) / BN) * ((m + BM - 1) / BM);
    const char *fp = forced_path();
    const bool ks1 = strcmp(fp, "gemm.ks1") == 0 ? true : strcmp(fp, "gemm.ks2") == 0 ? false
                                                     : tiles >= 2 * (int64_t)device_info().num_cus;
    if (ks1) launch_tiles<1, 2, EXP, false, FA>(w, m, plane, xq, xs, y, partials, s);
    else launch_tiles<2, 2, EXP, false, FA>(w, m, plane, xq, xs, y, partials, s);
    return FA ? "gemm.q6k.mfma-i8-32x32x32.hl-split" : "gemm.q6k.mfma-i8-32x32x32.hl-split.rowmajor-act";
}

// Pre-expansion of a q6_K matrix into the plane the EXP kernels load: for every weight,
// w' = sc * (q - 32) = 64 h + l with h = w' >> 6 (arithmetic) and l = w' & 63, in MFMA
// fragment order: [row group ceil(n/32)][32-block k/32][h, l][64 lanes][16 B], lane l
// holding row 32 g + l % 32 and k = 32 c + 16 (l / 32) .. + 15 (rows past n are zero).
// One thread per lane chunk (16 weights).
__global__ void __launch_bounds__(256) expand_q6k_planes(const uint8_t *__restrict__ ql, const uint8_t *__restrict__ qh,
                                                         const int8_t *__restrict__ sc, int8_t *__restrict__ plane,
                                                         int n, int k, int64_t nchunks) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nchunks) return;
    const int l = (int)(i & 63);
    const int64_t gc = i >> 6;
    const int nblk = k >> 5;
    const int64_t g = gc / nblk;
    const int c = (int)(gc - g * nblk);
    const int64_t row = 32 * g + (l & 31);
    uint8_t hb[16], lb[16];
    if (row < n) {
        const int k0 = 32 * c + 16 * (l >> 5), s = k0 >> 8, e0 = k0 & 255;
        const int h = e0 >> 7, t = (e0 >> 5) & 3, lo = e0 & 31;
        const uint8_t *a = ql + row * (k >> 1) + 128 * s + 64 * h + 32 * (t & 1) + lo;
        const uint8_t *b = qh + row * (k >> 2) + 64 * s + 32 * h + lo;
        const int scv = sc[row * (k >> 4) + 16 * s + (e0 >> 4)];
        for (int j = 0; j < 16; j++) {
            const int q = ((a[j] >> (4 * (t >> 1))) & 15) | (((b[j] >> (2 * t)) & 3) << 4);
            const int wv = scv * (q - 32);
            hb[j] = (uint8_t)(wv >> 6);
            lb[j] = (uint8_t)(wv & 63);
        }
    } else {
        for (int j = 0; j < 16; j++) hb[j] = lb[j] = 0;
    }
    int8_t *dst = plane + gc * 2048 + 16 * l;
    for (int j = 0; j < 16; j++) {
        dst[j] = (int8_t)hb[j];
        dst[1024 + j] = (int8_t)lb[j];
    }
}

}  // namespace

int64_t gemm_plane_bytes(int64_t n, int64_t k) { return 2 * ((n + 31) / 32) * 32 * k; }

const char *launch_gemm_q6k(const qmv_weights *w, int m, const int8_t *plane, const int8_t *xq, const float *xs,
                            float *y, int32_t *partials, hipStream_t s, bool frag) {
    const int64_t n = w->n, k = w->k;
    if (n > INT32_MAX - 64 || k > INT32_MAX || (int64_t)m * k > INT32_MAX || (m + BM - 1) / BM > 65535) return nullptr;
    // the workgroup's d values are staged in LDS once: 64 rows x k/256 fp16
    if (k / 256 > MAXSB) return nullptr;
    if (frag && !partials)
        return plane ? launch_gemm<true, true>(w, m, plane, xq, xs, y, nullptr, s)
                     : launch_gemm<false, true>(w, m, nullptr, xq, xs, y, nullptr, s);
    return plane ? launch_gemm<true, false>(w, m, plane, xq, xs, y, partials, s)
                 : launch_gemm<false, false>(w, m, nullptr, xq, xs, y, partials, s);
}

const char *launch_expand_q6k(const qmv_weights *w, int8_t *plane, hipStream_t s) {
    const int64_t nchunks = gemm_plane_bytes(w->n, w->k) / 32;
    if (nchunks > (int64_t)INT32_MAX * 256) return nullptr;
    hipLaunchKernelGGL(expand_q6k_planes, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, s,
                       (const uint8_t *)w->codes, (const uint8_t *)w->codes_hi, (const int8_t *)w->scales, plane,
                       (int)w->n, (int)w->k, nchunks);
    return "plane.q6k.expand";
}

}  // namespace qmv
