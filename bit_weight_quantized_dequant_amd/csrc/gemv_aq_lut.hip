// gemv_aq_lut.hip -- additive-code GEMV (2-bit and 3-bit, batch 1) through tables of
// codebook-entry dot products, for gfx950.
//
// Format as in gemv_aq.hip ("Chasing x100", "The kernel is ready": group g of row n holds NC
// 8-bit codes; its 8 weights are s[n] (C_1[c_1] + .. + C_NC[c_NC])).  The row's dot product
// with x regroups as
//     y[n] = s[n] * sum_g sum_b T_b[g][c_b(n, g)],   T_b[g][c] = sum_{j<8} C_b[c][j] x[8g + j],
// so with the tables T in LDS a group costs NC 4-byte lookups and NC adds, instead of NC
// 16-byte codebook-row gathers, eight activation reads and 8 NC multiply-adds ("LLMs on the
// Xiaomi TV Box", §19.1: a lookup kernel over tables of partial dot products that are built
// from the activations, there 16 entries per 4 activations for 1-bit weights).  A table
// holds 256 entries per (codebook, group) and is shared by every row of the matrix: each
// workgroup builds the part it needs, and the more rows it serves the less the build costs
// per row.
//
// Work split: workgroup (slice s, row chunk r) takes GS groups (8 GS weights; GS = 32 for the
// 2-bit code, 16 for the 3-bit one, so that the tables take 64 or 48 KiB of LDS) of 512 rows,
// one row per lane.  It
//   1. issues its loads: the slice's activations, the codebook rows its wave's table entries
//      need, then its rows' code bytes for the slice (NC * GS bytes per row, contiguous,
//      16-byte loads), which stay in flight while the tables are built;
//   2. builds the slice's tables in LDS, fp32 [NC][GS][256], on the matrix cores (one
//      32 x 32 x 16 fp16 product per wave and codebook, see below);
//   3. sums each row's lookups over the slice in group order and stores the partial sum to
//      the workspace, [slice][n].
// A second kernel adds each row's partials in slice order and scales by s[n].  The order of
// every sum is fixed, so the result does not depend on timing; the kernel boundary orders the
// partial stores before their loads.  Workgroups are numbered so that the slices of one row
// chunk run on the same XCD (launch order deals workgroups round-robin over the eight XCDs):
// adjacent slices share cache lines of the code rows.
//
// Measured on MI355X this is slower than the streaming kernel of gemv_aq.hip at the
// 14336 x 4096 and 4096 x 14336 shapes (table build, lookups and the partials' round trip
// together take longer than decoding each group directly), so qmv_gemv keeps that kernel;
// qmv_gemv_ws runs this one.
#include "device_common.h"
#include "qmv_internal.h"

namespace qmv {
namespace {

constexpr int THREADS = 512;

template <int NC>
struct LutShape {
    static constexpr int GS = NC == 2 ? 32 : 16;  // groups per slice: NC * GS * 1 KiB of LDS
};

// Row chunk and slice of this workgroup: consecutive numbers go to one XCD.
QMV_DEV void lut_place(int nsl, int &slice, int &chunk) {
    const int g = gridDim.x, b = blockIdx.x;
    const int l = (g & 7) == 0 ? (b & 7) * (g >> 3) + (b >> 3) : b;
    chunk = l / nsl;
    slice = l - chunk * nsl;
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Sum of the nsl partials of one row, in slice order (slices past nsl add +0).  LD loads one
// partial; 64 loads are issued before the first add.
template <class LD>
QMV_DEV float sum_partials(int nsl, LD ld) {
    float s = 0.f;
    for (int sl = 0; sl < nsl; sl += 64) {
        float p[64];
#pragma unroll
        for (int i = 0; i < 64; i++) p[i] = sl + i < nsl ? ld(sl + i) : 0.f;
#pragma unroll
        for (int i = 0; i < 64; i++) s += p[i];
    }
    return s;
}

template <int NC, int XT>
__global__ void __launch_bounds__(THREADS) aq_lut_kernel(const uint8_t *__restrict__ codes,
                                                         const uint16_t *__restrict__ cbk,
                                                         const void *__restrict__ x, float *__restrict__ part,
                                                         int n, int k) {
    constexpr int GS = LutShape<NC>::GS;
    constexpr int NQ = NC * GS / 16;      // 16-byte code loads per row
    __shared__ float tab[NC * GS * 256];  // [codebook][group][entry]
    const int nsl = k / (8 * GS);
    int slice, chunk;
    lut_place(nsl, slice, chunk);
    const int tid = threadIdx.x, lane = tid & 63, gl = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t k0 = (int64_t)slice * (8 * GS);

    // 1. loads, oldest first: the activations of group lane % 32 of the slice, this wave's
    // codebook rows (entry 32 wave + lane % 32 of each codebook), then the code bytes of this
    // lane's row.  The table build waits for the first two only.
    float xv[8];
    if (gl < GS) {
        ld_act8<XT>(x, k0 + 8 * gl, xv);
    } else {
#pragma unroll
        for (int j = 0; j < 8; j++) xv[j] = 0.f;
    }
    u32x4 cb[NC];
#pragma unroll
    for (int b = 0; b < NC; b++) cb[b] = *((const u32x4 *)cbk + b * 256 + 32 * wave + gl);
    const int row = chunk * THREADS + tid;
    uint32_t cw[4 * NQ];
    {
        const uint8_t *p = codes + ((int64_t)(row < n ? row : n - 1) * (k >> 3) + (int64_t)slice * GS) * NC;
#pragma unroll
        for (int i = 0; i < NQ; i++) {
            const uint4 v = ld_stream16(p + 16 * i);
            cw[4 * i] = v.x;
            cw[4 * i + 1] = v.y;
            cw[4 * i + 2] = v.z;
            cw[4 * i + 3] = v.w;
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. the slice's tables, on the matrix cores.  T_b[g][c] for the wave's 32 entries c and
    // all groups g is one 32 x 32 x 16 fp16 product: A[g][8h + j] = x_h[8g + j], B[8h + j][c] =
    // C_b[c][j], with x (scaled by a power of two 2^e that puts the slice's largest |x| in
    // [2^14, 2^15)) split as x_0 + x_1, x_0 = fp16(x), x_1 = fp16(x - x_0).  fp16 x fp16
    // products are exact in the fp32 accumulator, so the table entry is the fp32 dot product of
    // the codebook row with x to within 2^-22 of each |x| (and 2^-39 of the largest), then
    // scaled back by 2^-e.
    {
        float mx = 0.f;
#pragma unroll
        for (int j = 0; j < 8; j++) mx = fmaxf(mx, fabsf(xv[j]));
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        int ex = 0;
        (void)frexpf(mx, &ex);  // mx in [2^(ex-1), 2^ex)
        const float up = mx > 0.f ? ldexpf(1.f, 15 - ex) : 1.f;
        const float down = mx > 0.f ? ldexpf(1.f, ex - 15) : 1.f;
        f16x8 a;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float f = xv[j] * up;
            const _Float16 h = (_Float16)f;
            a[j] = lane < 32 ? h : (_Float16)(f - (float)h);
        }
        const f32x16 zero = {};
#pragma unroll
        for (int b = 0; b < NC; b++) {
            const f32x16 d = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(f16x8, cb[b]), zero, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < (GS == 32 ? 16 : 8); v++) {
                const int g = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                tab[(b * GS + g) * 256 + 32 * wave + gl] = d[v] * down;
            }
        }
    }
    lds_barrier();

    // 3. the row's lookups over the slice, in group order
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < GS; g++) {
        float t;
#pragma unroll
        for (int b = 0; b < NC; b++) {
            const int bi = NC * g + b;  // byte of code b of group g
            const uint32_t code = (cw[bi >> 2] >> (8 * (bi & 3))) & 0xFFu;
            const float v = tab[(b * GS + g) * 256 + code];
            t = b ? t + v : v;
        }
        acc = g ? acc + t : t;
    }
    if (row < n) part[(int64_t)slice * n + row] = acc;
}

// y[row] = s[row] * (sum of the row's partials in slice order).
__global__ void __launch_bounds__(256) aq_lut_reduce(const float *__restrict__ part, const uint16_t *__restrict__ srow,
                                                     float *__restrict__ y, int n, int nsl) {
    const int row = blockIdx.x * 256 + threadIdx.x;
    if (row >= n) return;
    const float s = sum_partials(nsl, [&](int sl) { return part[(int64_t)sl * n + row]; });
    y[row] = h2f(srow[row]) * s;
}

}  // namespace

int64_t aq_lut_workspace_bytes(const qmv_weights *w, int m) {
    if (m != 1 || (w->fmt != QMV_AQ2X8 && w->fmt != QMV_AQ3X8)) return 0;
    const int gs = w->fmt == QMV_AQ3X8 ? LutShape<3>::GS : LutShape<2>::GS;
    if (w->k % (8 * gs)) return 0;
    return (w->k / (8 * gs)) * w->n * 4;
}

const char *launch_gemv_aq_lut(const qmv_weights *w, const void *x, int xt, float *y, void *ws, hipStream_t s) {
    const int64_t n = w->n, k = w->k;
    const int nc = w->fmt == QMV_AQ3X8 ? 3 : 2;
    const int gs = nc == 2 ? LutShape<2>::GS : LutShape<3>::GS;
    const int64_t nsl = k / (8 * gs), chunks = (n + THREADS - 1) / THREADS;
    if (nsl * chunks > INT32_MAX) return nullptr;
    float *part = (float *)ws;
    const dim3 grid((unsigned)(nsl * chunks));
#define QMV_LUT(NC, XT)                                                                                       \
    hipLaunchKernelGGL((aq_lut_kernel<NC, XT>), grid, dim3(THREADS), 0, s, (const uint8_t *)w->codes,       \
                       (const uint16_t *)w->codebook, x, part, (int)n, (int)k)
    if (nc == 2) {
        if (xt == QMV_F32) QMV_LUT(2, 0);
        else QMV_LUT(2, 1);
    } else {
        if (xt == QMV_F32) QMV_LUT(3, 0);
        else QMV_LUT(3, 1);
    }
#undef QMV_LUT
    hipLaunchKernelGGL(aq_lut_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part,
                       (const uint16_t *)w->scales, y, (int)n, (int)nsl);
    return nc == 2 ? "aq2x8.lut-dot.split-k" : "aq3x8.lut-dot.split-k";
}

}  // namespace qmv
