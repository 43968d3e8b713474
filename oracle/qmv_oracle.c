/*
 * qmv_oracle.c -- the CPU oracle for the quantized GEMV / GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU library; it is plain, slow, scalar C:
 * every stored code is decoded to an exact integer, every weight is formed as
 * an exact real number from its fp16 / int8 fields (exact in double), and
 * every dot product is accumulated in double in plain k order.
 *
 * Sources followed (the web pages this method comes from):
 *   - "57 · r54 — MINFER_MMQ_Q6K_EXP", §2.1: the q6_K 6-bit value is the low
 *     nibble of ql joined with a 2-bit field of qh shifted up by four, minus 32;
 *     §2.3: that expansion is a pure integer transform (no rounding);
 *     §3.2 / §3.3: a raw q6_K super-block is 210 bytes for 256 weights.
 *   - "Chasing x100", "The kernel is ready": GEMVs are checked against a
 *     bit-faithful CPU reference; the format round trip is exact; the 4-bit
 *     codebook has 16 entries (quality table, "K=16"), the 8-bit one 256
 *     ("K=256"); the 2-bit and 3-bit formats are additive codes.
 *   - "LLMs on the Xiaomi TV Box", §11.5 E18: q4_0 costs 4.5 bits per weight
 *     (an fp16 scale per 32 4-bit codes).
 *   - quantprobe LAWS.md, Law 4: decode is a weight-byte stream (the GEMV).
 * Where the pages leave a layout open, the reading taken is stated at the
 * function that depends on it.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared
 * (no contraction, no fast math: the activation quantizer below must produce
 * the IEEE single-precision results its definition states).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { QO_Q4_0 = 1, QO_Q6_K = 2, QO_CB4 = 3, QO_AQ2X8 = 4, QO_CB8 = 5, QO_AQ3X8 = 6 };
enum { QO_F32 = 0, QO_BF16 = 1 };

/* One weight matrix, n rows (outputs) by k columns (inputs), as host planes.
 *   q4_0 : p0 = qs  u8[n][k/32][16]    p1 = d   f16[n][k/32]
 *   q6_K : p0 = ql  u8[n][k/256][128]  p1 = qh  u8[n][k/256][64]
 *          p2 = sc  i8[n][k/256][16]   p3 = d   f16[n][k/256]
 *   cb4  : p0 = idx u8[n][k/2]         p1 = cb  f16[n][k/128][16]
 *   aq2x8: p0 = codes u8[n][k/8][2]    p1 = cbk f16[2][256][8]   p2 = s f16[n]
 *   cb8  : p0 = idx u8[n][k]           p1 = cb  f16[n][256]
 *   aq3x8: p0 = codes u8[n][k/8][3]    p1 = cbk f16[3][256][8]   p2 = s f16[n]  */
typedef struct {
    int32_t fmt;
    int64_t n, k;
    const void *p0, *p1, *p2, *p3;
} qo_mat;

/* ---------------------------------------------------------------- scalars */

/* IEEE binary16 -> double, written from the format's definition:
 * sign, 5-bit exponent (bias 15), 10-bit fraction, subnormals at exponent 0. */
double qo_f16(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 1024), e - 25);
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double qo_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double act(const void *x, int32_t xt, int64_t i)
{
    if (xt == QO_F32)
        return (double)((const float *)x)[i];
    return qo_bf16(((const uint16_t *)x)[i]);
}

/* ------------------------------------------------------------ code fields */

/* q4_0, reading: block = 16 bytes for 32 weights; byte j carries weight j in
 * its low nibble and weight j+16 in its high nibble. */
int32_t qo_q4_0_code(const qo_mat *m, int64_t row, int64_t col)
{
    const uint8_t *qs = (const uint8_t *)m->p0 + row * (m->k / 2);
    int64_t blk = col / 32, i = col % 32;
    uint8_t byte = qs[blk * 16 + (i % 16)];
    return i < 16 ? (byte & 15) : (byte >> 4);
}

/* q6_K, reading: a 256-weight super-block is two halves of 128; inside a half,
 * weight r (0..127) has quarter t = r/32 and lane l = r%32.  Its low nibble is
 * in ql[64*half + l + 32*(t&1)], low half of the byte for t<2 and high half for
 * t>=2; its two high bits are bits 2t..2t+1 of qh[32*half + l].  The 6-bit
 * value is low | high<<4 (the r54 page's recombination formula). */
int32_t qo_q6k_code(const qo_mat *m, int64_t row, int64_t col)
{
    const uint8_t *ql = (const uint8_t *)m->p0 + row * (m->k / 2);
    const uint8_t *qh = (const uint8_t *)m->p1 + row * (m->k / 4);
    int64_t sb = col / 256, e = col % 256;
    int half = (int)(e / 128), r = (int)(e % 128), t = r / 32, l = r % 32;
    int low = (ql[sb * 128 + 64 * half + l + 32 * (t & 1)] >> (4 * (t >> 1))) & 15;
    int high = (qh[sb * 64 + 32 * half + l] >> (2 * t)) & 3;
    return low | (high << 4);
}

/* 4-bit codebook index, reading: byte i carries index 2i (low nibble) and
 * index 2i+1 (high nibble). */
int32_t qo_cb4_code(const qo_mat *m, int64_t row, int64_t col)
{
    const uint8_t *idx = (const uint8_t *)m->p0 + row * (m->k / 2);
    uint8_t byte = idx[col / 2];
    return (col & 1) ? (byte >> 4) : (byte & 15);
}

/* 8-bit codebook index, reading: one byte per weight, in k order. */
int32_t qo_cb8_code(const qo_mat *m, int64_t row, int64_t col)
{
    return ((const uint8_t *)m->p0)[row * m->k + col];
}

/* Codebooks of an additive code: 2 (2-bit format) or 3 (3-bit format). */
static int aq_books(const qo_mat *m) { return m->fmt == QO_AQ3X8 ? 3 : 2; }

/* Additive codes: each 8-weight group stores one byte per codebook, c1 first. */
int32_t qo_aq_code(const qo_mat *m, int64_t row, int64_t group, int which)
{
    int nb = aq_books(m);
    const uint8_t *c = (const uint8_t *)m->p0 + row * (m->k / 8) * nb;
    return c[group * nb + which];
}

/* --------------------------------------------------------------- weights */

static double f16_at(const void *p, int64_t i) { return qo_f16(((const uint16_t *)p)[i]); }

/* The exact real value of weight (row, col). */
double qo_weight(const qo_mat *m, int64_t row, int64_t col)
{
    switch (m->fmt) {
    case QO_Q4_0: {
        double d = f16_at(m->p1, row * (m->k / 32) + col / 32);
        return d * (double)(qo_q4_0_code(m, row, col) - 8);
    }
    case QO_Q6_K: {
        int64_t nsb = m->k / 256;
        double d = f16_at(m->p3, row * nsb + col / 256);
        int sc = ((const int8_t *)m->p2)[row * nsb * 16 + col / 16];
        return d * (double)sc * (double)(qo_q6k_code(m, row, col) - 32);
    }
    case QO_CB4: {
        int64_t g = row * (m->k / 128) + col / 128;
        return f16_at(m->p1, g * 16 + qo_cb4_code(m, row, col));
    }
    case QO_AQ2X8:
    case QO_AQ3X8: {
        /* weight = s[row] * (sum over codebooks b of C_b[c_b][j]); the sum of two or three
         * fp16 values and the product are exact in double */
        int64_t grp = col / 8, j = col % 8;
        double v = 0.0;
        for (int b = 0; b < aq_books(m); b++)
            v += f16_at(m->p1, (int64_t)b * 2048 + (int64_t)qo_aq_code(m, row, grp, b) * 8 + j);
        return f16_at(m->p2, row) * v;
    }
    case QO_CB8:
        /* reading: one 256-entry codebook per output row */
        return f16_at(m->p1, row * 256 + qo_cb8_code(m, row, col));
    }
    return NAN;
}

/* Dense dequantization: w[row][col] for every weight. */
void qo_dequant(const qo_mat *m, double *w)
{
    for (int64_t r = 0; r < m->n; r++)
        for (int64_t c = 0; c < m->k; c++)
            w[r * m->k + c] = qo_weight(m, r, c);
}

/* Exact integer codes (q4_0 / q6_K / cb4 / cb8 fields) as int32[n][k]. */
void qo_codes(const qo_mat *m, int32_t *out)
{
    for (int64_t r = 0; r < m->n; r++)
        for (int64_t c = 0; c < m->k; c++) {
            int32_t v = -1;
            if (m->fmt == QO_Q4_0) v = qo_q4_0_code(m, r, c);
            if (m->fmt == QO_Q6_K) v = qo_q6k_code(m, r, c);
            if (m->fmt == QO_CB4) v = qo_cb4_code(m, r, c);
            if (m->fmt == QO_CB8) v = qo_cb8_code(m, r, c);
            out[r * m->k + c] = v;
        }
}

/* ------------------------------------------------------------------ GEMV */

/* y[b][row] = sum_k w[row][k] * x[b][k] and bound[b][row] = sum_k |w||x|,
 * both in double, k ascending.  Only the listed rows are computed (rows == NULL
 * means all rows 0..n-1); outputs are indexed [b][i] over the listed rows. */
void qo_gemv_rows(const qo_mat *m, int32_t batch, const void *x, int32_t xt,
                  const int64_t *rows, int64_t nrows, double *y, double *bound,
                  int32_t nthreads)
{
    if (!rows) nrows = m->n;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t i = 0; i < nrows; i++) {
        int64_t row = rows ? rows[i] : i;
        for (int32_t b = 0; b < batch; b++) {
            double s = 0.0, a = 0.0;
            for (int64_t c = 0; c < m->k; c++) {
                double w = qo_weight(m, row, c);
                double v = act(x, xt, (int64_t)b * m->k + c);
                s += w * v;
                a += fabs(w) * fabs(v);
            }
            y[(int64_t)b * nrows + i] = s;
            if (bound) bound[(int64_t)b * nrows + i] = a;
        }
    }
}

void qo_gemv(const qo_mat *m, int32_t batch, const void *x, int32_t xt,
             double *y, double *bound, int32_t nthreads)
{
    qo_gemv_rows(m, batch, x, xt, NULL, 0, y, bound, nthreads);
}

/* SiLU(z) = z / (1 + e^-z). */
double qo_silu(double z) { return z / (1.0 + exp(-z)); }

/* --------------------------------------------------- activation quantizer */

/* Per row, per 32-element block: amax = max |x|, xs = amax / 127 and
 * xq = clamp(round-half-away-from-zero(x / xs), -127, 127), all in IEEE single
 * precision (this file is built without contraction or fast math); an all-zero
 * block gives xs = 0 and xq = 0. */
void qo_quant_act(const float *x, int64_t mrows, int64_t k, int8_t *xq, float *xs)
{
    for (int64_t r = 0; r < mrows; r++)
        for (int64_t c = 0; c < k / 32; c++) {
            const float *v = x + r * k + c * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; i++) {
                float a = fabsf(v[i]);
                if (a > amax) amax = a;
            }
            float scale = amax / 127.0f;
            xs[r * (k / 32) + c] = scale;
            for (int i = 0; i < 32; i++) {
                int q = 0;
                if (amax != 0.0f) {
                    float t = v[i] / scale;
                    float rq = roundf(t);
                    q = (int)rq;
                    if (q > 127) q = 127;
                    if (q < -127) q = -127;
                }
                xq[r * k + c * 32 + i] = (int8_t)q;
            }
        }
}

/* --------------------------------------------------- q6_K int8 contraction */

/* For sampled (m, n) pairs:
 *   P16[s][b] = sum over the 16 weights of sub-block b of (q - 32) * xq
 *   I32[s][c] = sc[2c] * P16[2c] + sc[2c+1] * P16[2c+1]   (32-activation block c)
 * written as int64 [pair][k/16] and [pair][k/32]. */
void qo_q6k_partials(const qo_mat *w, const int8_t *xq, const int64_t *mm, const int64_t *nn,
                     int64_t npairs, int64_t *p16, int64_t *i32)
{
    int64_t k = w->k;
    for (int64_t p = 0; p < npairs; p++) {
        int64_t m = mm[p], n = nn[p];
        const int8_t *sc = (const int8_t *)w->p2 + n * (k / 16);
        for (int64_t b = 0; b < k / 16; b++) {
            int64_t acc = 0;
            for (int64_t i = 0; i < 16; i++) {
                int64_t col = b * 16 + i;
                acc += (int64_t)(qo_q6k_code(w, n, col) - 32) * (int64_t)xq[m * k + col];
            }
            p16[p * (k / 16) + b] = acc;
        }
        for (int64_t c = 0; c < k / 32; c++)
            i32[p * (k / 32) + c] = (int64_t)sc[2 * c] * p16[p * (k / 16) + 2 * c] +
                                    (int64_t)sc[2 * c + 1] * p16[p * (k / 16) + 2 * c + 1];
    }
}

/* y[m][n] = sum over super-blocks s of d[n][s] * sum over c in s of xs[m][c] * I32[m][n][c],
 * in double, for sampled (m, n) pairs; bound = sum_k |w[n][k]| * |xs * xq|. */
void qo_q6k_gemm_pairs(const qo_mat *w, const int8_t *xq, const float *xs,
                       const int64_t *mm, const int64_t *nn, int64_t npairs,
                       double *y, double *bound, int32_t nthreads)
{
    int64_t k = w->k;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t p = 0; p < npairs; p++) {
        int64_t *p16 = (int64_t *)malloc(sizeof(int64_t) * (size_t)(k / 16));
        int64_t *i32 = (int64_t *)malloc(sizeof(int64_t) * (size_t)(k / 32));
        qo_q6k_partials(w, xq, mm + p, nn + p, 1, p16, i32);
        int64_t m = mm[p], n = nn[p];
        double acc = 0.0, bnd = 0.0;
        for (int64_t s = 0; s < k / 256; s++) {
            double d = f16_at(w->p3, n * (k / 256) + s);
            double inner = 0.0;
            for (int64_t c = s * 8; c < s * 8 + 8; c++)
                inner += (double)xs[m * (k / 32) + c] * (double)i32[c];
            acc += d * inner;
        }
        for (int64_t col = 0; col < k; col++)
            bnd += fabs(qo_weight(w, n, col)) *
                   fabs((double)xs[m * (k / 32) + col / 32] * (double)xq[m * k + col]);
        y[p] = acc;
        if (bound) bound[p] = bnd;
        free(p16);
        free(i32);
    }
}

/* ------------------------------------------- q4_0 with int8 activations */

/* The integer-dot form of the q4_0 GEMV (quantprobe LAWS.md, Law 4's per-format
 * amendment, L-15: on the standalone matvec the integer dot product over quantized
 * activations recovers most of what the unpack costs).  The activations are those of
 * the quantizer above (xq, xs per 32); per block b of row n:
 *   I[m][n][b] = sum over the block's 32 columns of (q - 8) * xq   (exact integer)
 *   y[m][n]    = sum_b d[n][b] * xs[m][b] * I[m][n][b]               (double)
 * bound = sum_k |w[n][k]| * |xs * xq|.  Sampled (m, n) pairs, like the GEMM above. */
void qo_q4_0_gemv_q8_pairs(const qo_mat *w, const int8_t *xq, const float *xs,
                           const int64_t *mm, const int64_t *nn, int64_t npairs,
                           double *y, double *bound, int32_t nthreads)
{
    int64_t k = w->k;
#ifdef _OPENMP
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t p = 0; p < npairs; p++) {
        int64_t m = mm[p], n = nn[p];
        double acc = 0.0, bnd = 0.0;
        for (int64_t b = 0; b < k / 32; b++) {
            int64_t isum = 0;
            for (int64_t i = 0; i < 32; i++) {
                int64_t col = b * 32 + i;
                isum += (int64_t)(qo_q4_0_code(w, n, col) - 8) * (int64_t)xq[m * k + col];
            }
            double d = f16_at(w->p1, n * (k / 32) + b);
            acc += d * (double)xs[m * (k / 32) + b] * (double)isum;
        }
        for (int64_t col = 0; col < k; col++)
            bnd += fabs(qo_weight(w, n, col)) *
                   fabs((double)xs[m * (k / 32) + col / 32] * (double)xq[m * k + col]);
        y[p] = acc;
        if (bound) bound[p] = bnd;
    }
}

/* --------------------------------------------------------------- encoders */

/* Pack integer codes [n][k] into the code planes (inverse of the readers above). */
void qo_pack_q4_0(const int32_t *q, int64_t n, int64_t k, uint8_t *qs)
{
    for (int64_t r = 0; r < n; r++)
        for (int64_t b = 0; b < k / 32; b++)
            for (int j = 0; j < 16; j++) {
                int lo = q[r * k + b * 32 + j] & 15, hi = q[r * k + b * 32 + j + 16] & 15;
                qs[r * (k / 2) + b * 16 + j] = (uint8_t)(lo | (hi << 4));
            }
}

void qo_pack_q6k(const int32_t *q, int64_t n, int64_t k, uint8_t *ql, uint8_t *qh)
{
    memset(ql, 0, (size_t)(n * k / 2));
    memset(qh, 0, (size_t)(n * k / 4));
    for (int64_t r = 0; r < n; r++)
        for (int64_t c = 0; c < k; c++) {
            int v = q[r * k + c] & 63;
            int64_t sb = c / 256, e = c % 256;
            int half = (int)(e / 128), rr = (int)(e % 128), t = rr / 32, l = rr % 32;
            ql[r * (k / 2) + sb * 128 + 64 * half + l + 32 * (t & 1)] |= (uint8_t)((v & 15) << (4 * (t >> 1)));
            qh[r * (k / 4) + sb * 64 + 32 * half + l] |= (uint8_t)((v >> 4) << (2 * t));
        }
}

void qo_pack_cb4(const int32_t *q, int64_t n, int64_t k, uint8_t *idx)
{
    for (int64_t r = 0; r < n; r++)
        for (int64_t i = 0; i < k / 2; i++)
            idx[r * (k / 2) + i] = (uint8_t)((q[r * k + 2 * i] & 15) | ((q[r * k + 2 * i + 1] & 15) << 4));
}

/* ------------------------------------------- block (array-of-structs) form */

/* q4_0 blocks of 18 bytes: fp16 d then 16 code bytes. */
void qo_q4_0_to_blocks(const uint8_t *qs, const uint16_t *d, int64_t nblocks, uint8_t *blk)
{
    for (int64_t b = 0; b < nblocks; b++) {
        memcpy(blk + b * 18, d + b, 2);
        memcpy(blk + b * 18 + 2, qs + b * 16, 16);
    }
}

void qo_q4_0_from_blocks(const uint8_t *blk, int64_t nblocks, uint8_t *qs, uint16_t *d)
{
    for (int64_t b = 0; b < nblocks; b++) {
        memcpy(d + b, blk + b * 18, 2);
        memcpy(qs + b * 16, blk + b * 18 + 2, 16);
    }
}

/* q6_K super-blocks of 210 bytes: ql[128], qh[64], sc[16], fp16 d. */
void qo_q6k_to_blocks(const uint8_t *ql, const uint8_t *qh, const int8_t *sc, const uint16_t *d,
                      int64_t nsb, uint8_t *blk)
{
    for (int64_t s = 0; s < nsb; s++) {
        memcpy(blk + s * 210, ql + s * 128, 128);
        memcpy(blk + s * 210 + 128, qh + s * 64, 64);
        memcpy(blk + s * 210 + 192, sc + s * 16, 16);
        memcpy(blk + s * 210 + 208, d + s, 2);
    }
}

void qo_q6k_from_blocks(const uint8_t *blk, int64_t nsb, uint8_t *ql, uint8_t *qh, int8_t *sc, uint16_t *d)
{
    for (int64_t s = 0; s < nsb; s++) {
        memcpy(ql + s * 128, blk + s * 210, 128);
        memcpy(qh + s * 64, blk + s * 210 + 128, 64);
        memcpy(sc + s * 16, blk + s * 210 + 192, 16);
        memcpy(d + s, blk + s * 210 + 208, 2);
    }
}

int32_t qo_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
