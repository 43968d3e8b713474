/*
 * qmv.h -- C ABI of libqmv: fused dequantize-and-multiply of block-quantized
 * weights on MI355X (gfx950).
 *
 * The operations (cited by page title and section):
 *   - the batch-1 decode GEMV y = W x over quantized W, a weight-byte stream
 *     whose speed is bytes over bandwidth with a per-format unpack tax
 *     (quantprobe LAWS.md, Law 4 and its L-15 amendment);
 *   - the q6_K prefill GEMM, an int8 contraction of expanded q6_K weights
 *     against per-32 int8 quantized activations ("57 · r54 —
 *     MINFER_MMQ_Q6K_EXP", §2.1 and §2.3);
 *   - the 4-bit 16-entry and 8-bit 256-entry codebook formats and the 2-bit and
 *     3-bit additive formats ("Chasing x100", "The kernel is ready" and the
 *     quality table).
 *
 * Conventions for every call:
 *   - All data pointers are DEVICE pointers unless a comment says otherwise.
 *     The caller allocates and owns every buffer; the library allocates no
 *     device memory and keeps no per-matrix state.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream); all
 *     GPU work is enqueued asynchronously on it.  Kernel faults surface at the
 *     caller's next synchronization.
 *   - Return value: QMV_OK (0) or a negative QMV_ERR_* code.  Arguments are
 *     validated on the host before any HIP call; on a validation error nothing
 *     is enqueued.  No C++ exception crosses this ABI.
 *   - Weight planes are row-major over output rows n, 16-byte aligned, with no
 *     padding between rows (layouts below).  Activations x are row-major
 *     [m][k]; outputs y are fp32 row-major [m][n].
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats. */
enum {
    QMV_Q4_0 = 1,  /* 32 weights per block: 16 code bytes + fp16 d; w = d*(q-8)                  */
    QMV_Q6_K = 2,  /* 256 per super-block: ql 128 B, qh 64 B, 16 int8 sc, fp16 d;
                      w = d*sc[e/16]*(q-32), q = low nibble | 2 high bits << 4                  */
    QMV_CB4 = 3,   /* 4-bit index into a 16-entry fp16 codebook per 128 weights along k         */
    QMV_AQ2X8 = 4, /* per 8 weights two 8-bit codes into two 256x8 fp16 codebooks, summed,
                      times an fp16 per-row scale                                               */
    QMV_CB8 = 5,   /* 8-bit index into a 256-entry fp16 codebook per output row (no block
                      structure; the GEMV and dequant kernels take k % 64 == 0)              */
    QMV_AQ3X8 = 6  /* as AQ2X8 with three codes and three codebooks per 8 weights              */
};

/* Activation element types. */
enum { QMV_F32 = 0, QMV_BF16 = 1 };

/* Status codes. */
enum {
    QMV_OK = 0,
    QMV_ERR_NULL = -1,      /* a required pointer is NULL                                        */
    QMV_ERR_SHAPE = -2,     /* n, k <= 0, or k not a multiple of the format's block (for
                               QMV_CB8 in qmv_validate and the calls that use it: of 64)     */
    QMV_ERR_FORMAT = -3,    /* unknown format, or an operation the format does not support       */
    QMV_ERR_DTYPE = -4,     /* unknown activation dtype                                          */
    QMV_ERR_ALIGN = -5,     /* a plane, x or y pointer is not 16-byte aligned                   */
    QMV_ERR_BATCH = -6,     /* m (batch rows) out of range                                       */
    QMV_ERR_WORKSPACE = -7, /* workspace NULL or smaller than qmm_workspace_bytes()             */
    QMV_ERR_HIP = -8,       /* a HIP call or kernel launch failed                                */
    QMV_ERR_LIMIT = -9      /* a size beyond what the kernels support (see each call)            */
};

#define QMV_MAX_BATCH 8

/*
 * One quantized weight matrix W (n rows = outputs, k columns = inputs).
 *
 *   fmt        codes                    codes_hi            scales               super            codebook
 *   Q4_0       qs u8[n][k/32][16]       NULL                d f16[n][k/32]       NULL             NULL
 *   Q6_K       ql u8[n][k/256][128]     qh u8[n][k/256][64] sc i8[n][k/256][16]  d f16[n][k/256]  NULL
 *   CB4        idx u8[n][k/2]           NULL                NULL                 NULL             cb f16[n][k/128][16]
 *   AQ2X8      codes u8[n][k/8][2]      NULL                s f16[n]             NULL             cbk f16[2][256][8]
 *   CB8        idx u8[n][k]             NULL                NULL                 NULL             cb f16[n][256]
 *   AQ3X8      codes u8[n][k/8][3]      NULL                s f16[n]             NULL             cbk f16[3][256][8]
 *
 * Element order inside the packed planes:
 *   Q4_0 : code byte j of a block holds weight j (bits 0-3) and weight j+16 (bits 4-7).
 *   Q6_K : in a super-block, weight e has half h=e/128, r=e%128, t=r/32, l=r%32; its low
 *          nibble is ql[64h+l+32(t&1)] bits 4(t>>1)..+3 and its high bits are
 *          qh[32h+l] bits 2t..2t+1 ("57 · r54 — MINFER_MMQ_Q6K_EXP", §2.1 recombination).
 *   CB4  : index byte i holds index 2i (bits 0-3) and index 2i+1 (bits 4-7).
 *   AQ2X8: group g of row n stores c1 then c2; weight 8g+j = s[n]*(C1[c1][j]+C2[c2][j]),
 *          C1 = cbk[0], C2 = cbk[1].
 *   CB8  : index byte j of row n holds weight j; weight = cb[n][idx].
 *   AQ3X8: group g stores c1, c2, c3; weight 8g+j = s[n]*(C1[c1][j]+C2[c2][j]+C3[c3][j]).
 * The same matrix stored as raw blocks (18 B per q4_0 block, 210 B per q6_K super-block)
 * has exactly the same bytes; these planes are that array split by field so that every
 * field can be read with aligned 128-bit loads.
 */
typedef struct {
    int32_t fmt;
    int64_t n, k;
    const void *codes;
    const void *codes_hi;
    const void *scales;
    const void *super;
    const void *codebook;
} qmv_weights;

/* Plane selectors for qmv_plane_bytes. */
enum { QMV_PLANE_CODES = 0, QMV_PLANE_CODES_HI = 1, QMV_PLANE_SCALES = 2, QMV_PLANE_SUPER = 3,
       QMV_PLANE_CODEBOOK = 4 };

/* Host only (no HIP call).  Bytes of one plane of an n x k matrix in format fmt
 * (0 for a plane the format does not use), or a negative QMV_ERR_* code.
 * Byte accounting of the stored format: a decode GEMV's time is its bytes over the
 * bandwidth (quantprobe LAWS.md, Law 4), so the plane sizes are the unit every
 * throughput figure is priced in ("57 · r54 — MINFER_MMQ_Q6K_EXP", §2.2: the bytes a
 * plane occupies reconcile exactly with its census). */
int64_t qmv_plane_bytes(int32_t fmt, int64_t n, int64_t k, int32_t plane);

/* Host only.  Sum of qmv_plane_bytes over all planes: the bytes a GEMV must stream
 * (quantprobe LAWS.md, Law 4 and its per-format amendment: scales and codebooks count,
 * the format's metadata density is part of its price).  Negative QMV_ERR_* code for an
 * unknown format (QMV_ERR_FORMAT) or a bad shape (QMV_ERR_SHAPE). */
int64_t qmv_weight_bytes(int32_t fmt, int64_t n, int64_t k);

/* Host only (no HIP call, no dereference of device pointers).  Checks the
 * descriptor for a GEMV with batch m and activation dtype xt: format, shape,
 * required planes non-NULL and 16-byte aligned, 1 <= m <= QMV_MAX_BATCH.
 * Returns QMV_OK or the first failing QMV_ERR_* code (FORMAT, SHAPE, DTYPE, BATCH,
 * NULL, ALIGN, LIMIT, in that order).  Every entry point runs it before launching, so a
 * bad descriptor fails loudly with a code instead of reaching a kernel ("57 · r54 —
 * MINFER_MMQ_Q6K_EXP", §3.1: a failure is explicit and named, never a silent path). */
int qmv_validate(const qmv_weights *w, int32_t m, int32_t xt);

/*
 * Decode GEMV: y[b][i] = sum_j W[i][j] * x[b][j] for b < m (Law 4's weight-byte
 * stream; L-15: the per-format unpack cost is the only other term).
 *   w   : weights (see qmv_weights); x: device [m][k] of dtype xt (QMV_F32 or QMV_BF16),
 *         16-byte aligned; y: device fp32 [m][n], 16-byte aligned.
 *   m   : 1..QMV_MAX_BATCH.  Each weight block is decoded once for all m rows.
 *   Accumulation is fp32; weights are formed exactly from their fields.
 *   Any n < 2^31 and k <= (2^31 - 1) / 8: activations that do not fit one workgroup's
 *   LDS are walked along k in chunks.
 *   Errors: any QMV_ERR_* from qmv_validate; QMV_ERR_NULL for x/y; QMV_ERR_LIMIT when n
 *   or k is beyond those bounds; QMV_ERR_HIP.
 */
int qmv_gemv(const qmv_weights *w, int32_t m, const void *x, int32_t xt, float *y, void *stream);

/*
 * Host only.  Workspace bytes qmv_gemv_ws needs for (w, m): 0 when its kernel for that
 * format and batch needs none (then qmv_gemv_ws is qmv_gemv).  Today only the additive
 * formats at m = 1 need one: one fp32 partial sum per k-slice and row, 4 * n * k / 256 bytes
 * for AQ2X8 (k % 256 == 0) and 4 * n * k / 128 for AQ3X8 (k % 128 == 0); other k need none.
 * Negative QMV_ERR_* code (NULL, FORMAT, SHAPE, BATCH) on a bad descriptor or m.
 */
int64_t qmv_gemv_workspace_bytes(const qmv_weights *w, int32_t m);

/*
 * Decode GEMV with a caller workspace: y as qmv_gemv computes it (fp32 accumulation; the
 * order of the sums differs), by kernels that split k over workgroups.  For the additive
 * formats at m = 1 ("Chasing x100", "The kernel is ready": the 2-bit and 3-bit additive
 * GEMVs; "LLMs on the Xiaomi TV Box", §19.1: a lookup kernel over tables of partial dot
 * products built from the activations): each workgroup builds, in LDS, the fp32 tables
 * T_b[g][c] = sum_j C_b[c][j] x[8g + j] of its k-slice, sums T_b[g][code] over its rows'
 * codes (one 4-byte lookup per code) and stores one partial per row and slice; a second
 * kernel adds each row's partials in slice order (so the result does not depend on timing)
 * and scales by s[n].  On MI355X this is slower than qmv_gemv's kernel at 14336 x 4096 and
 * 4096 x 14336, which is why qmv_gemv does not use it.
 *   w, m, x, xt, y, stream: as qmv_gemv.
 *   ws: device, 16-byte aligned, at least qmv_gemv_workspace_bytes(w, m) bytes (NULL is
 *   accepted when that is 0).  Nothing in it needs to start at zero.  Calls that share a
 *   workspace must be ordered (one stream): overlapping calls race.
 *   Errors: as qmv_gemv; QMV_ERR_WORKSPACE when the workspace is needed and ws is NULL or
 *   ws_bytes is smaller; QMV_ERR_ALIGN when ws is not 16-byte aligned.
 */
int qmv_gemv_ws(const qmv_weights *w, int32_t m, const void *x, int32_t xt, float *y, void *ws, int64_t ws_bytes,
                void *stream);

/*
 * Decode GEMV over per-32 int8 activations (the integer-dot form; quantprobe LAWS.md,
 * Law 4's per-format amendment, L-15: integer dot products over quantized activations
 * recover most of the unpack cost on a standalone matvec).  xq / xs are what
 * qmm_quant_act writes for x, so one quantization serves every GEMV that reads the same
 * activations.  Exact integer block sums, scaled and accumulated in fp32:
 *   q4_0: y[b][i] = sum_c d[i][c] * xs[b][c] * I[b][i][c],
 *         I = sum over the 32 weights of block c of (q - 8) * xq;
 *   q6_K: y[b][i] = sum_s d[i][s] * sum_{c in s} xs[b][c] * I[b][i][c],
 *         I = sum over the two 16-weight sub-blocks j of block c of
 *             sc[i][j] * sum (q - 32) * xq   (the arithmetic of qmm_gemm_q8).
 *   w : QMV_Q4_0 or QMV_Q6_K (QMV_ERR_FORMAT otherwise).
 *   xq: device int8 [m][k]; xs: device fp32 [m][k/32]; y: device fp32 [m][n]; each
 *       16-byte aligned (QMV_ERR_ALIGN).  m: 1..QMV_MAX_BATCH.
 *   Bounds: k <= 16384; the staged activations within one workgroup's LDS, i.e.
 *   40 * (64 * m * ceil(k / 2048) + 1) bytes for q4_0 and 24 * (256 * m * ceil(k / 4096)
 *   + 1) for q6_K (every m * k <= 65536 fits both); n < 2^31.  QMV_ERR_LIMIT otherwise.
 *   Errors: any QMV_ERR_* from qmv_validate; QMV_ERR_NULL; QMV_ERR_HIP.
 */
int qmv_gemv_q8(const qmv_weights *w, int32_t m, const int8_t *xq, const float *xs, float *y, void *stream);

/*
 * Dequantize W to dense fp32 out[n][k] (device).  Every q4_0, q6_K, CB4 and CB8
 * weight is exactly representable in fp32 and is written exactly; additive-code
 * weights are s times the fp32 sum of the codebook entries (exact when the entries
 * are below 1/4 in magnitude), rounded once more by the product.  Used to check the
 * unpack stage alone.
 */
int qmv_dequant(const qmv_weights *w, float *out, void *stream);

/*
 * Per-32 int8 activation quantizer (the q6_K GEMM's activation side):
 * for each row and each 32-element block, xs = max|x| / 127 and
 * xq = clamp(round-half-away-from-zero(x / xs), -127, 127) in IEEE binary32;
 * an all-zero block gives xs = 0, xq = 0.
 *   x: fp32 [m][k]; xq: int8 [m][k]; xs: fp32 [m][k/32]; k % 32 == 0, m >= 1.
 */
int qmm_quant_act(const float *x, int32_t m, int64_t k, int8_t *xq, float *xs, void *stream);

/*
 * Measurement: the stream-read ceiling ("LLMs on the Xiaomi TV Box", §11.5 E10: measure the
 * streaming-read ceiling first; quantprobe LAWS.md, Law 4: decode is bytes over bandwidth).
 * Reads `bytes` bytes at p with the GEMVs' access pattern (128-bit nontemporal loads, one
 * contiguous piece per workgroup) and does nothing else, so its time is the floor for a
 * kernel that reads that many bytes.  Not part of the GEMV or GEMM path.
 *   p: device, 16-byte aligned; bytes: > 0, a multiple of 16 (QMV_ERR_SHAPE otherwise);
 *   sink: device uint32, written only if the XOR of all words read equals 0x9E3779B9
 *   (practically never; it keeps the loads from being removed).
 *   Errors: QMV_ERR_NULL, QMV_ERR_SHAPE, QMV_ERR_ALIGN, QMV_ERR_LIMIT (more than 2^31
 *   workgroups), QMV_ERR_HIP.
 */
int qmv_read_ceiling(const void *p, int64_t bytes, uint32_t *sink, void *stream);

/* Host only.  Workspace bytes qmm_gemm needs for m activation rows: the int8 activations
 * and their per-32 scales in the GEMM's operand layout (with mp = m rounded up to a multiple
 * of 128: xq in int8 MFMA fragment order, [mp/32][k/32][64 lanes][16 B], lane l holding token
 * 32 g + l % 32 and k = 32 c + 16 (l / 32) .. + 15, mp * k bytes; then at a 256-byte aligned
 * offset xs fp32 [k/32][mp]), the activation side of the q6_K int8 contraction ("57 · r54 —
 * MINFER_MMQ_Q6K_EXP", §2.1: the kernel contracts int8 weights against int8 activations).
 * The caller allocates it; the library allocates nothing.  Negative QMV_ERR_* code (NULL,
 * FORMAT for a format other than q6_K, SHAPE, BATCH for m < 1) on a bad descriptor. */
int64_t qmm_workspace_bytes(const qmv_weights *w, int32_t m);

/*
 * q6_K prefill GEMM: y[r][i] = sum_s d[i][s] * sum_{c in s} xs[r][c] * I32[r][i][c],
 * I32[r][i][c] = sum over the 32 weights of activation block c of
 * sc[i][j/16] * (q[i][j] - 32) * xq[r][j], computed exactly in int32 by int8 MFMA,
 * then scaled and accumulated in fp32 ("57 · r54 — MINFER_MMQ_Q6K_EXP", §2.1: the
 * in-kernel ql/qh expansion into centred int8).
 *   w: QMV_Q6_K only; x: fp32 [m][k]; y: fp32 [m][n]; ws: device workspace of at least
 *   qmm_workspace_bytes(w, m) bytes, 256-byte aligned; on return it holds the quantized
 *   activations in the layout qmm_workspace_bytes describes (see qmm_gemm_ws).
 *   Runs qmm_quant_act, then the contraction.  m >= 1 (at most 65535 * 128); k % 256 == 0
 *   and k <= 20480 (each workgroup stages its 64 rows' d values for all of k in LDS beside
 *   a 54 KiB operand ring); QMV_ERR_LIMIT beyond.
 */
int qmm_gemm(const qmv_weights *w, int32_t m, const float *x, float *y, void *ws, int64_t ws_bytes,
             void *stream);

/*
 * qmm_gemm without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The same kernels as qmm_gemm; the quantized activations go to a library-owned device
 * array of QMV_NOALLOC_SCRATCH_BYTES (16 MiB), one per GPU, held until the process ends.
 *   w, m, x, y, stream: as qmm_gemm.  Nothing is allocated.
 *   Limit: qmm_workspace_bytes(w, m) <= QMV_NOALLOC_SCRATCH_BYTES (about 1.125 * m * k bytes;
 *   e.g. m = 512 tokens up to k = 28,928), else QMV_ERR_LIMIT.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one GPU (other
 *   streams or threads) race and must be ordered by the caller.  Nothing in the array needs
 *   to start at zero.
 *   Errors: as qmm_gemm (except QMV_ERR_WORKSPACE); QMV_ERR_HIP when the array's device
 *   address cannot be looked up.
 */
#define QMV_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
int qmm_gemm_noalloc(const qmv_weights *w, int32_t m, const float *x, float *y, void *stream);

/*
 * The contraction of qmm_gemm alone, on the quantized activations a previous qmm_gemm with
 * the same m and k left in ws: one quantization of the activations serves every q6_K weight
 * matrix that multiplies them (the projections of one layer).  ws is read only.
 *   Errors: as qmm_gemm (QMV_ERR_WORKSPACE when ws is NULL or smaller than
 *   qmm_workspace_bytes(w, m)).
 */
int qmm_gemm_ws(const qmv_weights *w, int32_t m, const void *ws, int64_t ws_bytes, float *y, void *stream);

/* The contraction of qmm_gemm alone, on already quantized activations
 * (xq int8 [m][k], xs fp32 [m][k/32]). */
int qmm_gemm_q8(const qmv_weights *w, int32_t m, const int8_t *xq, const float *xs, float *y,
                void *stream);

/* Debug / verification: the exact int32 partials I32[r][i][c] (int32 [m][n][k/32])
 * produced by the same MFMA code path that qmm_gemm_q8 uses. */
int qmm_partials(const qmv_weights *w, int32_t m, const int8_t *xq, int32_t *i32, void *stream);

/*
 * Pre-expanded q6_K planes for the GEMM ("57 · r54 — MINFER_MMQ_Q6K_EXP": a dense
 * int8 plane expanded once at registration so that the GEMM's weight staging is a plain
 * copy, §2.1; the expansion is an integer transform, so results are byte-identical with
 * and without it, §2.3; default on with an explicit "0" opt-out and a label that tells
 * the cases apart, §2.4 and §3.1).
 *
 * The plane: for every weight, w' = sc * (q - 32) = 64 H + L with H in [-64, 64] and L in
 * [0, 63], 2 bytes per weight, laid out in the int8 MFMA's fragment order so that the GEMM
 * loads it straight into LDS: [row group g < ceil(n/32)][32-block c < k/32][H, L][lane 64]
 * [16 bytes], lane l holding row 32 g + l % 32 and k = 32 c + 16 (l / 32) .. + 15 (rows past
 * n hold 0).
 *
 * qmm_plane_bytes: 2 * 32 * ceil(n / 32) * k for a valid QMV_Q6_K descriptor, else a
 *   QMV_ERR_* code.
 * qmm_register_plane: fills `plane` (device memory owned by the caller, at least
 *   qmm_plane_bytes(w) bytes, 256-byte aligned) from w's codes on `stream`, and records it
 *   for w, keyed by w->codes together with n, k and w's other plane pointers.  qmm_gemm,
 *   qmm_gemm_q8 and qmm_partials on w then copy their weight tiles from it.  The plane must
 *   stay allocated and unchanged, and w's codes unchanged, until qmm_unregister_plane(w);
 *   work on other streams must be ordered after the fill by the caller.  With
 *   QMV_Q6K_EXP=0 in the environment nothing is written or recorded and QMV_OK is returned.
 *   Errors: QMV_ERR_NULL, QMV_ERR_FORMAT (not q6_K), QMV_ERR_SHAPE, QMV_ERR_WORKSPACE
 *   (plane_bytes too small), QMV_ERR_ALIGN, QMV_ERR_HIP.  Thread-safe.
 * qmm_unregister_plane: forgets the plane recorded for w->codes (QMV_OK either way).
 * GEMM labels (qmv_last_path): "...hl-split.plane" when the plane is used; "...hl-split"
 *   when none is recorded; "...hl-split(exp=off)" when none is recorded and QMV_Q6K_EXP=0;
 *   "...hl-split(fallback!)" when one is recorded for w->codes with another geometry or
 *   other planes (it is not used; the codes are expanded in the kernel).
 */
int64_t qmm_plane_bytes(const qmv_weights *w);
int qmm_register_plane(const qmv_weights *w, void *plane, int64_t plane_bytes, void *stream);
int qmm_unregister_plane(const qmv_weights *w);

/*
 * Mixture-of-experts FFN over routed experts (batch 1 decode).  Per token only the
 * routed experts' 4-bit codebook weights are streamed, and they dominate the bytes of a
 * decode step ("Chasing x100", the "inversion" paragraph: routed-expert decode on 4-bit
 * codebooks runs near the memory read floor):
 *   for each listed expert e = ids[j]:  h[j] = SiLU(G_e x) * (U_e x),  y[j] = D_e h[j]
 * with SiLU(z) = z / (1 + e^-z).  No routing weights are applied; the caller
 * combines y[j].
 *   gate, up : descriptors of expert 0 (n = d_ff, k = d_model); down: of expert 0
 *              (n = d_model, k = d_ff); all three QMV_CB4 (QMV_ERR_FORMAT otherwise).
 *              Expert e's planes follow expert 0's contiguously:
 *              plane(e) = plane(0) + e * qmv_plane_bytes(...).
 *   n_experts: experts stored; ids: device int32 [n_ids]; ids outside
 *              [0, n_experts) produce NaN rows (their loads are redirected to
 *              expert 0, which stays in bounds; none of those bytes is used).
 *   x : device [d_model] of dtype xt; h: device fp32 [n_ids][d_ff] (written);
 *   y : device fp32 [n_ids][d_model].  1 <= n_ids <= 64.
 *   QMV_ERR_LIMIT when d_model or d_ff exceeds 16384 (an expert row is staged whole in
 *   LDS).
 */
int qmv_moe_ffn(const qmv_weights *gate, const qmv_weights *up, const qmv_weights *down,
                int32_t n_experts, const int32_t *ids, int32_t n_ids, const void *x, int32_t xt,
                float *h, float *y, void *stream);

/* Label of the kernel variant the calling thread's last successful call launched
 * (a thread-local string owned by the library; valid until that thread's next call).
 * With QMV_DEBUG=1 in the environment every call also prints
 * "qmv: <call> fmt=.. n=.. k=.. m=.. path=.." to stderr.  This is the liveness label of
 * "57 · r54 — MINFER_MMQ_Q6K_EXP", §2.4: parity cannot tell a fast path that never ran
 * from one that did, so every launch names its variant and tests and benchmarks count
 * the labels.  Empty before the thread's first successful call; never NULL. */
const char *qmv_last_path(void);

/* Static, library-owned description of a status code ("unknown status" for a code this
 * version does not define); never NULL.  Pairs with the named failure codes above
 * ("57 · r54 — MINFER_MMQ_Q6K_EXP", §3.1: a failure is loud and says what it was). */
const char *qmv_strerror(int code);

/* Library version string (static, library-owned). */
const char *qmv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QMV_H */
