/*
 * qgemv.h -- C ABI of the MI355X (gfx950) quantized-GEMV library.
 *
 * Symmetric absmax / absmean quantization of LLM weights and activations to
 * int8, ternary (1.58-bit, packed 2 bits per weight) and "1-bit sign backbone
 * + int8 residual", the packed batch-1 matrix-vector products that decode
 * runs on them, and a W8A8 prefill GEMM with an activation outlier-channel
 * split.
 *
 * Sources cited below (by short tag):
 *   [SEP]  "1-bit quantization is not magic": blog on separated
 *          quantization, m.lqnn.cn/news/241359.
 *   [VG]   "A Visual Guide to LLM Quantization" (Chinese translation),
 *          puppylpg.github.io.
 *   [OVR]  LLM quantization overview, 2048ai.net/68d1f9e38867235e13877cac.html.
 *   [DQ]   news report on ISTA-DASLab's quantization split by inference
 *          phase, ai4snews.wisdomeyes.cn/zh/news/786ff1c6c728dd1806bd2871.
 *   [T158] "1.58 bits vs FP8: what ternary weights actually buy",
 *          feinterview.poetries.top.
 *
 * Conventions (every entry point)
 *   - Pointers are DEVICE pointers unless a parameter says "host".  The caller
 *     allocates and owns every buffer, including workspaces (sized by the
 *     *_workspace_bytes queries).  The library never allocates, never frees
 *     and never synchronizes.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued asynchronously on it; results are valid once the
 *     stream has reached that point.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is launched and an error code is returned.  QG_ERR_HIP
 *     reports a launch failure (hipGetLastError after the launch).
 *   - Matrices are row-major with contiguous rows.  Base pointers that are
 *     streamed must be 16-byte aligned (QG_ERR_ALIGN otherwise).
 *   - Inputs are finite (non-finite inputs are a precondition violation; the
 *     kernels stay in bounds but the codes are unspecified).
 *   - Scales are the quantization MULTIPLIER s = 127 / max|x| ([VG]
 *     'Symmetric quantization', Fig. 17), except the ternary gamma and the
 *     sign-backbone alpha, which are dequantization steps (mean |W|).
 *   - Calls are stateless and may be issued from several host threads.
 *   - Debug mode: with QG_DEBUG=1 in the environment (read at every call),
 *     qg_quantize_absmax_split, qg_gather_columns_bf16 and
 *     qg_qgemm_w8a8_outlier also run device-side checks of the outlier path
 *     after their kernels (the index list as the kernels received it: in
 *     range and strictly increasing; the gathered outlier values, zero codes
 *     at the outlier columns and zero padding), then WAIT for the stream and
 *     return QG_ERR_DEVICE_CHECK if a check failed.  This breaks the
 *     never-synchronizes rule above on purpose, so it cannot be used while
 *     the stream is captured into a graph.  QG_DEBUG=2 runs the same checks
 *     expecting every gathered value with its lowest bit flipped, so that a
 *     correct call with at least one outlier reports QG_ERR_DEVICE_CHECK:
 *     a self-test of the reporting.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t qg_status;
#define QG_OK            0
#define QG_ERR_NULLPTR   1  /* a required pointer is NULL */
#define QG_ERR_SHAPE     2  /* a size is out of range or not a required multiple */
#define QG_ERR_ALIGN     3  /* a streamed pointer is not 16-byte aligned */
#define QG_ERR_ARG       4  /* unsupported format / mode / dtype, or bad index list */
#define QG_ERR_WORKSPACE 5  /* workspace missing or too small */
#define QG_ERR_HIP       6  /* the HIP runtime reported an error at launch */
#define QG_ERR_DEVICE_CHECK 7  /* QG_DEBUG=1 only: a device-side check of the outlier path failed */

/* element types */
#define QG_F32  0
#define QG_BF16 1

/* quantization granularity */
#define QG_PER_TENSOR 0
#define QG_PER_ROW    1

/* weight formats of qg_weight.fmt */
#define QG_WFMT_INT8       0  /* int8 codes [n][k], per-row scale s_w[n]            */
#define QG_WFMT_TERNARY2   1  /* 2-bit packed ternary [n][k/4], per-tensor gamma    */
#define QG_WFMT_SIGN1_RES8 2  /* 1-bit sign [n][k/8] + alpha[n], int8 residual      */
                              /* [n][k] + its own per-row scale s_r[n]              */
#define QG_WFMT_Q4K        3  /* 4-bit codes [n][k/2] in groups of 32 with zero-    */
                              /* points, two-level scales in [n][k/256][16] bytes   */
#define QG_WFMT_SIGN1_RES8Z 4 /* as SIGN1_RES8 with an asymmetric residual: codes   */
                              /* in [-128, 127], s_r[n] and a zero-point z_r[n]     */
#define QG_WFMT_TERNARY3   5  /* ternary, five per byte in base 3 (1.6 bits per     */
                              /* weight), [n][16 ceil(k/80)], per-tensor gamma      */
#define QG_WFMT_INT8_T16   6  /* the codes of QG_WFMT_INT8 in 16-row tiles for the  */
                              /* batch products (qg_pack_tiles16), s_w[n]           */

/* activation modes of qg_qgemv */
#define QG_ACT_INT8  0  /* x is quantized per tensor (absmax int8) inside the call */
#define QG_ACT_FLOAT 1  /* x is used as given (bf16), fp32 accumulation            */

/* limits */
#define QG_MAX_OUTLIERS 256     /* n_out of the outlier split                     */
#define QG_QGEMV_MAX_K  32768   /* k of qg_qgemv (bounded by the on-chip activation staging)  */
#define QG_MAX_GROUP    8       /* matrices per qg_qgemv_grouped launch              */
#define QG_OUT_LD_ALIGN 8       /* row stride (elements) of the outlier operands the
                                   prefill GEMMs read: a multiple of 8 bf16 = 16 B    */
#define QG_MAX_OUT_LD   65536   /* largest row stride of an outlier operand          */
#define QG_SEP_MAX_K    65536   /* k of the thresholded separated format             */
#define QG_BATCH_MAX_M  16      /* tokens of a qg_qgemv_batch launch                 */
#define QG_BATCH_MAX_K  262144  /* k of qg_qgemv_batch                               */
#define QG_MX_BLOCK     32      /* values per MXFP4 block (one E8M0 scale)           */
#define QG_QGEMM_MAX_K  133120  /* k of the W8A8 prefill GEMM: the largest multiple
                                   of 128 with k * 127^2 < 2^31, so that the int32
                                   sums are exact for any codes                      */

/* Human-readable text for a status code (static storage). */
const char* qg_status_str(qg_status s);

/* ABI version: major * 10000 + minor * 100 + patch. */
int32_t qg_abi_version(void);

/*
 * Symmetric absmax int8 quantization ([VG] 'Symmetric quantization', absmax,
 * Fig. 16-18; [OVR] section 3.1 steps 1-3; granularity per [OVR] section 2.3).
 *   alpha = max|x| over the group (a row, or the whole tensor);
 *   s = fl32(127 / alpha)  (IEEE fp32 division; s = 1 when alpha = 0);
 *   q = clip(round_half_even(fl32(x * s)), -127, 127).
 * x      : [rows][cols] of type xt (QG_F32 or QG_BF16), 16-B aligned.
 * q      : [rows][cols] int8 (out), 16-B aligned.
 * s      : [rows] (QG_PER_ROW) or [1] (QG_PER_TENSOR) fp32 (out).
 * ws     : workspace of qg_quantize_absmax_workspace_bytes() bytes (may be
 *          NULL when that is 0).
 * cols % 8 == 0; rows >= 1; cols >= 8.
 */
size_t qg_quantize_absmax_workspace_bytes(int64_t rows, int64_t cols, int32_t gran);
qg_status qg_quantize_absmax(const void* x, int32_t xt, int64_t rows, int64_t cols,
                             int32_t gran, int8_t* q, float* s,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * qg_quantize_absmax without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments (minus ws), checks and results, bit
 * for bit, as qg_quantize_absmax.  QG_PER_TENSOR keeps its partial maxima
 * (at most QG_ABSMAX_SCRATCH_PARTS floats, a bound no size exceeds: the first
 * pass never uses more workgroups) in a file-scope device array of the
 * library, one per device, set up on the first call on each device (the
 * device current at the call must be the stream's).  Every call on a device
 * shares that array; the first pass overwrites every entry the second reads,
 * so no clearing is needed, but calls that overlap on one device race and
 * must be serialized by the caller (one stream, or events).  QG_PER_ROW uses
 * no scratch.  Allocates nothing and calls no allocating routine.
 */
#define QG_ABSMAX_SCRATCH_PARTS 1024
qg_status qg_quantize_absmax_noalloc(const void* x, int32_t xt, int64_t rows, int64_t cols,
                                     int32_t gran, int8_t* q, float* s, void* stream);

/*
 * Activation outlier-channel split with per-token int8 quantization
 * ([SEP] section 2.2: a few channels tens of times larger are taken out and
 * kept in high precision; the rest go to int8; the channel list is found once
 * and cached).  For each row m:
 *   s[m]  = fl32(127 / max_{k not in idx} |x[m][k]|)  (1 when that max is 0);
 *   q[m][k] = clip(rne(fl32(x[m][k] * s[m])), -127, 127) for k not in idx,
 *             0 for k in idx;
 *   x_out[m][j] = x[m][idx[j]]  (bf16, copied bit for bit), j < n_out;
 *   x_out[m][j] = 0 for n_out <= j < x_out_ld (padding).
 * x      : [rows][cols] bf16, 16-B aligned.
 * idx    : HOST array of n_out int32, strictly increasing, in [0, cols)
 *          (QG_ERR_ARG otherwise); n_out in [0, QG_MAX_OUTLIERS]; may be NULL
 *          when n_out = 0.
 * q      : [rows][cols] int8 (out), 16-B aligned.  s: [rows] fp32 (out).
 * x_out  : [rows][x_out_ld] bf16 (out), n_out <= x_out_ld <= QG_MAX_OUT_LD;
 *          not touched (may be NULL) when n_out = 0.  A stride that is a
 *          multiple of QG_OUT_LD_ALIGN (and a 16-B aligned x_out) is what
 *          qg_qgemm_w8a8 reads.
 * cols % 8 == 0; cols <= 262144.
 */
qg_status qg_quantize_absmax_split(const void* x, int64_t rows, int64_t cols,
                                   const int32_t* idx, int32_t n_out,
                                   int8_t* q, float* s, void* x_out, int32_t x_out_ld,
                                   void* stream);

/*
 * Outlier-channel detection, run once on calibration activations ([SEP]
 * section 2.2: a few channels run tens of times larger than the rest; their
 * list is found once and cached).  The pages give no criterion; with a
 * budget of n_out channels:
 *   range[c] = max_m |x[m][c]|;
 *   idx = the n_out channels with the largest range (equal ranges: the lower
 *         channel index first), in ascending channel order -- the list that
 *         qg_quantize_absmax_split and qg_qgemm_w8a8_outlier take (copy it to
 *         the host).
 * x      : [rows][cols] bf16, 16-B aligned; rows >= 1; cols % 8 == 0,
 *          cols <= 262144.
 * n_out  : 0 <= n_out <= min(cols, QG_MAX_OUTLIERS) (QG_ERR_ARG otherwise);
 *          nothing is launched when 0.
 * idx    : [n_out] int32 (out, device).
 * ws     : qg_detect_outliers_workspace_bytes(cols) bytes, 16-B aligned
 *          (per-channel partial ranges; contents on entry do not matter).
 */
size_t qg_detect_outliers_workspace_bytes(int64_t cols);
qg_status qg_detect_outliers(const void* x, int64_t rows, int64_t cols, int32_t n_out,
                             int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * Gather the outlier channels' weights in high precision:
 * w_out[n][j] = bf16_rne(w[n][idx[j]]) ([SEP] section 2.2, high-precision path),
 * j < n_out; w_out[n][j] = 0 for n_out <= j < w_out_ld (padding).
 * w      : [n][k] fp32.   idx: HOST array as in qg_quantize_absmax_split.
 * w_out  : [n][w_out_ld] bf16 (out), n_out <= w_out_ld <= QG_MAX_OUT_LD; not
 *          touched (may be NULL) when n_out = 0.  The prefill GEMMs read a
 *          stride that is a multiple of QG_OUT_LD_ALIGN.
 */
qg_status qg_gather_columns_bf16(const float* w, int64_t n, int64_t k,
                                 const int32_t* idx, int32_t n_out,
                                 void* w_out, int32_t w_out_ld, void* stream);

/*
 * Ternary (BitNet b1.58) absmean quantization of a whole tensor ([VG]
 * 'BitNet b1.58', Fig. 58-60; [OVR] section 5.1):
 *   gamma = the fp32 nearest (ties to even) to the exact mean of |w|
 *           (computed exactly, independent of summation order);
 *   q = clip(rne(fl32(w / gamma)), -1, 1)  (all 0 when gamma = 0).
 * w      : [n][k] fp32, 16-B aligned.
 * q      : [n][k] int8 codes in {-1, 0, 1} (out), 16-B aligned.
 * gamma  : [1] fp32 (out).
 * ws     : qg_ternary_workspace_bytes() bytes, 8-B aligned.
 * n * k % 4 == 0; n * k < 2^39.
 */
size_t qg_ternary_workspace_bytes(int64_t n, int64_t k);
qg_status qg_quantize_ternary(const float* w, int64_t n, int64_t k, int8_t* q,
                              float* gamma, void* ws, size_t ws_bytes, void* stream);

/*
 * Separated quantization: 1-bit sign backbone + int8 residual, per output row
 * ([SEP] section 2.1: W ~ alpha*sign(W) + W_res, W_res = W - alpha*sign(W),
 * residual re-quantized to 8 bits; section 6.3: the residual keeps a scale of
 * its own; sign of a non-negative weight is +1 per [VG] 'BitNet', Fig. 55):
 *   sign[n][k] = +1 if w >= 0 (including -0.0), else -1;
 *   alpha[n]   = fp32 nearest to the exact mean of |w[n][:]|;
 *   R          = fl32(w - alpha[n] * sign);
 *   s_r[n]     = fl32(127 / max|R[n][:]|) (1 when 0);
 *   rq[n][k]   = clip(rne(fl32(R * s_r[n])), -127, 127).
 * w: [n][k] fp32; sign, rq: [n][k] int8 (out); alpha, s_r: [n] fp32 (out).
 * All 16-B aligned; k % 8 == 0; k < 2^31.
 */
qg_status qg_split_sign_residual(const float* w, int64_t n, int64_t k,
                                 int8_t* sign, float* alpha, int8_t* rq, float* s_r,
                                 void* stream);

/*
 * Asymmetric (zero-point) int8 quantization, one scale and zero-point per row
 * ([VG] 'Asymmetric quantization', figs. 22-26, in its multiplier notation;
 * [OVR] section 3 item 2 gives the same map with the reciprocal step).
 * The row's minimum beta and maximum alpha go to the ends of [-128, 127]:
 *   beta = min(min x[r][:], 0), alpha = max(max x[r][:], 0)  (the range is
 *          widened to contain 0, so 0 is exact and z fits in int8);
 *   d = fl32(alpha - beta);  s = fl32(255 / d)  (s = 1 when d = 0);
 *   z = clip(rne(fl32(-128 - fl32(s * beta))), -128, 127);
 *   q = clip(rne(fl32(fl32(x * s) + z)), -128, 127);
 *   dequantized value (q - z) / s.
 * x : [rows][cols] of type xt (QG_F32 or QG_BF16), 16-B aligned.
 * q : [rows][cols] int8 (out), 16-B aligned.  s: [rows] fp32 (out).
 * z : [rows] int8 (out).
 * cols % 8 == 0; rows >= 1; cols >= 8; cols < 2^31.
 */
qg_status qg_quantize_asym(const void* x, int32_t xt, int64_t rows, int64_t cols,
                           int8_t* q, float* s, int8_t* z, void* stream);

/*
 * Sign backbone + asymmetric int8 residual ([SEP] section 6.3: the residual
 * gets its own min / max, scale and zero-point, never the backbone's).
 * sign, alpha and R as in qg_split_sign_residual; then per row
 * (rq, s_r, z_r) = qg_quantize_asym of R.
 * w: [n][k] fp32; sign, rq: [n][k] int8 (out); alpha, s_r: [n] fp32 (out);
 * z_r: [n] int8 (out).  w, sign, rq 16-B aligned; k % 8 == 0; k < 2^31.
 */
qg_status qg_split_sign_residual_zp(const float* w, int64_t n, int64_t k,
                                    int8_t* sign, float* alpha, int8_t* rq, float* s_r,
                                    int8_t* z_r, void* stream);

/*
 * Group-wise 4-bit weights with zero-points and two-level scales ([VG] 'Why
 * Q4_K splits weights into blocks', 'Q4_K uses two-level blocks', figs.
 * 43-46).  Each row is cut along k into super-blocks of 256 = 8 groups of 32.
 * For group j of a super-block (fp32 arithmetic in the order written, round
 * half to even):
 *   scale_j = (max - min) / 15, min_j = min over the group's 32 weights;
 *   d    = fp16(max_j scale_j / 63),   sc_j = clip(rne(scale_j / d), 0, 63);
 *   dmin = fp16(max_j |min_j| / 31),   m_j = clip(rne(min_j / dmin), -31, 31);
 *   S_j = d * sc_j, M_j = dmin * m_j   (sc_j = 0 / m_j = 0 when d / dmin is 0);
 *   q = clip(rne((w - M_j) / S_j), 0, 15)   (0 when S_j = 0);
 *   w_hat = q * S_j + M_j.
 * Storage (144 bytes per 256 weights, 4.5 bits per weight):
 *   codes : [n][k/2] bytes, weight k of a row in byte k/2, low nibble first;
 *   meta  : [n][k/256][16] bytes; bytes 0-11 hold sixteen 6-bit fields,
 *           least significant first (sc_0..sc_7, then m_0+32..m_7+32); bytes
 *           12-13 d and 14-15 dmin as little-endian fp16.
 * w: [n][k] fp32, 16-B aligned; k % 256 == 0, k < 2^31; n * k < 2^40.
 */
qg_status qg_quantize_q4k(const float* w, int64_t n, int64_t k,
                          uint8_t* codes, uint8_t* meta, void* stream);

/*
 * Bit packing of low-bit codes (the storage format behind [SEP] section 3.2's
 * 0.125 byte per sign weight and [VG] 'BitNet b1.58''s log2(3) bits):
 *   bits = 2: field = q + 1 in {0, 1, 2} (q in {-1, 0, 1}), 4 per byte;
 *   bits = 1: field = 1 for q = +1, 0 for q = -1, 8 per byte.
 * Code k of a row is stored in byte k / (8/bits) at bit offset
 * bits * (k % (8/bits)), least significant field first; rows contiguous.
 * codes : [n][k] int8.   packed: [n][k*bits/8] uint8 (out).
 * k % (8 / bits) == 0.  Codes outside the allowed set give unspecified
 * (in-bounds) bytes.
 */
qg_status qg_pack(const int8_t* codes, int64_t n, int64_t k, int32_t bits,
                  uint8_t* packed, void* stream);
/* Inverse of qg_pack (field 3 of a 2-bit code decodes to +2). */
qg_status qg_unpack(const uint8_t* packed, int64_t n, int64_t k, int32_t bits,
                    int8_t* codes, void* stream);

/*
 * Base-3 packing of ternary codes, five per byte ([VG] 'BitNet b1.58': three
 * states carry log2(3) ~ 1.58 bits; 3^5 = 243 <= 256 gives 1.6 bits per
 * weight, against 2 for qg_pack's 2-bit fields).  The pages fix no layout;
 * this library's:
 *   digit f = q + 1 in {0, 1, 2};
 *   byte j of a row holds weights 5j .. 5j+4 as v = sum_i f[5j+i] 3^(4-i)
 *   (first weight = leading digit), stored as t = ceil(256 v / 243), so that
 *   digit i = (3 t_i) >> 8 with t_{i+1} = (3 t_i) & 255;
 *   a row takes qg_base3_row_bytes(k) = 16 * ceil(k / 80) bytes (80 weights
 *   per 16-byte chunk); weights past k are digit 1 (q = 0).
 * codes : [n][k] int8 in {-1, 0, 1} (other values give unspecified bytes).
 * packed: [n][qg_base3_row_bytes(k)] uint8.
 * qg_base3_row_bytes returns 0 for k < 1.
 */
int64_t qg_base3_row_bytes(int64_t k);
qg_status qg_pack_base3(const int8_t* codes, int64_t n, int64_t k, uint8_t* packed, void* stream);
qg_status qg_unpack_base3(const uint8_t* packed, int64_t n, int64_t k, int8_t* codes, void* stream);

/*
 * Int8 codes rearranged for the small-batch products' matrix-core fragments
 * (a layout of this library; the pages fix none).  Rows go in tiles of 16
 * (the last one zero-padded), k in units of 64: tile t, unit c is one
 * contiguous 1 KB block at byte (t * k/64 + c) * 1024, whose bytes
 * 16 L .. 16 L + 15 (L = 16 g + i; g < 4, i < 16) are the codes
 * [16 t + i][64 c + 16 g .. 64 c + 16 g + 15].  Lane L of a wave loads
 * exactly those 16 bytes as its fragment of row i, so one load instruction
 * reads one whole block; with row-major codes the same fragments take 64
 * bytes from each of 16 rows.  Same codes and scales as the row-major
 * matrix: as qg_weight, fmt QG_WFMT_INT8_T16 with codes = the tiled buffer;
 * qg_qgemv_batch, qg_qgemv_batch_grouped and qg_qgemv_batch_ws take it.
 * Results equal the row-major matrix's bit for bit where both run the same
 * kernel, and to fp32 rounding otherwise: with five or more 16-row tiles per
 * CU a launch on tiled codes gives each wave whole tiles, summed over k in
 * another order.
 * codes: [n][k] int8, 16-B aligned;  out: qg_tiles16_bytes(n, k) bytes
 * (16 ceil(n/16) k), 16-B aligned.  k % 128 == 0, k <= QG_BATCH_MAX_K;
 * 1 <= n < 2^31.  qg_tiles16_bytes returns 0 for shapes outside these.
 */
int64_t qg_tiles16_bytes(int64_t n, int64_t k);
qg_status qg_pack_tiles16(const int8_t* codes, int64_t n, int64_t k, int8_t* out, void* stream);

/*
 * A quantized weight matrix, described on the host (the struct lives in host
 * memory; its pointers are device pointers, all 16-B aligned).
 *   QG_WFMT_INT8      : codes = int8 [n][k];           scale = s_w[n]
 *   QG_WFMT_TERNARY2  : codes = packed 2-bit [n][k/4]; scale = &gamma (1 fp32)
 *   QG_WFMT_SIGN1_RES8: codes = packed 1-bit [n][k/8]; resid = int8 [n][k];
 *                       scale = alpha[n]; scale2 = s_r[n]
 *   QG_WFMT_Q4K       : codes = 4-bit plane [n][k/2]; resid = the metadata
 *                       plane [n][k/256][16] (as qg_quantize_q4k writes
 *                       them); scale, scale2 unused (may be NULL)
 *   QG_WFMT_TERNARY3  : codes = base-3 bytes [n][qg_base3_row_bytes(k)];
 *                       scale = &gamma (1 fp32)
 *   QG_WFMT_SIGN1_RES8Z: as SIGN1_RES8 (rq from qg_split_sign_residual_zp);
 *                       zero = z_r[n]
 * zero is read for QG_WFMT_SIGN1_RES8Z only (may be NULL otherwise).
 */
typedef struct qg_weight {
    int32_t fmt;
    int32_t reserved;
    int64_t n, k;
    const void* codes;
    const int8_t* resid;
    const float* scale;
    const float* scale2;
    const int8_t* zero;
} qg_weight;

/*
 * Batch-1 quantized matrix-vector product for decode ([SEP] section 3.1 and
 * [T158]: at batch 1 the time goes into reading the weights once per token;
 * [VG] 'GGUF' block-wise in-kernel dequantization: codes are decoded in
 * registers and used at once, never expanded in memory).
 *
 *   fmt INT8, amode QG_ACT_INT8 (W8A8, [VG] 'Why quantize activations'):
 *       xq, s_x = per-tensor absmax int8 of x (as qg_quantize_absmax);
 *       acc[n] = sum_k codes[n][k] * xq[k] (int32, exact);
 *       y[n] = acc[n] / (s_w[n] * s_x).
 *   fmt INT8, amode QG_ACT_FLOAT (weight-only W8A16):
 *       y[n] = (sum_k codes[n][k] * x[k]) / s_w[n], fp32 accumulation.
 *   fmt TERNARY2, amode QG_ACT_INT8 ([VG] 'BitNet b1.58' Fig. 58-59: +1 adds,
 *       0 skips, -1 subtracts the int8 activation):
 *       acc[n] = sum_k t[n][k] * xq[k] (int32, exact); y[n] = acc[n] * gamma / s_x.
 *   fmt TERNARY3, amode QG_ACT_INT8: the same product on base-3 packed codes.
 *   fmt SIGN1_RES8, amode QG_ACT_FLOAT ([SEP] sections 2.3 and 3.3: backbone
 *       and residual products in one fused kernel, results added):
 *       y[n] = alpha[n] * sum_k sign[n][k] x[k] + (sum_k rq[n][k] x[k]) / s_r[n],
 *       fp32 accumulation.
 *   fmt SIGN1_RES8Z, amode QG_ACT_FLOAT (the residual dequantized as
 *       (rq - z_r) / s_r, [VG] 'Asymmetric quantization', fig. 25):
 *       y[n] = alpha[n] * sum_k sign[n][k] x[k] + (sum_k (rq[n][k] - z_r[n]) x[k]) / s_r[n],
 *       fp32 accumulation of the differences (no z * sum_k x correction).
 *   fmt Q4K, amode QG_ACT_FLOAT (W4A16; the codes and group parameters are
 *       decoded in registers):
 *       y[n] = sum_groups (S_j * sum_{k in j} q[n][k] x[k] + M_j * sum_{k in j} x[k]),
 *       i.e. sum_k w_hat[n][k] x[k], fp32 accumulation; k % 256 == 0.
 * x       : [k] of type xt (QG_F32 or QG_BF16; SIGN1_RES8, SIGN1_RES8Z and Q4K
 *           need QG_BF16).
 * y       : [n] of type yt (QG_F32 or QG_BF16; bf16 is rounded to nearest even).
 * acc_out : [n] int32 raw accumulators (integer modes only); may be NULL.
 * k % 128 == 0, 128 <= k <= QG_QGEMV_MAX_K, n >= 1.
 */
qg_status qg_qgemv(const qg_weight* w, int32_t amode, const void* x, int32_t xt,
                   void* y, int32_t yt, int32_t* acc_out, void* stream);

/*
 * Several batch-1 products that read the same activation vector, in one
 * launch: y[m] = W[m] x for m < count (for example the q, k and v projections
 * of a layer, or its gate and up projections).  Each product follows
 * qg_qgemv's definition exactly and gives bit-identical outputs; a single
 * launch pays the kernel start-up and drain once instead of count times
 * ([SEP] section 3.3: launch overhead is one reason measured speed-ups fall
 * short of the bandwidth model; fusing operators into one kernel recovers it).
 * w       : HOST array of count descriptors; all share fmt and k.
 * y       : HOST array of count device pointers ([w[m].n] of type yt).
 * acc_out : HOST array of count device pointers (each may be NULL), or NULL.
 * count in [1, QG_MAX_GROUP]; other arguments as qg_qgemv.
 */
qg_status qg_qgemv_grouped(const qg_weight* w, int32_t count, int32_t amode, const void* x, int32_t xt,
                           void* const* y, int32_t yt, int32_t* const* acc_out, void* stream);

/*
 * The weight-only int8 products of a whole batch-1 decode step, with the
 * data dependencies between them, in ONE launch ([SEP] section 3.3: the
 * launch overhead of many small operators is one reason measured speed-ups
 * fall short of the bandwidth model ([SEP] section 3.1: decode time is the
 * time to read the weights once); this is the fused-operator remedy applied
 * across the step's products).
 *
 * A stage is 1..QG_MAX_GROUP products that read the same x:
 *     y_m[n] = (sum_k codes_m[n][k] * x[k]) / s_w_m[n]     (m < count)
 * exactly qg_qgemv's QG_WFMT_INT8 / QG_ACT_FLOAT product with bf16 x and
 * bf16 y (fp32 sums in another order, so results agree with qg_qgemv to
 * rounding, not bit for bit; one call's results are deterministic).  x of a
 * stage is read only after every output row of stage `dep` has been written
 * (dep < the stage's index; -1: x is ready when the call starts).  The
 * weights of every stage stream from the start of the call; only x waits.
 * Rules the caller keeps: a stage's y must not be any stage's x other than
 * that of stages depending on it (directly or through other stages), and
 * outputs must not overlap.
 *
 *   qg_chain_plan (host only, no GPU call) validates the stages and writes
 *   the plan IMAGE into host memory (a stage table and one record per slot
 *   of up to 128 rows): image_bytes >= qg_chain_plan_bytes(stages, nstages,
 *   workgroups), 16-B aligned.  `workgroups` is the grid of the launch (one
 *   per CU is what the kernel is sized for).
 *   qg_qgemv_chain runs the step: `image` is that host image, `plan` a
 *   device copy of it (16-B aligned, same bytes; the caller copies it once).
 *   The call updates control words in `plan` and restores them before it
 *   ends, so the same device copy serves any number of calls (and graph
 *   replays); calls that overlap on one plan race.
 *
 * Every wait inside the call is bounded (QG_CHAIN_TIMEOUT_TICKS of the
 * 100 MHz real-time counter).  A wait that runs past it sets bit 0 of the
 * uint32 at byte QG_CHAIN_ERROR_OFFSET of `plan`, the call ends normally
 * with unspecified outputs, and `plan` must be copied from the image again
 * before the next call.  The caller reads that word after the call.
 *
 * Stage: count in [1, QG_MAX_GROUP]; w = HOST array of count QG_WFMT_INT8
 * descriptors sharing k (16-B aligned codes, scale = s_w[n]); y = HOST array
 * of count device pointers (bf16 [w[m].n], 2-B aligned); x bf16 [k], 16-B
 * aligned; k % 128 == 0, QG_CHAIN_MIN_K <= k <= QG_CHAIN_MAX_K; 1 <= n < 2^31.
 * Errors: QG_ERR_ARG (count, dep, fmt, nstages, workgroups, or an image
 * that qg_chain_plan did not write), QG_ERR_SHAPE, QG_ERR_ALIGN,
 * QG_ERR_NULLPTR, QG_ERR_WORKSPACE (image too small).
 */
#define QG_CHAIN_MAX_STAGES    4096
#define QG_CHAIN_MIN_K         128
#define QG_CHAIN_MAX_K         16384
#define QG_CHAIN_ERROR_OFFSET  64
#define QG_CHAIN_TIMEOUT_TICKS 200000000ull   /* 2 s at 100 MHz */
typedef struct qg_chain_stage {
    int32_t count;
    int32_t dep;
    const void* x;
    const qg_weight* w;
    void* const* y;
} qg_chain_stage;
size_t qg_chain_plan_bytes(const qg_chain_stage* stages, int32_t nstages, int32_t workgroups);  /* 0 if invalid */
qg_status qg_chain_plan(const qg_chain_stage* stages, int32_t nstages, int32_t workgroups, void* image,
                        size_t image_bytes);
qg_status qg_qgemv_chain(const void* image, void* plan, void* stream);

/*
 * Weight-only int8 products for a small batch of tokens (decode of m
 * sequences at once; [SEP] section 3.1: at batch 1 every weight is read once
 * per token and the compute idles, so serving several tokens per read of
 * the weights is what batching buys).  For every token t < m:
 *   y[t][n] = (sum_k codes[n][k] * x[t][k]) / s_w[n]
 * i.e. qg_qgemv's INT8 / QG_ACT_FLOAT product of each row of x; the
 * products are exact and summed in fp32 (in another order than qg_qgemv's,
 * so results agree to rounding, not bit for bit).
 * w  : QG_WFMT_INT8 (codes [n][k] int8, scale = s_w[n]) or the same codes in
 *      16-row tiles (QG_WFMT_INT8_T16, qg_pack_tiles16; the same results to
 *      rounding); 16-B aligned codes.  A grouped launch takes one layout for
 *      all matrices.  Results of one call are deterministic; a grouped
 *      launch and the single launches of its matrices may differ by rounding
 *      (the kernel is chosen by the launch's number of tiles).
 * x  : [m][k] bf16 (xt must be QG_BF16), 16-B aligned; 1 <= m <= QG_BATCH_MAX_M.
 * y  : [m][n] of type yt (QG_F32 or QG_BF16, bf16 rounded to nearest even).
 * k % 128 == 0, 128 <= k <= QG_BATCH_MAX_K; 1 <= n < 2^31.
 * m = 1 (with k <= QG_QGEMV_MAX_K, row-major codes) runs qg_qgemv's batch-1
 * kernel.
 * The grouped form runs count (1..QG_MAX_GROUP) matrices that share k, m and
 * x in one launch (q, k and v; gate and up); w and y are HOST arrays of
 * count entries, y[j] holding [m][w[j].n] outputs.
 */
qg_status qg_qgemv_batch(const qg_weight* w, int32_t m, const void* x, int32_t xt, void* y, int32_t yt,
                         void* stream);

/*
 * qg_qgemv_batch with K split over workgroups, for a single matrix of at
 * most (CUs x 16) rows and 8192 <= k <= 16384 (the down projection at the
 * decode shapes): a workgroup takes up to four 16-row tiles and a quarter of
 * k, so it reads each activation row once for all its tiles instead of once
 * per tile.  Same definition as qg_qgemv_batch; the four partial sums of
 * each output are added in a fixed order (deterministic; rounding differs
 * from qg_qgemv_batch's order).
 * ws       : qg_qgemv_batch_workspace_bytes(n, k, m) bytes, 16-B aligned:
 *            partial tiles and one counter per row block.  The counters must
 *            be zero before the first call (e.g. zero-filled at allocation);
 *            every call leaves them zero.  Calls that overlap on one
 *            workspace race.
 * When that size is 0 (m = 1, more tiles than CUs, k below 8192 -- where the
 * partials' round trips through memory cost more than they save -- or k
 * above 16384) the call is qg_qgemv_batch and ws is not used.  Other arguments and checks as
 * qg_qgemv_batch.
 */
size_t qg_qgemv_batch_workspace_bytes(int64_t n, int64_t k, int32_t m);
qg_status qg_qgemv_batch_ws(const qg_weight* w, int32_t m, const void* x, int32_t xt, void* y, int32_t yt,
                            void* ws, size_t ws_bytes, void* stream);
qg_status qg_qgemv_batch_grouped(const qg_weight* w, int32_t count, int32_t m, const void* x, int32_t xt,
                                 void* const* y, int32_t yt, void* stream);

/*
 * Thresholded separated weights ([SEP] section 2.1: only the weights above a
 * threshold go into the 1-bit backbone, the others into the residual;
 * section 5.2: the threshold is a percentile of |W|, the 70th or 80th;
 * section 3.3: residual entries near zero are dropped and the residual is
 * stored sparse; section 5.3 (sep_linear): sign(W) times a scale on the
 * backbone plus an int8 residual).  Per row n, with m_k = |w[n][k]| and the
 * nearest-rank percentile P(p) = the j-th smallest m_k, j = ceil(p * k / 100):
 *   tau = P(pct_backbone); eps = P(pct_zero) (no zero class if pct_zero = 0);
 *   weight k is backbone if m_k > tau, zero if m_k <= eps, residual otherwise;
 *   alpha[n] = the fp32 nearest to the mean of m_k over the backbone (0 if
 *              the backbone is empty);
 *   s_r[n]   = fl32(127 / max m_k over the residual) (1 if that is 0 or the
 *              residual is empty);
 *   residual code = clip(rne(fl32(w * s_r[n])), -127, 127).
 * Storage:
 *   cls : [n][k/4] bytes; weight k's 2-bit class in byte k/4 at bits
 *         2*(k%4): 0 = backbone, w < 0 (-alpha); 1 = zero; 2 = backbone,
 *         w > 0 (+alpha); 3 = residual;
 *   rv  : [n][rv_ld] int8: row n's residual codes in increasing k, then
 *         zeros; rv_ld >= qg_sep_resid_ld(k, pct_zero), a multiple of 16.
 * w: [n][k] fp32; alpha, s_r: [n] fp32 (out).  1 <= pct_backbone <= 100,
 * 0 <= pct_zero <= pct_backbone; k % 128 == 0, 128 <= k <= QG_SEP_MAX_K;
 * 1 <= n, n * k < 2^40; w, cls, rv 16-B aligned.
 * qg_sep_resid_ld returns the smallest valid rv_ld (the residual count of a
 * row is at most k - j(pct_zero), rounded up to 16), or 0 for invalid
 * arguments.
 */
int64_t qg_sep_resid_ld(int64_t k, int32_t pct_zero);
qg_status qg_split_sep_threshold(const float* w, int64_t n, int64_t k, int32_t pct_backbone, int32_t pct_zero,
                                 uint8_t* cls, int8_t* rv, int64_t rv_ld, float* alpha, float* s_r,
                                 void* stream);

/*
 * Batch-1 product on thresholded separated weights with int8 activations
 * ([SEP] section 5.3: the backbone and residual products are computed and
 * added, here in one kernel; the residual product is an int8 product):
 *   xq, s_x  = per-tensor absmax int8 of x (as qg_quantize_absmax);
 *   acc_b[n] = sum over the backbone weights of sign(w) * xq[k]  (int32, exact);
 *   acc_r[n] = sum over the residual weights of code * xq[k]     (int32, exact);
 *   y[n]     = (alpha[n] * acc_b[n] + acc_r[n] / s_r[n]) / s_x  (fp32).
 * skip_residual != 0 is [SEP] section 3.3's fast path: y[n] = alpha[n] *
 * acc_b[n] / s_x; rv and s_r are not read (may be NULL) and acc_r is 0.
 * x: [k] of type xt (QG_F32 or QG_BF16), 16-B aligned.  y: [n] fp32 (out).
 * acc_out: [2][n] int32 (acc_b, then acc_r) or NULL.
 * 16 <= rv_ld <= k, rv_ld % 16 == 0; other sizes as qg_split_sep_threshold.
 */
qg_status qg_qgemv_sep(const uint8_t* cls, const int8_t* rv, int64_t rv_ld, const float* alpha,
                       const float* s_r, int64_t n, int64_t k, const void* x, int32_t xt,
                       int32_t skip_residual, float* y, int32_t* acc_out, void* stream);

/*
 * qg_qgemv_sep for 1..QG_MAX_GROUP matrices that read the same x, in one
 * launch ([SEP] section 3.3: the launch overhead of many small operators is
 * one reason measured speed-ups fall short of the bandwidth model; the
 * projections of a layer that share an input, such as q, k, v, are one
 * launch).  Matrix m holds the arrays and outputs of one qg_qgemv_sep call,
 * with the same meaning and limits; k, x, xt and skip_residual are shared.
 * Each y (and acc_out) is exactly what qg_qgemv_sep gives for that matrix
 * alone: every row is computed by the same code in the same order.
 * Outputs must not overlap one another or x.  QG_ERR_ARG for count outside
 * 1..QG_MAX_GROUP; the other errors as qg_qgemv_sep, for the first matrix
 * that fails (nothing is launched then).
 */
typedef struct qg_sep_matrix {
    const uint8_t* cls;   /* [n][k/4] classes                              */
    const int8_t* rv;     /* [n][rv_ld] residual codes (unused when skipping) */
    int64_t rv_ld;
    const float* alpha;   /* [n]                                           */
    const float* s_r;     /* [n] (unused when skipping)                    */
    int64_t n;
    float* y;             /* [n] fp32 (out)                                */
    int32_t* acc_out;     /* [2][n] int32 (out) or NULL                    */
} qg_sep_matrix;
qg_status qg_qgemv_sep_grouped(const qg_sep_matrix* m, int32_t count, int64_t k, const void* x, int32_t xt,
                               int32_t skip_residual, void* stream);

/*
 * MXFP4 block-scaled 4-bit floats for the format-separated prefill ([DQ]:
 * "format separation" runs the prefill on the accelerator's native low-bit
 * compute -- NVFP4 on the hardware it measures -- while decode keeps a
 * low-bit weight-only format).  MI355X's matrix cores take OCP MXFP4 natively:
 *   a block is QG_MX_BLOCK consecutive values of a row (along K);
 *   e = floor(log2 max|v|) - 2 of the block, clamped to [-127, 127] (0 for an
 *       all-zero block), stored as the E8M0 byte e + 127;
 *   element = the E2M1 value (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes
 *       0..7) nearest to v / 2^e, ties to the even code, saturating at 6;
 *       bit 3 is the sign, set for v < 0.
 * Storage (cols % 256 == 0): codes [rows][cols/2] bytes, element 2j in the
 * low nibble of byte j; scales [cols/256][rows][8] bytes: the 8 block scales
 * of 256 consecutive values of a row together, and those of all rows for
 * one 256-slice of the columns together (the slices the GEMM stages).
 *
 * qg_quantize_mxfp4: x [rows][cols] of type xt (QG_F32 or QG_BF16);
 *   cols % 256 == 0; rows >= 1; x and codes 16-B aligned.
 * qg_gemm_mxfp4: Y[m][n] = sum_k A[m][k] * B[n][k] over the decoded values,
 *   products exact, fp32 sums.  a, b: codes of [m][k] and [n][k]; as, bs
 *   their scales; y [m][n] fp32.  k % 256 == 0, 256 <= k <= 262144;
 *   1 <= m, n < 2^31, m * k and n * k <= 2^40; code and scale pointers
 *   16-B aligned.
 * qg_prefill_mxfp4: the format-separated prefill of activations x [m][k]
 *   bf16 against MXFP4 weights: qg_quantize_mxfp4 of x into the workspace
 *   (qg_prefill_mxfp4_workspace_bytes(m, k) bytes, 16-B aligned; its
 *   contents on entry do not matter), then qg_gemm_mxfp4.
 */
qg_status qg_quantize_mxfp4(const void* x, int32_t xt, int64_t rows, int64_t cols, uint8_t* codes,
                            uint8_t* scales, void* stream);
qg_status qg_gemm_mxfp4(const uint8_t* a, const uint8_t* a_scales, int64_t m, int64_t k, const uint8_t* b,
                        const uint8_t* b_scales, int64_t n, float* y, void* stream);
size_t qg_prefill_mxfp4_workspace_bytes(int64_t m, int64_t k);
qg_status qg_prefill_mxfp4(const void* x, int64_t m, int64_t k, const uint8_t* w, const uint8_t* w_scales,
                           int64_t n, float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * W8A8 prefill GEMM with the outlier-channel split ([SEP] section 2.2: outlier
 * channels in high precision, the rest int8, contributions summed; [T158]:
 * prefill is compute-bound, so the int8 part runs on the matrix cores).
 *   (xq, s_x, x_out) = qg_quantize_absmax_split(x, idx);
 *   acc[m][n] = sum_k xq[m][k] * wq[n][k]            (int32, exact);
 *   y[m][n]   = acc[m][n] / (s_x[m] * s_w[n])
 *             + sum_j x_out[m][j] * w_out[n][j]      (fp32).
 * x      : [m][k] bf16.   idx: HOST int32 list as in qg_quantize_absmax_split.
 * wq     : [n][k] int8 (per-row absmax codes of W, from qg_quantize_absmax).
 * s_w    : [n] fp32.
 * w_out  : [n][w_out_ld] bf16 (qg_gather_columns_bf16), 16-B aligned;
 *          w_out_ld a multiple of QG_OUT_LD_ALIGN, n_out <= w_out_ld <=
 *          QG_MAX_OUT_LD; columns >= n_out are never read.  Ignored (may be
 *          NULL) when n_out = 0.
 * y      : [m][n] fp32 (out).   acc_out: [m][n] int32 (out) or NULL.
 * ws     : qg_qgemm_workspace_bytes(m, k, n_out) bytes, 16-B aligned: the
 *          call's scratch for (xq, s_x, x_out); its contents on entry do not
 *          matter and are overwritten.
 * k % 128 == 0, k <= QG_QGEMM_MAX_K; 1 <= m, n < 2^31; m * k and n * k <= 2^40.
 */
size_t qg_qgemm_workspace_bytes(int64_t m, int64_t k, int32_t n_out);  /* 0 if out of range */
qg_status qg_qgemm_w8a8_outlier(const void* x, int64_t m, int64_t k,
                                const int32_t* idx, int32_t n_out,
                                const int8_t* wq, const float* s_w,
                                const void* w_out, int32_t w_out_ld,
                                int64_t n, float* y, int32_t* acc_out,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * The GEMM half of qg_qgemm_w8a8_outlier on activations that are already
 * split, e.g. one qg_quantize_absmax_split output shared by several
 * projections of the same tokens (q, k, v; gate, up).  Same definition and
 * bit-identical results:
 *   y[m][n] = acc[m][n] / (s_x[m] * s_w[n]) + sum_{j<n_out} x_out[m][j] * w_out[n][j].
 * xq     : [m][k] int8, 16-B aligned.  s_x: [m] fp32.
 * x_out  : [m][x_out_ld] bf16, 16-B aligned; x_out_ld a multiple of
 *          QG_OUT_LD_ALIGN, n_out <= x_out_ld <= QG_MAX_OUT_LD; columns >= n_out
 *          are never read.  Ignored (may be NULL) when n_out = 0.
 * wq, s_w, w_out, w_out_ld, n, y, acc_out, shape limits: as
 * qg_qgemm_w8a8_outlier; 0 <= n_out <= QG_MAX_OUTLIERS.
 */
qg_status qg_qgemm_w8a8(const int8_t* xq, const float* s_x, const void* x_out, int32_t x_out_ld,
                        int64_t m, int64_t k, int32_t n_out,
                        const int8_t* wq, const float* s_w, const void* w_out, int32_t w_out_ld,
                        int64_t n, float* y, int32_t* acc_out, void* stream);

/*
 * Measurement aid, not a step of the method: the streaming-read probe that
 * gives the HBM read rate the qgemv kernels are compared with.  Reads the
 * first qg_probe_stream_read_bytes(bytes, workgroups) bytes of buf (its
 * largest prefix that splits into equal per-workgroup blocks of whole passes
 * of 512 threads x 16 B x 8 loads) exactly once with 128-bit non-temporal
 * loads, the access the weight streams use; computes nothing but an XOR.
 * buf    : device buffer of at least that many bytes, 16-B aligned.
 * sink   : device buffer of workgroups uint32 (practically never written).
 * workgroups in [1, 65535]; each block must stay below 2^31 bytes
 * (QG_ERR_SHAPE otherwise, also when the prefix is empty).
 */
size_t qg_probe_stream_read_bytes(int64_t bytes, int32_t workgroups);
qg_status qg_probe_stream_read(const void* buf, int64_t bytes, int32_t workgroups, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QGEMV_H */
