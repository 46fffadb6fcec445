// api.cpp -- the C ABI of include/qgemv.h: host-side argument validation,
// workspace carving and dispatch to the launchers.  Every check runs before
// any HIP call, so invalid arguments are rejected without touching a device.
#include "../../include/qgemv.h"

#include <hip/hip_runtime.h>

#include <string.h>

#include "qg_chain.h"
#include "qg_debug.h"
#include "qg_launch.h"

namespace {

// rows per slot of a chained stage of `rows` rows in total: about one slot
// per workgroup and stage (so that every workgroup works on every stage),
// whole rows for each worker wave, at most kMaxRows
int64_t chain_rows_per_slot(int64_t rows, int32_t workgroups) {
    using namespace qg::chain;
    int64_t r = (rows + (int64_t)workgroups - 1) / (int64_t)workgroups;
    r = (r + kWorkers - 1) / kWorkers * kWorkers;
    return r > kMaxRows ? kMaxRows : r;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline qg_status from_hip(hipError_t e) { return e == hipSuccess ? QG_OK : QG_ERR_HIP; }

// QG_DEBUG=1 in the environment (read at every call): the outlier-path
// calls run the device-side checks of qg_debug.h after their kernels, wait
// for the stream and report a failed check as QG_ERR_DEVICE_CHECK.
// QG_DEBUG=2: the same with the checks' self-test expectation (a correct call
// with outliers reports QG_ERR_DEVICE_CHECK).  0: off.
int debug_mode() {
    const char* e = getenv("QG_DEBUG");
    if (!e || e[1] != 0) return 0;
    return e[0] == '1' ? 1 : e[0] == '2' ? 2 : 0;
}
qg_status debug_result(hipStream_t st) {
    uint32_t flags = 0;
    if (qg::debug_take_flags(st, &flags) != hipSuccess) return QG_ERR_HIP;
    return flags ? QG_ERR_DEVICE_CHECK : QG_OK;
}

// Validates a host index list: strictly increasing, inside [0, cols).
qg_status check_idx(const int32_t* idx, int32_t n_out, int64_t cols, qg::OutlierIdx* out) {
    if (n_out < 0 || n_out > QG_MAX_OUTLIERS) return QG_ERR_ARG;
    if (n_out > 0 && !idx) return QG_ERR_NULLPTR;
    for (int i = 0; i < qg::kMaxOutliers; ++i) out->v[i] = 0;
    for (int32_t j = 0; j < n_out; ++j) {
        if (idx[j] < 0 || idx[j] >= cols) return QG_ERR_ARG;
        if (j > 0 && idx[j] <= idx[j - 1]) return QG_ERR_ARG;
        out->v[j] = idx[j];
    }
    return QG_OK;
}

// Workspace of the prefill call: the split activations xq [m][k] int8 |
// s_x [m] fp32 | x_out [m][ld] bf16 with ld = n_out rounded up to
// QG_OUT_LD_ALIGN, each part 256-B aligned.
int out_ld(int32_t n_out) { return (int)align_up((size_t)n_out, QG_OUT_LD_ALIGN); }
size_t qgemm_layout(int64_t m, int64_t k, int32_t n_out, size_t* off_sx, size_t* off_xo) {
    const size_t xq = (size_t)m * (size_t)k;
    const size_t sx = align_up(xq, 256);
    const size_t xo = align_up(sx + (size_t)m * sizeof(float), 256);
    const size_t total = align_up(xo + (size_t)m * (size_t)out_ld(n_out) * 2, 256);
    if (off_sx) *off_sx = sx;
    if (off_xo) *off_xo = xo;
    return total;
}

// An outlier operand the GEMM reads: [rows][ld] bf16, 16-B aligned rows.
qg_status check_out_operand(const void* p, int32_t ld, int32_t n_out) {
    if (n_out == 0) return QG_OK;
    if (!p) return QG_ERR_NULLPTR;
    if (ld < n_out || ld > QG_MAX_OUT_LD || ld % QG_OUT_LD_ALIGN != 0) return QG_ERR_SHAPE;
    if (!aligned16(p)) return QG_ERR_ALIGN;
    return QG_OK;
}

// Sizes the prefill GEMM supports: K in whole 128-column steps and small
// enough that the int32 sums are exact (K * 127^2 < 2^31), indices of the
// [m][k] / [n][k] operands within 2^40 elements, m and n below 2^31.
qg_status check_gemm_shape(int64_t m, int64_t k, int64_t n) {
    if (m < 1 || n < 1 || m >= ((int64_t)1 << 31) || n >= ((int64_t)1 << 31)) return QG_ERR_SHAPE;
    if (k < 128 || k % 128 != 0 || k > QG_QGEMM_MAX_K) return QG_ERR_SHAPE;
    if (m > ((int64_t)1 << 40) / k || n > ((int64_t)1 << 40) / k) return QG_ERR_SHAPE;
    return QG_OK;
}

}  // namespace

extern "C" {

const char* qg_status_str(qg_status s) {
    switch (s) {
        case QG_OK: return "ok";
        case QG_ERR_NULLPTR: return "a required pointer is NULL";
        case QG_ERR_SHAPE: return "a size is out of range or not a required multiple";
        case QG_ERR_ALIGN: return "a streamed pointer is not 16-byte aligned";
        case QG_ERR_ARG: return "unsupported format/mode/dtype or bad index list";
        case QG_ERR_WORKSPACE: return "workspace missing or too small";
        case QG_ERR_HIP: return "HIP runtime error at launch";
        case QG_ERR_DEVICE_CHECK: return "a QG_DEBUG device-side check of the outlier path failed";
        default: return "unknown status";
    }
}

int32_t qg_abi_version(void) { return 20600; }

size_t qg_quantize_absmax_workspace_bytes(int64_t rows, int64_t cols, int32_t gran) {
    if (gran != QG_PER_TENSOR || rows < 1 || cols < 8) return 0;
    return (size_t)qg::absmax_tensor_parts(rows * cols) * sizeof(float);
}

qg_status qg_quantize_absmax(const void* x, int32_t xt, int64_t rows, int64_t cols, int32_t gran, int8_t* q,
                             float* s, void* ws, size_t ws_bytes, void* stream) {
    if (!x || !q || !s) return QG_ERR_NULLPTR;
    if (xt != QG_F32 && xt != QG_BF16) return QG_ERR_ARG;
    if (gran != QG_PER_TENSOR && gran != QG_PER_ROW) return QG_ERR_ARG;
    if (rows < 1 || cols < 8 || cols % 8 != 0 || rows > ((int64_t)1 << 40) / cols) return QG_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q)) return QG_ERR_ALIGN;
    if (gran == QG_PER_ROW) return from_hip(qg::launch_absmax_rows(x, xt, rows, cols, q, s, as_stream(stream)));
    const size_t need = qg_quantize_absmax_workspace_bytes(rows, cols, gran);
    if (!ws || ws_bytes < need) return QG_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 3u) != 0) return QG_ERR_ALIGN;
    return from_hip(qg::launch_absmax_tensor(x, xt, rows * cols, q, s, static_cast<float*>(ws), as_stream(stream)));
}

qg_status qg_quantize_absmax_noalloc(const void* x, int32_t xt, int64_t rows, int64_t cols, int32_t gran, int8_t* q,
                                     float* s, void* stream) {
    if (!x || !q || !s) return QG_ERR_NULLPTR;
    if (xt != QG_F32 && xt != QG_BF16) return QG_ERR_ARG;
    if (gran != QG_PER_TENSOR && gran != QG_PER_ROW) return QG_ERR_ARG;
    if (rows < 1 || cols < 8 || cols % 8 != 0 || rows > ((int64_t)1 << 40) / cols) return QG_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q)) return QG_ERR_ALIGN;
    if (gran == QG_PER_ROW) return from_hip(qg::launch_absmax_rows(x, xt, rows, cols, q, s, as_stream(stream)));
    static_assert(QG_ABSMAX_SCRATCH_PARTS == qg::kAbsmaxScratchParts, "header and library agree");
    if (qg::absmax_tensor_parts(rows * cols) > QG_ABSMAX_SCRATCH_PARTS) return QG_ERR_WORKSPACE;
    return from_hip(qg::launch_absmax_tensor_noalloc(x, xt, rows * cols, q, s, as_stream(stream)));
}

qg_status qg_quantize_absmax_split(const void* x, int64_t rows, int64_t cols, const int32_t* idx, int32_t n_out,
                                   int8_t* q, float* s, void* x_out, int32_t x_out_ld, void* stream) {
    if (!x || !q || !s) return QG_ERR_NULLPTR;
    if (n_out > 0 && !x_out) return QG_ERR_NULLPTR;
    if (rows < 1 || cols < 8 || cols % 8 != 0 || cols > 262144 || rows > ((int64_t)1 << 40) / cols)
        return QG_ERR_SHAPE;
    if (n_out > 0 && (x_out_ld < n_out || x_out_ld > QG_MAX_OUT_LD)) return QG_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q)) return QG_ERR_ALIGN;
    qg::OutlierIdx oi;
    const qg_status st = check_idx(idx, n_out, cols, &oi);
    if (st != QG_OK) return st;
    const int ld = n_out > 0 ? x_out_ld : 0;
    hipError_t e = qg::launch_absmax_split(static_cast<const uint16_t*>(x), rows, cols, oi, n_out, q, s,
                                           static_cast<uint16_t*>(x_out), ld, as_stream(stream));
    if (e != hipSuccess || !debug_mode()) return from_hip(e);
    e = qg::debug_check_split(static_cast<const uint16_t*>(x), rows, cols, oi, n_out, q,
                              static_cast<const uint16_t*>(x_out), ld, debug_mode() == 2, as_stream(stream));
    return e != hipSuccess ? QG_ERR_HIP : debug_result(as_stream(stream));
}

size_t qg_detect_outliers_workspace_bytes(int64_t cols) {
    if (cols < 1 || cols > 262144) return 0;
    return (size_t)qg::detect_row_blocks(cols) * (size_t)cols * sizeof(uint32_t);
}

qg_status qg_detect_outliers(const void* x, int64_t rows, int64_t cols, int32_t n_out, int32_t* idx, void* ws,
                             size_t ws_bytes, void* stream) {
    if (!x) return QG_ERR_NULLPTR;
    if (rows < 1 || cols < 8 || cols % 8 != 0 || cols > 262144 || rows > ((int64_t)1 << 40) / cols)
        return QG_ERR_SHAPE;
    if (n_out < 0 || n_out > QG_MAX_OUTLIERS || n_out > cols) return QG_ERR_ARG;
    if (n_out == 0) return QG_OK;
    if (!idx) return QG_ERR_NULLPTR;
    if (!aligned16(x)) return QG_ERR_ALIGN;
    if (!ws || ws_bytes < qg_detect_outliers_workspace_bytes(cols)) return QG_ERR_WORKSPACE;
    if (!aligned16(ws)) return QG_ERR_ALIGN;
    return from_hip(qg::launch_detect_outliers(static_cast<const uint16_t*>(x), rows, cols, n_out, idx,
                                               static_cast<uint32_t*>(ws), as_stream(stream)));
}

qg_status qg_gather_columns_bf16(const float* w, int64_t n, int64_t k, const int32_t* idx, int32_t n_out,
                                 void* w_out, int32_t w_out_ld, void* stream) {
    if (!w) return QG_ERR_NULLPTR;
    if (n_out > 0 && !w_out) return QG_ERR_NULLPTR;
    if (n < 1 || k < 1) return QG_ERR_SHAPE;
    if (n_out > 0 && (w_out_ld < n_out || w_out_ld > QG_MAX_OUT_LD)) return QG_ERR_SHAPE;
    qg::OutlierIdx oi;
    const qg_status st = check_idx(idx, n_out, k, &oi);
    if (st != QG_OK) return st;
    hipError_t e = qg::launch_gather_cols_bf16(w, n, k, oi, n_out, static_cast<uint16_t*>(w_out), w_out_ld,
                                               as_stream(stream));
    if (e != hipSuccess || !debug_mode()) return from_hip(e);
    e = qg::debug_check_gather(w, n, k, oi, n_out, static_cast<const uint16_t*>(w_out), w_out_ld,
                               debug_mode() == 2, as_stream(stream));
    return e != hipSuccess ? QG_ERR_HIP : debug_result(as_stream(stream));
}

qg_status qg_quantize_q4k(const float* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* meta, void* stream) {
    if (!w || !codes || !meta) return QG_ERR_NULLPTR;
    if (n < 1 || k < 256 || k % 256 != 0 || k >= ((int64_t)1 << 31) || n > ((int64_t)1 << 40) / k)
        return QG_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(codes) || !aligned16(meta)) return QG_ERR_ALIGN;
    return from_hip(qg::launch_quantize_q4k(w, n, k, codes, meta, as_stream(stream)));
}

// Nearest rank ceil(pct * k / 100) of a percentile (0 for pct = 0).
static int64_t nearest_rank(int32_t pct, int64_t k) { return (pct * k + 99) / 100; }

static qg_status check_sep_shape(int64_t n, int64_t k) {
    if (n < 1 || k < 128 || k % 128 != 0 || k > QG_SEP_MAX_K) return QG_ERR_SHAPE;
    if (n > ((int64_t)1 << 40) / k) return QG_ERR_SHAPE;
    return QG_OK;
}

int64_t qg_sep_resid_ld(int64_t k, int32_t pct_zero) {
    if (k < 1 || k > QG_SEP_MAX_K || pct_zero < 0 || pct_zero > 100) return 0;
    const int64_t ld = (k - nearest_rank(pct_zero, k) + 15) / 16 * 16;
    return ld < 16 ? 16 : ld;
}

qg_status qg_split_sep_threshold(const float* w, int64_t n, int64_t k, int32_t pct_backbone, int32_t pct_zero,
                                 uint8_t* cls, int8_t* rv, int64_t rv_ld, float* alpha, float* s_r, void* stream) {
    if (!w || !cls || !rv || !alpha || !s_r) return QG_ERR_NULLPTR;
    const qg_status sh = check_sep_shape(n, k);
    if (sh != QG_OK) return sh;
    if (pct_backbone < 1 || pct_backbone > 100 || pct_zero < 0 || pct_zero > pct_backbone) return QG_ERR_ARG;
    if (rv_ld % 16 != 0 || rv_ld < qg_sep_resid_ld(k, pct_zero) || rv_ld > k) return QG_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(cls) || !aligned16(rv)) return QG_ERR_ALIGN;
    return from_hip(qg::launch_sep_split(w, n, k, (int)nearest_rank(pct_backbone, k), (int)nearest_rank(pct_zero, k),
                                         cls, rv, rv_ld, alpha, s_r, as_stream(stream)));
}

static qg_status sep_args(const qg_sep_matrix& m, int64_t k, const void* x, int32_t xt, bool skip, qg::SepArgs* a) {
    if (!m.cls || !m.alpha || !x || !m.y || (!skip && (!m.rv || !m.s_r))) return QG_ERR_NULLPTR;
    const qg_status sh = check_sep_shape(m.n, k);
    if (sh != QG_OK) return sh;
    if (m.n >= ((int64_t)1 << 31)) return QG_ERR_SHAPE;
    if (xt != QG_F32 && xt != QG_BF16) return QG_ERR_ARG;
    if (!skip && (m.rv_ld < 16 || m.rv_ld > k || m.rv_ld % 16 != 0)) return QG_ERR_SHAPE;
    if (!aligned16(m.cls) || !aligned16(x) || (!skip && !aligned16(m.rv))) return QG_ERR_ALIGN;
    a->cls = m.cls;
    a->rv = skip ? nullptr : m.rv;
    a->ld = skip ? 16 : m.rv_ld;
    a->alpha = m.alpha;
    a->s_r = m.s_r;
    a->n = m.n;
    a->k = k;
    a->x = x;
    a->xt = xt;
    a->skip = skip;
    a->y = m.y;
    a->acc_out = m.acc_out;
    return QG_OK;
}

qg_status qg_qgemv_sep(const uint8_t* cls, const int8_t* rv, int64_t rv_ld, const float* alpha, const float* s_r,
                       int64_t n, int64_t k, const void* x, int32_t xt, int32_t skip_residual, float* y,
                       int32_t* acc_out, void* stream) {
    const qg_sep_matrix m{cls, rv, rv_ld, alpha, s_r, n, y, acc_out};
    return qg_qgemv_sep_grouped(&m, 1, k, x, xt, skip_residual, stream);
}

qg_status qg_qgemv_sep_grouped(const qg_sep_matrix* m, int32_t count, int64_t k, const void* x, int32_t xt,
                               int32_t skip_residual, void* stream) {
    if (!m) return QG_ERR_NULLPTR;
    if (count < 1 || count > QG_MAX_GROUP) return QG_ERR_ARG;
    qg::SepArgs a[QG_MAX_GROUP];
    for (int32_t i = 0; i < count; ++i) {
        const qg_status st = sep_args(m[i], k, x, xt, skip_residual != 0, &a[i]);
        if (st != QG_OK) return st;
    }
    return from_hip(qg::launch_sep_qgemv_group(a, count, as_stream(stream)));
}

size_t qg_ternary_workspace_bytes(int64_t n, int64_t k) {
    (void)n;
    (void)k;
    return 256 * sizeof(uint64_t);
}

qg_status qg_quantize_ternary(const float* w, int64_t n, int64_t k, int8_t* q, float* gamma, void* ws,
                              size_t ws_bytes, void* stream) {
    if (!w || !q || !gamma) return QG_ERR_NULLPTR;
    if (n < 1 || k < 1) return QG_ERR_SHAPE;
    if (n > ((int64_t)1 << 39) / k) return QG_ERR_SHAPE;
    const int64_t count = n * k;
    if (count % 4 != 0) return QG_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(q)) return QG_ERR_ALIGN;
    if (!ws || ws_bytes < qg_ternary_workspace_bytes(n, k)) return QG_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 7u) != 0) return QG_ERR_ALIGN;
    return from_hip(qg::launch_ternary(w, count, q, gamma, static_cast<uint64_t*>(ws), as_stream(stream)));
}

qg_status qg_split_sign_residual(const float* w, int64_t n, int64_t k, int8_t* sign, float* alpha, int8_t* rq,
                                 float* s_r, void* stream) {
    if (!w || !sign || !alpha || !rq || !s_r) return QG_ERR_NULLPTR;
    if (n < 1 || k < 8 || k % 8 != 0 || k >= ((int64_t)1 << 31)) return QG_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(sign) || !aligned16(rq)) return QG_ERR_ALIGN;
    return from_hip(qg::launch_split_sign_residual(w, n, k, sign, alpha, rq, s_r, nullptr, as_stream(stream)));
}

qg_status qg_split_sign_residual_zp(const float* w, int64_t n, int64_t k, int8_t* sign, float* alpha, int8_t* rq,
                                    float* s_r, int8_t* z_r, void* stream) {
    if (!w || !sign || !alpha || !rq || !s_r || !z_r) return QG_ERR_NULLPTR;
    if (n < 1 || k < 8 || k % 8 != 0 || k >= ((int64_t)1 << 31)) return QG_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(sign) || !aligned16(rq)) return QG_ERR_ALIGN;
    return from_hip(qg::launch_split_sign_residual(w, n, k, sign, alpha, rq, s_r, z_r, as_stream(stream)));
}

qg_status qg_quantize_asym(const void* x, int32_t xt, int64_t rows, int64_t cols, int8_t* q, float* s, int8_t* z,
                           void* stream) {
    if (!x || !q || !s || !z) return QG_ERR_NULLPTR;
    if (xt != QG_F32 && xt != QG_BF16) return QG_ERR_ARG;
    if (rows < 1 || cols < 8 || cols % 8 != 0 || cols >= ((int64_t)1 << 31)) return QG_ERR_SHAPE;
    if (rows > ((int64_t)1 << 40) / cols) return QG_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q)) return QG_ERR_ALIGN;
    return from_hip(qg::launch_asym_rows(x, xt, rows, cols, q, s, z, as_stream(stream)));
}

qg_status qg_pack(const int8_t* codes, int64_t n, int64_t k, int32_t bits, uint8_t* packed, void* stream) {
    if (!codes || !packed) return QG_ERR_NULLPTR;
    if (bits != 1 && bits != 2) return QG_ERR_ARG;
    if (n < 1 || k < 1 || k % (8 / bits) != 0 || n > ((int64_t)1 << 40) / k) return QG_ERR_SHAPE;
    if (!aligned16(codes)) return QG_ERR_ALIGN;
    return from_hip(qg::launch_pack(codes, n * k, bits, packed, as_stream(stream)));
}

qg_status qg_unpack(const uint8_t* packed, int64_t n, int64_t k, int32_t bits, int8_t* codes, void* stream) {
    if (!codes || !packed) return QG_ERR_NULLPTR;
    if (bits != 1 && bits != 2) return QG_ERR_ARG;
    if (n < 1 || k < 1 || k % (8 / bits) != 0 || n > ((int64_t)1 << 40) / k) return QG_ERR_SHAPE;
    if (!aligned16(codes)) return QG_ERR_ALIGN;
    return from_hip(qg::launch_unpack(packed, n * k, bits, codes, as_stream(stream)));
}

int64_t qg_base3_row_bytes(int64_t k) {
    if (k < 1 || k >= ((int64_t)1 << 40)) return 0;
    return 16 * ((k + 79) / 80);
}

int64_t qg_tiles16_bytes(int64_t n, int64_t k) {
    if (n < 1 || n >= ((int64_t)1 << 31) || k < 128 || k % 128 != 0 || k > QG_BATCH_MAX_K) return 0;
    return qg::tiles16_bytes(n, k);
}

qg_status qg_pack_tiles16(const int8_t* codes, int64_t n, int64_t k, int8_t* out, void* stream) {
    if (!codes || !out) return QG_ERR_NULLPTR;
    if (qg_tiles16_bytes(n, k) == 0) return QG_ERR_SHAPE;
    if (!aligned16(codes) || !aligned16(out)) return QG_ERR_ALIGN;
    return from_hip(qg::launch_pack_tiles16(codes, n, k, out, as_stream(stream)));
}

qg_status qg_pack_base3(const int8_t* codes, int64_t n, int64_t k, uint8_t* packed, void* stream) {
    if (!codes || !packed) return QG_ERR_NULLPTR;
    if (n < 1 || k < 1 || n > ((int64_t)1 << 40) / k) return QG_ERR_SHAPE;
    return from_hip(qg::launch_pack3(codes, n, k, packed, as_stream(stream)));
}

qg_status qg_unpack_base3(const uint8_t* packed, int64_t n, int64_t k, int8_t* codes, void* stream) {
    if (!codes || !packed) return QG_ERR_NULLPTR;
    if (n < 1 || k < 1 || n > ((int64_t)1 << 40) / k) return QG_ERR_SHAPE;
    return from_hip(qg::launch_unpack3(packed, n, k, codes, as_stream(stream)));
}

static qg_status check_qgemv(const qg_weight* w, int32_t amode, const void* x, int32_t xt, const void* y,
                             int32_t yt, const int32_t* acc_out) {
    if (!w || !x || !y) return QG_ERR_NULLPTR;
    if (!w->codes || (!w->scale && w->fmt != QG_WFMT_Q4K)) return QG_ERR_NULLPTR;
    if (xt != QG_F32 && xt != QG_BF16) return QG_ERR_ARG;
    if (yt != QG_F32 && yt != QG_BF16) return QG_ERR_ARG;
    if (amode != QG_ACT_INT8 && amode != QG_ACT_FLOAT) return QG_ERR_ARG;
    switch (w->fmt) {
        case QG_WFMT_INT8: break;
        case QG_WFMT_TERNARY2:
        case QG_WFMT_TERNARY3:
            if (amode != QG_ACT_INT8) return QG_ERR_ARG;
            break;
        case QG_WFMT_SIGN1_RES8:
            if (amode != QG_ACT_FLOAT || xt != QG_BF16) return QG_ERR_ARG;
            if (!w->resid || !w->scale2) return QG_ERR_NULLPTR;
            break;
        case QG_WFMT_SIGN1_RES8Z:
            if (amode != QG_ACT_FLOAT || xt != QG_BF16) return QG_ERR_ARG;
            if (!w->resid || !w->scale2 || !w->zero) return QG_ERR_NULLPTR;
            break;
        case QG_WFMT_Q4K:
            if (amode != QG_ACT_FLOAT || xt != QG_BF16) return QG_ERR_ARG;
            if (!w->resid) return QG_ERR_NULLPTR;
            if (w->k % 256 != 0) return QG_ERR_SHAPE;
            break;
        default: return QG_ERR_ARG;
    }
    if (acc_out && amode != QG_ACT_INT8) return QG_ERR_ARG;
    if (w->n < 1 || w->n >= ((int64_t)1 << 31)) return QG_ERR_SHAPE;
    if (w->k < 128 || w->k % 128 != 0 || w->k > QG_QGEMV_MAX_K) return QG_ERR_SHAPE;
    if (!aligned16(w->codes) || !aligned16(x)) return QG_ERR_ALIGN;
    if ((w->fmt == QG_WFMT_SIGN1_RES8 || w->fmt == QG_WFMT_SIGN1_RES8Z || w->fmt == QG_WFMT_Q4K) &&
        !aligned16(w->resid))
        return QG_ERR_ALIGN;
    return QG_OK;
}

static qg::QgemvArgs qgemv_args(const qg_weight* w, int32_t amode, const void* x, int32_t xt, void* y, int32_t yt,
                                int32_t* acc_out) {
    qg::QgemvArgs a;
    a.fmt = w->fmt;
    a.amode = amode;
    a.xt = xt;
    a.yt = yt;
    a.n = w->n;
    a.k = w->k;
    a.codes = w->codes;
    a.resid = w->resid;
    a.scale = w->scale;
    a.scale2 = w->scale2;
    a.zero = w->fmt == QG_WFMT_SIGN1_RES8Z ? w->zero : nullptr;
    a.x = x;
    a.y = y;
    a.acc_out = acc_out;
    return a;
}

qg_status qg_qgemv(const qg_weight* w, int32_t amode, const void* x, int32_t xt, void* y, int32_t yt,
                   int32_t* acc_out, void* stream) {
    const qg_status st = check_qgemv(w, amode, x, xt, y, yt, acc_out);
    if (st != QG_OK) return st;
    return from_hip(qg::launch_qgemv(qgemv_args(w, amode, x, xt, y, yt, acc_out), as_stream(stream)));
}

qg_status qg_qgemv_grouped(const qg_weight* w, int32_t count, int32_t amode, const void* x, int32_t xt,
                           void* const* y, int32_t yt, int32_t* const* acc_out, void* stream) {
    if (!w || !y) return QG_ERR_NULLPTR;
    if (count < 1 || count > QG_MAX_GROUP) return QG_ERR_ARG;
    qg::QgemvArgs a[QG_MAX_GROUP];
    for (int32_t m = 0; m < count; ++m) {
        int32_t* acc = acc_out ? acc_out[m] : nullptr;
        const qg_status st = check_qgemv(&w[m], amode, x, xt, y[m], yt, acc);
        if (st != QG_OK) return st;
        if (w[m].fmt != w[0].fmt) return QG_ERR_ARG;
        if (w[m].k != w[0].k) return QG_ERR_SHAPE;
        a[m] = qgemv_args(&w[m], amode, x, xt, y[m], yt, acc);
    }
    return from_hip(qg::launch_qgemv_group(a, count, as_stream(stream)));
}

qg_status qg_qgemv_batch_grouped(const qg_weight* w, int32_t count, int32_t m, const void* x, int32_t xt,
                                 void* const* y, int32_t yt, void* stream) {
    if (!w || !y || !x) return QG_ERR_NULLPTR;
    if (count < 1 || count > QG_MAX_GROUP) return QG_ERR_ARG;
    if (xt != QG_BF16 || (yt != QG_F32 && yt != QG_BF16)) return QG_ERR_ARG;
    if (m < 1 || m > QG_BATCH_MAX_M) return QG_ERR_SHAPE;
    if (!aligned16(x)) return QG_ERR_ALIGN;
    qg::BatchArgs a[QG_MAX_GROUP];
    for (int32_t j = 0; j < count; ++j) {
        const qg_weight& wj = w[j];
        if (!wj.codes || !wj.scale || !y[j]) return QG_ERR_NULLPTR;
        if (wj.fmt != QG_WFMT_INT8 && wj.fmt != QG_WFMT_INT8_T16) return QG_ERR_ARG;
        if (wj.fmt != w[0].fmt) return QG_ERR_ARG;  // one layout per launch
        if (wj.n < 1 || wj.n >= ((int64_t)1 << 31)) return QG_ERR_SHAPE;
        if (wj.k < 128 || wj.k % 128 != 0 || wj.k > QG_BATCH_MAX_K || wj.k != w[0].k) return QG_ERR_SHAPE;
        if (!aligned16(wj.codes)) return QG_ERR_ALIGN;
        a[j].n = wj.n;
        a[j].k = wj.k;
        a[j].m = m;
        a[j].wq = static_cast<const int8_t*>(wj.codes);
        a[j].s_w = wj.scale;
        a[j].x = x;
        a[j].y = y[j];
        a[j].yt = yt;
        a[j].t16 = wj.fmt == QG_WFMT_INT8_T16;
    }
    if (m == 1 && w[0].k <= QG_QGEMV_MAX_K && w[0].fmt == QG_WFMT_INT8) {
        // one token: the batch-1 kernel (same definition, y [1][n] is y [n])
        qg::QgemvArgs b[QG_MAX_GROUP];
        for (int32_t j = 0; j < count; ++j) b[j] = qgemv_args(&w[j], QG_ACT_FLOAT, x, xt, y[j], yt, nullptr);
        return from_hip(qg::launch_qgemv_group(b, count, as_stream(stream)));
    }
    return from_hip(qg::launch_qgemv_batch(a, count, as_stream(stream)));
}

qg_status qg_qgemv_batch(const qg_weight* w, int32_t m, const void* x, int32_t xt, void* y, int32_t yt,
                         void* stream) {
    void* ys[1] = {y};
    return qg_qgemv_batch_grouped(w, 1, m, x, xt, ys, yt, stream);
}

size_t qg_qgemv_batch_workspace_bytes(int64_t n, int64_t k, int32_t m) {
    if (n < 1 || n >= ((int64_t)1 << 31) || k < 128 || k % 128 != 0 || k > QG_BATCH_MAX_K) return 0;
    if (m < 2 || m > QG_BATCH_MAX_M) return 0;
    return qg::qgemv_batch_splitk_workspace(n, k);
}

qg_status qg_qgemv_batch_ws(const qg_weight* w, int32_t m, const void* x, int32_t xt, void* y, int32_t yt, void* ws,
                            size_t ws_bytes, void* stream) {
    if (!w) return QG_ERR_NULLPTR;
    const size_t need = qg_qgemv_batch_workspace_bytes(w->n, w->k, m);
    if (need == 0) return qg_qgemv_batch(w, m, x, xt, y, yt, stream);  // no split for this shape
    if (!x || !y || !w->codes || !w->scale) return QG_ERR_NULLPTR;
    if (w->fmt != QG_WFMT_INT8 && w->fmt != QG_WFMT_INT8_T16) return QG_ERR_ARG;
    if (xt != QG_BF16 || (yt != QG_F32 && yt != QG_BF16)) return QG_ERR_ARG;
    if (!aligned16(x) || !aligned16(w->codes)) return QG_ERR_ALIGN;
    if (!ws || ws_bytes < need) return QG_ERR_WORKSPACE;
    if (!aligned16(ws)) return QG_ERR_ALIGN;
    qg::BatchArgs a;
    a.n = w->n;
    a.k = w->k;
    a.m = m;
    a.wq = static_cast<const int8_t*>(w->codes);
    a.s_w = w->scale;
    a.x = x;
    a.y = y;
    a.yt = yt;
    a.t16 = w->fmt == QG_WFMT_INT8_T16;
    return from_hip(qg::launch_qgemv_batch_splitk(a, ws, as_stream(stream)));
}

qg_status qg_quantize_mxfp4(const void* x, int32_t xt, int64_t rows, int64_t cols, uint8_t* codes,
                            uint8_t* scales, void* stream) {
    if (!x || !codes || !scales) return QG_ERR_NULLPTR;
    if (xt != QG_F32 && xt != QG_BF16) return QG_ERR_ARG;
    if (rows < 1 || cols < 256 || cols % 256 != 0 || rows > ((int64_t)1 << 40) / cols)
        return QG_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(codes)) return QG_ERR_ALIGN;
    return from_hip(qg::launch_quantize_mxfp4(x, xt, rows, cols, codes, scales, as_stream(stream)));
}

static qg_status check_mx_gemm(int64_t m, int64_t k, int64_t n) {
    if (m < 1 || n < 1 || m >= ((int64_t)1 << 31) || n >= ((int64_t)1 << 31)) return QG_ERR_SHAPE;
    if (k < 256 || k % 256 != 0 || k > 262144) return QG_ERR_SHAPE;
    if (m > ((int64_t)1 << 40) / k || n > ((int64_t)1 << 40) / k) return QG_ERR_SHAPE;
    return QG_OK;
}

qg_status qg_gemm_mxfp4(const uint8_t* a, const uint8_t* a_scales, int64_t m, int64_t k, const uint8_t* b,
                        const uint8_t* b_scales, int64_t n, float* y, void* stream) {
    if (!a || !a_scales || !b || !b_scales || !y) return QG_ERR_NULLPTR;
    const qg_status st = check_mx_gemm(m, k, n);
    if (st != QG_OK) return st;
    if (!aligned16(a) || !aligned16(a_scales) || !aligned16(b) || !aligned16(b_scales)) return QG_ERR_ALIGN;
    return from_hip(qg::launch_gemm_mxfp4(a, a_scales, m, k, b, b_scales, n, y, as_stream(stream)));
}

// workspace of the MXFP4 prefill: codes [m][k/2] | scales [k/256][m][8], 256-B aligned parts
static size_t mx_layout(int64_t m, int64_t k, size_t* off_scales) {
    const size_t codes = align_up((size_t)m * (size_t)(k / 2), 256);
    if (off_scales) *off_scales = codes;
    return codes + align_up((size_t)m * (size_t)(k / 32), 256);
}

size_t qg_prefill_mxfp4_workspace_bytes(int64_t m, int64_t k) {
    if (check_mx_gemm(m, k, 1) != QG_OK) return 0;
    return mx_layout(m, k, nullptr);
}

qg_status qg_prefill_mxfp4(const void* x, int64_t m, int64_t k, const uint8_t* w, const uint8_t* w_scales,
                           int64_t n, float* y, void* ws, size_t ws_bytes, void* stream) {
    if (!x || !w || !w_scales || !y) return QG_ERR_NULLPTR;
    const qg_status st = check_mx_gemm(m, k, n);
    if (st != QG_OK) return st;
    if (!aligned16(x) || !aligned16(w) || !aligned16(w_scales)) return QG_ERR_ALIGN;
    size_t off_s = 0;
    const size_t need = mx_layout(m, k, &off_s);
    if (!ws || ws_bytes < need) return QG_ERR_WORKSPACE;
    if (!aligned16(ws)) return QG_ERR_ALIGN;
    uint8_t* xc = static_cast<uint8_t*>(ws);
    uint8_t* xs = xc + off_s;
    hipStream_t s = as_stream(stream);
    hipError_t e = qg::launch_quantize_mxfp4(x, QG_BF16, m, k, xc, xs, s);
    if (e != hipSuccess) return QG_ERR_HIP;
    return from_hip(qg::launch_gemm_mxfp4(xc, xs, m, k, w, w_scales, n, y, s));
}

size_t qg_qgemm_workspace_bytes(int64_t m, int64_t k, int32_t n_out) {
    if (m < 1 || k < 1 || k > QG_QGEMM_MAX_K || n_out < 0 || n_out > QG_MAX_OUTLIERS) return 0;
    if (m > ((int64_t)1 << 40) / k) return 0;
    return qgemm_layout(m, k, n_out, nullptr, nullptr);
}

qg_status qg_qgemm_w8a8(const int8_t* xq, const float* s_x, const void* x_out, int32_t x_out_ld, int64_t m,
                        int64_t k, int32_t n_out, const int8_t* wq, const float* s_w, const void* w_out,
                        int32_t w_out_ld, int64_t n, float* y, int32_t* acc_out, void* stream) {
    if (!xq || !s_x || !wq || !s_w || !y) return QG_ERR_NULLPTR;
    if (n_out < 0 || n_out > QG_MAX_OUTLIERS) return QG_ERR_ARG;
    qg_status st = check_gemm_shape(m, k, n);
    if (st != QG_OK) return st;
    if ((st = check_out_operand(x_out, x_out_ld, n_out)) != QG_OK) return st;
    if ((st = check_out_operand(w_out, w_out_ld, n_out)) != QG_OK) return st;
    if (!aligned16(xq) || !aligned16(wq)) return QG_ERR_ALIGN;
    qg::QgemmArgs a;
    a.m = m;
    a.k = k;
    a.n = n;
    a.xq = xq;
    a.s_x = s_x;
    a.x_out = static_cast<const uint16_t*>(x_out);
    a.x_out_ld = x_out_ld;
    a.wq = wq;
    a.s_w = s_w;
    a.w_out = static_cast<const uint16_t*>(w_out);
    a.w_out_ld = w_out_ld;
    a.n_out = n_out;
    a.y = y;
    a.acc_out = acc_out;
    return from_hip(qg::launch_qgemm(a, as_stream(stream)));
}

qg_status qg_qgemm_w8a8_outlier(const void* x, int64_t m, int64_t k, const int32_t* idx, int32_t n_out,
                                const int8_t* wq, const float* s_w, const void* w_out, int32_t w_out_ld, int64_t n,
                                float* y, int32_t* acc_out, void* ws, size_t ws_bytes, void* stream) {
    if (!x || !wq || !s_w || !y) return QG_ERR_NULLPTR;
    if (n_out < 0 || n_out > QG_MAX_OUTLIERS) return QG_ERR_ARG;
    qg_status st = check_gemm_shape(m, k, n);
    if (st != QG_OK) return st;
    if ((st = check_out_operand(w_out, w_out_ld, n_out)) != QG_OK) return st;
    if (!aligned16(x) || !aligned16(wq)) return QG_ERR_ALIGN;
    qg::OutlierIdx oi;
    st = check_idx(idx, n_out, k, &oi);
    if (st != QG_OK) return st;
    size_t off_sx = 0, off_xo = 0;
    const size_t need = qgemm_layout(m, k, n_out, &off_sx, &off_xo);
    if (!ws || ws_bytes < need) return QG_ERR_WORKSPACE;
    if (!aligned16(ws)) return QG_ERR_ALIGN;
    uint8_t* base = static_cast<uint8_t*>(ws);
    int8_t* xq = reinterpret_cast<int8_t*>(base);
    float* s_x = reinterpret_cast<float*>(base + off_sx);
    uint16_t* x_out = reinterpret_cast<uint16_t*>(base + off_xo);
    const int ld = out_ld(n_out);
    hipError_t e = qg::launch_absmax_split(static_cast<const uint16_t*>(x), m, k, oi, n_out, xq, s_x, x_out, ld,
                                           as_stream(stream));
    if (e != hipSuccess) return QG_ERR_HIP;
    const int dbg = debug_mode();
    if (dbg && qg::debug_check_split(static_cast<const uint16_t*>(x), m, k, oi, n_out, xq, x_out, ld, dbg == 2,
                                     as_stream(stream)) != hipSuccess)
        return QG_ERR_HIP;
    qg::QgemmArgs a;
    a.m = m;
    a.k = k;
    a.n = n;
    a.xq = xq;
    a.s_x = s_x;
    a.x_out = x_out;
    a.x_out_ld = ld;
    a.wq = wq;
    a.s_w = s_w;
    a.w_out = static_cast<const uint16_t*>(w_out);
    a.w_out_ld = w_out_ld;
    a.n_out = n_out;
    a.y = y;
    a.acc_out = acc_out;
    e = qg::launch_qgemm(a, as_stream(stream));
    if (e != hipSuccess || !dbg) return from_hip(e);
    return debug_result(as_stream(stream));
}

size_t qg_probe_stream_read_bytes(int64_t bytes, int32_t workgroups) {
    if (bytes < 1 || workgroups < 1 || workgroups > 65535) return 0;
    const int64_t blk = qg::stream_read_block(bytes, workgroups);
    if (blk < 1 || blk >= ((int64_t)1 << 31)) return 0;
    return (size_t)(blk * workgroups);
}

qg_status qg_probe_stream_read(const void* buf, int64_t bytes, int32_t workgroups, uint32_t* sink, void* stream) {
    if (!buf || !sink) return QG_ERR_NULLPTR;
    if (qg_probe_stream_read_bytes(bytes, workgroups) == 0) return QG_ERR_SHAPE;
    if (!aligned16(buf)) return QG_ERR_ALIGN;
    return from_hip(qg::launch_stream_read(buf, bytes, workgroups, sink, as_stream(stream)));
}

}  // extern "C"

namespace {

// Validates the stages of a chained step and counts its slots.
qg_status chain_check(const qg_chain_stage* stages, int32_t nstages, int32_t workgroups, int64_t* total_slots) {
    using namespace qg::chain;
    if (!stages) return QG_ERR_NULLPTR;
    if (nstages < 1 || nstages > QG_CHAIN_MAX_STAGES) return QG_ERR_ARG;
    if (workgroups < 1 || workgroups > 65535) return QG_ERR_ARG;
    int64_t total = 0;
    for (int32_t s = 0; s < nstages; ++s) {
        const qg_chain_stage& st = stages[s];
        if (st.count < 1 || st.count > QG_MAX_GROUP) return QG_ERR_ARG;
        if (st.dep < -1 || st.dep >= s) return QG_ERR_ARG;  // an earlier stage only
        if (!st.w || !st.y || !st.x) return QG_ERR_NULLPTR;
        if (!aligned16(st.x)) return QG_ERR_ALIGN;
        const int64_t k = st.w[0].k;
        if (k < QG_CHAIN_MIN_K || k > QG_CHAIN_MAX_K || k % 128 != 0) return QG_ERR_SHAPE;
        int64_t rows = 0;
        for (int32_t m = 0; m < st.count; ++m) {
            const qg_weight& w = st.w[m];
            if (w.fmt != QG_WFMT_INT8) return QG_ERR_ARG;
            if (!w.codes || !w.scale || !st.y[m]) return QG_ERR_NULLPTR;
            if (w.k != k) return QG_ERR_SHAPE;
            if (w.n < 1 || w.n >= ((int64_t)1 << 31)) return QG_ERR_SHAPE;
            if (!aligned16(w.codes)) return QG_ERR_ALIGN;
            if ((reinterpret_cast<uintptr_t>(st.y[m]) & 1u) != 0) return QG_ERR_ALIGN;
            rows += w.n;
        }
        const int64_t r = chain_rows_per_slot(rows, workgroups);
        for (int32_t m = 0; m < st.count; ++m) total += (st.w[m].n + r - 1) / r;
        // slot records are addressed with 32-bit byte offsets
        if (total * (int64_t)sizeof(SlotD) >= ((int64_t)1 << 31)) return QG_ERR_SHAPE;
    }
    *total_slots = total;
    return QG_OK;
}

}  // namespace

extern "C" {

size_t qg_chain_plan_bytes(const qg_chain_stage* stages, int32_t nstages, int32_t workgroups) {
    int64_t total = 0;
    if (chain_check(stages, nstages, workgroups, &total) != QG_OK) return 0;
    return (size_t)qg::chain::plan_bytes(nstages, total);
}

qg_status qg_chain_plan(const qg_chain_stage* stages, int32_t nstages, int32_t workgroups, void* image,
                        size_t image_bytes) {
    using namespace qg::chain;
    if (!image) return QG_ERR_NULLPTR;
    int64_t total = 0;
    const qg_status chk = chain_check(stages, nstages, workgroups, &total);
    if (chk != QG_OK) return chk;
    if (!aligned16(image)) return QG_ERR_ALIGN;
    const uint64_t bytes = plan_bytes(nstages, total);
    if (image_bytes < bytes) return QG_ERR_WORKSPACE;

    uint8_t* img = static_cast<uint8_t*>(image);
    memset(img, 0, (size_t)bytes);
    Header* h = reinterpret_cast<Header*>(img);
    h->magic = kMagic;
    h->version = kVersion;
    h->nstages = nstages;
    h->total_slots = (int32_t)total;
    h->stride = done_stride(nstages);
    h->grid = workgroups;
    h->stages_off = (uint64_t)kOffDone + (uint64_t)kRep * (uint64_t)h->stride * 4u;
    h->slots_off = (h->stages_off + (uint64_t)nstages * sizeof(StageD) + 63) / 64 * 64;
    h->timeout_ticks = QG_CHAIN_TIMEOUT_TICKS;
    h->bytes = bytes;
    StageD* sd = reinterpret_cast<StageD*>(img + h->stages_off);
    SlotD* sl = reinterpret_cast<SlotD*>(img + h->slots_off);
    int64_t slot = 0;
    int32_t max_k = 0, nc = 0;
    for (int32_t s = 0; s < nstages; ++s) {
        const qg_chain_stage& st = stages[s];
        const int32_t k = (int32_t)st.w[0].k;
        int64_t rows = 0;
        for (int32_t m = 0; m < st.count; ++m) rows += st.w[m].n;
        const int64_t r = chain_rows_per_slot(rows, workgroups);
        StageD& d = sd[s];
        d.x = reinterpret_cast<uint64_t>(st.x);
        d.k = k;
        d.dep = st.dep;
        d.slot0 = (int32_t)slot;
        d.nseg = (k + kItemChunks * 16 - 1) / (kItemChunks * 16);
        for (int32_t m = 0; m < st.count; ++m) {
            const qg_weight& w = st.w[m];
            for (int64_t row0 = 0; row0 < w.n; row0 += r) {
                SlotD& t = sl[slot++];
                t.codes = reinterpret_cast<uint64_t>(w.codes) + (uint64_t)row0 * (uint64_t)k;
                t.scale = reinterpret_cast<uint64_t>(w.scale) + 4u * (uint64_t)row0;
                t.y = reinterpret_cast<uint64_t>(st.y[m]) + 2u * (uint64_t)row0;
                t.rows = (int32_t)(w.n - row0 < r ? w.n - row0 : r);
                t.k = k;
                t.nseg = d.nseg;
                t.stage = s;
            }
        }
        d.nslots = (int32_t)(slot - d.slot0);
        if (k > max_k) max_k = k;
        if (d.nseg * kItemChunks > nc) nc = d.nseg * kItemChunks;
    }
    h->max_k = max_k;
    h->nc = nc;
    return QG_OK;
}

qg_status qg_qgemv_chain(const void* image, void* plan, void* stream) {
    using namespace qg::chain;
    if (!image || !plan) return QG_ERR_NULLPTR;
    if (!aligned16(image) || !aligned16(plan)) return QG_ERR_ALIGN;
    const Header* h = static_cast<const Header*>(image);
    if (h->magic != kMagic || h->version != kVersion) return QG_ERR_ARG;
    if (h->nstages < 1 || h->nstages > QG_CHAIN_MAX_STAGES || h->grid < 1 || h->grid > 65535) return QG_ERR_ARG;
    return from_hip(qg::launch_chain(image, plan, as_stream(stream)));
}

}  // extern "C"
