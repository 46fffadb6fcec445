// qg_launch.h -- host-side launchers implemented in the .hip translation
// units and called by the C ABI layer (api.cpp) after argument validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

constexpr int kMaxOutliers = 256;

// The cached outlier channel list travels by value in the kernel arguments.
struct OutlierIdx {
    int32_t v[kMaxOutliers];
};

hipError_t launch_absmax_rows(const void* x, int xt, int64_t rows, int64_t cols, int8_t* q, float* s,
                              hipStream_t st);
int absmax_tensor_parts(int64_t elems);
hipError_t launch_absmax_tensor(const void* x, int xt, int64_t elems, int8_t* q, float* s, float* partial,
                                hipStream_t st);
// The same two passes with the partial maxima in a file-scope device array
// (no workspace); absmax_tensor_parts() never exceeds its size.
constexpr int kAbsmaxScratchParts = 1024;
constexpr int kMaxDevices = 64;
hipError_t launch_absmax_tensor_noalloc(const void* x, int xt, int64_t elems, int8_t* q, float* s,
                                        hipStream_t st);
hipError_t launch_absmax_split(const uint16_t* x, int64_t rows, int64_t cols, const OutlierIdx& idx, int n_out,
                               int8_t* q, float* s, uint16_t* x_out, int x_out_ld, hipStream_t st);
// Row blocks of the detection's range pass (a function of cols only, so the
// workspace size is too): about 1024 workgroups, at most 64 row blocks.
inline int detect_row_blocks(int64_t cols) {
    const int64_t gx = (cols / 8 + 255) / 256;
    int64_t gy = (1024 + gx - 1) / gx;
    return (int)(gy < 1 ? 1 : gy > 64 ? 64 : gy);
}
hipError_t launch_detect_outliers(const uint16_t* x, int64_t rows, int64_t cols, int n_out, int32_t* idx,
                                  uint32_t* partial, hipStream_t st);
hipError_t launch_gather_cols_bf16(const float* w, int64_t n, int64_t k, const OutlierIdx& idx, int n_out,
                                   uint16_t* w_out, int w_out_ld, hipStream_t st);
hipError_t launch_ternary(const float* w, int64_t count, int8_t* q, float* gamma, uint64_t* hist, hipStream_t st);
// z_r == nullptr: symmetric residual; otherwise the zero-point residual
hipError_t launch_split_sign_residual(const float* w, int64_t n, int64_t k, int8_t* sign, float* alpha, int8_t* rq,
                                      float* s_r, int8_t* z_r, hipStream_t st);
hipError_t launch_asym_rows(const void* x, int xt, int64_t rows, int64_t cols, int8_t* q, float* s, int8_t* z,
                            hipStream_t st);
hipError_t launch_quantize_q4k(const float* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* meta, hipStream_t st);
hipError_t launch_pack(const int8_t* codes, int64_t count, int bits, uint8_t* packed, hipStream_t st);
hipError_t launch_unpack(const uint8_t* packed, int64_t count, int bits, int8_t* codes, hipStream_t st);
hipError_t launch_pack3(const int8_t* codes, int64_t n, int64_t k, uint8_t* packed, hipStream_t st);
int64_t tiles16_bytes(int64_t n, int64_t k);
hipError_t launch_pack_tiles16(const int8_t* codes, int64_t n, int64_t k, int8_t* out, hipStream_t st);
hipError_t launch_unpack3(const uint8_t* packed, int64_t n, int64_t k, int8_t* codes, hipStream_t st);

struct QgemvArgs {
    int fmt, amode, xt, yt;
    int64_t n, k;
    const void* codes;
    const int8_t* resid;
    const float* scale;
    const float* scale2;
    const int8_t* zero;
    const void* x;
    void* y;
    int32_t* acc_out;
};
hipError_t launch_qgemv(const QgemvArgs& a, hipStream_t st);
constexpr int kMaxGroupLaunch = 8;
hipError_t launch_qgemv_group(const QgemvArgs* a, int count, hipStream_t st);

// The W8A8 GEMM over split activations (xq, s_x, x_out [m][x_out_ld]);
// outlier operand strides are multiples of 8 elements, rows 16-B aligned.
struct QgemmArgs {
    int64_t m, k, n;
    const int8_t* xq;
    const float* s_x;
    const uint16_t* x_out;
    int x_out_ld;
    const int8_t* wq;
    const float* s_w;
    const uint16_t* w_out;
    int w_out_ld;
    int n_out;
    float* y;
    int32_t* acc_out;
};
hipError_t launch_qgemm(const QgemmArgs& a, hipStream_t st);

// Thresholded separated weights: j_b, j_z are the nearest ranks of the two
// percentiles (j_z = 0: no zero class).
hipError_t launch_sep_split(const float* w, int64_t n, int64_t k, int j_b, int j_z, uint8_t* cls, int8_t* rv,
                            int64_t ld, float* alpha, float* s_r, hipStream_t st);
struct SepArgs {
    const uint8_t* cls;
    const int8_t* rv;
    int64_t ld;
    const float* alpha;
    const float* s_r;
    int64_t n, k;
    const void* x;
    int xt;
    bool skip;
    float* y;
    int32_t* acc_out;
};
hipError_t launch_sep_qgemv(const SepArgs& a, hipStream_t st);
// 1..kMaxGroupLaunch matrices sharing x, k, xt and skip in one launch
hipError_t launch_sep_qgemv_group(const SepArgs* a, int count, hipStream_t st);

// Weight-only int8 products for a batch of m tokens (x bf16 [m][k]); the
// entries of one launch share k, m, x and yt.
struct BatchArgs {
    int64_t n, k;
    int m;
    const int8_t* wq;
    const float* s_w;
    const void* x;
    void* y;
    int yt;
    bool t16;  // codes in 16-row tiles (else row-major)
};
hipError_t launch_qgemv_batch(const BatchArgs* a, int count, hipStream_t st);
// One matrix with K split over workgroups (partials and row-block counters
// in the workspace); 0 bytes when that path does not apply to (n, k).
size_t qgemv_batch_splitk_workspace(int64_t n, int64_t k);
hipError_t launch_qgemv_batch_splitk(const BatchArgs& a, void* ws, hipStream_t st);

// MXFP4: codes [rows][cols/2] (low nibble first) and E8M0 scales
// [rows][cols/32]; GEMM Y[m][n] = sum_k A[m][k] B[n][k] (fp32).
hipError_t launch_quantize_mxfp4(const void* x, int xt, int64_t rows, int64_t cols, uint8_t* codes,
                                 uint8_t* scales, hipStream_t st);
hipError_t launch_gemm_mxfp4(const uint8_t* a, const uint8_t* as, int64_t m, int64_t k, const uint8_t* b,
                             const uint8_t* bs, int64_t n, float* y, hipStream_t st);

int device_cu_count();

// Streaming-read probe: workgroups of kQProbeThreads each read one block of
// stream_read_block(bytes, wgs) bytes (a multiple of the per-pass span).
constexpr int kQProbeThreads = 512;
int64_t stream_read_block(int64_t bytes, int wgs);
hipError_t launch_stream_read(const void* buf, int64_t bytes, int wgs, uint32_t* sink, hipStream_t st);

}  // namespace qg
