// debug.hip -- the QG_DEBUG=1 checks of the outlier path (qg_debug.h).
// Each check reads the index list from its kernel argument, exactly as the
// split and gather kernels receive theirs, and compares the outputs of those
// kernels with what the list and the inputs define; every memory access is
// guarded by the bounds of its buffer, so a bad list cannot make a check
// read out of range.  In self-test mode (QG_DEBUG=2) the checks expect every
// gathered value with its lowest bit flipped, so that a call whose outlier
// path is correct and has at least one outlier reports a failed check: the
// way to see the reporting work end to end.
#include <mutex>

#include "qg_debug.h"
#include "qg_device.h"

namespace qg {

// the flag word (the first of the array), one per device; host code takes
// its device address
static __device__ __align__(256) uint32_t dbg_flags[64];

namespace {
constexpr int kDbgThreads = 256;
static_assert(kDbgThreads >= kMaxOutliers, "one thread per list entry");

std::mutex dbg_mu;
uint32_t* dbg_dev[kMaxDevices] = {};

hipError_t flag_ptr(uint32_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(dbg_mu);
    if (!dbg_dev[dev]) {  // once per device, with that device current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(dbg_flags));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        dbg_dev[dev] = static_cast<uint32_t*>(p);
    }
    *out = dbg_dev[dev];
    return hipSuccess;
}

// the list itself: entries in range and strictly increasing
__device__ __forceinline__ bool idx_ok(const OutlierIdx& idx, int j, int64_t cols) {
    const int c = idx.v[j];
    return c >= 0 && c < cols && (j == 0 || c > idx.v[j - 1]);
}
}  // namespace

__global__ __launch_bounds__(kDbgThreads) void dbg_split_kernel(const uint16_t* x, int64_t rows, int64_t cols,
                                                                OutlierIdx idx, int n_out, const int8_t* q,
                                                                const uint16_t* x_out, int ld, uint16_t flip,
                                                                uint32_t* flags) {
    const int j = threadIdx.x;
    uint32_t bad = 0;
    if (blockIdx.x == 0 && j < n_out && !idx_ok(idx, j, cols)) bad |= kDbgIdx;
    if (j < ld) {
        const int c = j < n_out ? idx.v[j] : -1;
        const bool in = c >= 0 && c < cols;
        for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
            const uint16_t g = x_out[r * ld + j];
            if (j < n_out) {
                if (in && ((g ^ flip) != x[r * cols + c] || q[r * cols + c] != 0)) bad |= kDbgSplit;
            } else if (g != 0) {
                bad |= kDbgSplit;
            }
        }
    }
    if (bad) atomicOr(flags, bad);
}

__global__ __launch_bounds__(kDbgThreads) void dbg_gather_kernel(const float* w, int64_t n, int64_t k, OutlierIdx idx,
                                                                 int n_out, const uint16_t* w_out, int ld,
                                                                 uint16_t flip, uint32_t* flags) {
    const int j = threadIdx.x;
    uint32_t bad = 0;
    if (blockIdx.x == 0 && j < n_out && !idx_ok(idx, j, k)) bad |= kDbgIdx;
    if (j < ld) {
        const int c = j < n_out ? idx.v[j] : -1;
        const bool in = c >= 0 && c < k;
        for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
            const uint16_t g = w_out[r * ld + j];
            if (j < n_out) {
                if (in && (g ^ flip) != (uint16_t)f32_to_bf16(w[r * k + c])) bad |= kDbgGather;
            } else if (g != 0) {
                bad |= kDbgGather;
            }
        }
    }
    if (bad) atomicOr(flags, bad);
}

static int dbg_grid(int64_t rows) { return (int)(rows < 1024 ? (rows < 1 ? 1 : rows) : 1024); }

hipError_t debug_check_split(const uint16_t* x, int64_t rows, int64_t cols, const OutlierIdx& idx, int n_out,
                             const int8_t* q, const uint16_t* x_out, int ld, bool selftest, hipStream_t st) {
    uint32_t* f = nullptr;
    const hipError_t e = flag_ptr(&f);
    if (e != hipSuccess) return e;
    if (n_out == 0) ld = 0;  // no x_out
    dbg_split_kernel<<<dbg_grid(rows), kDbgThreads, 0, st>>>(x, rows, cols, idx, n_out, q, x_out, ld,
                                                            selftest ? (uint16_t)1 : (uint16_t)0, f);
    return hipGetLastError();
}

hipError_t debug_check_gather(const float* w, int64_t n, int64_t k, const OutlierIdx& idx, int n_out,
                              const uint16_t* w_out, int ld, bool selftest, hipStream_t st) {
    if (n_out == 0) return hipSuccess;  // nothing was written
    uint32_t* f = nullptr;
    const hipError_t e = flag_ptr(&f);
    if (e != hipSuccess) return e;
    dbg_gather_kernel<<<dbg_grid(n), kDbgThreads, 0, st>>>(w, n, k, idx, n_out, w_out, ld,
                                                          selftest ? (uint16_t)1 : (uint16_t)0, f);
    return hipGetLastError();
}

hipError_t debug_take_flags(hipStream_t st, uint32_t* flags) {
    uint32_t* f = nullptr;
    hipError_t e = flag_ptr(&f);
    if (e != hipSuccess) return e;
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
    if ((e = hipMemcpy(flags, f, sizeof(uint32_t), hipMemcpyDeviceToHost)) != hipSuccess) return e;
    return hipMemset(f, 0, sizeof(uint32_t));
}

}  // namespace qg
