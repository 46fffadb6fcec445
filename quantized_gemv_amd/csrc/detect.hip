// detect.hip -- outlier-channel detection from calibration activations.
//
// [SEP] section 2.2: the few channels whose activations run tens of times
// larger than the rest are found once and the list is cached.  A channel's
// range is its max |x| over the calibration rows; the n_out channels with the
// largest ranges are chosen (equal ranges: the lower channel index first) and
// written in ascending channel order, the form the split takes.
//
// Ranges are kept as fp32 bit patterns: |x| >= 0, so bit patterns order like
// the values and integer max is exact.
// Pass 1 (many workgroups): row block j writes partial[j][c], the max over
// its rows -- no atomics (thousands of workgroups contending for the same
// few thousand addresses would serialize).
// Pass 2 (one workgroup): folds the partials into range[c] = partial[0][c],
// runs a radix select of the n_out-th largest range over its 32 bits (four
// 8-bit digits, histograms in LDS), then one sweep over the channels in index
// order emits every channel above that value and, in index order, as many
// channels equal to it as are still needed.
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

// Thread t of block (bx, by) owns the 8 channels of 16-byte piece
// bx * kThreads + t and the rows by, by + gridDim.y, ...; it writes their
// maxima to row block by's partials.
__global__ __launch_bounds__(kThreads) void channel_range_kernel(const uint16_t* x, int64_t rows, int64_t cols,
                                                                 uint32_t* partial) {
    const int64_t c8 = cols / 8;
    const int64_t piece = blockIdx.x * (int64_t)kThreads + threadIdx.x;
    if (piece >= c8) return;
    uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        const uint4 h = *reinterpret_cast<const uint4*>(x + r * cols + piece * 8);
        const uint32_t w[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // |bf16| as the fp32 bit pattern of the same value
            m[2 * e] = max(m[2 * e], (w[e] & 0x7FFFu) << 16);
            m[2 * e + 1] = max(m[2 * e + 1], (w[e] >> 16 & 0x7FFFu) << 16);
        }
    }
    uint4* out = reinterpret_cast<uint4*>(partial + blockIdx.y * cols + piece * 8);
    out[0] = make_uint4(m[0], m[1], m[2], m[3]);
    out[1] = make_uint4(m[4], m[5], m[6], m[7]);
}

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

// Exclusive prefix count of a 0/1 flag over the workgroup, in thread order;
// returns this thread's offset and sets `total`.  Two barriers.
__device__ __forceinline__ int block_flag_scan(bool flag, int* wave_cnt, int& total) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const uint64_t b = __ballot(flag);
    const int below = __popcll(b & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[w] = __popcll(b);
    lds_barrier();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) {
        const int c = wave_cnt[i];
        off += (i < w) ? c : 0;
        tot += c;
    }
    lds_barrier();
    total = tot;
    return off + below;
}

__global__ __launch_bounds__(kSelThreads) void select_channels_kernel(uint32_t* partial, int blocks, int cols,
                                                                      int n_out, int32_t* idx) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh_prefix, sh_need;
    __shared__ int wave_cnt[kSelWaves];
    const int tid = threadIdx.x;
    // fold the row blocks' partials into row 0 (each thread owns its channels)
    uint32_t* range = partial;
    for (int c = tid; c < cols; c += kSelThreads) {
        uint32_t v = partial[c];
#pragma unroll 8
        for (int j = 1; j < blocks; ++j) v = max(v, partial[(int64_t)j * cols + c]);
        range[c] = v;
    }
    __syncthreads();  // the folded ranges are read by other threads below
    // --- radix select: the n_out-th largest range (ranked with repeats)
    uint32_t prefix = 0, mask = 0, need = (uint32_t)n_out;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0u;
        lds_barrier();
        for (int c = tid; c < cols; c += kSelThreads) {
            const uint32_t v = range[c];
            if ((v & mask) == prefix) atomicAdd(&hist[(v >> shift) & 255u], 1u);
        }
        lds_barrier();
        if (tid < kWave) {
            // the bucket holding the need-th element from the top: lane l sums
            // buckets 4l .. 4l+3; a suffix sum over the lanes finds the lane
            // whose buckets hold it, and that lane walks its four
            const int l = tid;
            uint32_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) h[i] = hist[4 * l + i];
            const uint32_t own = h[0] + h[1] + h[2] + h[3];
            uint32_t incl = own;  // buckets >= 4l
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const uint32_t t = __shfl_down(incl, off, kWave);
                if (l + off < kWave) incl += t;
            }
            uint32_t above = incl - own;  // buckets > 4l + 3
            if (above < need && need <= incl) {
                int i = 3;
                for (; i > 0; --i) {
                    if (above + h[i] >= need) break;
                    above += h[i];
                }
                sh_prefix = prefix | ((uint32_t)(4 * l + i) << shift);
                sh_need = need - above;
            }
        }
        lds_barrier();
        prefix = sh_prefix;
        need = sh_need;
        mask |= 255u << shift;
    }
    // prefix is now the n_out-th largest range; `need` (>= 1) of the channels
    // equal to it are taken, the lowest indices first
    int emitted = 0, equal_seen = 0;
    for (int base = 0; base < cols; base += kSelThreads) {
        const int c = base + tid;
        const uint32_t v = (c < cols) ? range[c] : 0u;
        const bool live = c < cols;
        int eq_total;
        const int eq_rank = block_flag_scan(live && v == prefix, wave_cnt, eq_total) + equal_seen;
        const bool take = live && (v > prefix || (v == prefix && eq_rank < (int)need));
        int take_total;
        const int pos = block_flag_scan(take, wave_cnt, take_total) + emitted;
        if (take) idx[pos] = c;
        emitted += take_total;
        equal_seen += eq_total;
    }
}

hipError_t launch_detect_outliers(const uint16_t* x, int64_t rows, int64_t cols, int n_out, int32_t* idx,
                                  uint32_t* partial, hipStream_t st) {
    if (n_out == 0) return hipSuccess;
    const int gx = (int)((cols / 8 + kThreads - 1) / kThreads);
    const int gy = detect_row_blocks(cols);  // row blocks without rows write zeros
    channel_range_kernel<<<dim3(gx, gy), kThreads, 0, st>>>(x, rows, cols, partial);
    select_channels_kernel<<<1, kSelThreads, 0, st>>>(partial, gy, (int)cols, n_out, idx);
    return hipGetLastError();
}

}  // namespace qg
