// probe.hip -- the streaming-read probe that measures the HBM read rate the
// qgemv kernels are compared with: every byte of a buffer read once with
// 128-bit non-temporal loads, the same access the weight streams use, and
// nothing computed but an XOR that keeps the loads live.  A measurement aid,
// not a step of the method.
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per lane

// Workgroup g reads the block [g * blk, (g + 1) * blk); blk is a multiple of
// 512 threads x 16 B x kProbeUnroll, so every load is in range.
__global__ __launch_bounds__(kQProbeThreads) void stream_read_kernel(const uint8_t* p, uint32_t blk, uint32_t* sink) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(p + (uint64_t)blockIdx.x * blk, blk);
    constexpr uint32_t kStep = kQProbeThreads * 16u * kProbeUnroll;
    uint32_t acc = 0;
    for (uint32_t o = threadIdx.x * 16u; o < blk; o += kStep) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = load16_nt(r, o + u * kQProbeThreads * 16u);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;  // practically never: keeps the loads from being removed
}

int64_t stream_read_block(int64_t bytes, int wgs) {
    const int64_t q = (int64_t)kQProbeThreads * 16 * kProbeUnroll;
    return bytes / wgs / q * q;
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, int wgs, uint32_t* sink, hipStream_t st) {
    const int64_t blk = stream_read_block(bytes, wgs);
    stream_read_kernel<<<wgs, kQProbeThreads, 0, st>>>(static_cast<const uint8_t*>(buf), (uint32_t)blk, sink);
    return hipGetLastError();
}

}  // namespace qg
