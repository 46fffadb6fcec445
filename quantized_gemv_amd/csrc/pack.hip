// pack.hip -- bit packing of ternary (2-bit) and sign (1-bit) codes.
//
// Layout: code k of a row sits in byte k / v at bit offset bits * (k % v),
// least significant field first, v = 8 / bits.  Since every row length is a
// multiple of v, rows pack back to back and the kernels work on the flat
// code array: one thread per packed byte.
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

__global__ __launch_bounds__(kThreads) void pack2_kernel(const int8_t* codes, int64_t nbytes, uint8_t* out) {
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < nbytes; i += (int64_t)gridDim.x * kThreads) {
        const uint32_t c = reinterpret_cast<const uint32_t*>(codes)[i];
        uint32_t b = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) b |= ((((c >> (8 * j)) & 0xFFu) + 1u) & 3u) << (2 * j);
        out[i] = (uint8_t)b;
    }
}

__global__ __launch_bounds__(kThreads) void pack1_kernel(const int8_t* codes, int64_t nbytes, uint8_t* out) {
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < nbytes; i += (int64_t)gridDim.x * kThreads) {
        const uint2 c = reinterpret_cast<const uint2*>(codes)[i];
        const uint32_t w[2] = {c.x, c.y};
        uint32_t b = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int8_t q = (int8_t)((w[j >> 2] >> (8 * (j & 3))) & 0xFFu);
            b |= (q > 0 ? 1u : 0u) << j;
        }
        out[i] = (uint8_t)b;
    }
}

__global__ __launch_bounds__(kThreads) void unpack2_kernel(const uint8_t* in, int64_t nbytes, int8_t* codes) {
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < nbytes; i += (int64_t)gridDim.x * kThreads) {
        const uint32_t b = in[i];
        uint32_t o = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) o |= (uint32_t)((((b >> (2 * j)) & 3u) - 1u) & 0xFFu) << (8 * j);
        reinterpret_cast<uint32_t*>(codes)[i] = o;
    }
}

__global__ __launch_bounds__(kThreads) void unpack1_kernel(const uint8_t* in, int64_t nbytes, int8_t* codes) {
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < nbytes; i += (int64_t)gridDim.x * kThreads) {
        const uint32_t b = in[i];
        uint32_t o[2] = {0, 0};
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j >> 2] |= (((b >> j) & 1u) ? 0x01u : 0xFFu) << (8 * (j & 3));
        reinterpret_cast<uint2*>(codes)[i] = make_uint2(o[0], o[1]);
    }
}

static int pack_grid(int64_t nbytes) {
    int64_t g = (nbytes + kThreads * 4 - 1) / (kThreads * 4);
    if (g < 1) g = 1;
    if (g > 16384) g = 16384;
    return (int)g;
}

hipError_t launch_pack(const int8_t* codes, int64_t count, int bits, uint8_t* packed, hipStream_t st) {
    const int64_t nbytes = count * bits / 8;
    if (nbytes == 0) return hipSuccess;
    if (bits == 2) pack2_kernel<<<pack_grid(nbytes), kThreads, 0, st>>>(codes, nbytes, packed);
    else pack1_kernel<<<pack_grid(nbytes), kThreads, 0, st>>>(codes, nbytes, packed);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* packed, int64_t count, int bits, int8_t* codes, hipStream_t st) {
    const int64_t nbytes = count * bits / 8;
    if (nbytes == 0) return hipSuccess;
    if (bits == 2) unpack2_kernel<<<pack_grid(nbytes), kThreads, 0, st>>>(packed, nbytes, codes);
    else unpack1_kernel<<<pack_grid(nbytes), kThreads, 0, st>>>(packed, nbytes, codes);
    return hipGetLastError();
}

}  // namespace qg
