// pack.hip -- bit packing of ternary (2-bit), sign (1-bit) and base-3
// ternary (five per byte) codes; int8 codes in 16-row tiles for the
// small-batch products.
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

// ---------------------------------------------------------------- base 3
// Five ternary digits f = q + 1 per byte, leading digit first, stored as the
// base-3 fraction rounded up to 8 bits, t = ceil(256 v / 243); a row takes
// rb = 16 * ceil(k / 80) bytes and the weights past k are digit 1 (q = 0).
// One thread per packed byte.
__global__ __launch_bounds__(kThreads) void pack3_kernel(const int8_t* codes, int64_t n, int64_t k, int64_t rb,
                                                         uint8_t* out) {
    const int64_t total = n * rb;
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
        const int64_t r = i / rb, j = i - r * rb;
        uint32_t v = 0;
#pragma unroll
        for (int t = 0; t < 5; ++t) {
            const int64_t c = 5 * j + t;
            const uint32_t f = c < k ? (uint32_t)((int)codes[r * k + c] + 1) : 1u;
            v = 3u * v + f;
        }
        out[i] = (uint8_t)((256u * v + 242u) / 243u);
    }
}

// digits by repeated multiplication by 3: digit = (3 t) >> 8, t = (3 t) & 255
__global__ __launch_bounds__(kThreads) void unpack3_kernel(const uint8_t* in, int64_t n, int64_t k, int64_t rb,
                                                           int8_t* codes) {
    const int64_t total = n * rb;
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
        const int64_t r = i / rb, j = i - r * rb;
        uint32_t t = in[i];
#pragma unroll
        for (int d = 0; d < 5; ++d) {
            const uint32_t m = 3u * t;
            t = m & 255u;
            const int64_t c = 5 * j + d;
            if (c < k) codes[r * k + c] = (int8_t)((int)(m >> 8) - 1);
        }
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

// 16-row tiles: output chunk q (16 bytes) is lane L = q % 64 of unit
// c = (q / 64) % C of tile t = q / (64 C): row 16 t + L % 16, codes
// 64 c + 16 (L / 16) .. + 15; rows past n are zeros.  Writes are contiguous.
__global__ __launch_bounds__(kThreads) void pack_tiles16_kernel(const int8_t* codes, int64_t n, int64_t k,
                                                                int64_t chunks, int8_t* out) {
    const int64_t C = k / 64;
    for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < chunks; q += (int64_t)gridDim.x * kThreads) {
        const int L = (int)(q & 63);
        const int64_t c = (q >> 6) % C;
        const int64_t t = (q >> 6) / C;
        const int64_t row = 16 * t + (L & 15);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row < n) v = *reinterpret_cast<const u32x4*>(codes + row * k + 64 * c + 16 * (L >> 4));
        *reinterpret_cast<u32x4*>(out + 16 * q) = v;
    }
}

int64_t tiles16_bytes(int64_t n, int64_t k) { return (n + 15) / 16 * 16 * k; }

hipError_t launch_pack_tiles16(const int8_t* codes, int64_t n, int64_t k, int8_t* out, hipStream_t st) {
    const int64_t chunks = tiles16_bytes(n, k) / 16;
    pack_tiles16_kernel<<<pack_grid(chunks), kThreads, 0, st>>>(codes, n, k, chunks, out);
    return hipGetLastError();
}

hipError_t launch_pack3(const int8_t* codes, int64_t n, int64_t k, uint8_t* packed, hipStream_t st) {
    const int64_t rb = 16 * ((k + 79) / 80);
    pack3_kernel<<<pack_grid(n * rb), kThreads, 0, st>>>(codes, n, k, rb, packed);
    return hipGetLastError();
}

hipError_t launch_unpack3(const uint8_t* packed, int64_t n, int64_t k, int8_t* codes, hipStream_t st) {
    const int64_t rb = 16 * ((k + 79) / 80);
    unpack3_kernel<<<pack_grid(n * rb), kThreads, 0, st>>>(packed, n, k, rb, codes);
    return hipGetLastError();
}

}  // namespace qg
