// qg_device.h -- device helpers shared by the gfx950 kernels.
//
// Everything here is written for CDNA4 wave64: 256-thread workgroups are
// four waves, wave-level reductions use cross-lane shuffles, and streamed
// loads go through buffer resources so that out-of-range lanes read zeros
// instead of faulting.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "exact_mean.h"

namespace qg {

constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// Round-to-nearest-even narrowing of a finite fp32 to bf16 bits.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// ------------------------------------------------------------------ absmax step
// s = 127 / alpha as one IEEE fp32 division (the build keeps division
// correctly rounded); an all-zero group gets s = 1 so its codes are 0.  For
// alpha below about 3.7e-37 the quotient overflows: s is clamped to FLT_MAX,
// so codes stay finite (|x * s| < 127) and zeros stay 0.
__device__ __forceinline__ float absmax_scale(float alpha) {
    return alpha == 0.0f ? 1.0f : __builtin_fminf(127.0f / alpha, 3.40282347e38f);
}

// clip(round_half_even(fl32(x * s)), -127, 127).  The build disables FP
// contraction, so the product is rounded on its own before rint.
__device__ __forceinline__ int qcode(float x, float s) {
    float t = x * s;
    t = __builtin_rintf(t);
    t = __builtin_fminf(__builtin_fmaxf(t, -127.0f), 127.0f);
    return (int)t;
}

// ------------------------------------------------------------------ asymmetric step
// The range [lo, hi] of a group, widened to contain 0, goes to [-128, 127]:
// s = 255 / (hi - lo) (1 for an empty range) and z = rne(-128 - s * lo),
// clipped to int8; every product and sum is rounded on its own.
__device__ __forceinline__ void asym_params(float lo, float hi, float& s, float& z) {
    lo = __builtin_fminf(lo, 0.0f);
    hi = __builtin_fmaxf(hi, 0.0f);
    const float d = hi - lo;
    s = d == 0.0f ? 1.0f : __builtin_fminf(255.0f / d, 3.40282347e38f);  // clamped like absmax_scale
    const float t = s * lo;
    const float u = -128.0f - t;
    z = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(u), -128.0f), 127.0f);
}

// clip(round_half_even(fl32(fl32(x * s) + z)), -128, 127)
__device__ __forceinline__ int qcode_zp(float x, float s, float z) {
    const float t = x * s;
    float u = t + z;
    u = __builtin_rintf(u);
    u = __builtin_fminf(__builtin_fmaxf(u, -128.0f), 127.0f);
    return (int)u;
}

// ------------------------------------------------------------------ reductions

// DPP (data-parallel primitive) reductions: each step adds a lane permutation
// of the value within rows of 16 lanes (quad swaps, half-row and row
// mirrors), then row_bcast15 / row_bcast31 carry row totals into the upper
// rows.  The full 64-lane sum ends in lane 63.  No LDS round trips, and the
// chains of several rows are independent, so they interleave.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_mov(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

__device__ __forceinline__ float wave_sum_to_lane63(float v) {
    v += __int_as_float(dpp_mov<0xB1>(__float_as_int(v)));        // quad_perm [1,0,3,2]
    v += __int_as_float(dpp_mov<0x4E>(__float_as_int(v)));        // quad_perm [2,3,0,1]
    v += __int_as_float(dpp_mov<0x141>(__float_as_int(v)));       // row_half_mirror
    v += __int_as_float(dpp_mov<0x140>(__float_as_int(v)));       // row_mirror
    v += __int_as_float(dpp_mov<0x142, 0xA>(__float_as_int(v)));  // row_bcast:15 into rows 1, 3
    v += __int_as_float(dpp_mov<0x143, 0xC>(__float_as_int(v)));  // row_bcast:31 into rows 2, 3
    return v;
}

// max of non-negative values over the wave, in lane 63 (the lanes that the
// row_bcast steps leave out combine with 0, which cannot raise the max)
__device__ __forceinline__ float wave_max_to_lane63(float v) {
    v = __builtin_fmaxf(v, __int_as_float(dpp_mov<0xB1>(__float_as_int(v))));
    v = __builtin_fmaxf(v, __int_as_float(dpp_mov<0x4E>(__float_as_int(v))));
    v = __builtin_fmaxf(v, __int_as_float(dpp_mov<0x141>(__float_as_int(v))));
    v = __builtin_fmaxf(v, __int_as_float(dpp_mov<0x140>(__float_as_int(v))));
    v = __builtin_fmaxf(v, __int_as_float(dpp_mov<0x142, 0xA>(__float_as_int(v))));
    v = __builtin_fmaxf(v, __int_as_float(dpp_mov<0x143, 0xC>(__float_as_int(v))));
    return v;
}

__device__ __forceinline__ int wave_sum_to_lane63(int v) {
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0x141>(v);
    v += dpp_mov<0x140>(v);
    v += dpp_mov<0x142, 0xA>(v);
    v += dpp_mov<0x143, 0xC>(v);
    return v;
}

// Whole-wave reductions broadcast to every lane: the DPP chain to lane 63,
// then v_readlane (no LDS round trips).  All 64 lanes must be active.
// wave_max takes non-negative values only (see wave_max_to_lane63).
__device__ __forceinline__ float wave_max(float v) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_max_to_lane63(v)), 63));
}
__device__ __forceinline__ int wave_sum(int v) { return __builtin_amdgcn_readlane(wave_sum_to_lane63(v), 63); }

// Workgroup barrier for LDS traffic: waits for this wave's LDS (and scalar)
// operations only.  A fenced __syncthreads would also wait for every global
// load in flight, i.e. for prefetched data that the barrier does not guard.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Block-wide max / sum over a workgroup of NW waves; `scratch` holds >= NW
// elements of shared memory.  All threads receive the result.  Contains two
// barriers, so every thread of the block must call it.
template <int NW = kWaves>
__device__ __forceinline__ float block_max(float v, float* scratch) {
    v = wave_max(v);
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    if (lane == 0) scratch[w] = v;
    lds_barrier();
    float r = scratch[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) r = __builtin_fmaxf(r, scratch[i]);
    lds_barrier();
    return r;
}

template <int NW = kWaves>
__device__ __forceinline__ int block_sum_int(int v, int* scratch) {
    v = wave_sum(v);
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    if (lane == 0) scratch[w] = v;
    lds_barrier();
    int r = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) r += scratch[i];
    lds_barrier();
    return r;
}

// ------------------------------------------------------------------ buffer loads
// Raw buffer resource over [base, base + bytes): loads whose range ends past
// `bytes` return zeros (hardware range check), so tails need no branches.
// Word 3 0x00020000 is the gfx9-family raw 32-bit data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint16_t load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint8_t load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// Non-temporal loads (the gfx9.4/9.5 NT cache-policy bit, aux = 2) for data a
// launch reads exactly once, i.e. the weight streams: they do not displace
// the lines that are reused (the activations, tables) from the CU and L2
// caches.  Measured on the W8A16 decode step: 4254 -> 4597 GB/s.  Only for
// loads whose instruction consumes whole 128-byte lines: where two
// instructions share a line, the second one fetches it again.
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ u32x4 load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicyNT);
}
__device__ __forceinline__ uint32_t load4_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCachePolicyNT);
}

}  // namespace qg
