// qg_gemm.h -- pieces shared by the matrix-core GEMM kernels (gfx950):
// fragment types, the LDS chunk swizzle, direct global->LDS loads, vmcnt
// waits and the tile / stage configuration.
#pragma once

#include "qg_launch.h"

namespace qg {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Physical 16-byte chunk of logical chunk c in tile row r, for CPR chunks per
// row.  The gfx950 LDS has 64 banks of 4 bytes and serves a 128-bit read 16
// lanes at a time; a fragment load's 16 lanes read 16 consecutive rows at the
// same logical chunk.  A row of CPR * 16 bytes covers 4 * CPR banks, so rows
// r and r + 64 / (4 * CPR) start on the same bank: XOR-ing the chunk with
// r / (64 / (4 * CPR)) gives the 16 rows 16 different 4-bank groups (measured
// on the prefill GEMM: no bank-conflict cycles, against 4 per read with the
// 8-row pattern of a 32-bank LDS).
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
    if constexpr (CPR == 4) return c ^ ((r >> 2) & 3);
    else return c ^ ((r >> 1) & 7);
}

// One 16-byte-per-lane direct global->LDS load; lane i's bytes land at
// lds_dst + 16 i.  (Kept in a non-template device function: the LDS
// address-space cast inside a lambda of the kernel template makes the host
// pass drop the kernel's host-side instantiation.)
__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_dst, 16, 0, 0);
}

// s_waitcnt vmcnt(n) with expcnt / lgkmcnt left unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// wait until at most `later` stages of LPS loads each are outstanding
template <int LPS, int MAXL>
__device__ __forceinline__ void wait_stage(int later) {
    if constexpr (MAXL >= 3) { if (later >= 3) { wait_vmcnt<3 * LPS>(); return; } }
    if constexpr (MAXL >= 2) { if (later == 2) { wait_vmcnt<2 * LPS>(); return; } }
    if constexpr (MAXL >= 1) { if (later == 1) { wait_vmcnt<LPS>(); return; } }
    wait_vmcnt<0>();
}

// Tile configuration: WAVES_M x WAVES_N waves, each computing WTM x WTN MFMA
// tiles of 32 x 32; K steps of BK through a ring of STAGES LDS buffers.
template <int WAVES_M, int WAVES_N, int WTM, int WTN, int BK_, int STAGES>
struct Cfg {
    static constexpr int kWavesT = WAVES_M * WAVES_N;
    static constexpr int kThreadsT = 64 * kWavesT;
    static constexpr int BM = WAVES_M * WTM * 32;
    static constexpr int BN = WAVES_N * WTN * 32;
    static constexpr int BK = BK_;
    static constexpr int CPR = BK / 16;                 // 16-byte chunks per row
    static constexpr int kRowsPerLoad = 64 / CPR;       // rows filled by one 1 KB wave load
    static constexpr int kStageA = BM * BK;
    static constexpr int kStageB = BN * BK;
    static constexpr int kStageBytes = kStageA + kStageB;
    static constexpr int kLoads = kStageBytes / 1024;   // wave loads per stage
    static constexpr int kLPS = kLoads / kWavesT;       // per wave
    static_assert(kLoads % kWavesT == 0, "stage must split evenly over the waves");
    static_assert(CPR == 4 || CPR == 8, "BK 64 or 128");
    static constexpr size_t kLds = (size_t)STAGES * kStageBytes;
};


// One 4-byte-per-lane direct global->LDS load; lane i's bytes land at
// lds_dst + 4 i.
__device__ __forceinline__ void dma4(const void* src, void* lds_dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_dst, 4, 0, 0);
}

}  // namespace qg
