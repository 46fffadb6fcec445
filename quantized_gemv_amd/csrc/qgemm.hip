// qgemm.hip -- W8A8 prefill GEMM with the activation outlier split (gfx950).
//
// Y[m][n] = acc[m][n] / (s_x[m] * s_w[n]) + sum_j X_out[m][j] * W_out[n][j]
// acc     = Xq . Wq^T over K (int32, exact), both operands K-contiguous.
//
// Prefill is the one dense contraction on the path, so the int8 part runs on
// the matrix cores (v_mfma_i32_32x32x32_i8: a 32x32 int32 tile, K = 32 per
// instruction).  The outlier channels (a few, zero-padded to a multiple of
// 16) are added in the epilogue with v_mfma_f32_32x32x16_bf16, whose fp32
// accumulator starts from the rescaled int32 result.
//
// Tiling: a 256-thread workgroup computes a 256 (M) x 128 (N) tile, each of
// its four waves a 128 x 64 sub-tile (4 x 2 MFMA tiles, 128 accumulator
// registers).  K advances 64 at a time through a 4-stage LDS ring filled by
// direct global->LDS loads (global_load_lds_dwordx4: lane i's 16 bytes land
// at LDS base + 16 i), so staging costs no registers and three K steps are in
// flight while one is multiplied.  Rows are stored in LDS with their four
// 16-byte chunks XOR-permuted by (row / 2) mod 4, so the eight rows read
// together by a fragment load fall in eight different bank groups.
// Workgroups are mapped XCD-aware: the 32 workgroups that share an XCD (and
// its L2) cover a 4 x 8 block of tiles, so A and B panels are reused there.
//
// MFMA operand convention: lane l supplies row (l % 32) of A (column (l % 32)
// of B) and a contiguous run of K elements selected by (l / 32); A and B use
// the same selection, so the instruction's internal pairing of K elements
// always yields the full dot product.  The 32x32 result tile has column
// l % 32 and row 8 * (r / 4) + 4 * (l / 32) + (r % 4) for accumulator r.
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int kStages = 4;
constexpr int kStageA = BM * BK;               // bytes of A per stage
constexpr int kStageB = BN * BK;               // bytes of B per stage
constexpr int kStageBytes = kStageA + kStageB;  // 24 KB
constexpr int kLoadsPerStage = (kStageBytes / 1024) / kWaves;  // 1 KB wave loads per wave per stage (6)

struct GemmParams {
    const int8_t* xq;       // [M][K]
    const int8_t* wq;       // [N][K]
    const float* s_x;       // [M]
    const float* s_w;       // [N]
    const uint16_t* x_out;  // [M][ld] bf16, zero beyond n_out
    const uint16_t* w_out;  // [N][n_out] bf16
    float* y;               // [M][N]
    int32_t* acc_out;       // [M][N] or null
    int M, N, K, n_out, ld;
    int tiles_m, tiles_n;
};

// physical 16-byte chunk of logical chunk c in tile row r
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 3); }

// s_waitcnt vmcnt(n) with expcnt / lgkmcnt left unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__global__ __launch_bounds__(kThreads) void qgemm_w8a8_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves of 128 x 64

    // ---------------------------------------------------------------- tile
    // XCD-aware order: consecutive dispatches go to different XCDs, so give
    // each XCD a contiguous run of the tile sequence, rasterised in
    // supertiles of 4 M-tiles (a run of 32 covers a 4 x 8 block).
    const int G = gridDim.x;
    int t = blockIdx.x;
    if ((G & 7) == 0) t = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const int st_rows = 4 * p.tiles_n;
    const int st = t / st_rows;
    const int u = t - st * st_rows;
    const int h = min(4, p.tiles_m - 4 * st);
    const int tile_m = 4 * st + u % h;
    const int tile_n = u / h;
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    // ---------------------------------------------------------------- DMA plan
    // Stage layout: A rows 0..255 then B rows 0..127, 64 bytes each.  A wave
    // load fills 16 consecutive rows (1 KB); wave w issues loads
    // w, w + 4, ... (6 per stage).  Lane i fills row (i / 4), physical chunk
    // (i % 4), i.e. it fetches logical chunk swz(row, i % 4).
    const int8_t* src[kLoadsPerStage];
#pragma unroll
    for (int l = 0; l < kLoadsPerStage; ++l) {
        const int blk = wave + kWaves * l;     // 0..23: 16-row block of the stage
        const int row = blk * 16 + (lane >> 2);  // 0..383
        const int pc = lane & 3;
        if (row < BM) {
            const int gm = min(m0 + row, p.M - 1);
            src[l] = p.xq + (int64_t)gm * p.K + 16 * swz(row, pc);
        } else {
            const int rb = row - BM;
            const int gn = min(n0 + rb, p.N - 1);
            src[l] = p.wq + (int64_t)gn * p.K + 16 * swz(rb, pc);
        }
    }
    auto issue_stage = [&](int ks) {
        uint8_t* base = smem + (ks % kStages) * kStageBytes;
#pragma unroll
        for (int l = 0; l < kLoadsPerStage; ++l) {
            const int blk = wave + kWaves * l;
            __builtin_amdgcn_global_load_lds(src[l] + (int64_t)ks * BK, (lds_ptr_t)(base + blk * 1024), 16, 0, 0);
        }
    };

    i32x16 acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

    const int nk = p.K / BK;
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < nk) issue_stage(s);

    for (int ks = 0; ks < nk; ++ks) {
        // stage ks has landed once at most the loads of the later issued
        // stages are outstanding (loads retire in order)
        if (ks + 2 < nk) wait_vmcnt<2 * kLoadsPerStage>();
        else if (ks + 1 < nk) wait_vmcnt<kLoadsPerStage>();
        else wait_vmcnt<0>();
        // Every wave's part of stage ks is in LDS and stage ks-1 is no longer
        // read (its fragments were consumed by MFMAs, so their LDS reads are
        // complete).  A fenced __syncthreads would also wait for the DMA of
        // the stages still in flight; this barrier does not.
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (ks + kStages - 1 < nk) issue_stage(ks + kStages - 1);

        const uint8_t* sa = smem + (ks % kStages) * kStageBytes;
        const uint8_t* sb = sa + kStageA;
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            const int c = kk * 2 + (lane >> 5);
            i32x4 fa[4], fb[2];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int r = wm * 128 + a * 32 + (lane & 31);
                fa[a] = *reinterpret_cast<const i32x4*>(sa + r * BK + 16 * swz(r, c));
            }
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int r = wn * 64 + b * 32 + (lane & 31);
                fb[b] = *reinterpret_cast<const i32x4*>(sb + r * BK + 16 * swz(r, c));
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[a], fb[b], acc[a][b], 0, 0, 0);
        }
    }

    // ---------------------------------------------------------------- epilogue
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int tm = m0 + wm * 128 + a * 32;  // 32x32 tile origin
            const int tn = n0 + wn * 64 + b * 32;
            const int col = tn + (lane & 31);
            const float sw = p.s_w[min(col, p.N - 1)];
            f32x16 f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = tm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const float sx = p.s_x[min(row, p.M - 1)];
                f[r] = (float)acc[a][b][r] / (sx * sw);
            }
            for (int kb = 0; kb < p.ld; kb += 16) {
                const int kc = kb + (lane >> 5) * 8;
                const int arow = min(tm + (lane & 31), p.M - 1);
                const uint4 xa = *reinterpret_cast<const uint4*>(p.x_out + (int64_t)arow * p.ld + kc);
                uint32_t wb[4];
                const int bcol = min(col, p.N - 1);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int k0 = kc + 2 * q, k1 = k0 + 1;
                    const uint32_t lo = k0 < p.n_out ? p.w_out[(int64_t)bcol * p.n_out + k0] : 0u;
                    const uint32_t hi = k1 < p.n_out ? p.w_out[(int64_t)bcol * p.n_out + k1] : 0u;
                    wb[q] = lo | (hi << 16);
                }
                const uint4 wv = make_uint4(wb[0], wb[1], wb[2], wb[3]);
                f = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa),
                                                            __builtin_bit_cast(bf16x8, wv), f, 0, 0, 0);
            }
            if (col < p.N) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = tm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (row < p.M) {
                        p.y[(int64_t)row * p.N + col] = f[r];
                        if (p.acc_out) p.acc_out[(int64_t)row * p.N + col] = acc[a][b][r];
                    }
                }
            }
        }
    }
}

hipError_t launch_qgemm(const QgemmArgs& a, const OutlierIdx& idx, hipStream_t st) {
    hipError_t e = launch_absmax_split(a.x, a.m, a.k, idx, a.n_out, a.xq, a.s_x, a.x_out, a.x_out_ld, st);
    if (e != hipSuccess) return e;
    GemmParams p;
    p.xq = a.xq;
    p.wq = a.wq;
    p.s_x = a.s_x;
    p.s_w = a.s_w;
    p.x_out = a.x_out;
    p.w_out = a.w_out;
    p.y = a.y;
    p.acc_out = a.acc_out;
    p.M = (int)a.m;
    p.N = (int)a.n;
    p.K = (int)a.k;
    p.n_out = a.n_out;
    p.ld = a.x_out_ld;
    p.tiles_m = (int)((a.m + BM - 1) / BM);
    p.tiles_n = (int)((a.n + BN - 1) / BN);
    const size_t lds = (size_t)kStages * kStageBytes;  // 96 KB
    static bool attr_set = false;
    if (!attr_set) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(qgemm_w8a8_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int grid = p.tiles_m * p.tiles_n;
    qgemm_w8a8_kernel<<<grid, kThreads, lds, st>>>(p);
    return hipGetLastError();
}

}  // namespace qg
