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
// Tiling: a 512-thread workgroup computes a 256 (M) x 128 (N) tile, each of
// its eight waves a 64 x 64 sub-tile (2 x 2 MFMA tiles; two waves per SIMD,
// so one wave's LDS waits are covered by the other's MFMAs).  K advances 128
// at a time through a 3-stage LDS ring filled by direct global->LDS loads
// (global_load_lds_dwordx4: lane i's 16 bytes land at LDS base + 16 i), so
// staging costs no registers and two K steps are in flight while one is
// multiplied.  Rows are stored in LDS with their 16-byte chunks
// XOR-permuted by the row index, so the eight rows read together by a
// fragment load fall in eight different bank groups.
// Workgroups are mapped XCD-aware: the 32 workgroups that share an XCD (and
// its L2) cover a 4 x 8 block of tiles, so A and B panels are reused there.
//
// MFMA operand convention: lane l supplies row (l % 32) of A (column (l % 32)
// of B) and a contiguous run of K elements selected by (l / 32); A and B use
// the same selection, so the instruction's internal pairing of K elements
// always yields the full dot product.  The 32x32 result tile has column
// l % 32 and row 8 * (r / 4) + 4 * (l / 32) + (r % 4) for accumulator r.
#include "qg_device.h"
#include "qg_gemm.h"

namespace qg {


struct GemmParams {
    const int8_t* xq;       // [M][K]
    const int8_t* wq;       // [N][K]
    const float* s_x;       // [M]
    const float* s_w;       // [N]
    const uint16_t* x_out;  // [M][x_ld] bf16, x_ld % 8 == 0 (columns < n_out are used)
    const uint16_t* w_out;  // [N][w_ld] bf16, w_ld % 8 == 0 (columns < n_out are used)
    float* y;               // [M][N]
    int32_t* acc_out;       // [M][N] or null
    int M, N, K, n_out, x_ld, w_ld;
    int tiles_m, tiles_n;
};

template <int WAVES_M, int WAVES_N, int WTM, int WTN, int BK_, int STAGES>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void qgemm_w8a8_kernel(GemmParams p) {
    typedef Cfg<WAVES_M, WAVES_N, WTM, WTN, BK_, STAGES> CF;
    constexpr int BM = CF::BM, BN = CF::BN, BK = CF::BK, CPR = CF::CPR;
    constexpr int kStageA = CF::kStageA, kStageBytes = CF::kStageBytes;
    constexpr int kLoadsPerStage = CF::kLPS;
    constexpr int kNW = CF::kWavesT;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

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
    // Stage layout: A rows 0..BM-1 then B rows 0..BN-1, BK bytes each.  A
    // wave load fills 64 / CPR consecutive rows (1 KB); wave w issues loads
    // w, w + kNW, ...  Lane i fills row i / CPR, physical chunk i % CPR, i.e.
    // it fetches logical chunk swz(row, i % CPR).
    const int8_t* src[kLoadsPerStage];
#pragma unroll
    for (int l = 0; l < kLoadsPerStage; ++l) {
        const int blk = wave + kNW * l;  // 1 KB block of the stage
        const int row = blk * CF::kRowsPerLoad + lane / CPR;
        const int pc = lane % CPR;
        if (row < BM) {
            const int gm = min(m0 + row, p.M - 1);
            src[l] = p.xq + (int64_t)gm * p.K + 16 * swz<CPR>(row, pc);
        } else {
            const int rb = row - BM;
            const int gn = min(n0 + rb, p.N - 1);
            src[l] = p.wq + (int64_t)gn * p.K + 16 * swz<CPR>(rb, pc);
        }
    }
    auto issue_stage = [&](int ks) {
        uint8_t* base = smem + (ks % STAGES) * kStageBytes;
#pragma unroll
        for (int l = 0; l < kLoadsPerStage; ++l) {
            const int blk = wave + kNW * l;
            dma16(src[l] + (int64_t)ks * BK, base + blk * 1024);
        }
    };

    i32x16 acc[WTM][WTN];
#pragma unroll
    for (int a = 0; a < WTM; ++a)
#pragma unroll
        for (int b = 0; b < WTN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

    const int nk = p.K / BK;
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) issue_stage(s);

    for (int ks = 0; ks < nk; ++ks) {
        // stage ks has landed once at most the loads of the later issued
        // stages are outstanding (loads retire in order)
        wait_stage<kLoadsPerStage, STAGES - 2>(min(STAGES - 2, nk - 1 - ks));
        // Every wave's part of stage ks is in LDS and stage ks-1 is no longer
        // read (its fragments were consumed by MFMAs, so their LDS reads are
        // complete).  A fenced __syncthreads would also wait for the DMA of
        // the stages still in flight; this barrier does not.
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (ks + STAGES - 1 < nk) issue_stage(ks + STAGES - 1);

        const uint8_t* sa = smem + (ks % STAGES) * kStageBytes;
        const uint8_t* sb = sa + kStageA;
        auto frags = [&](int kk, i32x4 (&fa)[WTM], i32x4 (&fb)[WTN]) {
            const int c = kk * 2 + (lane >> 5);
#pragma unroll
            for (int a = 0; a < WTM; ++a) {
                const int r = wm * (WTM * 32) + a * 32 + (lane & 31);
                fa[a] = *reinterpret_cast<const i32x4*>(sa + r * BK + 16 * swz<CPR>(r, c));
            }
#pragma unroll
            for (int b = 0; b < WTN; ++b) {
                const int r = wn * (WTN * 32) + b * 32 + (lane & 31);
                fb[b] = *reinterpret_cast<const i32x4*>(sb + r * BK + 16 * swz<CPR>(r, c));
            }
        };
        // fragments in two register sets: the LDS reads of step kk + 1 are
        // issued before the MFMAs of step kk (kept there by the scheduling
        // barrier), so their latency runs under those MFMAs
        i32x4 fa[2][WTM], fb[2][WTN];
        frags(0, fa[0], fb[0]);
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            if (kk + 1 < BK / 32) frags(kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int a = 0; a < WTM; ++a)
#pragma unroll
                for (int b = 0; b < WTN; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[kk & 1][a], fb[kk & 1][b], acc[a][b], 0, 0, 0);
        }
    }

    // ---------------------------------------------------------------- epilogue
    // Rescale: y = acc * (1 / s_x[m]) * (1 / s_w[n]) with v_rcp_f32
    // reciprocals (a few ulp in all, far inside the fp32 tolerance) instead of
    // one IEEE division per element.
    const int wr0 = m0 + wm * (WTM * 32);  // wave tile origin
    const int wc0 = n0 + wn * (WTN * 32);
    float inv_sw[WTN];
#pragma unroll
    for (int b = 0; b < WTN; ++b) inv_sw[b] = __builtin_amdgcn_rcpf(p.s_w[min(wc0 + b * 32 + (lane & 31), p.N - 1)]);
    f32x16 f[WTM][WTN];
#pragma unroll
    for (int a = 0; a < WTM; ++a) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = wr0 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const float isx = __builtin_amdgcn_rcpf(p.s_x[min(row, p.M - 1)]);
#pragma unroll
            for (int b = 0; b < WTN; ++b) f[a][b][r] = (float)acc[a][b][r] * isx * inv_sw[b];
        }
    }
    // Outlier channels: bf16 MFMA over the gathered activations [M][x_ld] and
    // the outlier weights [N][w_ld], K = 16 per instruction, added on top.
    // Rows are 16-B aligned (strides are multiples of 8 elements), so each
    // fragment is one 16-byte load; lanes whose 8 columns start at or past
    // the stride load nothing, and columns >= n_out are zeroed in registers
    // (the padding of the operands is never trusted).
    auto frag8 = [&](const uint16_t* row, int ld, int kc) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (kc < ld) v = *reinterpret_cast<const uint4*>(row + kc);
        const int live = p.n_out - kc;  // columns of this fragment that are real
        if (live < 8) {
            uint32_t h[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (2 * e >= live) h[e] = 0u;
                else if (2 * e + 1 >= live) h[e] &= 0xFFFFu;
            }
            v = make_uint4(h[0], h[1], h[2], h[3]);
        }
        return v;
    };
    for (int kb = 0; kb < p.n_out; kb += 16) {
        const int kc = kb + (lane >> 5) * 8;
        uint4 xa[WTM], wb[WTN];
#pragma unroll
        for (int a = 0; a < WTM; ++a)
            xa[a] = frag8(p.x_out + (int64_t)min(wr0 + a * 32 + (lane & 31), p.M - 1) * p.x_ld, p.x_ld, kc);
#pragma unroll
        for (int b = 0; b < WTN; ++b)
            wb[b] = frag8(p.w_out + (int64_t)min(wc0 + b * 32 + (lane & 31), p.N - 1) * p.w_ld, p.w_ld, kc);
#pragma unroll
        for (int a = 0; a < WTM; ++a)
#pragma unroll
            for (int b = 0; b < WTN; ++b)
                f[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa[a]),
                                                                  __builtin_bit_cast(bf16x8, wb[b]), f[a][b], 0, 0, 0);
    }
#pragma unroll
    for (int a = 0; a < WTM; ++a) {
#pragma unroll
        for (int b = 0; b < WTN; ++b) {
            const int col = wc0 + b * 32 + (lane & 31);
            if (col < p.N) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wr0 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (row < p.M) {
                        p.y[(int64_t)row * p.N + col] = f[a][b][r];
                        if (p.acc_out) p.acc_out[(int64_t)row * p.N + col] = acc[a][b][r];
                    }
                }
            }
        }
    }
}

template <int WAVES_M, int WAVES_N, int WTM, int WTN, int BK_, int STAGES>
static hipError_t run_gemm(const GemmParams& p0, hipStream_t st) {
    typedef Cfg<WAVES_M, WAVES_N, WTM, WTN, BK_, STAGES> C;
    auto kern = qgemm_w8a8_kernel<WAVES_M, WAVES_N, WTM, WTN, BK_, STAGES>;
    GemmParams p = p0;
    p.tiles_m = (p.M + C::BM - 1) / C::BM;
    p.tiles_n = (p.N + C::BN - 1) / C::BN;
    static bool attr_set = false;  // per instantiation
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::kLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    kern<<<p.tiles_m * p.tiles_n, C::kThreadsT, C::kLds, st>>>(p);
    return hipGetLastError();
}

hipError_t launch_qgemm(const QgemmArgs& a, hipStream_t st) {
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
    p.x_ld = a.x_out_ld;
    p.w_ld = a.w_out_ld;
    // 8 waves of 64 x 64 in a 256 x 128 tile, K steps of 128, 3 stages
    // (fastest of the configurations measured on MI355X at 2048 x 4096 x 4096)
    return run_gemm<4, 2, 2, 2, 128, 3>(p, st);
}

}  // namespace qg
