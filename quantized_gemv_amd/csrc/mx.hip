// mx.hip -- MXFP4 (OCP microscaling: E2M1 elements, one E8M0 scale per 32
// along K) quantization and GEMM for the format-separated prefill (gfx950).
//
// [DQ] (quantization split by inference phase): "format separation" runs
// the prefill on the accelerator's native low-bit compute while decode keeps
// a low-bit weight-only format.  MI355X's matrix cores take MXFP4 natively
// (v_mfma_scale_f32_32x32x64_f8f6f4, twice the int8 rate), so the prefill
// quantizes the activations per 32-block and multiplies them with MXFP4
// weights.
//
// Format (rows of K values):
//   codes  [R][K/2] bytes: element 2j in the low nibble of byte j; a code is
//          sign (bit 3) | E2M1 magnitude code (0..7 = 0, 0.5, 1, 1.5, 2, 3, 4, 6);
//   scales [K/256][R][8] E8M0 bytes (the 8 block scales of 256 values of a
//          row, all rows of one 256-slice of K together; K % 256 == 0):
//          block exponent e + 127, with
//          e = floor(log2 max|v|) - 2 clamped to [-127, 127] (0 for an
//          all-zero block); an element is the E2M1 value nearest to v / 2^e
//          (ties to the even code, saturating at 6).
//
// GEMM: Y[m][n] = sum_k A[m][k] B[n][k] in fp32 (products exact, the scales
// applied by the instruction).  The tiling is the int8 prefill GEMM's (256 x
// 128 workgroup tile, 8 waves of 2 x 2 tiles of 32 x 32, a 3-stage LDS ring
// fed by direct global->LDS loads, XOR-swizzled 16-byte chunks), with K
// steps of 256 elements (128 bytes per row) and the stage's scale bytes (8
// per row, contiguous over rows in the slice-major layout, so a 256-byte
// wave load of them touches two cache lines) staged beside the codes: a
// 16-byte fragment chunk is exactly one 32-element block, so lane l of a
// fragment also reads its block's scale.
#include "qg_device.h"
#include "qg_gemm.h"

namespace qg {

// ------------------------------------------------------------------ quantizer
// One thread per 8 consecutive values; the 4 threads of a 32-block are
// consecutive lanes (shuffles give the block max).
template <int XT>
__global__ __launch_bounds__(kThreads) void mxfp4_quantize_kernel(const void* x, int64_t rows, int64_t cols,
                                                                  uint8_t* codes, uint8_t* scales) {
    const int64_t n8 = rows * cols / 8;
    const int64_t nb = cols / 32;  // blocks per row
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < n8; g += stride) {
        float v[8];
        if constexpr (XT == 1) {
            const uint4 h = reinterpret_cast<const uint4*>(x)[g];
            const uint32_t w[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
                v[2 * e + 1] = bf16_to_f32(w[e] >> 16);
            }
        } else {
            const float4 a = reinterpret_cast<const float4*>(x)[2 * g];
            const float4 b = reinterpret_cast<const float4*>(x)[2 * g + 1];
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        }
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(v[j]));
        m = __builtin_fmaxf(m, __shfl_xor(m, 1, kWave));
        m = __builtin_fmaxf(m, __shfl_xor(m, 2, kWave));
        // floor(log2 m) is the unbiased exponent of m (exact); subnormal m
        // and the lowest binade clamp to -127
        const int E = (int)(__float_as_uint(m) >> 23);
        const int e = (m == 0.0f) ? 0 : max(E - 129, -127);
        const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e (127 - e in [2, 254])
        uint32_t packed = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float a = __builtin_fabsf(v[j]) * inv;  // exact
            // nearest E2M1 value: count the midpoints below, ties to the even code
            const uint32_t mag = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                                 (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                                 (uint32_t)(a > 5.0f);
            packed |= (mag | (v[j] < 0.0f ? 8u : 0u)) << (4 * j);
        }
        reinterpret_cast<uint32_t*>(codes)[g] = packed;
        if ((g & 3) == 0) {
            const int64_t r = (g >> 2) / nb, b = (g >> 2) - r * nb;  // row, block
            scales[((b >> 3) * rows + r) * 8 + (b & 7)] = (uint8_t)(e + 127);
        }
    }
}

hipError_t launch_quantize_mxfp4(const void* x, int xt, int64_t rows, int64_t cols, uint8_t* codes,
                                 uint8_t* scales, hipStream_t st) {
    const int64_t n8 = rows * cols / 8;
    const int64_t want = (n8 + kThreads - 1) / kThreads;
    const int grid = (int)(want < 16384 ? want : 16384);
    if (xt == 1) mxfp4_quantize_kernel<1><<<grid, kThreads, 0, st>>>(x, rows, cols, codes, scales);
    else mxfp4_quantize_kernel<0><<<grid, kThreads, 0, st>>>(x, rows, cols, codes, scales);
    return hipGetLastError();
}

// ------------------------------------------------------------------ GEMM
struct MxParams {
    const uint8_t* a;   // [M][K/2]
    const uint8_t* as;  // [K/256][M][8]
    const uint8_t* b;   // [N][K/2]
    const uint8_t* bs;  // [K/256][N][8]
    float* y;           // [M][N]
    int M, N, K;
    int tiles_m, tiles_n;
};

template <int WAVES_M, int WAVES_N, int WTM, int WTN, int STAGES>
struct MxCfg {
    typedef Cfg<WAVES_M, WAVES_N, WTM, WTN, 128, STAGES> C;  // 128 bytes = 256 elements per row per stage
    static constexpr int kScaleBytes = (C::BM + C::BN) * 8;    // 8 scale bytes per row per stage
    static constexpr int kScaleLoads = kScaleBytes / 256;      // 4-byte DMA: 256 bytes per wave load
    static constexpr int kSLPW = (kScaleLoads + C::kWavesT - 1) / C::kWavesT;  // per wave (extra ones repeat the last)
    static constexpr int kStage = C::kStageBytes + kScaleBytes;
    static constexpr int kLPS = C::kLPS + kSLPW;
    static constexpr size_t kLds = (size_t)STAGES * kStage;
    static_assert(kScaleBytes % 256 == 0, "scale rows fill whole wave loads");
};

template <int WAVES_M, int WAVES_N, int WTM, int WTN, int STAGES>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_mxfp4_kernel(MxParams p) {
    typedef MxCfg<WAVES_M, WAVES_N, WTM, WTN, STAGES> MC;
    typedef typename MC::C CF;
    constexpr int BM = CF::BM, BN = CF::BN, BK = CF::BK, CPR = CF::CPR;
    constexpr int kStageA = CF::kStageA;
    constexpr int kNW = CF::kWavesT;
    constexpr int kDataLoads = CF::kLPS;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int KB = p.K / 2;    // code bytes per row

    // XCD-aware tile order (as the int8 GEMM): each XCD gets a contiguous run
    // of the tile sequence, rasterised in supertiles of 4 M-tiles
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

    // ---- DMA plan: the codes as in the int8 GEMM (A rows, then B rows, BK
    // bytes each, chunks swizzled), then the scales: row R's 8 bytes of the
    // stage at kStageBytes + 8 R (wave load j covers rows 32 j .. 32 j + 31;
    // in global memory slice ks of row r is at (ks * rows + r) * 8)
    const uint8_t* src[kDataLoads];
#pragma unroll
    for (int l = 0; l < kDataLoads; ++l) {
        const int blk = wave + kNW * l;
        const int row = blk * CF::kRowsPerLoad + lane / CPR;
        const int pc = lane % CPR;
        if (row < BM) {
            const int gm = min(m0 + row, p.M - 1);
            src[l] = p.a + (int64_t)gm * KB + 16 * swz<CPR>(row, pc);
        } else {
            const int rb = row - BM;
            const int gn = min(n0 + rb, p.N - 1);
            src[l] = p.b + (int64_t)gn * KB + 16 * swz<CPR>(rb, pc);
        }
    }
    const uint8_t* ssrc[MC::kSLPW];
    int sdst[MC::kSLPW];
#pragma unroll
    for (int l = 0; l < MC::kSLPW; ++l) {
        const int j = min(wave + kNW * l, MC::kScaleLoads - 1);
        const int R = 32 * j + lane / 2;
        const int d = lane & 1;
        if (R < BM) ssrc[l] = p.as + (int64_t)min(m0 + R, p.M - 1) * 8 + 4 * d;
        else ssrc[l] = p.bs + (int64_t)min(n0 + R - BM, p.N - 1) * 8 + 4 * d;
        sdst[l] = CF::kStageBytes + 256 * j;
    }
    int64_t sstr[MC::kSLPW];  // bytes per K slice of the A or B scales this lane loads
#pragma unroll
    for (int l = 0; l < MC::kSLPW; ++l)
        sstr[l] = (32 * min(wave + kNW * l, MC::kScaleLoads - 1) + lane / 2) < BM ? (int64_t)p.M * 8 : (int64_t)p.N * 8;
    auto issue_stage = [&](int ks) {
        uint8_t* base = smem + (ks % STAGES) * MC::kStage;
#pragma unroll
        for (int l = 0; l < kDataLoads; ++l) {
            const int blk = wave + kNW * l;
            dma16(src[l] + (int64_t)ks * BK, base + blk * 1024);
        }
#pragma unroll
        for (int l = 0; l < MC::kSLPW; ++l) dma4(ssrc[l] + (int64_t)ks * sstr[l], base + sdst[l]);
    };

    f32x16 acc[WTM][WTN];
#pragma unroll
    for (int a = 0; a < WTM; ++a)
#pragma unroll
        for (int b = 0; b < WTN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    const int nk = p.K / 256;
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        if (s < nk) issue_stage(s);

    const int hs = 8 * (lane >> 5);  // this lane's block within a 64-element MFMA step: bit shift of its scale byte
    for (int ks = 0; ks < nk; ++ks) {
        wait_stage<MC::kLPS, STAGES - 2>(min(STAGES - 2, nk - 1 - ks));
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (ks + STAGES - 1 < nk) issue_stage(ks + STAGES - 1);

        const uint8_t* sa = smem + (ks % STAGES) * MC::kStage;
        const uint8_t* sb = sa + kStageA;
        const uint8_t* sc = sa + CF::kStageBytes;
        uint2 scA[WTM], scB[WTN];  // the 8 block scales of each fragment row
#pragma unroll
        for (int a = 0; a < WTM; ++a)
            scA[a] = *reinterpret_cast<const uint2*>(sc + 8 * (wm * (WTM * 32) + a * 32 + (lane & 31)));
#pragma unroll
        for (int b = 0; b < WTN; ++b)
            scB[b] = *reinterpret_cast<const uint2*>(sc + 8 * (BM + wn * (WTN * 32) + b * 32 + (lane & 31)));
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            const int c = kk * 2 + (lane >> 5);  // 16-byte chunk = one 32-element block
            i32x4 fa[WTM], fb[WTN];
            int xa[WTM], xb[WTN];
#pragma unroll
            for (int a = 0; a < WTM; ++a) {
                const int r = wm * (WTM * 32) + a * 32 + (lane & 31);
                fa[a] = *reinterpret_cast<const i32x4*>(sa + r * BK + 16 * swz<CPR>(r, c));
                xa[a] = (int)((kk < 2 ? scA[a].x : scA[a].y) >> (16 * (kk & 1) + hs));
            }
#pragma unroll
            for (int b = 0; b < WTN; ++b) {
                const int r = wn * (WTN * 32) + b * 32 + (lane & 31);
                fb[b] = *reinterpret_cast<const i32x4*>(sb + r * BK + 16 * swz<CPR>(r, c));
                xb[b] = (int)((kk < 2 ? scB[b].x : scB[b].y) >> (16 * (kk & 1) + hs));
            }
#pragma unroll
            for (int a = 0; a < WTM; ++a)
#pragma unroll
                for (int b = 0; b < WTN; ++b) {
                    const i32x8 A = {fa[a][0], fa[a][1], fa[a][2], fa[a][3], 0, 0, 0, 0};
                    const i32x8 B = {fb[b][0], fb[b][1], fb[b][2], fb[b][3], 0, 0, 0, 0};
                    // cbsz = blgp = 4: both operands E2M1; scale byte 0 of xa / xb
                    acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[a][b], 4, 4, 0, xa[a], 0,
                                                                                xb[b]);
                }
        }
    }

    // ---- epilogue: lane l holds column l % 32, rows 8 (r / 4) + 4 (l / 32) + r % 4
    const int wr0 = m0 + wm * (WTM * 32);
    const int wc0 = n0 + wn * (WTN * 32);
#pragma unroll
    for (int a = 0; a < WTM; ++a) {
#pragma unroll
        for (int b = 0; b < WTN; ++b) {
            const int col = wc0 + b * 32 + (lane & 31);
            if (col < p.N) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = wr0 + a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (row < p.M) p.y[(int64_t)row * p.N + col] = acc[a][b][r];
                }
            }
        }
    }
}

template <int WAVES_M, int WAVES_N, int WTM, int WTN, int STAGES>
static hipError_t run_mx(MxParams p, hipStream_t st) {
    typedef MxCfg<WAVES_M, WAVES_N, WTM, WTN, STAGES> MC;
    auto kern = gemm_mxfp4_kernel<WAVES_M, WAVES_N, WTM, WTN, STAGES>;
    p.tiles_m = (p.M + MC::C::BM - 1) / MC::C::BM;
    p.tiles_n = (p.N + MC::C::BN - 1) / MC::C::BN;
    static bool attr_set = false;  // per instantiation
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)MC::kLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    kern<<<p.tiles_m * p.tiles_n, MC::C::kThreadsT, MC::kLds, st>>>(p);
    return hipGetLastError();
}

hipError_t launch_gemm_mxfp4(const uint8_t* a, const uint8_t* as, int64_t m, int64_t k, const uint8_t* b,
                             const uint8_t* bs, int64_t n, float* y, hipStream_t st) {
    MxParams p;
    p.a = a;
    p.as = as;
    p.b = b;
    p.bs = bs;
    p.y = y;
    p.M = (int)m;
    p.N = (int)n;
    p.K = (int)k;
    return run_mx<4, 2, 2, 2, 3>(p, st);
}

}  // namespace qg
