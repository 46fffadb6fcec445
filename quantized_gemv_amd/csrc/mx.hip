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
// One thread per 8 consecutive values, kMxQU such groups kThreads apart with
// all loads issued first (clamped into range, so none waits behind a branch);
// the 4 threads of a 32-block are consecutive lanes of one quad (DPP quad
// permutes give the block max).
//
// The rounding is gfx950's scaled conversion (v_cvt_scalef32_pk_fp4_*): it
// divides each input by the E8M0 scale given in a float's exponent field and
// rounds to the nearest E2M1 value, ties to even, saturating at 6 -- the
// element rule above, two values per instruction.  One difference is removed
// before it: the instruction keeps the sign of -0, whose code here is +0, so
// negative zeros are cleared first (a negative value that rounds to zero
// keeps its sign bit, as the element rule says).
constexpr int kMxQU = 2;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// the bf16 pair in w with a -0 half turned into +0
__device__ __forceinline__ uint32_t bf16x2_clear_neg_zero(uint32_t w) {
    const uint32_t mag = w & 0x7FFF7FFFu;
    const uint32_t nonzero = (mag + 0x7FFF7FFFu) & 0x80008000u;  // bit 15 / 31 set where a half is nonzero
    return mag | (w & nonzero);
}

template <int XT>
__global__ __launch_bounds__(kThreads) void mxfp4_quantize_kernel(const void* x, int64_t rows, int64_t cols,
                                                                 uint8_t* codes, uint8_t* scales) {
    const int64_t n8 = rows * cols / 8;
    const int64_t nb = cols / 32;  // blocks per row
    const bool idx32 = rows * nb <= (int64_t)0xFFFFFFFF;  // block index fits 32 bits: cheaper division
    const int64_t stride = (int64_t)gridDim.x * kThreads * kMxQU;
    for (int64_t g0 = (int64_t)blockIdx.x * kThreads * kMxQU + threadIdx.x; g0 < n8; g0 += stride) {
        uint32_t w[kMxQU][8];  // bf16: 4 pairs; fp32: 8 values (bits)
#pragma unroll
        for (int u = 0; u < kMxQU; ++u) {
            const int64_t g = min(g0 + (int64_t)u * kThreads, n8 - 1);
            if constexpr (XT == 1) {
                const uint4 h = reinterpret_cast<const uint4*>(x)[g];
                w[u][0] = h.x; w[u][1] = h.y; w[u][2] = h.z; w[u][3] = h.w;
            } else {
                const uint4 a = reinterpret_cast<const uint4*>(x)[2 * g];
                const uint4 b = reinterpret_cast<const uint4*>(x)[2 * g + 1];
                w[u][0] = a.x; w[u][1] = a.y; w[u][2] = a.z; w[u][3] = a.w;
                w[u][4] = b.x; w[u][5] = b.y; w[u][6] = b.z; w[u][7] = b.w;
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // keep every load issued before the first use
#pragma unroll
        for (int u = 0; u < kMxQU; ++u) {
            // block max |v| (as bits: magnitudes of finite values order as integers)
            uint32_t mb;
            if constexpr (XT == 1) {
                u16x2_t m2 = __builtin_bit_cast(u16x2_t, w[u][0] & 0x7FFF7FFFu);
#pragma unroll
                for (int j = 1; j < 4; ++j)
                    m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_t, w[u][j] & 0x7FFF7FFFu));
                mb = (uint32_t)max(m2.x, m2.y) << 16;
            } else {
                mb = w[u][0] & 0x7FFFFFFFu;
#pragma unroll
                for (int j = 1; j < 8; ++j) mb = max(mb, w[u][j] & 0x7FFFFFFFu);
            }
            mb = max(mb, (uint32_t)dpp_mov<0xB1>((int)mb));  // quad_perm [1,0,3,2]
            mb = max(mb, (uint32_t)dpp_mov<0x4E>((int)mb));  // quad_perm [2,3,0,1]
            // floor(log2 m) is the unbiased exponent of m (exact); subnormal m
            // and the lowest binade clamp to -127
            const int E = (int)(mb >> 23);
            const int e = (mb == 0u) ? 0 : max(E - 129, -127);
            const float sc = __uint_as_float((uint32_t)(e + 127) << 23);  // E8M0 scale in the exponent field
            uint32_t packed = 0;
            if constexpr (XT == 1) {
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, bf16x2_clear_neg_zero(w[u][0])), sc, 0);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, bf16x2_clear_neg_zero(w[u][1])), sc, 1);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, bf16x2_clear_neg_zero(w[u][2])), sc, 2);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, bf16x2_clear_neg_zero(w[u][3])), sc, 3);
            } else {
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(w[u][j]) + 0.0f;  // -0 + 0 = +0
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[0], v[1], sc, 0);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[2], v[3], sc, 1);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[4], v[5], sc, 2);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[6], v[7], sc, 3);
            }
            const int64_t g = g0 + (int64_t)u * kThreads;
            if (g < n8) {
                reinterpret_cast<uint32_t*>(codes)[g] = packed;
                if ((g & 3) == 0) {
                    int64_t r, b;  // row, block
                    if (idx32) {
                        const uint32_t gb = (uint32_t)(g >> 2), r32 = gb / (uint32_t)nb;
                        r = r32;
                        b = gb - r32 * (uint32_t)nb;
                    } else {
                        r = (g >> 2) / nb;
                        b = (g >> 2) - r * nb;
                    }
                    scales[((b >> 3) * rows + r) * 8 + (b & 7)] = (uint8_t)(e + 127);
                }
            }
        }
    }
}

hipError_t launch_quantize_mxfp4(const void* x, int xt, int64_t rows, int64_t cols, uint8_t* codes,
                                 uint8_t* scales, hipStream_t st) {
    const int64_t n8 = rows * cols / 8;
    const int64_t want = (n8 + (int64_t)kThreads * kMxQU - 1) / ((int64_t)kThreads * kMxQU);
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
        auto frags = [&](int kk, i32x4 (&fa)[WTM], i32x4 (&fb)[WTN], int (&xa)[WTM], int (&xb)[WTN]) {
            const int c = kk * 2 + (lane >> 5);  // 16-byte chunk = one 32-element block
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
        };
        // two register sets: the reads of step kk + 1 go out before the MFMAs of step kk
        i32x4 fa[2][WTM], fb[2][WTN];
        int xa[2][WTM], xb[2][WTN];
        frags(0, fa[0], fb[0], xa[0], xb[0]);
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            if (kk + 1 < BK / 32) frags(kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1], xa[(kk + 1) & 1], xb[(kk + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int a = 0; a < WTM; ++a)
#pragma unroll
                for (int b = 0; b < WTN; ++b) {
                    const i32x4 fA = fa[kk & 1][a], fB = fb[kk & 1][b];
                    const i32x8 A = {fA[0], fA[1], fA[2], fA[3], 0, 0, 0, 0};
                    const i32x8 B = {fB[0], fB[1], fB[2], fB[3], 0, 0, 0, 0};
                    // cbsz = blgp = 4: both operands E2M1; scale byte 0 of xa / xb
                    acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[a][b], 4, 4, 0, xa[kk & 1][a],
                                                                                0, xb[kk & 1][b]);
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
