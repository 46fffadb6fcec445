// qgemm.hip -- W8A8 prefill GEMM with the activation outlier split (gfx950).
//
// Y[m][n] = acc[m][n] / (s_x[m] * s_w[n]) + sum_j X_out[m][j] * W_out[n][j]
// acc     = Xq . Wq^T over K (int32, exact), both operands K-contiguous.
//
// Prefill is the one dense contraction on the path, so the int8 part runs on
// the matrix cores: v_mfma_i32_32x32x32_i8 (32x32 int32 tile, K = 32 per
// instruction).  The outlier channels (a few, zero-padded to a multiple of
// 16) are added in the epilogue with v_mfma_f32_32x32x16_bf16, whose fp32
// accumulator starts from the rescaled int32 result.
//
// MFMA operand convention used throughout: lane l supplies row (l % 32) of A
// (column (l % 32) of B) and a contiguous run of K elements selected by
// (l / 32).  A and B use the same K-selection, so the hardware's pairing of
// those elements yields the full dot product whatever its internal order.
// The 32x32 result tile is laid out with column = l % 32 and
// row = 8 * (r / 4) + 4 * (l / 32) + (r % 4) for accumulator register r.
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 16;  // 80 B rows: 8 lanes x 16 B reads hit disjoint banks

struct GemmParams {
    const int8_t* xq;    // [M][K]
    const int8_t* wq;    // [N][K]
    const float* s_x;    // [M]
    const float* s_w;    // [N]
    const uint16_t* x_out;  // [M][ld] bf16, zero beyond n_out
    const uint16_t* w_out;  // [N][n_out] bf16
    float* y;               // [M][N]
    int32_t* acc_out;       // [M][N] or null
    int M, N, K, n_out, ld;
};

__global__ __launch_bounds__(kThreads) void qgemm_w8a8_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(16))) int8_t As[BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) int8_t Bs[BN * LDS_STRIDE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves, 64 x 64 each
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

    // global -> LDS staging: each thread moves 2 x 16 B of A and of B per K step
    int ga_row[2], ga_col[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int piece = tid + kThreads * i;  // 0..511: 128 rows x 4 pieces of 16 B
        ga_row[i] = piece >> 2;
        ga_col[i] = (piece & 3) * 16;
    }
    const int8_t* a_src[2];
    const int8_t* b_src[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int am = min(m0 + ga_row[i], p.M - 1);
        const int bn = min(n0 + ga_row[i], p.N - 1);
        a_src[i] = p.xq + (int64_t)am * p.K + ga_col[i];
        b_src[i] = p.wq + (int64_t)bn * p.K + ga_col[i];
    }

    i32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

    uint4 ra[2], rb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        ra[i] = *reinterpret_cast<const uint4*>(a_src[i]);
        rb[i] = *reinterpret_cast<const uint4*>(b_src[i]);
    }

    const int ksteps = p.K / BK;
    for (int ks = 0; ks < ksteps; ++ks) {
        __syncthreads();  // previous step's LDS reads are done
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            *reinterpret_cast<uint4*>(As + ga_row[i] * LDS_STRIDE + ga_col[i]) = ra[i];
            *reinterpret_cast<uint4*>(Bs + ga_row[i] * LDS_STRIDE + ga_col[i]) = rb[i];
        }
        __syncthreads();
        if (ks + 1 < ksteps) {  // prefetch the next K step into registers
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + (ks + 1) * BK);
                rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + (ks + 1) * BK);
            }
        }
#pragma unroll
        for (int kb = 0; kb < BK / 32; ++kb) {
            i32x4 fa[2], fb[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ar = wm * 64 + t * 32 + (lane & 31);
                const int br = wn * 64 + t * 32 + (lane & 31);
                const int kc = kb * 32 + (lane >> 5) * 16;
                fa[t] = *reinterpret_cast<const i32x4*>(As + ar * LDS_STRIDE + kc);
                fb[t] = *reinterpret_cast<const i32x4*>(Bs + br * LDS_STRIDE + kc);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[a], fb[b], acc[a][b], 0, 0, 0);
        }
    }

    // ------------------------------------------------------------ epilogue
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int tm = m0 + wm * 64 + a * 32;  // tile origin
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
    dim3 grid((unsigned)((a.n + BN - 1) / BN), (unsigned)((a.m + BM - 1) / BM));
    qgemm_w8a8_kernel<<<grid, kThreads, 0, st>>>(p);
    return hipGetLastError();
}

}  // namespace qg
