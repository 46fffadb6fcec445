// qgemv_batch.hip -- weight-only int8 products for a small batch of tokens.
//
// Decoding M sequences at once (M = 1..16) multiplies every weight row with
// M activation vectors: the weights are still read once per launch, but the
// arithmetic per weight byte grows M-fold (2M flops per byte at M = 16 is
// more than the fp32 VALU can sustain at HBM speed), so the products run on
// the matrix cores: the int8 codes are widened to bf16 in registers (exact:
// |q| <= 127 needs 7 significant bits) and multiplied with the bf16 tokens by
// v_mfma_f32_16x16x32_bf16 into fp32 accumulators.  The result is the
// batch-1 weight-only product of every token: y[t][n] = (sum_k q[n][k] *
// x[t][k]) / s_w[n].
//
// Work: a workgroup owns one 16-row tile of a matrix (a grouped launch
// covers several matrices that share x); its 8 waves split K in units of 64
// (wave w takes units w, w + 8, ...).  In a unit, lane l loads 16 codes of
// row l % 16 and the same 16 activations (k group l / 16) of token l % 16
// (tokens >= M read zeros through the range check, no traffic): the A and B
// fragments of two MFMAs.  Four units per iteration, double-buffered.  The
// eight partial 16x16 tiles are summed through LDS; lane l of wave 0 then
// holds token l % 16, rows 4 (l / 16) + r, r < 4.
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBThreads = 512;
constexpr int kBWaves = kBThreads / kWave;
constexpr int kBUnit = 64;  // k per unit: 4 lane groups x 16
constexpr int kBJS = 4;     // units per iteration

struct BMat {
    const int8_t* wq;
    const float* s_w;
    void* y;
    int32_t n;
};
struct BGroup {
    int32_t count, k, m;
    const uint16_t* x;
    int32_t wg_start[kMaxGroupLaunch + 1];
    BMat mats[kMaxGroupLaunch];
};

// 16 int8 codes -> two bf16x8 (codes 0-7, 8-15): fp32 by an exact integer
// conversion, then the upper halves of two fp32 values form a bf16 pair
__device__ __forceinline__ void widen16(const u32x4& w, bf16x8& a0, bf16x8& a1) {
    uint32_t h[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t v = w[d];
        const float f0 = (float)(int)(int8_t)(v & 0xFFu);
        const float f1 = (float)(int)(int8_t)((v >> 8) & 0xFFu);
        const float f2 = (float)(int)(int8_t)((v >> 16) & 0xFFu);
        const float f3 = (float)(int)(int8_t)(v >> 24);
        h[2 * d] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
        h[2 * d + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    }
    a0 = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    a1 = __builtin_bit_cast(bf16x8, u32x4{h[4], h[5], h[6], h[7]});
}

template <int YT>
__global__ __launch_bounds__(kBThreads) void qgemv_batch_kernel(BGroup grp) {
    __shared__ f32x4 part[kBWaves][kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int mi = 0;
    while (mi + 1 < grp.count && (int)blockIdx.x >= grp.wg_start[mi + 1]) ++mi;
    const BMat& mat = grp.mats[mi];
    const int K = grp.k, M = grp.m;
    const int row0 = ((int)blockIdx.x - grp.wg_start[mi]) * 16;
    const int rows = min(16, mat.n - row0);
    const int i = lane & 15, g = lane >> 4;  // A row / B token, k group
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(mat.wq + (int64_t)row0 * K, (uint32_t)(rows * K));
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(grp.x, (uint32_t)(M * K * 2));
    const uint32_t oob_w = (uint32_t)(rows * K), oob_x = (uint32_t)(M * K * 2);
    const int C = K / kBUnit;
    const int mine = C > wave ? (C - wave + kBWaves - 1) / kBWaves : 0;  // units of this wave
    const int nit = (mine + kBJS - 1) / kBJS;

    struct Frag {
        u32x4 w[kBJS], xa[kBJS], xb[kBJS];
    };
    auto issue = [&](int it, Frag& f) {
#pragma unroll
        for (int j = 0; j < kBJS; ++j) {
            const int u = kBJS * it + j;
            const int c = wave + kBWaves * u;
            const bool ok = u < mine;
            const int kk = c * kBUnit + 16 * g;
            f.w[j] = load16(rw, (ok && i < rows) ? (uint32_t)(i * K + kk) : oob_w);
            const uint32_t xo = (uint32_t)((i * K + kk) * 2);
            f.xa[j] = load16(rx, (ok && i < M) ? xo : oob_x);
            f.xb[j] = load16(rx, (ok && i < M) ? xo + 16u : oob_x);
        }
    };
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto consume = [&](const Frag& f) {
#pragma unroll
        for (int j = 0; j < kBJS; ++j) {
            bf16x8 a0, a1;
            widen16(f.w[j], a0, a1);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(bf16x8, f.xa[j]), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8, f.xb[j]), acc, 0, 0, 0);
        }
    };
    Frag fa, fb;
    issue(0, fa);
    // two buffers in turn (no register copy waits for a load in flight); the
    // last round may consume one iteration past the wave's last, all zeros.
    // The scheduling barriers keep each iteration's loads ahead of the
    // arithmetic on the previous one.
    for (int it = 0; it < nit; it += 2) {
        issue(it + 1, fb);
        __builtin_amdgcn_sched_barrier(0);
        consume(fa);
        __builtin_amdgcn_sched_barrier(0);
        issue(it + 2, fa);
        __builtin_amdgcn_sched_barrier(0);
        consume(fb);
        __builtin_amdgcn_sched_barrier(0);
    }
    part[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        f32x4 s = part[0][lane];
#pragma unroll
        for (int w = 1; w < kBWaves; ++w) {
            const f32x4 t = part[w][lane];
            s[0] += t[0];
            s[1] += t[1];
            s[2] += t[2];
            s[3] += t[3];
        }
        const int t = lane & 15;  // token
        if (t < M) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * (lane >> 4) + r;
                if (row < rows) {
                    const float o = s[r] / mat.s_w[row0 + row];
                    const int64_t at = (int64_t)t * mat.n + row0 + row;
                    if constexpr (YT == 0) static_cast<float*>(mat.y)[at] = o;
                    else static_cast<uint16_t*>(mat.y)[at] = (uint16_t)f32_to_bf16(o);
                }
            }
        }
    }
}

hipError_t launch_qgemv_batch(const BatchArgs* a, int count, hipStream_t st) {
    BGroup g;
    g.count = count;
    g.k = (int32_t)a[0].k;
    g.m = a[0].m;
    g.x = static_cast<const uint16_t*>(a[0].x);
    int wg = 0;
    for (int j = 0; j < count; ++j) {
        g.mats[j].wq = a[j].wq;
        g.mats[j].s_w = a[j].s_w;
        g.mats[j].y = a[j].y;
        g.mats[j].n = (int32_t)a[j].n;
        g.wg_start[j] = wg;
        wg += (int)((a[j].n + 15) / 16);
    }
    for (int j = count; j <= kMaxGroupLaunch; ++j) g.wg_start[j] = wg;
    if (a[0].yt == 0) qgemv_batch_kernel<0><<<wg, kBThreads, 0, st>>>(g);
    else qgemv_batch_kernel<1><<<wg, kBThreads, 0, st>>>(g);
    return hipGetLastError();
}

}  // namespace qg
