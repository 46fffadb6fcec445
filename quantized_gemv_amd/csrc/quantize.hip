// quantize.hip -- quantizers for gfx950: absmax int8 (per row / per tensor),
// the activation outlier split, the outlier-weight gather, ternary absmean
// and the sign-backbone + int8-residual split.
//
// These run offline (weights) or once per step on small activations, so
// they favour plain, exact code over speed: one 256-thread workgroup per row
// where a row-wide statistic is needed, 16-byte vector loads along the row.
#include <mutex>

#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

// Load 8 consecutive elements starting at element index e (e % 8 == 0) as fp32.
template <int XT>
__device__ __forceinline__ void load8(const void* base, int64_t e, float v[8]) {
    if constexpr (XT == 0) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + e);
        float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 h = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + e);
        const uint32_t w[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
            v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
        }
    }
}

__device__ __forceinline__ void store8_codes(int8_t* q, int64_t e, const int c[8]) {
    uint2 o;
    o.x = (uint32_t)(c[0] & 0xFF) | ((uint32_t)(c[1] & 0xFF) << 8) | ((uint32_t)(c[2] & 0xFF) << 16) |
          ((uint32_t)(c[3] & 0xFF) << 24);
    o.y = (uint32_t)(c[4] & 0xFF) | ((uint32_t)(c[5] & 0xFF) << 8) | ((uint32_t)(c[6] & 0xFF) << 16) |
          ((uint32_t)(c[7] & 0xFF) << 24);
    *reinterpret_cast<uint2*>(q + e) = o;
}

// ---------------------------------------------------------------- absmax per row
template <int XT>
__global__ __launch_bounds__(kThreads) void absmax_rows_kernel(const void* x, int64_t rows, int64_t cols,
                                                                int8_t* q, float* s) {
    __shared__ float red[kWaves];
    const int64_t c8 = cols / 8;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        float m = 0.0f;
        for (int64_t i = threadIdx.x; i < c8; i += kThreads) {
            float v[8];
            load8<XT>(x, r * cols + i * 8, v);
#pragma unroll
            for (int j = 0; j < 8; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(v[j]));
        }
        const float sc = absmax_scale(block_max(m, red));
        if (threadIdx.x == 0) s[r] = sc;
        for (int64_t i = threadIdx.x; i < c8; i += kThreads) {
            float v[8];
            int c[8];
            load8<XT>(x, r * cols + i * 8, v);
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = qcode(v[j], sc);
            store8_codes(q, r * cols + i * 8, c);
        }
    }
}

// ---------------------------------------------------------------- asymmetric per row
// [VG] 'Asymmetric quantization': one workgroup per row finds the row's
// minimum and maximum, derives (s, z) and writes the codes.
template <int XT>
__global__ __launch_bounds__(kThreads) void asym_rows_kernel(const void* x, int64_t rows, int64_t cols, int8_t* q,
                                                             float* s, int8_t* z) {
    __shared__ float red[kWaves];
    const int64_t c8 = cols / 8;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        float lo = 0.0f, hi = 0.0f;  // the range always contains 0
        for (int64_t i = threadIdx.x; i < c8; i += kThreads) {
            float v[8];
            load8<XT>(x, r * cols + i * 8, v);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                lo = __builtin_fminf(lo, v[j]);
                hi = __builtin_fmaxf(hi, v[j]);
            }
        }
        hi = block_max(hi, red);
        lo = -block_max(-lo, red);
        float sc, zp;
        asym_params(lo, hi, sc, zp);
        if (threadIdx.x == 0) {
            s[r] = sc;
            z[r] = (int8_t)(int)zp;
        }
        for (int64_t i = threadIdx.x; i < c8; i += kThreads) {
            float v[8];
            int c[8];
            load8<XT>(x, r * cols + i * 8, v);
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = qcode_zp(v[j], sc, zp);
            store8_codes(q, r * cols + i * 8, c);
        }
    }
}

// ---------------------------------------------------------------- absmax per tensor
// Pass 1: each workgroup writes the max |x| of its grid-stride share.
template <int XT>
__global__ __launch_bounds__(kThreads) void absmax_partial_kernel(const void* x, int64_t n8, float* partial) {
    __shared__ float red[kWaves];
    float m = 0.0f;
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n8; i += (int64_t)gridDim.x * kThreads) {
        float v[8];
        load8<XT>(x, i * 8, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(v[j]));
    }
    m = block_max(m, red);
    if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// Pass 2: every workgroup folds all partial maxima (max is exact and
// order-free), derives s and quantizes its share.
template <int XT>
__global__ __launch_bounds__(kThreads) void absmax_apply_kernel(const void* x, int64_t n8, const float* partial,
                                                                 int nparts, int8_t* q, float* s) {
    __shared__ float red[kWaves];
    float m = 0.0f;
    for (int i = threadIdx.x; i < nparts; i += kThreads) m = __builtin_fmaxf(m, partial[i]);
    const float sc = absmax_scale(block_max(m, red));
    if (blockIdx.x == 0 && threadIdx.x == 0) s[0] = sc;
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n8; i += (int64_t)gridDim.x * kThreads) {
        float v[8];
        int c[8];
        load8<XT>(x, i * 8, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = qcode(v[j], sc);
        store8_codes(q, i * 8, c);
    }
}

// ---------------------------------------------------------------- outlier split
// One workgroup per token row (grid-stride when there are more rows than
// workgroups).  The outlier channel set is a bitmap in LDS built from the
// host-validated, sorted index list passed by value.  Everything a row needs
// from memory -- its values and its outlier activations -- is requested
// before the bitmap is built (those barriers wait for LDS traffic only), so a
// row costs one memory round trip.  Rows of up to NP * 2048 columns stay in
// registers between the max pass and the quantize pass; longer rows (NP = 0)
// are read again, from cache, for the second pass.
// n_out <= kThreads (at most 256 outliers): thread j handles outlier j.
static_assert(kThreads <= kMaxOutliers, "every thread reads one entry of the index list");
template <int NP>
__global__ __launch_bounds__(kThreads) void absmax_split_kernel(const uint16_t* x, int64_t rows, int64_t cols,
                                                                 OutlierIdx idx, int n_out, int8_t* q, float* s,
                                                                 uint16_t* x_out, int x_out_ld) {
    extern __shared__ uint32_t bitmap[];  // ceil(cols / 32) words
    __shared__ float red[kWaves];
    const int nwords = (int)((cols + 31) / 32);
    const int64_t c8 = cols / 8;
    const int tid = threadIdx.x;
    // this thread's outlier channel (n_out <= kThreads), requested before the
    // row so that the gather below waits for it alone (loads retire in order)
    const int c_raw = idx.v[tid];
    __builtin_amdgcn_sched_barrier(0);
    const int my_c = (tid < n_out) ? c_raw : 0;
    // Row loads go through a buffer resource over the row: offsets past its
    // end read zeros, so every load is issued unconditionally (a branch
    // around a load makes the compiler wait for all loads at the join).
    const uint32_t row_bytes = (uint32_t)(cols * 2);
    u32x4 keep[NP > 0 ? NP : 1];
    uint16_t gath = 0;  // this thread's outlier activation (tid < n_out)
    auto fetch = [&](int64_t row) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(x + row * cols, row_bytes);
        if constexpr (NP > 0) {
#pragma unroll
            for (int t = 0; t < NP; ++t) {
                const int64_t i = tid + (int64_t)kThreads * t;
                keep[t] = load16(rs, (i < c8) ? (uint32_t)(i * 16) : row_bytes);
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // the row loads go out before the gather waits for its index
        gath = load2(rs, (tid < n_out) ? (uint32_t)(2 * my_c) : row_bytes);
    };
    int64_t r = blockIdx.x;  // < rows: the grid never exceeds the row count
    fetch(r);
    for (int i = tid; i < nwords; i += kThreads) bitmap[i] = 0u;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (tid < n_out) atomicOr(&bitmap[my_c >> 5], 1u << (my_c & 31));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    auto unpack8 = [](u32x4 h, float v[8]) {
        const uint32_t w[4] = {h[0], h[1], h[2], h[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
            v[2 * e + 1] = bf16_to_f32(w[e] >> 16);
        }
    };
    // bit j set: column 8 i + j is not an outlier
    auto inliers = [&](int64_t i) { return ~(bitmap[(i * 8) >> 5] >> ((i * 8) & 31)) & 0xFFu; };
    for (; r < rows; r += gridDim.x) {
        const uint16_t* xr = x + r * cols;
        float m = 0.0f;
        auto piece_max = [&](int64_t i, u32x4 h) {
            float v[8];
            unpack8(h, v);
            const uint32_t in = inliers(i);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if ((in >> j) & 1u) m = __builtin_fmaxf(m, __builtin_fabsf(v[j]));
        };
        auto piece_quant = [&](int64_t i, u32x4 h, float sc) {
            float v[8];
            int c[8];
            unpack8(h, v);
            const uint32_t in = inliers(i);
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = ((in >> j) & 1u) ? qcode(v[j], sc) : 0;
            store8_codes(q, r * cols + i * 8, c);
        };
        float sc;
        if constexpr (NP > 0) {
#pragma unroll
            for (int t = 0; t < NP; ++t) {
                const int64_t i = tid + (int64_t)kThreads * t;
                if (i < c8) piece_max(i, keep[t]);
            }
            sc = absmax_scale(block_max(m, red));
#pragma unroll
            for (int t = 0; t < NP; ++t) {
                const int64_t i = tid + (int64_t)kThreads * t;
                if (i < c8) piece_quant(i, keep[t], sc);
            }
        } else {
            for (int64_t i = tid; i < c8; i += kThreads) piece_max(i, *reinterpret_cast<const u32x4*>(xr + i * 8));
            sc = absmax_scale(block_max(m, red));
            for (int64_t i = tid; i < c8; i += kThreads)
                piece_quant(i, *reinterpret_cast<const u32x4*>(xr + i * 8), sc);
        }
        if (tid == 0) s[r] = sc;
        // gathered outlier activations, zero-padded up to the row stride
        if (n_out > 0)
            for (int j = tid; j < x_out_ld; j += kThreads) x_out[r * x_out_ld + j] = (j < n_out) ? gath : (uint16_t)0;
        if (r + gridDim.x < rows) fetch(r + gridDim.x);
    }
}

// ---------------------------------------------------------------- outlier weight gather
// w_out [n][ld]: column j < n_out holds bf16(w[r][idx[j]]), the rest zero.
__global__ __launch_bounds__(kThreads) void gather_cols_bf16_kernel(const float* w, int64_t n, int64_t k,
                                                                     OutlierIdx idx, int n_out, uint16_t* w_out,
                                                                     int ld) {
    const int64_t total = n * ld;
    for (int64_t t = blockIdx.x * (int64_t)kThreads + threadIdx.x; t < total; t += (int64_t)gridDim.x * kThreads) {
        const int64_t r = t / ld;
        const int j = (int)(t - r * ld);
        w_out[t] = (j < n_out) ? (uint16_t)f32_to_bf16(w[r * k + idx.v[j]]) : (uint16_t)0;
    }
}

// ---------------------------------------------------------------- ternary absmean
__global__ void zero_u64_kernel(uint64_t* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// Binade histogram of |w| over the whole tensor: per-workgroup LDS
// histogram, then one 64-bit global add per non-empty bin.  Integer sums:
// the result does not depend on scheduling.
__global__ __launch_bounds__(kThreads) void abs_binade_hist_kernel(const float* w, int64_t n4, uint64_t* hist) {
    __shared__ unsigned long long h[256];
    h[threadIdx.x] = 0ull;
    __syncthreads();
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads) {
        const float4 v = reinterpret_cast<const float4*>(w)[i];
        const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t sh, m;
            abs_binade(e[j], sh, m);
            if (m) atomicAdd(&h[sh], (unsigned long long)m);
        }
    }
    __syncthreads();
    const unsigned long long mine = h[threadIdx.x];
    if (mine) atomicAdd(reinterpret_cast<unsigned long long*>(hist) + threadIdx.x, mine);
}

__global__ void mean_finalize_kernel(const uint64_t* hist, uint64_t count, float* out) {
    if (blockIdx.x == 0 && threadIdx.x == 0) out[0] = round_mean_from_binades(hist, count);
}

__global__ __launch_bounds__(kThreads) void ternary_codes_kernel(const float* w, int64_t n4, const float* gamma,
                                                                  int8_t* q) {
    const float g = gamma[0];
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads) {
        const float4 v = reinterpret_cast<const float4*>(w)[i];
        const float e[4] = {v.x, v.y, v.z, v.w};
        uint32_t o = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int c = 0;
            if (g != 0.0f) {
                float t = __builtin_rintf(e[j] / g);
                t = __builtin_fminf(__builtin_fmaxf(t, -1.0f), 1.0f);
                c = (int)t;
            }
            o |= (uint32_t)(c & 0xFF) << (8 * j);
        }
        reinterpret_cast<uint32_t*>(q)[i] = o;
    }
}

// ---------------------------------------------------------------- sign + residual
// One workgroup per weight row: exact mean |w| -> alpha, then the residual
// R = w - alpha * sign(w), its absmax scale and int8 codes.
template <bool ZP>
__global__ __launch_bounds__(kThreads) void split_sign_residual_kernel(const float* w, int64_t n, int64_t k,
                                                                        int8_t* sign, float* alpha, int8_t* rq,
                                                                        float* s_r, int8_t* z_r) {
    __shared__ unsigned long long h[256];
    __shared__ float red[kWaves];
    __shared__ float alpha_sh;
    const int64_t k4 = k / 4;
    for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
        const float4* row = reinterpret_cast<const float4*>(w + r * k);
        h[threadIdx.x] = 0ull;
        __syncthreads();
        for (int64_t i = threadIdx.x; i < k4; i += kThreads) {
            const float4 v = row[i];
            const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t sh, m;
                abs_binade(e[j], sh, m);
                if (m) atomicAdd(&h[sh], (unsigned long long)m);
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            const float a = round_mean_from_binades(reinterpret_cast<const uint64_t*>(h), (uint64_t)k);
            alpha_sh = a;
            alpha[r] = a;
        }
        __syncthreads();
        const float a = alpha_sh;
        float m = 0.0f, lo = 0.0f;  // max |R| (symmetric) or max R and min R (zero-point)
        for (int64_t i = threadIdx.x; i < k4; i += kThreads) {
            const float4 v = row[i];
            const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float res = e[j] - (e[j] >= 0.0f ? a : -a);
                if constexpr (ZP) {
                    m = __builtin_fmaxf(m, res);
                    lo = __builtin_fminf(lo, res);
                } else {
                    m = __builtin_fmaxf(m, __builtin_fabsf(res));
                }
            }
        }
        float sc, zp = 0.0f;
        if constexpr (ZP) {
            const float hi = block_max(m, red);
            lo = -block_max(-lo, red);
            asym_params(lo, hi, sc, zp);
            if (threadIdx.x == 0) z_r[r] = (int8_t)(int)zp;
        } else {
            sc = absmax_scale(block_max(m, red));
        }
        if (threadIdx.x == 0) s_r[r] = sc;
        for (int64_t i = threadIdx.x; i < k4; i += kThreads) {
            const float4 v = row[i];
            const float e[4] = {v.x, v.y, v.z, v.w};
            uint32_t so = 0, ro = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool pos = e[j] >= 0.0f;
                const float res = e[j] - (pos ? a : -a);
                so |= (uint32_t)(pos ? 0x01u : 0xFFu) << (8 * j);
                const int qc = ZP ? qcode_zp(res, sc, zp) : qcode(res, sc);
                ro |= (uint32_t)(qc & 0xFF) << (8 * j);
            }
            reinterpret_cast<uint32_t*>(sign + r * k)[i] = so;
            reinterpret_cast<uint32_t*>(rq + r * k)[i] = ro;
        }
        __syncthreads();  // h and alpha_sh are reused by the next row
    }
}

// ---------------------------------------------------------------- 4-bit groups, two-level scales
// [VG] 'Q4_K uses two-level blocks': one wave per super-block of 256
// weights.  Lane l holds weights 4l .. 4l+3, which lie in group l / 8: group
// min / max over 8 lanes, super-block maxima over the wave (shuffles), then
// every lane codes its 4 weights and lane 0 writes the 16-byte metadata
// record.  fp32 arithmetic in the order of the definition; fp16 by RNE.
__global__ __launch_bounds__(kThreads) void q4k_quantize_kernel(const float* w, int64_t n, int64_t k, uint8_t* codes,
                                                                 uint8_t* meta) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t per_row = k / 256;
    const int64_t total = n * per_row;
    for (int64_t sb = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); sb < total; sb += (int64_t)gridDim.x * kWaves) {
        const int64_t r = sb / per_row, b = sb - r * per_row;
        const float4 v4 = *reinterpret_cast<const float4*>(w + r * k + b * 256 + 4 * lane);
        const float v[4] = {v4.x, v4.y, v4.z, v4.w};
        float lo = __builtin_fminf(__builtin_fminf(v[0], v[1]), __builtin_fminf(v[2], v[3]));
        float hi = __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), __builtin_fmaxf(v[2], v[3]));
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) {  // the 8 lanes of a group
            lo = __builtin_fminf(lo, __shfl_xor(lo, off, kWave));
            hi = __builtin_fmaxf(hi, __shfl_xor(hi, off, kWave));
        }
        const float scale = (hi - lo) / 15.0f;
        float smax = scale, amax = __builtin_fabsf(lo);
#pragma unroll
        for (int off = 8; off < kWave; off <<= 1) {  // across the 8 groups
            smax = __builtin_fmaxf(smax, __shfl_xor(smax, off, kWave));
            amax = __builtin_fmaxf(amax, __shfl_xor(amax, off, kWave));
        }
        const _Float16 d16 = (_Float16)(smax / 63.0f);
        const _Float16 dm16 = (_Float16)(amax / 31.0f);
        const float d = (float)d16, dm = (float)dm16;
        const float scq = (d == 0.0f) ? 0.0f : __builtin_fminf(__builtin_fmaxf(rintf(scale / d), 0.0f), 63.0f);
        const float mq = (dm == 0.0f) ? 0.0f : __builtin_fminf(__builtin_fmaxf(rintf(lo / dm), -31.0f), 31.0f);
        const float S = d * scq, M = dm * mq;
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int q = (S == 0.0f) ? 0 : (int)__builtin_fminf(__builtin_fmaxf(rintf((v[e] - M) / S), 0.0f), 15.0f);
            packed |= (uint32_t)q << (4 * e);
        }
        reinterpret_cast<uint16_t*>(codes + r * (k / 2) + b * 128)[lane] = (uint16_t)packed;
        // the record: field i (sc_0..sc_7, then m_0+32..m_7+32) at bits 6i..6i+5
        const int fsc = (int)scq, fm = (int)mq + 32;
        uint32_t rec[3] = {0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t f = (uint32_t)__shfl(i < 8 ? fsc : fm, 8 * (i & 7), kWave);
            const int p = 6 * i, wd = p >> 5, sh = p & 31;
            rec[wd] |= f << sh;
            if (sh > 26) rec[wd + 1] |= f >> (32 - sh);
        }
        if (lane == 0) {
            const uint32_t dd = (uint32_t)__builtin_bit_cast(uint16_t, d16) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, dm16) << 16);
            *reinterpret_cast<uint4*>(meta + sb * 16) = make_uint4(rec[0], rec[1], rec[2], dd);
        }
    }
}

// ---------------------------------------------------------------- launchers
static int grid_for(int64_t work_items, int per_block_items, int cap) {
    int64_t g = (work_items + per_block_items - 1) / per_block_items;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (int)g;
}

hipError_t launch_absmax_rows(const void* x, int xt, int64_t rows, int64_t cols, int8_t* q, float* s,
                              hipStream_t st) {
    const int g = grid_for(rows, 1, 65535);
    if (xt == 0) absmax_rows_kernel<0><<<g, kThreads, 0, st>>>(x, rows, cols, q, s);
    else absmax_rows_kernel<1><<<g, kThreads, 0, st>>>(x, rows, cols, q, s);
    return hipGetLastError();
}

int absmax_tensor_parts(int64_t elems) { return grid_for(elems / 8, kThreads * 4, 1024); }

hipError_t launch_absmax_tensor(const void* x, int xt, int64_t elems, int8_t* q, float* s, float* partial,
                                hipStream_t st) {
    const int parts = absmax_tensor_parts(elems);
    const int64_t n8 = elems / 8;
    if (xt == 0) {
        absmax_partial_kernel<0><<<parts, kThreads, 0, st>>>(x, n8, partial);
        absmax_apply_kernel<0><<<parts, kThreads, 0, st>>>(x, n8, partial, parts, q, s);
    } else {
        absmax_partial_kernel<1><<<parts, kThreads, 0, st>>>(x, n8, partial);
        absmax_apply_kernel<1><<<parts, kThreads, 0, st>>>(x, n8, partial, parts, q, s);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- no-allocation variant
// The per-tensor quantizer's only scratch is its partial maxima, one per
// workgroup of the first pass (absmax_tensor_parts(elems) <= 1024 floats).
// For callers that cannot allocate, they live in this file-scope array: one
// copy per device, held until the process ends.  The partial pass writes
// every entry that the apply pass reads, so nothing needs clearing between
// calls; calls that overlap on one device race for it.
static __device__ __align__(256) float scratch[kAbsmaxScratchParts];

namespace {
std::mutex scratch_mu;
float* scratch_dev[kMaxDevices] = {};  // device address of `scratch`, per device
}  // namespace

hipError_t launch_absmax_tensor_noalloc(const void* x, int xt, int64_t elems, int8_t* q, float* s,
                                        hipStream_t st) {
    if (absmax_tensor_parts(elems) > kAbsmaxScratchParts) return hipErrorInvalidValue;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    float* ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(scratch_mu);
        if (!scratch_dev[dev]) {  // once per device, with that device current
            void* p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            scratch_dev[dev] = static_cast<float*>(p);
        }
        ptr = scratch_dev[dev];
    }
    // the kernels take the device address, never the host-side name
    return launch_absmax_tensor(x, xt, elems, q, s, ptr, st);
}

hipError_t launch_absmax_split(const uint16_t* x, int64_t rows, int64_t cols, const OutlierIdx& idx, int n_out,
                               int8_t* q, float* s, uint16_t* x_out, int x_out_ld, hipStream_t st) {
    const int g = grid_for(rows, 1, 65535);
    const size_t lds = (size_t)((cols + 31) / 32) * sizeof(uint32_t);
    const int64_t per_thread = (cols / 8 + kThreads - 1) / kThreads;  // 16-byte pieces per thread
    if (per_thread <= 1)
        absmax_split_kernel<1><<<g, kThreads, lds, st>>>(x, rows, cols, idx, n_out, q, s, x_out, x_out_ld);
    else if (per_thread <= 2)
        absmax_split_kernel<2><<<g, kThreads, lds, st>>>(x, rows, cols, idx, n_out, q, s, x_out, x_out_ld);
    else if (per_thread <= 4)
        absmax_split_kernel<4><<<g, kThreads, lds, st>>>(x, rows, cols, idx, n_out, q, s, x_out, x_out_ld);
    else
        absmax_split_kernel<0><<<g, kThreads, lds, st>>>(x, rows, cols, idx, n_out, q, s, x_out, x_out_ld);
    return hipGetLastError();
}

hipError_t launch_gather_cols_bf16(const float* w, int64_t n, int64_t k, const OutlierIdx& idx, int n_out,
                                   uint16_t* w_out, int w_out_ld, hipStream_t st) {
    if (n_out == 0) return hipSuccess;
    const int g = grid_for(n * w_out_ld, kThreads, 65535);
    gather_cols_bf16_kernel<<<g, kThreads, 0, st>>>(w, n, k, idx, n_out, w_out, w_out_ld);
    return hipGetLastError();
}

hipError_t launch_ternary(const float* w, int64_t count, int8_t* q, float* gamma, uint64_t* hist, hipStream_t st) {
    const int64_t n4 = count / 4;
    zero_u64_kernel<<<1, 256, 0, st>>>(hist, 256);
    const int g = grid_for(n4, kThreads * 16, 2048);
    abs_binade_hist_kernel<<<g, kThreads, 0, st>>>(w, n4, hist);
    mean_finalize_kernel<<<1, 64, 0, st>>>(hist, (uint64_t)count, gamma);
    ternary_codes_kernel<<<grid_for(n4, kThreads * 4, 8192), kThreads, 0, st>>>(w, n4, gamma, q);
    return hipGetLastError();
}

hipError_t launch_split_sign_residual(const float* w, int64_t n, int64_t k, int8_t* sign, float* alpha, int8_t* rq,
                                      float* s_r, int8_t* z_r, hipStream_t st) {
    const int g = grid_for(n, 1, 65535);
    if (z_r) split_sign_residual_kernel<true><<<g, kThreads, 0, st>>>(w, n, k, sign, alpha, rq, s_r, z_r);
    else split_sign_residual_kernel<false><<<g, kThreads, 0, st>>>(w, n, k, sign, alpha, rq, s_r, nullptr);
    return hipGetLastError();
}

hipError_t launch_asym_rows(const void* x, int xt, int64_t rows, int64_t cols, int8_t* q, float* s, int8_t* z,
                            hipStream_t st) {
    const int g = grid_for(rows, 1, 65535);
    if (xt == 0) asym_rows_kernel<0><<<g, kThreads, 0, st>>>(x, rows, cols, q, s, z);
    else asym_rows_kernel<1><<<g, kThreads, 0, st>>>(x, rows, cols, q, s, z);
    return hipGetLastError();
}

hipError_t launch_quantize_q4k(const float* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* meta, hipStream_t st) {
    const int64_t blocks = (n * (k / 256) + kWaves - 1) / kWaves;  // one wave per super-block
    q4k_quantize_kernel<<<(int)(blocks < 16384 ? blocks : 16384), kThreads, 0, st>>>(w, n, k, codes, meta);
    return hipGetLastError();
}

}  // namespace qg
