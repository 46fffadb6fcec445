// sepq.hip -- thresholded separated weights: the split and the batch-1 product.
//
// [SEP] sections 2.1 and 5.2: only the weights above a per-row percentile of
// |W| form the 1-bit backbone (+-alpha); section 3.3: the small weights below
// a second percentile are dropped and the rest form a sparse int8 residual;
// section 5.3: the two products are added (one kernel, no intermediate).
//
// Storage: a 2-bit class per weight ([N][K/4] bytes, weight k in byte k/4 at
// bits 2(k%4): 0 = -alpha, 1 = zero, 2 = +alpha, 3 = residual) and, per row,
// the residual codes in increasing k ([N][ld] int8, zero-filled).
//
// The product (activations quantized per tensor to int8 in the prologue):
//   * a wave step covers 1024 weights of a row: lane l owns weights
//     16l .. 16l+15, i.e. one dword of classes;
//   * backbone: the residual classes are turned into zeros (3 -> 1), the
//     four 2-bit planes of the dword are masked into bytes and fed to v_dot4
//     against x permuted to the same order; sum (class - 1) x is that minus
//     sum x;
//   * residual: the wave loads the step's slice of the row's residual stream
//     (contiguous: the lanes' runs follow each other) into LDS; a lane's run
//     starts at the exclusive prefix (DPP scan) of the lanes' residual
//     counts.  For 4 weights at a time, a 256-entry table maps the 4 residual
//     flags to a byte selector, v_perm places the next codes of the run in
//     the flagged byte slots (zeros elsewhere), and v_dot4 multiplies them
//     with x in natural order;
//   * the class dwords and residual slices of the next step are requested
//     before the current one is computed (one step in flight per wave).
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

constexpr int kSepStep = 1024;   // weights per wave step (64 lanes x 16)
constexpr int kSepStage = 1056;  // staged bytes per row: 1024 codes + 15 misalignment + 8 window over-read

// --------------------------------------------------------------------------- helpers
// Exclusive prefix sum over the workgroup (thread order) of small
// non-negative counts; sets `total`.  Two barriers.
__device__ __forceinline__ int block_excl_scan(int v, int* wave_tot, int& total) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    int inc = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int t = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += t;
    }
    if (lane == kWave - 1) wave_tot[w] = inc;
    lds_barrier();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int c = wave_tot[i];
        before += (i < w) ? c : 0;
        tot += c;
    }
    lds_barrier();
    total = tot;
    return before + inc - v;
}

// Inclusive prefix sum over the 64 lanes of a wave: row_shr 1, 2, 4, 8 within
// rows of 16 lanes, then the row totals are carried by row_bcast15 / 31.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += dpp_mov<0x111>(v);
    v += dpp_mov<0x112>(v);
    v += dpp_mov<0x114>(v);
    v += dpp_mov<0x118>(v);
    v += dpp_mov<0x142, 0xA>(v);
    v += dpp_mov<0x143, 0xC>(v);
    return v;
}

__device__ __forceinline__ uint32_t mag_key(float w) { return __float_as_uint(w) & 0x7FFFFFFFu; }

// --------------------------------------------------------------------------- the split
// One workgroup per row (grid-stride).  Passes over the row (L2 resident):
// 4 radix passes select the two order statistics at once (8-bit digits,
// histograms in LDS); one pass gathers the backbone's exact binade sums and
// count and the residual's max magnitude; one pass writes the classes and
// the compacted residual codes (block scan of the per-thread counts); the
// stream's tail is zero-filled.
__global__ __launch_bounds__(kThreads) void sep_split_kernel(const float* w, int64_t n, int64_t k, int j_b, int j_z,
                                                             uint8_t* cls, int8_t* rv, int64_t ld, float* alpha,
                                                             float* s_r) {
    __shared__ uint32_t hist[2][256];
    __shared__ unsigned long long h64[256];
    __shared__ uint32_t sh_prefix[2], sh_need[2];
    __shared__ float red[kWaves];
    __shared__ int redi[kWaves];
    __shared__ float sh_alpha, sh_sr;
    const int tid = threadIdx.x;
    const int64_t k4 = k / 4;
    const int nsel = (j_z > 0) ? 2 : 1;
    for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
        const float4* row = reinterpret_cast<const float4*>(w + r * k);
        // ---- order statistics: the j_b-th and j_z-th smallest magnitudes
        uint32_t prefix[2] = {0u, 0u}, mask = 0u, need[2] = {(uint32_t)j_b, (uint32_t)(j_z > 0 ? j_z : 1)};
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 512; i += kThreads) (&hist[0][0])[i] = 0u;
            __syncthreads();
            for (int64_t i = tid; i < k4; i += kThreads) {
                const float4 v = row[i];
                const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t key = mag_key(e[j]);
                    if ((key & mask) == prefix[0]) atomicAdd(&hist[0][(key >> shift) & 255u], 1u);
                    if (nsel == 2 && (key & mask) == prefix[1]) atomicAdd(&hist[1][(key >> shift) & 255u], 1u);
                }
            }
            __syncthreads();
            const int wv = tid / kWave, l = tid & (kWave - 1);
            if (wv < nsel) {
                // the bucket holding the need-th smallest: lane l owns buckets 4l .. 4l+3
                uint32_t h[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) h[i] = hist[wv][4 * l + i];
                const uint32_t own = h[0] + h[1] + h[2] + h[3];
                uint32_t incl = own;
#pragma unroll
                for (int off = 1; off < kWave; off <<= 1) {
                    const uint32_t t = __shfl_up(incl, off, kWave);
                    if (l >= off) incl += t;
                }
                uint32_t before = incl - own;
                const uint32_t nd = wv == 0 ? need[0] : need[1];
                const uint32_t pf = wv == 0 ? prefix[0] : prefix[1];
                if (before < nd && nd <= incl) {
                    uint32_t bucket = 4u * l + 3u;
#pragma unroll
                    for (int i = 0; i < 3; ++i) {
                        if (bucket == 4u * l + 3u) {
                            if (before + h[i] >= nd) bucket = 4u * l + i;
                            else before += h[i];
                        }
                    }
                    sh_prefix[wv] = pf | (bucket << shift);
                    sh_need[wv] = nd - before;
                }
            }
            __syncthreads();
            prefix[0] = sh_prefix[0];
            need[0] = sh_need[0];
            if (nsel == 2) {
                prefix[1] = sh_prefix[1];
                need[1] = sh_need[1];
            }
            mask |= 255u << shift;
        }
        const uint32_t tau = prefix[0];
        const bool has_z = j_z > 0;
        const uint32_t eps = prefix[1];
        // ---- backbone exact sums and count; residual max magnitude
        h64[tid] = 0ull;
        __syncthreads();
        int nb = 0;
        uint32_t mx = 0u;
        for (int64_t i = tid; i < k4; i += kThreads) {
            const float4 v = row[i];
            const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t key = mag_key(e[j]);
                if (key > tau) {
                    uint32_t sh, m;
                    abs_binade(e[j], sh, m);
                    atomicAdd(&h64[sh], (unsigned long long)m);
                    ++nb;
                } else if (!has_z || key > eps) {
                    mx = max(mx, key);
                }
            }
        }
        nb = block_sum_int(nb, redi);
        const float rmax = block_max(__uint_as_float(mx), red);  // after block_sum_int's barriers: h64 complete
        if (tid == 0) {
            const float a = nb ? round_mean_from_binades(reinterpret_cast<const uint64_t*>(h64), (uint64_t)nb) : 0.0f;
            const float sc = absmax_scale(rmax);
            alpha[r] = a;
            s_r[r] = sc;
            sh_alpha = a;
            sh_sr = sc;
        }
        __syncthreads();
        const float sc = sh_sr;
        // ---- classes and compacted residual codes, 1024 weights per pass
        int64_t base = 0;
        for (int64_t c0 = 0; c0 < k4; c0 += kThreads) {
            const int64_t i = c0 + tid;
            float e[4] = {0.f, 0.f, 0.f, 0.f};
            if (i < k4) {
                const float4 v = row[i];
                e[0] = v.x; e[1] = v.y; e[2] = v.z; e[3] = v.w;
            }
            uint32_t f[4];
            int cnt = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t key = mag_key(e[j]);
                if (key > tau) f[j] = (e[j] > 0.0f) ? 2u : 0u;
                else if (has_z && key <= eps) f[j] = 1u;
                else f[j] = 3u;
                cnt += (f[j] == 3u) ? 1 : 0;
            }
            if (i >= k4) cnt = 0;
            int total;
            const int off = block_excl_scan(cnt, redi, total);
            if (i < k4) {
                cls[r * k4 + i] = (uint8_t)(f[0] | f[1] << 2 | f[2] << 4 | f[3] << 6);
                int8_t* dst = rv + r * ld + base + off;
                int rank = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (f[j] == 3u) dst[rank++] = (int8_t)qcode(e[j], sc);
                }
            }
            base += total;
        }
        for (int64_t i = base + tid; i < ld; i += kThreads) rv[r * ld + i] = 0;
        __syncthreads();  // LDS is reused by the next row
    }
}

hipError_t launch_sep_split(const float* w, int64_t n, int64_t k, int j_b, int j_z, uint8_t* cls, int8_t* rv,
                            int64_t ld, float* alpha, float* s_r, hipStream_t st) {
    const int grid = (int)(n < 8192 ? n : 8192);
    sep_split_kernel<<<grid, kThreads, 0, st>>>(w, n, k, j_b, j_z, cls, rv, ld, alpha, s_r);
    return hipGetLastError();
}

// --------------------------------------------------------------------------- the product
struct SepParams {
    const uint8_t* cls;
    const int8_t* rv;
    const float* alpha;
    const float* s_r;
    const void* x;
    float* y;
    int32_t* acc_out;
    int64_t ld;
    int32_t n, k, rows_per_wg;
};

__device__ __forceinline__ int sdot4i(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

template <int XT, int U, bool SKIP>
__global__ __launch_bounds__(kThreads) void sep_qgemv_kernel(SepParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t sm[];
    __shared__ float redf[kWaves];
    __shared__ int redi[kWaves];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = p.k;
    const int nsteps = (K + kSepStep - 1) / kSepStep;
    const int Kp = nsteps * kSepStep;
    uint32_t* lut = reinterpret_cast<uint32_t*>(sm);  // 256 selectors
    uint8_t* xn = sm + 1024;                          // int8 x, natural order [Kp]
    uint8_t* xp = xn + Kp;                            // int8 x, 4x4 byte-transposed per 16 [Kp]
    const uint32_t stage0 = 1024u + 2u * (uint32_t)Kp + (uint32_t)(wave * U * kSepStage);  // LDS byte offset

    const int row0 = (int)blockIdx.x * p.rows_per_wg;
    const int rows = min(p.rows_per_wg, p.n - row0);
    const int rowC = K / 4;  // class bytes per row
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.cls + (int64_t)row0 * rowC, (uint32_t)(rows * rowC));
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(SKIP ? nullptr : p.rv + (int64_t)row0 * p.ld,
                                                SKIP ? 0u : (uint32_t)((int64_t)rows * p.ld));
    const uint32_t oob_c = (uint32_t)(rows * rowC);
    const uint32_t oob_r = SKIP ? 0u : (uint32_t)((int64_t)rows * p.ld);
    const uint32_t ld = (uint32_t)p.ld;

    const int ngroups = (rows + U - 1) / U;
    const int my_groups = ngroups > wave ? (ngroups - wave + kWaves - 1) / kWaves : 0;
    const int nit = my_groups * nsteps;

    // class dwords and residual slices of one item (U rows x one step), and
    // the residual count of each row before that step
    struct Buf {
        uint32_t D[U];
        u32x4 V1[U], V2[U];
        int base[U];
    };
    // items past the wave's last read zeros through out-of-range offsets
    auto issue = [&](int it, Buf& b) {
        const int g = wave + kWaves * (it / nsteps);
        const int s = it % nsteps;
        const bool live = it < nit;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = g * U + u;
            const bool ok = live && r < rows && s * kSepStep + 16 * lane < K;
            b.D[u] = load4(rc, ok ? (uint32_t)(r * rowC + s * (kSepStep / 4) + 4 * lane) : oob_c);
            if constexpr (!SKIP) {
                const bool okr = live && r < rows;
                const uint32_t a0 = (uint32_t)r * ld + ((uint32_t)b.base[u] & ~15u);
                b.V1[u] = load16(rr, okr ? a0 + 16u * lane : oob_r);
                b.V2[u] = load16(rr, (okr && lane == 0) ? a0 + (uint32_t)kSepStep : oob_r);
            }
        }
    };
    Buf fa, fb;
#pragma unroll
    for (int u = 0; u < U; ++u) fa.base[u] = 0;
    issue(0, fa);
    __builtin_amdgcn_sched_barrier(0);

    // ---------------------------------------------------------------- prologue
    {   // selector for 4 residual flags (bits 0, 2, 4, 6 of the index): the
        // i-th flagged slot takes byte 4 + (flags below it) of the window
        // operand, an unflagged slot byte 0 of the zero operand
        uint32_t sel = 0;
        int pre = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int f = (tid >> (2 * i)) & 1;
            sel |= (uint32_t)(f ? 4 + pre : 0) << (8 * i);
            pre += f;
        }
        lut[tid] = sel;
    }
    constexpr int kElems = (XT == 0) ? 4 : 8;
    const int npieces = K / kElems;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (uint32_t)(K * (XT == 0 ? 4 : 2)));
    auto piece = [&](int pi, float v[kElems]) {
        const u32x4 r = load16(rx, (uint32_t)(16 * pi));
        if constexpr (XT == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(r[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = bf16_to_f32(r[e] & 0xFFFFu);
                v[2 * e + 1] = bf16_to_f32(r[e] >> 16);
            }
        }
    };
    float m = 0.0f;
    for (int pi = tid; pi < npieces; pi += kThreads) {
        float v[kElems];
        piece(pi, v);
#pragma unroll
        for (int e = 0; e < kElems; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e]));
    }
    const float sx = absmax_scale(block_max(m, redf));
    int sum_xq = 0;
    for (int pi = tid; pi < npieces; pi += kThreads) {
        float v[kElems];
        piece(pi, v);
#pragma unroll
        for (int e = 0; e < kElems; ++e) {
            const int q = qcode(v[e], sx);
            sum_xq += q;
            const int c = pi * kElems + e;
            const int l = c & 15;
            xn[c] = (uint8_t)(q & 0xFF);
            xp[(c - l) + 4 * (l & 3) + (l >> 2)] = (uint8_t)(q & 0xFF);
        }
    }
    for (int i = K / 4 + tid; i < Kp / 4; i += kThreads) {
        reinterpret_cast<uint32_t*>(xn)[i] = 0u;
        reinterpret_cast<uint32_t*>(xp)[i] = 0u;
    }
    sum_xq = block_sum_int(sum_xq, redi);  // its barriers also publish the LDS tables

    int accb[U], accr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) { accb[u] = 0; accr[u] = 0; }

    // one item: scan the residual flags, request the next item (whose stream
    // offsets that scan gives), stage this item's residual slice, multiply
    auto body = [&](int it, Buf& cur, Buf& nxt) {
        const int s = it % nsteps;
        const int g = wave + kWaves * (it / nsteps);
        float al[U], sr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {  // requested ahead of the next item's data
            const int rcl = min(g * U + u, rows - 1);
            al[u] = p.alpha[(int64_t)row0 + rcl];
            sr[u] = SKIP ? 1.0f : p.s_r[(int64_t)row0 + rcl];
        }
        uint32_t R[U];
        int excl[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            R[u] = cur.D[u] & (cur.D[u] >> 1) & 0x55555555u;  // residual flags at even bits
            const int cnt = __builtin_popcount(R[u]);
            const int incl = wave_incl_scan(cnt);
            excl[u] = incl - cnt;
            const int tot = __builtin_amdgcn_readlane(incl, kWave - 1);
            nxt.base[u] = (s + 1 < nsteps) ? cur.base[u] + tot : 0;
        }
        issue(it + 1, nxt);
        if constexpr (!SKIP) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                *reinterpret_cast<u32x4*>(sm + stage0 + u * kSepStage + 16 * lane) = cur.V1[u];
                if (lane == 0) *reinterpret_cast<u32x4*>(sm + stage0 + u * kSepStage + kSepStep) = cur.V2[u];
            }
        }
        const u32x4 xnat = *reinterpret_cast<const u32x4*>(xn + s * kSepStep + 16 * lane);
        const u32x4 xper = *reinterpret_cast<const u32x4*>(xp + s * kSepStep + 16 * lane);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t dz = cur.D[u] ^ (R[u] << 1);  // residual class 3 -> 1 (no backbone term)
            accb[u] = sdot4i(dz & 0x03030303u, xper[0], accb[u]);
            accb[u] = sdot4i((dz >> 2) & 0x03030303u, xper[1], accb[u]);
            accb[u] = sdot4i((dz >> 4) & 0x03030303u, xper[2], accb[u]);
            accb[u] = sdot4i((dz >> 6) & 0x03030303u, xper[3], accb[u]);
            if constexpr (!SKIP) {
                uint32_t a = stage0 + (uint32_t)(u * kSepStage) + ((uint32_t)cur.base[u] & 15u) + (uint32_t)excl[u];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t fl = (R[u] >> (8 * q)) & 0xFFu;
                    const uint32_t sel = lut[fl];
                    const uint32_t aw = a & ~3u;
                    const uint32_t w0 = *reinterpret_cast<const uint32_t*>(sm + aw);
                    const uint32_t w1 = *reinterpret_cast<const uint32_t*>(sm + aw + 4);
                    const uint32_t win = __builtin_amdgcn_alignbyte(w1, w0, a);
                    const uint32_t vals = __builtin_amdgcn_perm(win, 0u, sel);
                    accr[u] = sdot4i(vals, xnat[q], accr[u]);
                    a += (uint32_t)__builtin_popcount(fl);
                }
            }
        }
        if (s == nsteps - 1) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = g * U + u;
                const int tb = wave_sum_to_lane63(accb[u]);
                const int tr = SKIP ? 0 : wave_sum_to_lane63(accr[u]);
                if (lane == kWave - 1 && r < rows) {
                    const int64_t row = (int64_t)row0 + r;
                    const int ab = tb - sum_xq;  // sum (class - 1) x over the row
                    const float tbk = al[u] * (float)ab;
                    const float t = SKIP ? tbk : tbk + (float)tr / sr[u];
                    p.y[row] = t / sx;
                    if (p.acc_out) {
                        p.acc_out[row] = ab;
                        p.acc_out[(int64_t)p.n + row] = tr;
                    }
                }
                accb[u] = 0;
                accr[u] = 0;
            }
        }
    };
    // two buffers in turn, so that no register copy waits for a load in
    // flight; an odd item count ends with one item past the wave's last,
    // which reads zeros and stores nothing
    for (int it = 0; it < nit; it += 2) {
        body(it, fa, fb);
        body(it + 1, fb, fa);
    }
}

template <int XT, int U, bool SKIP>
static hipError_t run_sep(const SepArgs& a, hipStream_t st) {
    const int K = (int)a.k;
    const int nsteps = (K + kSepStep - 1) / kSepStep;
    const size_t lds = 1024 + 2 * (size_t)nsteps * kSepStep + (size_t)kWaves * U * kSepStage;
    const int cus = device_cu_count();
    const int64_t N = a.n;
    const int64_t quantum = (int64_t)kWaves * U;
    int64_t rpw = (N + 2 * cus - 1) / (2 * cus);  // about two workgroups per CU
    rpw = (rpw + quantum - 1) / quantum * quantum;
    // buffer ranges stay below 2 GiB
    const int64_t per_row = a.ld > K / 4 ? a.ld : K / 4;
    const int64_t cap = (((int64_t)1 << 31) / per_row) / quantum * quantum;
    if (rpw > cap) rpw = cap > quantum ? cap : quantum;
    SepParams p;
    p.cls = a.cls;
    p.rv = a.rv;
    p.alpha = a.alpha;
    p.s_r = a.s_r;
    p.x = a.x;
    p.y = a.y;
    p.acc_out = a.acc_out;
    p.ld = a.ld;
    p.n = (int32_t)N;
    p.k = K;
    p.rows_per_wg = (int32_t)rpw;
    const int grid = (int)((N + rpw - 1) / rpw);
    auto kern = sep_qgemv_kernel<XT, U, SKIP>;
    if (lds > 64 * 1024) {
        static bool attr_set = false;  // per instantiation
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            attr_set = true;
        }
    }
    kern<<<grid, kThreads, lds, st>>>(p);
    return hipGetLastError();
}

hipError_t launch_sep_qgemv(const SepArgs& a, hipStream_t st) {
    if (a.xt == 0) return a.skip ? run_sep<0, 2, true>(a, st) : run_sep<0, 2, false>(a, st);
    return a.skip ? run_sep<1, 2, true>(a, st) : run_sep<1, 2, false>(a, st);
}

}  // namespace qg
