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
//   * an item covers 4096 weights of each of U rows: lane l owns weights
//     64l .. 64l+63, i.e. 16 bytes (four dwords) of classes per row;
//   * backbone: the residual classes are turned into zeros (3 -> 1), the
//     four 2-bit planes of each dword are masked into bytes and fed to v_dot4
//     against x transposed (in registers, shared by the U rows) to the same
//     order; sum (class - 1) x is that minus sum x;
//   * residual: the wave loads the step's slice of the row's residual stream
//     (contiguous: the lanes' runs follow each other) into LDS; a lane's run
//     starts at the exclusive prefix (DPP scan) of the lanes' residual
//     counts.  For 4 weights at a time, a 256-entry table maps the 4 residual
//     flags to a byte selector, v_perm places the next codes of the run in
//     the flagged byte slots (zeros elsewhere), and v_dot4 multiplies them
//     with x in natural order;
//   * the classes run two items ahead and the residual slice one item ahead
//     of the item being computed; a slice is read in whole 16-byte blocks,
//     only those that hold its codes.
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

constexpr int kSepStep = 4096;   // weights per row per item (64 lanes x 64)
constexpr int kSepStage = 4128;  // staged bytes per row: 4096 codes + 16 (misalignment) + 16 (window over-read)

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

constexpr int kSepThreads = 512;  // 8 waves, two per SIMD
constexpr int kSepWaves = kSepThreads / kWave;
constexpr uint32_t kSepLdsHead = 1024 + 64 + 16;  // selectors + reduction scratch + group counter
constexpr int kSepXR = 4;  // 16-byte pieces of x per thread held in registers in the prologue

__device__ __forceinline__ int sdot4i(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// 4x4 byte transpose: t[j] = bytes (a0.j, a1.j, a2.j, a3.j), i.e. the
// activations 4b + j (b = 0..3) of a 16-activation slice, the order in which
// (classes >> 2j) & 0x03030303 holds the classes of those weights.
__device__ __forceinline__ void transpose4x4(const u32x4& a, uint32_t t[4]) {
    const uint32_t lo01 = __builtin_amdgcn_perm(a[1], a[0], 0x05010400u);
    const uint32_t hi01 = __builtin_amdgcn_perm(a[1], a[0], 0x07030602u);
    const uint32_t lo23 = __builtin_amdgcn_perm(a[3], a[2], 0x05010400u);
    const uint32_t hi23 = __builtin_amdgcn_perm(a[3], a[2], 0x07030602u);
    t[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
    t[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
    t[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
    t[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// Work: a workgroup owns rows_per_wg consecutive rows in groups of U rows;
// wave w takes groups w and w + 8, then the next free group from a counter in
// the LDS head; an item is one group x one step, and a wave runs the steps
// of its group in order.  The classes of the item two ahead and the residual
// slice of the next item are in flight while an item is computed: the
// classes run two items ahead so that the slice of the
// next item (its start: the running residual count; its length: the scan of
// its classes) is known when it is requested, and only the 16-byte blocks it
// covers are read.
// The matrices of one launch (1, 3 or 8 slots, the fewest that fit): they
// share x and K; matrix blockIdx.y takes workgroups blockIdx.x = 0, 1, ...
// of rows_per_wg rows each, and workgroups past its rows exit at once.
template <int MG>
struct SepGroup {
    SepParams mats[MG];
};

template <int XT, int U, bool SKIP, bool XPL, int MG>
__global__ __launch_bounds__(kSepThreads) void sep_qgemv_kernel(SepGroup<MG> grp) {
    const SepParams& p = grp.mats[blockIdx.y];
    // The kernel's only LDS is this dynamic block (so it starts at address 0
    // and byte offsets are addresses): 256 selectors | reduction scratch |
    // int8 x (zero-padded to Kp) | with XPL the same x 4x4-byte-transposed |
    // the waves' residual slices.  x is stored lane-interleaved: the 16
    // activations that lane l multiplies as dword d of item s sit at
    // s * 4096 + 1024 d + 16 l, so a wave's 16-byte reads are consecutive.
    extern __shared__ __attribute__((aligned(16))) uint8_t sm[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = p.k;
    const int nsteps = (K + kSepStep - 1) / kSepStep;
    const int Kp = nsteps * kSepStep;
    uint32_t* lut = reinterpret_cast<uint32_t*>(sm);
    float* redf = reinterpret_cast<float*>(sm + 1024);
    int* redi = reinterpret_cast<int*>(sm + 1024 + 4 * kSepWaves);
    uint8_t* xn = sm + kSepLdsHead;
    uint8_t* xp = xn + Kp;
    const uint32_t stage0 = kSepLdsHead + (uint32_t)Kp * (XPL ? 2u : 1u) + (uint32_t)(wave * U * kSepStage);
    // LDS offset of 16-activation block b (b = 256 s + 4 l + d)
    auto lane_slot = [](int b) -> uint32_t {
        return (uint32_t)((b >> 8) * kSepStep + ((b & 3) << 10) + (((b >> 2) & 63) << 4));
    };

    const int row0 = (int)blockIdx.x * p.rows_per_wg;
    if (row0 >= p.n) return;  // a smaller matrix of the group needs fewer workgroups (before any barrier)
    const int rows = min(p.rows_per_wg, p.n - row0);
    const int rowC = K / 4;  // class bytes per row
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.cls + (int64_t)row0 * rowC, (uint32_t)(rows * rowC));
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(SKIP ? nullptr : p.rv + (int64_t)row0 * p.ld,
                                                SKIP ? 0u : (uint32_t)((int64_t)rows * p.ld));
    const uint32_t oob_c = (uint32_t)(rows * rowC);
    const uint32_t oob_r = SKIP ? 0u : (uint32_t)((int64_t)rows * p.ld);
    const uint32_t ld = (uint32_t)p.ld;

    // Row groups: waves w and w + 4 (and the other workgroup's waves on the
    // CU) share a SIMD, and the older issues first; with a fixed share the
    // younger waves of a workgroup finished about 5 us after the older ones
    // (per-wave timestamps on MI355X).  So a wave takes groups w and w + 8,
    // then the next free group from a counter in the LDS head, fetched one
    // group ahead of its use.
    const int ngroups = (rows + U - 1) / U;
    typedef __attribute__((address_space(3))) int lds_int;
    lds_int* const ctr = (lds_int*)reinterpret_cast<int*>(sm + 1024 + 8 * kSepWaves);
    if (tid == 0) *reinterpret_cast<int*>(sm + 1024 + 8 * kSepWaves) = 2 * kSepWaves;  // read after the prologue's barriers
    int started = 1;  // groups this wave has started
    int g_pend = 0;   // lane 0: the group after the current one (LDS atomic in flight)
    auto fetch_group = [&]() {
        if (lane == 0) g_pend = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };

    // classes of one item and what their scan gives
    struct Slot {
        int g, s;  // the item: row group and step (wave-uniform)
        u32x4 D[U];
        int excl[U];  // residual codes of the row's item before this lane's 64 weights
        int T[U];     // residual codes in the row's item (wave-uniform)
        int base[U];  // residual codes of the row before the item (wave-uniform)
    };
    u32x4 V[U][4];     // the residual slice in flight: lane l holds blocks l + 64 j,
    uint32_t X4[U];    // and lanes 0-3 the four dwords after them

    // the item after b's in the wave's sequence, into c
    auto next_into = [&](const Slot& b, Slot& c) {
        if (b.s + 1 < nsteps) {
            c.g = b.g;
            c.s = b.s + 1;
            return;
        }
        if (started == 1) {
            c.g = wave + kSepWaves;
        } else {
            c.g = __builtin_amdgcn_readfirstlane(g_pend);
            fetch_group();
        }
        ++started;
        c.s = 0;
    };
    // groups past the last read zeros through out-of-range offsets
    auto issue_codes = [&](Slot& c) {
        const int g = c.g;
        const int s = c.s;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = g * U + u;
            const bool ok = r < rows && s * kSepStep + 64 * lane < K;
            c.D[u] = load16_nt(rc, ok ? (uint32_t)(r * rowC + s * (kSepStep / 4) + 16 * lane) : oob_c);
        }
    };
    // residual flags, their per-lane exclusive prefix and the step's total;
    // `prev` is the item before (same rows, previous step) unless s == 0
    auto scan = [&](Slot& b, const Slot& prev, bool first) {
        const int s = b.s;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int cnt = 0;
#pragma unroll
            for (int d = 0; d < 4; ++d) cnt += __builtin_popcount(b.D[u][d] & (b.D[u][d] >> 1) & 0x55555555u);
            const int incl = wave_incl_scan(cnt);
            b.excl[u] = incl - cnt;
            b.T[u] = __builtin_amdgcn_readlane(incl, kWave - 1);
            b.base[u] = (first || s == 0) ? 0 : prev.base[u] + prev.T[u];
        }
    };
    auto issue_vals = [&](const Slot& b) {
        const int g = b.g;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = g * U + u;
            const uint32_t mis = (uint32_t)b.base[u] & 15u;
            const uint32_t a0 = (uint32_t)r * ld + ((uint32_t)b.base[u] - mis);
            const uint32_t end = mis + (uint32_t)b.T[u];  // bytes of the slice from a0
            const bool okr = r < rows;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t o = 16u * (64u * j + lane);
                V[u][j] = load16(rr, (okr && o < end) ? a0 + o : oob_r);  // slices start anywhere in a line: normal loads
            }
            const uint32_t o4 = (uint32_t)kSepStep + 4u * lane;
            X4[u] = load4(rr, (okr && lane < 4 && o4 < end) ? a0 + o4 : oob_r);
        }
    };

    Slot S0, S1, S2;
    S0.g = wave;
    S0.s = 0;
    next_into(S0, S1);  // the wave's own first two groups: no LDS access
    issue_codes(S0);
    issue_codes(S1);
    // x pieces (16 B: 4 fp32 or 8 bf16) of this thread, requested next
    constexpr int kElems = (XT == 0) ? 4 : 8;
    const int npieces = K / kElems;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (uint32_t)(K * (XT == 0 ? 4 : 2)));
    const uint32_t xend = (uint32_t)(K * (XT == 0 ? 4 : 2));
    u32x4 xr[kSepXR];
#pragma unroll
    for (int l = 0; l < kSepXR; ++l) {
        const int pi = tid + kSepThreads * l;
        xr[l] = load16(rx, pi < npieces ? (uint32_t)(16 * pi) : xend);  // past K: zeros
    }
    __builtin_amdgcn_sched_barrier(0);
    // item 0's residual slice goes out before the prologue arithmetic
    scan(S0, S0, true);
    if constexpr (!SKIP) issue_vals(S0);
    __builtin_amdgcn_sched_barrier(0);

    // ---------------------------------------------------------------- prologue
    if (tid < 256) {
        // selector for 4 residual flags (bits 0, 2, 4, 6 of the index): the
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
    auto vals_of = [&](const u32x4& r, float v[kElems]) {
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
    // visit every piece once: the register window, then (K beyond it) loads
    auto for_pieces = [&](auto&& f) {
#pragma unroll
        for (int l = 0; l < kSepXR; ++l) {
            float v[kElems];
            vals_of(xr[l], v);
            f(tid + kSepThreads * l, v);
        }
        for (int pi = tid + kSepThreads * kSepXR; pi < npieces; pi += kSepThreads) {
            float v[kElems];
            vals_of(load16(rx, (uint32_t)(16 * pi)), v);
            f(pi, v);
        }
    };
    float m = 0.0f;
    for_pieces([&](int, const float* v) {
#pragma unroll
        for (int e = 0; e < kElems; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e]));
    });
    const float sx = absmax_scale(block_max<kSepWaves>(m, redf));
    int sum_xq = 0;
    for_pieces([&](int pi, const float* v) {
        if (pi >= npieces) return;  // register-window pieces past K
        uint32_t packed[kElems / 4];
#pragma unroll
        for (int w4 = 0; w4 < kElems / 4; ++w4) packed[w4] = 0;
#pragma unroll
        for (int e = 0; e < kElems; ++e) {
            const int q = qcode(v[e], sx);
            sum_xq += q;
            packed[e / 4] |= (uint32_t)(q & 0xFF) << (8 * (e % 4));
        }
        // activation c = 16 * blk + i goes to lane_slot(blk) + i; a piece lies in one block
        const int c0 = pi * kElems;
        const uint32_t off = lane_slot(c0 >> 4) + (uint32_t)(c0 & 15);
#pragma unroll
        for (int w4 = 0; w4 < kElems / 4; ++w4) *reinterpret_cast<uint32_t*>(xn + off + 4 * w4) = packed[w4];
    });
    for (int i = K / 4 + tid; i < Kp / 4; i += kSepThreads) {
        const uint32_t off = lane_slot(i >> 2) + 4u * (uint32_t)(i & 3);
        *reinterpret_cast<uint32_t*>(xn + off) = 0u;
    }
    if constexpr (XPL) {
        // the transposed copy, one 16-activation block per thread
        lds_barrier();
        for (int b = tid; b < Kp / 16; b += kSepThreads) {
            const uint32_t off = lane_slot(b);
            const u32x4 a = *reinterpret_cast<const u32x4*>(xn + off);
            uint32_t t[4];
            transpose4x4(a, t);
            *reinterpret_cast<u32x4*>(xp + off) = u32x4{t[0], t[1], t[2], t[3]};
        }
    }
    sum_xq = block_sum_int<kSepWaves>(sum_xq, redi);  // its barriers also publish the LDS tables (and the counter)
    fetch_group();

    int accb[U], accr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) { accb[u] = 0; accr[u] = 0; }

    // A holds the classes of the item computed now (scanned), B the next
    // item's (in flight), C receives the classes of the item after B
    auto body = [&](Slot& A, Slot& B, Slot& C) {
        const int s = A.s;
        const int g = A.g;
        float al[U], sr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {  // requested ahead of the next items' data
            const int rcl = min(g * U + u, rows - 1);
            al[u] = p.alpha[(int64_t)row0 + rcl];
            sr[u] = SKIP ? 1.0f : p.s_r[(int64_t)row0 + rcl];
        }
        next_into(B, C);
        issue_codes(C);
        scan(B, A, false);
        if constexpr (!SKIP) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<u32x4*>(sm + stage0 + u * kSepStage + 16 * (64 * j + lane)) = V[u][j];
                if (lane < 4) *reinterpret_cast<uint32_t*>(sm + stage0 + u * kSepStage + kSepStep + 4 * lane) = X4[u];
            }
            issue_vals(B);
        }
        uint32_t a[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            a[u] = stage0 + (uint32_t)(u * kSepStage) + ((uint32_t)A.base[u] & 15u) + (uint32_t)A.excl[u];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t xo = (uint32_t)(s * kSepStep + 1024 * d + 16 * lane);
            const u32x4 xnat = *reinterpret_cast<const u32x4*>(xn + xo);
            uint32_t xper[4];
            if constexpr (XPL) {
                const u32x4 t = *reinterpret_cast<const u32x4*>(xp + xo);
                xper[0] = t[0]; xper[1] = t[1]; xper[2] = t[2]; xper[3] = t[3];
            } else {
                transpose4x4(xnat, xper);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t D = A.D[u][d];
                const uint32_t R = D & (D >> 1) & 0x55555555u;
                const uint32_t dz = D ^ (R << 1);  // residual class 3 -> 1 (no backbone term)
                accb[u] = sdot4i(dz & 0x03030303u, xper[0], accb[u]);
                accb[u] = sdot4i((dz >> 2) & 0x03030303u, xper[1], accb[u]);
                accb[u] = sdot4i((dz >> 4) & 0x03030303u, xper[2], accb[u]);
                accb[u] = sdot4i((dz >> 6) & 0x03030303u, xper[3], accb[u]);
                if constexpr (!SKIP) {
                    // the 4 groups' window offsets first, then all their LDS
                    // reads, then the arithmetic (one LDS round trip per dword)
                    uint32_t fl[4], ag[4], sel[4], w0[4], w1[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        fl[q] = (R >> (8 * q)) & 0xFFu;
                        ag[q] = a[u];
                        a[u] += (uint32_t)__builtin_popcount(fl[q]);
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        sel[q] = lut[fl[q]];
                        const uint32_t aw = ag[q] & ~3u;
                        w0[q] = *reinterpret_cast<const uint32_t*>(sm + aw);
                        w1[q] = *reinterpret_cast<const uint32_t*>(sm + aw + 4);
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t win = __builtin_amdgcn_alignbyte(w1[q], w0[q], ag[q]);
                        const uint32_t vals = __builtin_amdgcn_perm(win, 0u, sel[q]);
                        accr[u] = sdot4i(vals, xnat[q], accr[u]);
                    }
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
    // three slots in turn, so that no register copy waits for a load in
    // flight.  The wave's groups are increasing: the loop ends when the next
    // item to compute is past the last group.  Its loads (and the ones of
    // the item after it) read zeros; they are folded into an opaque use at
    // the exit, since a load left unused there would be sunk by the compiler
    // below the exit test, after the arithmetic it is meant to run under.
    while (true) {
        body(S0, S1, S2);
        if (S1.g >= ngroups) break;
        body(S1, S2, S0);
        if (S2.g >= ngroups) break;
        body(S2, S0, S1);
        if (S0.g >= ngroups) break;
    }
    uint32_t inflight = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int d = 0; d < 4; ++d) inflight ^= S0.D[u][d] ^ S1.D[u][d] ^ S2.D[u][d];
        if constexpr (!SKIP) {
#pragma unroll
            for (int j = 0; j < 4; ++j) inflight ^= V[u][j][0] ^ V[u][j][1] ^ V[u][j][2] ^ V[u][j][3];
            inflight ^= X4[u];
        }
    }
    asm volatile("" ::"v"(inflight));
}

template <int XT, int U, bool SKIP, bool XPL, int MG>
static hipError_t run_sep(const SepArgs* a, int count, hipStream_t st) {
    const int K = (int)a[0].k;
    const int nsteps = (K + kSepStep - 1) / kSepStep;
    const size_t lds = kSepLdsHead + (size_t)nsteps * kSepStep * (XPL ? 2 : 1) + (SKIP ? 0 : (size_t)kSepWaves * U * kSepStage);
    const int cus = device_cu_count();
    int64_t total = 0, ld_max = K / 4;
    for (int i = 0; i < count; ++i) {
        total += a[i].n;
        if (a[i].ld > ld_max) ld_max = a[i].ld;
    }
    const int64_t quantum = (int64_t)kSepWaves * U;
    int64_t rpw = (total + 2 * cus - 1) / (2 * cus);  // about two workgroups per CU over the whole launch
    rpw = (rpw + quantum - 1) / quantum * quantum;
    // buffer ranges stay below 2 GiB
    const int64_t cap = (((int64_t)1 << 31) / ld_max) / quantum * quantum;
    if (rpw > cap) rpw = cap > quantum ? cap : quantum;
    SepGroup<MG> g;
    int64_t gx = 1;
    for (int i = 0; i < count; ++i) {
        SepParams& p = g.mats[i];
        p.cls = a[i].cls;
        p.rv = a[i].rv;
        p.alpha = a[i].alpha;
        p.s_r = a[i].s_r;
        p.x = a[i].x;
        p.y = a[i].y;
        p.acc_out = a[i].acc_out;
        p.ld = a[i].ld;
        p.n = (int32_t)a[i].n;
        p.k = K;
        p.rows_per_wg = (int32_t)rpw;
        const int64_t wgs = (a[i].n + rpw - 1) / rpw;
        if (wgs > gx) gx = wgs;
    }
    auto kern = sep_qgemv_kernel<XT, U, SKIP, XPL, MG>;
    if (lds > 64 * 1024) {
        static bool attr_set = false;  // per instantiation
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            attr_set = true;
        }
    }
    kern<<<dim3((unsigned)gx, (unsigned)count), kSepThreads, lds, st>>>(g);
    return hipGetLastError();
}

template <int XT, int U, bool SKIP, bool XPL>
static hipError_t run_sep_mg(const SepArgs* a, int count, hipStream_t st) {
    if (count == 1) return run_sep<XT, U, SKIP, XPL, 1>(a, count, st);
    if (count <= 3) return run_sep<XT, U, SKIP, XPL, 3>(a, count, st);
    return run_sep<XT, U, SKIP, XPL, kMaxGroupLaunch>(a, count, st);
}

hipError_t launch_sep_qgemv_group(const SepArgs* a, int count, hipStream_t st) {
    if (count < 1 || count > kMaxGroupLaunch) return hipErrorInvalidValue;
    // One row per item: at two rows the slices' LDS leaves room for only one
    // workgroup per CU, which measured slower on MI355X; the skip path has no
    // slices and takes two.  The transposed copy of x stays in LDS while
    // K <= 32768 (else it is formed in registers).
    const bool skip = a[0].skip;
    if (a[0].k <= 32768) {
        if (a[0].xt == 0) return skip ? run_sep_mg<0, 2, true, true>(a, count, st) : run_sep_mg<0, 1, false, true>(a, count, st);
        return skip ? run_sep_mg<1, 2, true, true>(a, count, st) : run_sep_mg<1, 1, false, true>(a, count, st);
    }
    if (a[0].xt == 0) return skip ? run_sep_mg<0, 2, true, false>(a, count, st) : run_sep_mg<0, 1, false, false>(a, count, st);
    return skip ? run_sep_mg<1, 2, true, false>(a, count, st) : run_sep_mg<1, 1, false, false>(a, count, st);
}

hipError_t launch_sep_qgemv(const SepArgs& a, hipStream_t st) { return launch_sep_qgemv_group(&a, 1, st); }

}  // namespace qg
