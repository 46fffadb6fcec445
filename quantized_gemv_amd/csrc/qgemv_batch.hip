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
// Work: the tiles are 16 rows of a matrix (a grouped launch covers several
// matrices that share x); a workgroup takes tiles in turn (the grid is one
// round of resident workgroups) and its 8 waves split K in units of 64
// (wave w takes a contiguous range of them, so each row is read in long
// runs).  In a unit, lane l loads 16 codes of
// row l % 16 and the same 16 activations (k group l / 16) of token l % 16
// (tokens >= M read zeros through the range check, no traffic): the A and B
// fragments of two MFMAs.  Four units per iteration, double-buffered.  The
// eight partial 16x16 tiles are summed through LDS; lane l of wave 0 then
// holds token l % 16, rows 4 (l / 16) + r, r < 4.
//
// A wave's K range is the same for every tile, so its activation fragments
// are too.  When a workgroup walks several tiles and the fragments of all
// eight waves fit in LDS (K <= 4608: 32 B per lane and unit), every wave
// loads its fragments once, keeps them in its own LDS region and the items
// then carry only weights: at 16 tokens the activations are twice the weight
// bytes of a 16-row tile, and re-reading them from L2 for every tile was the
// larger part of the time (measured: a grouped 3 x 4096 x 4096 launch at 16
// tokens took 22.8 us, 13.5 us with no activation reads at all).  The sums
// are the same operations in the same order either way.
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBThreads = 512;
constexpr int kBWaves = kBThreads / kWave;
constexpr int kBUnit = 64;  // k per unit: 4 lane groups x 16
constexpr int kBJS = 4;     // units per iteration
// LDS for the activation fragments of the eight waves (with the 8 KB of
// partial tiles, within the 160 KB of a CU): K <= 4608
constexpr size_t kBatchXlMaxLds = 144 * 1024;
constexpr int kBXlUnits = 9;  // units per wave that fit: 8 waves x 9 x 2 KB = 144 KB
static_assert((size_t)kBXlUnits * 8 * 2 * 64 * 16 == kBatchXlMaxLds, "LDS budget and unit count agree");

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

template <int YT, bool XL>
__global__ __launch_bounds__(kBThreads) void qgemv_batch_kernel(BGroup grp) {
    __shared__ f32x4 part[kBWaves][kWave];
    extern __shared__ u32x4 xsh[];  // XL: [wave][unit][xa | xb][lane]
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = grp.k, M = grp.m;
    const int i = lane & 15, g = lane >> 4;  // A row / B token, k group
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(grp.x, (uint32_t)(M * K * 2));
    const uint32_t oob_x = (uint32_t)(M * K * 2);
    const int C = K / kBUnit;
    // iterations per tile: the same for every wave (the largest share), since
    // the tile-end barriers are counted in items; shorter shares read zeros
    const int most = (C + kBWaves - 1) / kBWaves;
    const int nit = most > 0 ? (most + kBJS - 1) / kBJS : 1;
    const int ntiles = grp.wg_start[grp.count];
    // the workgroup's tiles are blockIdx.x + gridDim.x * j; every wave walks
    // the flat sequence of (tile, iteration) items of them, so the next
    // tile's loads are in flight while a tile is reduced
    const int my_tiles = ntiles > (int)blockIdx.x ? (ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 0;
    const int nitems = my_tiles * nit;

    struct Tile {
        const BMat* mat;
        int row0, rows;
    };
    auto tile_of = [&](int it) {
        const int tile = (int)blockIdx.x + (int)gridDim.x * (it / nit);
        int mi = 0;
        while (mi + 1 < grp.count && tile >= grp.wg_start[mi + 1]) ++mi;
        Tile t;
        t.mat = &grp.mats[mi];
        t.row0 = (tile - grp.wg_start[mi]) * 16;
        t.rows = it < nitems ? min(16, t.mat->n - t.row0) : 0;  // past the last item: nothing to read
        return t;
    };
    struct Frag {
        u32x4 w[kBJS], xa[XL ? 1 : kBJS], xb[XL ? 1 : kBJS];
        float sw[4];  // this lane's four row scales (used by wave 0)
    };
    u32x4* const xw = xsh + (size_t)wave * most * 2 * kWave;  // XL: this wave's fragments
    auto issue = [&](int it, Frag& f) {
        const Tile t = tile_of(it);
        const int itn = it % nit;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(t.mat->s_w + t.row0, (uint32_t)(t.rows * 4));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * g + r;
            f.sw[r] = __uint_as_float(load4(rs, row < t.rows ? (uint32_t)(4 * row) : (uint32_t)(t.rows * 4)));
        }
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(t.mat->wq + (int64_t)t.row0 * K, (uint32_t)(t.rows * K));
        const uint32_t oob_w = (uint32_t)(t.rows * K);
#pragma unroll
        for (int j = 0; j < kBJS; ++j) {
            const int u = kBJS * itn + j;
            const int c = wave * most + u;  // this wave's contiguous range of units
            const bool ok = u < most && c < C && t.rows > 0;
            const int kk = c * kBUnit + 16 * g;
            f.w[j] = load16(rw, (ok && i < t.rows) ? (uint32_t)(i * K + kk) : oob_w);
            if constexpr (!XL) {
                const uint32_t xo = (uint32_t)((i * K + kk) * 2);
                f.xa[j] = load16(rx, (ok && i < M) ? xo : oob_x);
                f.xb[j] = load16(rx, (ok && i < M) ? xo + 16u : oob_x);
            }
        }
    };
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto consume = [&](int it, const Frag& f) {
        const int itn = it % nit;
#pragma unroll
        for (int j = 0; j < kBJS; ++j) {
            bf16x8 a0, a1;
            widen16(f.w[j], a0, a1);
            u32x4 xa, xb;
            if constexpr (XL) {
                // units past the wave's range hold zeros in registers, never read LDS
                const int u = kBJS * itn + j;
                const bool in = u < most;
                xa = in ? xw[(2 * u) * kWave + lane] : u32x4{0u, 0u, 0u, 0u};
                xb = in ? xw[(2 * u + 1) * kWave + lane] : u32x4{0u, 0u, 0u, 0u};
            } else {
                xa = f.xa[j];
                xb = f.xb[j];
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(bf16x8, xa), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8, xb), acc, 0, 0, 0);
        }
        if (it % nit == nit - 1 && it < nitems) {
            // end of a tile: sum the eight waves' partial tiles (LDS-only
            // barriers: the next items' loads stay in flight)
            part[wave][lane] = acc;
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
            lds_barrier();
            if (wave == 0) {
                const Tile t = tile_of(it);
                f32x4 s = part[0][lane];
#pragma unroll
                for (int w = 1; w < kBWaves; ++w) {
                    const f32x4 q = part[w][lane];
                    s[0] += q[0];
                    s[1] += q[1];
                    s[2] += q[2];
                    s[3] += q[3];
                }
                const int tok = lane & 15;
                if (tok < M) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 4 * g + r;
                        if (row < t.rows) {
                            const float o = s[r] / f.sw[r];
                            const int64_t at = (int64_t)tok * t.mat->n + t.row0 + row;
                            if constexpr (YT == 0) static_cast<float*>(t.mat->y)[at] = o;
                            else static_cast<uint16_t*>(t.mat->y)[at] = (uint16_t)f32_to_bf16(o);
                        }
                    }
                }
            }
            lds_barrier();  // part[] is reused by the next tile
        }
    };
    Frag fa, fb;
    if constexpr (XL) {
        // this wave's activation fragments, once.  All of them are requested
        // (unconditionally: units past the range read zeros), then the first
        // item's weights, and only then are they written to LDS, so the
        // writes wait for the activations while the weights stay in flight.
        // Each wave reads only what it wrote: no barrier, the LDS counter
        // orders its own writes before its reads.
        u32x4 v0[kBXlUnits], v1[kBXlUnits];
#pragma unroll
        for (int u = 0; u < kBXlUnits; ++u) {
            const int c = wave * most + u;
            const bool ok = u < most && c < C && i < M;
            const uint32_t xo = (uint32_t)((i * K + c * kBUnit + 16 * g) * 2);
            v0[u] = load16(rx, ok ? xo : oob_x);
            v1[u] = load16(rx, ok ? xo + 16u : oob_x);
        }
        __builtin_amdgcn_sched_barrier(0);
        issue(0, fa);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kBXlUnits; ++u) {
            if (u < most) {
                xw[(2 * u) * kWave + lane] = v0[u];
                xw[(2 * u + 1) * kWave + lane] = v1[u];
            }
        }
    } else {
        issue(0, fa);
    }
    // two buffers in turn (no register copy waits for a load in flight); the
    // last round may run one item past the wave's last, which reads zeros
    // and stores nothing.  The scheduling barriers keep each item's loads
    // ahead of the arithmetic on the previous one.
    for (int it = 0; it < nitems; it += 2) {
        issue(it + 1, fb);
        __builtin_amdgcn_sched_barrier(0);
        consume(it, fa);
        __builtin_amdgcn_sched_barrier(0);
        issue(it + 2, fa);
        __builtin_amdgcn_sched_barrier(0);
        consume(it + 1, fb);
        __builtin_amdgcn_sched_barrier(0);
    }
}

hipError_t launch_qgemv_batch(const BatchArgs* a, int count, hipStream_t st) {
    BGroup g;
    g.count = count;
    g.k = (int32_t)a[0].k;
    g.m = a[0].m;
    g.x = static_cast<const uint16_t*>(a[0].x);
    int tiles = 0;
    for (int j = 0; j < count; ++j) {
        g.mats[j].wq = a[j].wq;
        g.mats[j].s_w = a[j].s_w;
        g.mats[j].y = a[j].y;
        g.mats[j].n = (int32_t)a[j].n;
        g.wg_start[j] = tiles;
        tiles += (int)((a[j].n + 15) / 16);
    }
    for (int j = count; j <= kMaxGroupLaunch; ++j) g.wg_start[j] = tiles;
    const int cus = device_cu_count();
    const int C = (int)(a[0].k / kBUnit);
    const int most = (C + kBWaves - 1) / kBWaves;
    const size_t xl_bytes = (size_t)kBWaves * most * 2 * kWave * sizeof(u32x4);
    if (tiles > cus && xl_bytes <= kBatchXlMaxLds) {
        // activations kept in LDS: one workgroup per CU, each walking its
        // tiles with the fragments loaded once
        const int grid = cus;
        auto k0 = qgemv_batch_kernel<0, true>;
        auto k1 = qgemv_batch_kernel<1, true>;
        static bool attr_set = false;
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k0),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)kBatchXlMaxLds);
            if (e == hipSuccess)
                e = hipFuncSetAttribute(reinterpret_cast<const void*>(k1), hipFuncAttributeMaxDynamicSharedMemorySize,
                                        (int)kBatchXlMaxLds);
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        if (a[0].yt == 0) k0<<<grid, kBThreads, xl_bytes, st>>>(g);
        else k1<<<grid, kBThreads, xl_bytes, st>>>(g);
        return hipGetLastError();
    }
    // two resident workgroups per CU (the register budget); more tiles than
    // that are walked by the workgroups in turn
    const int slots = 2 * cus;
    const int grid = tiles < slots ? tiles : slots;
    if (a[0].yt == 0) qgemv_batch_kernel<0, false><<<grid, kBThreads, 0, st>>>(g);
    else qgemv_batch_kernel<1, false><<<grid, kBThreads, 0, st>>>(g);
    return hipGetLastError();
}

}  // namespace qg
