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
    int32_t count, k, m, t16;
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

// Weight fragments: lane L = 16 g + i takes the 16 codes of row i of the
// tile, k = 64 c + 16 g .. + 15.  Row-major codes hold them at i K + 64 c +
// 16 g of the tile (64 bytes of each of 16 rows per load); the 16-row tiled
// layout at 1024 c + 16 L (one contiguous 1 KB block per load, so the loads
// can be non-temporal).  A tile is 16 K bytes in both (the tiled one
// zero-padded past the last row).
template <int YT, bool XL, bool T16>
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
        // the tiled layout's last tile is padded to 16 rows (zeros)
        const uint32_t oob_w = (uint32_t)((T16 && t.rows > 0 ? 16 : t.rows) * K);
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(t.mat->wq + (int64_t)t.row0 * K, oob_w);
#pragma unroll
        for (int j = 0; j < kBJS; ++j) {
            const int u = kBJS * itn + j;
            const int c = wave * most + u;  // this wave's contiguous range of units
            const bool ok = u < most && c < C && t.rows > 0;
            const int kk = c * kBUnit + 16 * g;
            if constexpr (T16) f.w[j] = load16_nt(rw, ok ? (uint32_t)(c * 1024 + lane * 16) : oob_w);  // whole 1 KB blocks
            else f.w[j] = load16(rw, (ok && i < t.rows) ? (uint32_t)(i * K + kk) : oob_w);
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

// ------------------------------------------ activations in registers
// Grouped launches with more 16-row tiles than CUs and K <= 4608: one
// workgroup per CU; wave w keeps the activation fragments of its MOST units
// of K in registers (loaded once: 4 MOST VGPRs, no LDS copy to write and
// read back; measured 15.9 -> 15.6 us for q, k, v at 16 tokens against the
// LDS copy) and the workgroup walks its tiles blockIdx.x + gridDim.x * j.  Per tile a wave loads its MOST units of
// weights (16 rows x 64 k each) and the tile's row scales in one go, the
// next tile's loads in flight while it multiplies; MOST is a template
// parameter, so there is no branch between the loads and the products.
// The waves' partial tiles meet in LDS (two buffers, one barrier per tile)
// and wave j % 8 reduces tile j, so the reductions are spread over the
// waves and the others go on to the next tile at once.  The same products
// and the same summation order as the tile loop above.
template <int YT, int MOST>
__global__ __launch_bounds__(kBThreads) void qgemv_batch_xl_kernel(BGroup grp) {
    __shared__ f32x4 part[2][kBWaves][kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = grp.k, M = grp.m;
    const int i = lane & 15, g = lane >> 4;  // A row / B token, k group
    const int C = K / kBUnit;
    const int c0 = wave * MOST;  // this wave's units c0 .. c0 + MOST - 1 (those >= C read zeros)
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(grp.x, (uint32_t)(M * K * 2));
    const uint32_t oob_x = (uint32_t)(M * K * 2);
    const int ntiles = grp.wg_start[grp.count];
    const int my_tiles =
        ntiles > (int)blockIdx.x ? (ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 0;

    // the tile's matrix, selected with constant indices into the kernel
    // argument (a computed index would take it through memory and make the
    // buffer descriptors non-uniform: a loop over lanes around every load)
    struct Tile {
        BMat mat;
        int row0, rows;
    };
    auto tile_of = [&](int j) {
        const int tile = (int)blockIdx.x + (int)gridDim.x * j;
        Tile t;
        t.mat = grp.mats[0];
        int start = 0;
#pragma unroll
        for (int q = 1; q < kMaxGroupLaunch; ++q) {
            if (q < grp.count && tile >= grp.wg_start[q]) {
                t.mat = grp.mats[q];
                start = grp.wg_start[q];
            }
        }
        t.row0 = (tile - start) * 16;
        t.rows = j < my_tiles ? min(16, t.mat.n - t.row0) : 0;  // past the last tile: nothing to read
        return t;
    };
    struct Frag {
        u32x4 w[MOST];
        float sw[4];  // this lane's four row scales (used by the reducing wave)
    };
    auto issue = [&](int j, Frag& f) {
        const Tile t = tile_of(j);
        // the last tile is padded to 16 rows (zeros)
        const uint32_t tile_bytes = (uint32_t)((t.rows > 0 ? 16 : 0) * K);
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(t.mat.wq + (int64_t)t.row0 * K, tile_bytes);
#pragma unroll
        for (int u = 0; u < MOST; ++u) {
            const int c = c0 + u;
            // whole 1 KB blocks, each read once: non-temporal
            f.w[u] = load16_nt(rw, c < C ? (uint32_t)(c * 1024 + lane * 16) : tile_bytes);
        }
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(t.mat.s_w + t.row0, (uint32_t)(t.rows * 4));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * g + r;
            f.sw[r] = __uint_as_float(load4(rs, row < t.rows ? (uint32_t)(4 * row) : (uint32_t)(t.rows * 4)));
        }
    };
    u32x4 xr0[MOST], xr1[MOST];  // this wave's activation fragments (units >= C: zeros)
    auto consume = [&](int j, const Frag& f) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < MOST; ++u) {
            bf16x8 a0, a1;
            widen16(f.w[u], a0, a1);
            const u32x4 xa = xr0[u];
            const u32x4 xb = xr1[u];
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(bf16x8, xa), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8, xb), acc, 0, 0, 0);
        }
        part[j & 1][wave][lane] = acc;
        lds_barrier();
        if (wave == j % kBWaves) {
            const Tile t = tile_of(j);
            f32x4 s = part[j & 1][0][lane];
#pragma unroll
            for (int v = 1; v < kBWaves; ++v) {
                const f32x4 q = part[j & 1][v][lane];
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
                        const int64_t at = (int64_t)tok * t.mat.n + t.row0 + row;
                        if constexpr (YT == 0) static_cast<float*>(t.mat.y)[at] = o;
                        else static_cast<uint16_t*>(t.mat.y)[at] = (uint16_t)f32_to_bf16(o);
                    }
                }
            }
        }
        // part[j & 1] is written again at tile j + 2, after every wave has
        // passed tile j + 1's barrier, which the reducing wave reaches only
        // after its reads above
    };
    // this wave's activation fragments, requested before the first tile's
    // weights (the first products wait for them in issue order)
    Frag fa, fb;
#pragma unroll
    for (int u = 0; u < MOST; ++u) {
        const int c = c0 + u;
        const bool ok = c < C && i < M;
        const uint32_t xo = (uint32_t)((i * K + c * kBUnit + 16 * g) * 2);
        xr0[u] = load16(rx, ok ? xo : oob_x);
        xr1[u] = load16(rx, ok ? xo + 16u : oob_x);
    }
    __builtin_amdgcn_sched_barrier(0);
    issue(0, fa);
    __builtin_amdgcn_sched_barrier(0);
    // two tiles per round, each buffer reloaded right after its products; a
    // last round past my_tiles reads zeros and its tile stores nothing
    for (int j = 0; j < my_tiles; j += 2) {
        issue(j + 1, fb);
        __builtin_amdgcn_sched_barrier(0);
        consume(j, fa);
        if (j + 1 >= my_tiles) break;
        issue(j + 2, fa);
        __builtin_amdgcn_sched_barrier(0);
        consume(j + 1, fb);
    }
}

template <int YT>
static hipError_t launch_xl(int most, int grid, const BGroup& g, hipStream_t st) {
    switch (most) {
        case 1: qgemv_batch_xl_kernel<YT, 1><<<grid, kBThreads, 0, st>>>(g); break;
        case 2: qgemv_batch_xl_kernel<YT, 2><<<grid, kBThreads, 0, st>>>(g); break;
        case 3: qgemv_batch_xl_kernel<YT, 3><<<grid, kBThreads, 0, st>>>(g); break;
        case 4: qgemv_batch_xl_kernel<YT, 4><<<grid, kBThreads, 0, st>>>(g); break;
        case 5: qgemv_batch_xl_kernel<YT, 5><<<grid, kBThreads, 0, st>>>(g); break;
        case 6: qgemv_batch_xl_kernel<YT, 6><<<grid, kBThreads, 0, st>>>(g); break;
        case 7: qgemv_batch_xl_kernel<YT, 7><<<grid, kBThreads, 0, st>>>(g); break;
        case 8: qgemv_batch_xl_kernel<YT, 8><<<grid, kBThreads, 0, st>>>(g); break;
        case 9: qgemv_batch_xl_kernel<YT, 9><<<grid, kBThreads, 0, st>>>(g); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ------------------------------------------ one tile per wave (tiled)
// Grouped launches of 16-row tiled codes with more tiles than CUs and
// K <= 4608: one workgroup per CU holds the activation fragments of all of
// K in LDS (loaded once), and each wave multiplies whole tiles alone -- all
// K of its 16 rows -- so after the first tile the waves never wait for each
// other.  With three or four tiles per CU (q, k, v: 768 tiles) that would
// leave most waves idle, so there (H = 2) waves 2j and 2j + 1 take one half
// of K of tile j each and add their halves through LDS once at the end:
// 15.5 -> 13.1 us for q, k, v at 16 tokens against the shared-tile kernel.  The fragments arrive in phases of 8 units (one per wave), each
// written behind its own barrier, and the first tile's products of a phase
// start as soon as it is in LDS (at 16 tokens the fragments are 128 KB per
// CU, twice a tile's weights).  A wave's tiles are blockIdx.x + gridDim.x
// (w + 8 q); its units (tile, unit c) form one stream that a ring of D loads
// in flight runs through, across tile ends (D divides 8 and the units per
// tile, so phases and tiles end between two turns of the ring and the loop
// body has no memory operation under a branch).  Per unit: the 1 KB block of codes (non-temporal, read once),
// widened to bf16, and the two activation fragments of unit c from LDS into
// two MFMAs; after a tile's last unit its 16 x 16 products are complete
// (summed in unit order), rescaled by the row scales (each lane's four,
// loaded when the tile starts) and stored.

template <int YT, int D, int MG, int H>
__global__ __launch_bounds__(kBThreads) void qgemv_batch_wt_kernel(BGroup grp) {
    static_assert(H == 1 || H == 2, "whole tiles or halves");
    extern __shared__ u32x4 xsh[];  // [unit][xa | xb][lane]
    __shared__ f32x4 hpart[H == 2 ? kBWaves / 2 : 1][kWave];  // H = 2: the second halves' partial tiles
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = grp.k, M = grp.m;
    const int i = lane & 15, g = lane >> 4;  // A row / B token, k group
    const int C = K / kBUnit;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(grp.x, (uint32_t)(M * K * 2));
    const uint32_t oob_x = (uint32_t)(M * K * 2);
    const int ntiles = grp.wg_start[grp.count];
    const int my_tiles =
        ntiles > (int)blockIdx.x ? (ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 0;
    // H = 1: wave w multiplies tiles w, w + 8, ... of the workgroup over all
    // of K.  H = 2 (at most 4 tiles per workgroup): waves 2j and 2j + 1 take
    // the two halves of K of tile j, one piece each.
    const int CH = C / H;                     // units of a piece
    const int half = H == 2 ? (wave & 1) : 0;
    const int cbase = half * CH;              // the piece's first unit
    const int wt = H == 1 ? (my_tiles > wave ? (my_tiles - wave + kBWaves - 1) / kBWaves : 0)
                          : (wave / 2 < my_tiles ? 1 : 0);  // this wave's pieces

    struct Tile {
        BMat mat;
        int row0, rows;
    };
    // the wave's tile q, with its matrix selected by constant indices (the
    // buffer descriptors stay uniform; MG >= count slots are looked at)
    auto tile_of = [&](int q) {
        const int tile = (int)blockIdx.x + (int)gridDim.x * (H == 1 ? wave + kBWaves * q : wave / 2 + 4 * q);
        Tile t;
        t.mat = grp.mats[0];
        int start = 0;
#pragma unroll
        for (int mq = 1; mq < MG; ++mq) {
            if (mq < grp.count && tile >= grp.wg_start[mq]) {
                t.mat = grp.mats[mq];
                start = grp.wg_start[mq];
            }
        }
        t.row0 = (tile - start) * 16;
        t.rows = q < wt ? min(16, t.mat.n - t.row0) : 0;
        return t;
    };
    // the prefetch cursor: tile pq, unit pc, and the tile's codes (tiles
    // past the wave's last read zeros)
    int pq = 0, pc = 0;
    __amdgpu_buffer_rsrc_t prw;
    {
        const Tile t = tile_of(0);
        prw = make_rsrc(t.mat.wq + (int64_t)t.row0 * K, (uint32_t)((t.rows > 0 ? 16 : 0) * K));
    }
    auto fetch = [&]() -> u32x4 {
        const u32x4 v = load16_nt(prw, (uint32_t)((cbase + pc) * 1024 + lane * 16));
        if (++pc == CH) {
            pc = 0;
            ++pq;
            const Tile t = tile_of(pq);
            prw = make_rsrc(t.mat.wq + (int64_t)t.row0 * K, (uint32_t)((t.rows > 0 ? 16 : 0) * K));
        }
        return v;
    };

    // activations: phase p holds 8 units, one written by each wave (H = 1:
    // units 8p .. 8p + 7; H = 2: units 4p .. 4p + 3 of each half).  Wave w
    // requests its unit of the first kXD phases, then the ring's first D
    // units of weights; the unit of phase p + kXD is requested when phase p
    // starts.  (Every phase requested up front -- 128 KB per CU at 16 tokens,
    // from all CUs at once -- delayed the first phase to 4.8 us after the
    // launch, per-wave timestamps on MI355X.)
    constexpr int kXU = (kBatchXlMaxLds / 2048 + kBWaves - 1) / kBWaves;  // phases (units per wave) at most
    constexpr int kXD = 2;                                                // phases requested ahead
    auto phase_unit = [&](int q) -> int {  // C when past the last unit
        if constexpr (H == 1) return min(wave + kBWaves * q, C);
        const int u = 4 * q + (wave & 3);
        return u < CH ? (wave < 4 ? 0 : CH) + u : C;
    };
    u32x4 v0[kXU], v1[kXU];
    auto load_x = [&](int q) {  // unconditional: units past C read zeros
        const int c = phase_unit(q);
        const bool ok = c < C && i < M;
        const uint32_t xo = (uint32_t)((i * K + c * kBUnit + 16 * g) * 2);
        v0[q] = load16(rx, ok ? xo : oob_x);
        v1[q] = load16(rx, ok ? xo + 16u : oob_x);
    };
#pragma unroll
    for (int q = 0; q < kXD; ++q) load_x(q);
    __builtin_amdgcn_sched_barrier(0);
    u32x4 ring[D];
#pragma unroll
    for (int d = 0; d < D; ++d) ring[d] = fetch();
    __builtin_amdgcn_sched_barrier(0);

    // this lane's four row scales (rows 4 (l / 16) + r of the tile; rows
    // past the matrix read zero and are never stored), vector loads issued
    // when the tile starts: they complete long before the tile ends, so the
    // wait for them does not wait for the ring
    auto scales = [&](const Tile& ct, float (&sw)[4]) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(ct.mat.s_w + ct.row0, (uint32_t)(ct.rows * 4));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * g + r;
            sw[r] = __uint_as_float(load4(rs, row < ct.rows ? (uint32_t)(4 * row) : (uint32_t)(ct.rows * 4)));
        }
    };
    // one turn of the ring: units cb .. cb + D - 1 of the current tile, the
    // ring refilled unit by unit (a wave without tiles only keeps the
    // prefetch cursor going: its loads read zeros, it multiplies nothing)
    auto turn = [&](int cb, bool live, f32x4& acc) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int c = cb + d;
            const u32x4 w = ring[d];
            ring[d] = fetch();
            if (live) {
                bf16x8 a0, a1;
                widen16(w, a0, a1);
                const u32x4 xa = xsh[(2 * c) * kWave + lane];
                const u32x4 xb = xsh[(2 * c + 1) * kWave + lane];
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(bf16x8, xa), acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8, xb), acc, 0, 0, 0);
            } else {
                asm volatile("" ::"v"(w));  // the load is waited for in issue order either way
            }
        }
    };
    // lane l holds token l % 16, rows 4 (l / 16) + r
    auto store = [&](const Tile& ct, const float (&sw)[4], const f32x4& acc) {
        const int tok = lane & 15;
        if (tok < M) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * g + r;
                if (row < ct.rows) {
                    const float o = acc[r] / sw[r];
                    const int64_t at = (int64_t)tok * ct.mat.n + ct.row0 + row;
                    if constexpr (YT == 0) static_cast<float*>(ct.mat.y)[at] = o;
                    else static_cast<uint16_t*>(ct.mat.y)[at] = (uint16_t)f32_to_bf16(o);
                }
            }
        }
    };
    // The first tile, with every wave taking part: phase p of the
    // activations is written to LDS behind a barrier of its own, and the
    // tile's products over that phase's units follow at once, while the
    // later phases are still arriving.  Waves without a tile write their
    // units and pass the barriers.
    {
        const bool live = wt > 0;
        const Tile ct = tile_of(0);
        float sw[4];
        scales(ct, sw);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < kXU; ++p) {
            if (p + kXD < kXU) load_x(p + kXD);  // outside the branch below: no load under a branch
            if (kBWaves * p < C) {  // uniform: every wave passes the same barriers
                const int c = phase_unit(p);
                if (c < C) {
                    xsh[(2 * c) * kWave + lane] = v0[p];
                    xsh[(2 * c + 1) * kWave + lane] = v1[p];
                }
                lds_barrier();
                if constexpr (H == 1) {
                    const int ce = min(kBWaves * (p + 1), C);  // D divides 8 and C
                    for (int cb = kBWaves * p; cb < ce; cb += D) turn(cb, live, acc);
                } else {
#pragma unroll
                    for (int cb = 0; cb < 4; cb += D) turn(cbase + 4 * p + cb, live, acc);  // 8 divides C
                }
            }
        }
        if constexpr (H == 1) {
            if (live) store(ct, sw, acc);
        } else {
            // the pair's halves meet in LDS: first half + second half, in
            // that order whichever finishes first
            if (half == 1) hpart[wave >> 1][lane] = acc;
            lds_barrier();
            if (half == 0 && live) {
                const f32x4 o = hpart[wave >> 1][lane];
                f32x4 s;
#pragma unroll
                for (int r = 0; r < 4; ++r) s[r] = acc[r] + o[r];
                store(ct, sw, s);
            }
        }
    }
    for (int q = 1; q < wt; ++q) {
        const Tile ct = tile_of(q);
        float sw[4];
        scales(ct, sw);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int cb = 0; cb < CH; cb += D) turn(cbase + cb, true, acc);  // H = 1 only: one piece per wave otherwise
        store(ct, sw, acc);
    }
}

// ring depth: 4 units (4 KB per wave in flight) where it divides the units
// per tile, else 2 (C is even).  Measured on MI355X at 16 tokens, 1376 tiles
// of 4096 columns: 16 units 24.1 us, 8 23.3 us, 4 22.85 us, 2 28.3 us.
static int wt_ring(int C) { return C % 4 == 0 ? 4 : 2; }

template <int YT, int D, int MG, int H>
static hipError_t launch_wt_d(int grid, size_t lds, const BGroup& g, hipStream_t st) {
    auto fn = qgemv_batch_wt_kernel<YT, D, MG, H>;
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)kBatchXlMaxLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    fn<<<grid, kBThreads, lds, st>>>(g);
    return hipGetLastError();
}
template <int YT, int MG>
static hipError_t launch_wt_mg(int C, bool halves, int grid, size_t lds, const BGroup& g, hipStream_t st) {
    if (halves) return launch_wt_d<YT, 4, MG, 2>(grid, lds, g, st);  // C % 8 == 0
    switch (wt_ring(C)) {
        case 4: return launch_wt_d<YT, 4, MG, 1>(grid, lds, g, st);
        default: return launch_wt_d<YT, 2, MG, 1>(grid, lds, g, st);
    }
}
// matrix slots the kernel looks at: 1, 3 (q, k, v; gate, up) or all
template <int YT>
static hipError_t launch_wt(int C, bool halves, int grid, size_t lds, const BGroup& g, hipStream_t st) {
    if (g.count == 1) return launch_wt_mg<YT, 1>(C, halves, grid, lds, g, st);
    if (g.count <= 3) return launch_wt_mg<YT, 3>(C, halves, grid, lds, g, st);
    return launch_wt_mg<YT, kMaxGroupLaunch>(C, halves, grid, lds, g, st);
}

// ---------------------------------------------------------------- split K
// One matrix whose 16-row tiles number no more than the CUs (o, down at the
// decode shapes): with one tile per workgroup, every workgroup would read all
// m activation rows (twice its weight bytes at 16 tokens).  Here a workgroup
// takes T consecutive tiles (a row block) and one of kSkS
// quarters of K: every wave loads the activation fragments of its units of
// that quarter once, into registers, and uses them for all T tiles.  The
// waves' partial tiles are summed through LDS; the workgroup stores its fp32
// partial tiles in the workspace and counts itself in on its row block's
// counter.  The workgroup that arrives last (no waiting: the others have
// finished their stores already) adds the kSkS partials of each tile in
// split order -- the same order whoever comes last, so results are
// deterministic -- rescales, stores y and sets the counter back to 0 for the
// next launch.
//
// Visibility across the eight XCDs (each with its own L2) without cache
// maintenance: the partials are stored and loaded with the agent scope bit
// (sc1), so they are coherent across the XCDs by themselves; a store's
// completion (vmcnt) means it has reached that level, so each wave waits for
// its stores before the workgroup barrier that precedes the counter's
// atomic add.  An agent-scope release / acquire fence would write back /
// invalidate the whole L2 of the XCD instead (buffer_wbl2 / buffer_inv):
// measured at 32 us for the 4096 x 4096 launch at 16 tokens, against 8 us
// for the launch without split.
constexpr int kCachePolicyAgent = 16;  // sc1: agent scope (gfx9.4/9.5 cache-policy bits)
constexpr int kSkS = 4;          // splits of K
constexpr int kSkDepth = 2;      // tiles of weights in flight per wave
constexpr int kSkMaxT = kSkS;    // tiles per workgroup at most: T <= kSkS when tiles <= CUs
constexpr int kSkMaxUnits = 8;   // units of 64 k per wave in registers (K / kSkS <= 8 x 8 x 64)

struct SkPlan {
    int tiles, T, nrb, C, Cs, most;
};
static SkPlan splitk_plan(int64_t n, int64_t k) {
    SkPlan p;
    p.tiles = (int)((n + 15) / 16);
    const int cus = device_cu_count();
    p.T = (p.tiles * kSkS + cus - 1) / cus;  // about one workgroup per CU
    if (p.T < 1) p.T = 1;
    if (p.T == 3) p.T = 4;                    // instantiated tile counts: 1, 2, 4
    if (p.T > kSkMaxT) p.T = kSkMaxT;
    p.nrb = (p.tiles + p.T - 1) / p.T;
    p.C = (int)(k / kBUnit);
    p.Cs = (p.C + kSkS - 1) / kSkS;
    p.most = (p.Cs + kBWaves - 1) / kBWaves;
    return p;
}

// 0 when the split path does not apply: more tiles than CUs, K per split
// beyond the register-resident fragments, or K below kSkMinK (there the
// reduction's three memory round trips cost more than the activation reads
// they save: 4096 x 4096 at 4 tokens 8.0 against 6.6 us unsplit, tiled)
constexpr int64_t kSkMinK = 8192;
size_t qgemv_batch_splitk_workspace(int64_t n, int64_t k) {
    const SkPlan p = splitk_plan(n, k);
    if (k < kSkMinK || p.tiles > device_cu_count() || p.most > kSkMaxUnits || p.most < 1) return 0;
    const size_t parts = (size_t)kSkS * p.tiles * kWave * sizeof(f32x4);
    return parts + ((size_t)p.nrb * sizeof(uint32_t) + 255) / 256 * 256;
}

struct SkParams {
    const int8_t* wq;
    const float* s_w;
    const uint16_t* x;
    void* y;
    f32x4* part;     // [kSkS][tiles][64 lanes]
    uint32_t* ctr;   // [nrb], zero between launches
    int n, k, m, tiles, C, Cs;
};

// MOST units of 64 k per wave, T tiles per workgroup: the wave's activation
// fragments are requested with the first tile's weights, unit by unit, and
// kept in registers for all T tiles; the other tiles' weights follow two
// tiles ahead of the products, with no branches between the loads and the
// products, so the waits count down through the loads in order.  (Every
// tile requested up front measured 14.4 us for the 4096 x 11008 product at
// 16 tokens, two tiles ahead 13.2 us, one 13.6 us: with the whole share in
// flight no product starts before all of it has arrived; the activations
// interleaved with the first tile: 13.0 us.)
template <int YT, int MOST, int T, bool T16>
__global__ __launch_bounds__(kBThreads) void qgemv_batch_splitk_kernel(SkParams p) {
    __shared__ f32x4 red[T][kBWaves][kWave];
    __shared__ int last;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = lane & 15, g = lane >> 4;  // A row / B token, k group
    const int rb = (int)blockIdx.x / kSkS, sp = (int)blockIdx.x % kSkS;
    const int t0 = rb * T, nt = min(T, p.tiles - t0);
    const int K = p.k, M = p.m;
    // this wave's units: [c0, c1) of the split's [sp * Cs, min((sp + 1) * Cs, C))
    const int s0 = sp * p.Cs, s1 = min(s0 + p.Cs, p.C);
    const int c0 = s0 + wave * MOST, c1 = min(c0 + MOST, s1);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (uint32_t)(M * K * 2));
    const uint32_t oob_x = (uint32_t)(M * K * 2);
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.part, (uint32_t)(kSkS * p.tiles * kWave * 16));
    // weights of tile t (rows past n and units past the range read zeros
    // through the range check)
    u32x4 w[T][MOST];
    auto issue_t = [&](int t) {
        const int row0 = (t0 + t) * 16;
        const int rows = t < nt ? min(16, p.n - row0) : 0;
        // the tiled layout's last tile is padded to 16 rows (zeros)
        const uint32_t tile_bytes = (uint32_t)((T16 && rows > 0 ? 16 : rows) * K);
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.wq + (int64_t)min(row0, p.n) * K, tile_bytes);
#pragma unroll
        for (int u = 0; u < MOST; ++u) {
            const int c = c0 + u;
            if constexpr (T16) {
                // whole 1 KB blocks, each read once: non-temporal
                w[t][u] = load16_nt(rw, c < c1 ? (uint32_t)(c * 1024 + lane * 16) : tile_bytes);
            } else {
                w[t][u] = load16(rw, (c < c1 && i < rows) ? (uint32_t)(i * K + c * kBUnit + 16 * g) : tile_bytes);
            }
        }
    };
    // the activation fragments of the wave's units (tokens >= m read zeros)
    u32x4 xa[MOST], xb[MOST];
    {  // tile 0's weights interleaved with the activations, unit by unit, so
       // that its first products wait for their own unit only
        const int row0 = t0 * 16;
        const int rows = 0 < nt ? min(16, p.n - row0) : 0;
        const uint32_t tile_bytes = (uint32_t)((T16 && rows > 0 ? 16 : rows) * K);
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.wq + (int64_t)min(row0, p.n) * K, tile_bytes);
#pragma unroll
        for (int u = 0; u < MOST; ++u) {
            const int c = c0 + u;
            const bool ok = c < c1 && i < M;
            const uint32_t xo = (uint32_t)((i * K + c * kBUnit + 16 * g) * 2);
            xa[u] = load16(rx, ok ? xo : oob_x);
            xb[u] = load16(rx, ok ? xo + 16u : oob_x);
            if constexpr (T16) {  // whole 1 KB blocks, each read once: non-temporal
                w[0][u] = load16_nt(rw, c < c1 ? (uint32_t)(c * 1024 + lane * 16) : tile_bytes);
            } else {
                w[0][u] = load16(rw, (c < c1 && i < rows) ? (uint32_t)(i * K + c * kBUnit + 16 * g) : tile_bytes);
            }
        }
    }
    // kSkDepth tiles in flight: tile t + kSkDepth - 1 is requested when
    // tile t's products begin
#pragma unroll
    for (int t = 1; t < (T < kSkDepth ? T : kSkDepth); ++t) issue_t(t);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        if (t > 0 && t - 1 + kSkDepth < T) {
            __builtin_amdgcn_sched_barrier(0);
            issue_t(t - 1 + kSkDepth);
            __builtin_amdgcn_sched_barrier(0);
        }
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < MOST; ++u) {
            bf16x8 a0, a1;
            widen16(w[t][u], a0, a1);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(bf16x8, xa[u]), acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8, xb[u]), acc[t], 0, 0, 0);
        }
        red[t][wave][lane] = acc[t];
    }
    __syncthreads();
    // the waves' partial tiles, summed by wave t for tile t (fixed order);
    // lane l holds token l % 16, so lanes of tokens >= m store nothing
    const int tok = lane & 15;
    if (wave < nt) {
        f32x4 sum = red[wave][0][lane];
#pragma unroll
        for (int v = 1; v < kBWaves; ++v) {
            const f32x4 q = red[wave][v][lane];
            sum[0] += q[0];
            sum[1] += q[1];
            sum[2] += q[2];
            sum[3] += q[3];
        }
        if (tok < M)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sum), rp,
                                                   (uint32_t)((((size_t)sp * p.tiles + t0 + wave) * kWave + lane) * 16),
                                                   0, kCachePolicyAgent);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the partial has reached agent scope
    }
    __syncthreads();
    if (tid == 0) {
        const uint32_t before = __hip_atomic_fetch_add(p.ctr + rb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = before == kSkS - 1;
    }
    __syncthreads();
    if (!last) return;
    if (wave < nt && tok < M) {
        // the loads follow the counter's value (control dependency through
        // the barrier) and read at agent scope
        const int tile = t0 + wave;
        f32x4 q[kSkS];
#pragma unroll
        for (int s2 = 0; s2 < kSkS; ++s2)
            q[s2] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rp, (uint32_t)((((size_t)s2 * p.tiles + tile) * kWave + lane) * 16),
                                                  0, kCachePolicyAgent));
        f32x4 sum = q[0];
#pragma unroll
        for (int s2 = 1; s2 < kSkS; ++s2) {
            sum[0] += q[s2][0];
            sum[1] += q[s2][1];
            sum[2] += q[s2][2];
            sum[3] += q[s2][3];
        }
        const int row0 = tile * 16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = row0 + 4 * g + r;
            if (row < p.n) {
                const float o = sum[r] / p.s_w[row];
                const int64_t at = (int64_t)tok * p.n + row;
                if constexpr (YT == 0) static_cast<float*>(p.y)[at] = o;
                else static_cast<uint16_t*>(p.y)[at] = (uint16_t)f32_to_bf16(o);
            }
        }
    }
    if (tid == 0) __hip_atomic_store(p.ctr + rb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int YT, int MOST, bool T16>
static void launch_sk_t(int T, int grid, const SkParams& p, hipStream_t st) {
    if (T == 1) qgemv_batch_splitk_kernel<YT, MOST, 1, T16><<<grid, kBThreads, 0, st>>>(p);
    else if (T == 2) qgemv_batch_splitk_kernel<YT, MOST, 2, T16><<<grid, kBThreads, 0, st>>>(p);
    else qgemv_batch_splitk_kernel<YT, MOST, 4, T16><<<grid, kBThreads, 0, st>>>(p);
}
template <int YT, bool T16>
static void launch_sk(int most, int T, int grid, const SkParams& p, hipStream_t st) {
    switch (most) {
        case 1: launch_sk_t<YT, 1, T16>(T, grid, p, st); break;
        case 2: launch_sk_t<YT, 2, T16>(T, grid, p, st); break;
        case 3: launch_sk_t<YT, 3, T16>(T, grid, p, st); break;
        case 4: launch_sk_t<YT, 4, T16>(T, grid, p, st); break;
        case 5: launch_sk_t<YT, 5, T16>(T, grid, p, st); break;
        case 6: launch_sk_t<YT, 6, T16>(T, grid, p, st); break;
        case 7: launch_sk_t<YT, 7, T16>(T, grid, p, st); break;
        default: launch_sk_t<YT, 8, T16>(T, grid, p, st); break;
    }
}

hipError_t launch_qgemv_batch_splitk(const BatchArgs& a, void* ws, hipStream_t st) {
    const SkPlan pl = splitk_plan(a.n, a.k);
    if (pl.most < 1 || pl.most > kSkMaxUnits || pl.tiles > device_cu_count()) return hipErrorInvalidValue;
    SkParams p;
    p.wq = a.wq;
    p.s_w = a.s_w;
    p.x = static_cast<const uint16_t*>(a.x);
    p.y = a.y;
    p.part = static_cast<f32x4*>(ws);
    p.ctr = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + (size_t)kSkS * pl.tiles * kWave * sizeof(f32x4));
    p.n = (int)a.n;
    p.k = (int)a.k;
    p.m = a.m;
    p.tiles = pl.tiles;
    p.C = pl.C;
    p.Cs = pl.Cs;
    const int grid = pl.nrb * kSkS;
    if (a.yt == 0) a.t16 ? launch_sk<0, true>(pl.most, pl.T, grid, p, st) : launch_sk<0, false>(pl.most, pl.T, grid, p, st);
    else a.t16 ? launch_sk<1, true>(pl.most, pl.T, grid, p, st) : launch_sk<1, false>(pl.most, pl.T, grid, p, st);
    return hipGetLastError();
}

hipError_t launch_qgemv_batch(const BatchArgs* a, int count, hipStream_t st) {
    BGroup g;
    g.count = count;
    g.k = (int32_t)a[0].k;
    g.m = a[0].m;
    g.t16 = a[0].t16 ? 1 : 0;
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
        // activations loaded once per workgroup (into LDS, or into the
        // waves' registers where the eight waves share each tile): one
        // workgroup per CU, each walking its tiles
        const int grid = cus;
        if (a[0].t16) {
            // five or more tiles per workgroup keep five or more waves busy
            // with one tile each; three or four keep six to eight busy with
            // half a tile each; fewer, and the eight waves share each tile
            // (measured on MI355X at 16 tokens: 1376 tiles 21.4 against
            // 25.4 us; 768 tiles 13.1 in halves, 18.6 whole, 15.6 shared)
            const int per = (tiles + cus - 1) / cus;
            const bool halves = per >= 3 && per <= 4 && C % 8 == 0;
            if (per >= 5 || halves) {
                const size_t wt_bytes = (size_t)C * 2 * kWave * sizeof(u32x4);
                return a[0].yt == 0 ? launch_wt<0>(C, halves, grid, wt_bytes, g, st)
                                    : launch_wt<1>(C, halves, grid, wt_bytes, g, st);
            }
            return a[0].yt == 0 ? launch_xl<0>(most, grid, g, st) : launch_xl<1>(most, grid, g, st);
        }
        auto k0 = qgemv_batch_kernel<0, true, false>;
        auto k1 = qgemv_batch_kernel<1, true, false>;
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
    if (a[0].t16) {
        if (a[0].yt == 0) qgemv_batch_kernel<0, false, true><<<grid, kBThreads, 0, st>>>(g);
        else qgemv_batch_kernel<1, false, true><<<grid, kBThreads, 0, st>>>(g);
    } else {
        if (a[0].yt == 0) qgemv_batch_kernel<0, false, false><<<grid, kBThreads, 0, st>>>(g);
        else qgemv_batch_kernel<1, false, false><<<grid, kBThreads, 0, st>>>(g);
    }
    return hipGetLastError();
}

}  // namespace qg
