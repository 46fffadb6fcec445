// qgemv.hip -- batch-1 quantized matrix-vector products for gfx950.
//
// At batch 1 every weight byte is read once per token and the arithmetic per
// byte is a handful of ALU operations, so the kernel is bound by HBM
// bandwidth: the design goal is to keep enough 16-byte loads in flight on
// every CU and to keep the per-byte ALU work well under the VALU budget.
//
// Layout of the work
//   * grid: about one 512-thread workgroup (8 waves, 2 per SIMD) per CU, each
//     owning a contiguous block of rows; a grouped launch covers several
//     matrices that share x (q, k, v or gate, up) with workgroups handed out
//     in proportion to their rows;
//   * each wave takes groups of U rows; an "item" is U rows x JS chunk
//     columns per lane; items are double-buffered in registers so the next
//     item's loads are in flight while the current one is reduced; the
//     groups of a workgroup are a fixed share per wave (w, w + 8, ...), or,
//     for the sign + residual formats, two fixed groups and then the next
//     free one from an LDS counter (the younger wave of each SIMD pair
//     otherwise finishes far behind the older);
//   * the activation vector: for int8 weights with bf16 / fp32 x, every item
//     loads its own 16-activation slice next to its weights (x is L2
//     resident; no LDS and no barrier); the other formats stage x once per
//     workgroup in LDS in the form the inner loop wants (int8 codes quantized
//     in-kernel; codes permuted to the ternary unpack order; bf16 pairs for
//     the sign path), zero-padded so ragged K needs no branches;
//   * weights are read through buffer resources: out-of-range lanes (ragged
//     rows or chunks) get zeros from the hardware range check;
//   * per-row partial sums are reduced across the wave with DPP row / bank
//     moves, and lane 63, which ends up with the sums, applies the per-row
//     scale and stores.
//
// Formats (codes as stored by the library's packing):
//   INT8 (x float) : 16 B chunk = 16 int8 weights; v_cvt_f32_i32 (SDWA byte
//                    select) + FMA against fp32 x.
//   INT8 (x int8)  : 16 B chunk = 16 weights; v_dot4 against in-kernel int8 x.
//   TERNARY2       : 16 B chunk = 64 weights as 2-bit fields q+1; each dword
//                    is split into 4 masked byte planes (fields stay in place,
//                    i.e. scaled by 1, 4, 16, 16) and fed to v_dot4 against x
//                    permuted to the same order; sum_k (q+1) x - sum_k x.
//   SIGN1_RES8     : 32-column unit = 32 B int8 residual + 4 B sign bits; the
//                    residual becomes bf16 pairs (col j, col j+16) and the sign
//                    bits become +-1.0 bf16 pairs with one bit-field insert;
//                    both go through v_dot2_f32_bf16 against bf16 x pairs.
//   TERNARY3       : 16 B chunk = 80 weights, five per byte as the base-3
//                    fraction t = ceil(256 v / 243).  The four bytes of a
//                    dword sit in four 16-bit lanes of a 64-bit value; one
//                    64-bit shift-add multiplies every lane by 3, which moves
//                    the next digit into bits 8-9 of the lane; one v_perm
//                    gathers the four digits, v_dot4 takes them against x
//                    staged in the same (dword, digit) order, and a mask
//                    keeps the fraction; then sum_k (q+1) x - sum_k x as for
//                    TERNARY2.
//   SIGN1_RES8Z    : the same units; every residual pair also goes through
//                    one more v_dot2 with the pair (-z, -z), so the sum is
//                    sum_k (rq - z) x[k] as it accumulates (a z * sum_k x[k]
//                    correction at the end would cancel in fp32 whenever the
//                    activations have a large mean).
//   Q4K            : 16 B chunk = one group of 32 4-bit codes; the chunk's
//                    16-byte super-block record gives the group's S and M
//                    (6-bit fields, fp16 d / dmin); a byte's two codes become
//                    the bf16 pair (128 + q, 128 + q') by one v_perm and an
//                    OR, v_dot2_f32_bf16 takes it against the x pair, and
//                    S * that + (M - 128 S) * sum_k x removes the offset.
#include <type_traits>

#include "qg_device.h"
#include "qg_launch.h"

namespace qg {

enum { F_INT8F = 0, F_INT8I = 1, F_TERN = 2, F_SR = 3, F_Q4 = 4, F_SRZ = 5, F_TERN3 = 6, F_INT8L = 7 };
// the sign + residual formats (symmetric residual, or with a zero-point)
template <int F>
constexpr bool kSignRes = (F == F_SR || F == F_SRZ);

struct KParams {
    const uint8_t* codes;
    const int8_t* resid;
    const float* scale;
    const float* scale2;
    const int8_t* zero;
    const void* x;
    void* y;
    int32_t* acc_out;
    int32_t n, k, rows_per_wg;
};

// A launch covers up to kMaxGroup weight matrices that share K and x (for
// example the q, k and v projections of a layer).  Workgroups are handed out
// per matrix in proportion to its rows; matrix m is grid row blockIdx.y = m.
// The argument holds MG slots (1, 3 or 8, the fewest that fit the launch):
// on MI355X a launch in a HIP graph costs about 0.15 us more with the full
// 8-slot (576-byte) argument than with a small one.
constexpr int kMaxGroup = 8;
template <int MG>
struct KGroup {
    KParams mats[MG];
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}


template <int F>
struct Fmt;
template <>
struct Fmt<F_INT8F> {
    static constexpr int kColsPerChunk = 16;
    static constexpr int kLdsBytesPerCol = 0;  // x travels with each item instead
    struct Frag { u32x4 w; u32x4 x[4]; };      // x: 16 activations (bf16: x[0..1], fp32: x[0..3])
};
// int8 weights with float x staged once per workgroup in LDS as fp32 (rows
// longer than one item of register-resident x): chunk c's 16 activations are
// four 16-byte pieces, stored as four planes [piece][chunk]
template <>
struct Fmt<F_INT8L> {
    static constexpr int kColsPerChunk = 16;
    static constexpr int kLdsBytesPerCol = 4;
    struct Frag { u32x4 w; };
};
template <>
struct Fmt<F_INT8I> {
    static constexpr int kColsPerChunk = 16;
    static constexpr int kLdsBytesPerCol = 1;
    struct Frag { u32x4 w; };
};
template <>
struct Fmt<F_TERN> {
    static constexpr int kColsPerChunk = 64;
    static constexpr int kLdsBytesPerCol = 1;
    struct Frag { u32x4 w; };
};
template <>
struct Fmt<F_TERN3> {
    static constexpr int kColsPerChunk = 80;  // 16 B of base-3 bytes, 5 weights each
    static constexpr int kLdsBytesPerCol = 1;
    struct Frag { u32x4 w; };
};
template <>
struct Fmt<F_SR> {
    static constexpr int kColsPerChunk = 32;
    static constexpr int kLdsBytesPerCol = 2;
    struct Frag { u32x4 r0, r1; uint32_t s; };
};
template <>
struct Fmt<F_SRZ> {
    static constexpr int kColsPerChunk = 32;
    static constexpr int kLdsBytesPerCol = 2;
    struct Frag { u32x4 r0, r1; uint32_t s, z; };  // z: the row's zero-point (j = 0 only)
};
template <>
struct Fmt<F_Q4> {
    static constexpr int kColsPerChunk = 32;   // one group: 16 B of 4-bit codes
    static constexpr int kLdsBytesPerCol = 0;  // x (bf16) travels with each item
    struct Frag { u32x4 w; u32x4 meta; u32x4 x[4]; };
};

// LDS byte of activation column c for the base-3 format: chunk c / 80 holds
// 20 dwords, dword 5 d + i carrying column 80 g + 20 d + 5 b + i in byte b.
__device__ __forceinline__ int tern3_slot(int c) {
    const int g = c / 80, r = c - 80 * g;
    const int d = r / 20, r2 = r - 20 * d;
    const int b = r2 / 5, i = r2 - 5 * b;
    return 80 * g + 4 * (5 * d + i) + b;
}

// Workgroup shape: 8 waves (2 per SIMD, so one wave's LDS / ALU latency is
// covered by the other's work), one workgroup per CU.
constexpr int kQThreads = 512;
constexpr int kQWaves = kQThreads / kWave;
constexpr int kXL = 4;  // x pieces of 16 B held in registers per thread (K <= 16384 bf16 / 8192 fp32)

// XREG (items spanning the whole row; int8 weights with float x, or 4-bit
// groups): lane l only ever multiplies the columns of its chunks
// c = l + 64 j (j < JS), so it loads and converts that x (and, for the 4-bit
// groups, the groups' sums) once before the first item; the items then carry
// weights (and super-block records) only.
// NPF > 0: every item of a wave (at most NPF, which the host checks) goes
// out in the prologue, so all of the wave's weights are in flight while x is
// prepared and the decode work is spread over all waves (short rows, few per
// wave: the ternary formats at the decode shapes).
template <int F, int XT, int YT, int U, int JS, bool XREG = false, int NPF = 0, int MG = kMaxGroup>
__global__ __launch_bounds__(kQThreads) void qgemv_kernel(KGroup<MG> grp) {
    using Frag = typename Fmt<F>::Frag;
    constexpr int kCols = Fmt<F>::kColsPerChunk;
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
    __shared__ float redf[kQWaves];
    __shared__ int redi[kQWaves];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // the matrix is blockIdx.y: its parameters come in the first round of
    // kernel-argument reads, with no search over the group before them
    // (measured 0.19 us per launch at the decode shapes)
    constexpr bool kDynamic = kSignRes<F>;  // row groups handed out dynamically (see below)
    // int8 weights with x staged in LDS: the row groups of the two waves of
    // a SIMD form one pool, taken from both ends (see below).  Measured on
    // MI355X at 4096 x 11008: 10.6 -> 10.1 us.  Not for register-resident x:
    // there the compiler reuses a register of the prefetched item for the
    // LDS read and waits for every load at the loop head (4096 x 4096:
    // 4.85 -> 5.14 us).
    constexpr bool kPaired = F == F_INT8L;
    constexpr bool kDynItems = kDynamic || kPaired;  // items named by (group, segment)
    const int mi = blockIdx.y;
    const KParams& p = grp.mats[mi];
    const int K = p.k;
    const int row0 = (int)blockIdx.x * p.rows_per_wg;
    if (row0 >= p.n) return;  // a smaller matrix of the group needs fewer workgroups
    const int rows = min(p.rows_per_wg, p.n - row0);
    const int C = (K + kCols - 1) / kCols;  // chunks per row (the last may be partly padding)
    const int J = (C + 63) / 64;       // chunk iterations per lane per row
    const int nseg = (J + JS - 1) / JS;
    // x is staged (zero-padded) for every chunk iteration a segment can touch
    const int padded_cols = nseg * JS * 64 * kCols;
    // ternary 2-bit and sign + residual: a chunk's x is four 16-byte pieces,
    // stored as four planes [piece][chunk], so that the 16 lanes of an LDS
    // read phase take 16 consecutive 16-byte slots (one piece per lane at a
    // 64-byte stride would put lanes l and l + 4 on the same banks)
    const int NC = nseg * JS * 64;  // chunks in the staged copy

    // ------------------------------------------------------------ stream
    const int rowB = (F == F_TERN) ? K / 4 : kSignRes<F> ? K / 8 : (F == F_Q4) ? K / 2 : (F == F_TERN3) ? 16 * C : K;  // code bytes per row (K for int8)
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.codes + (int64_t)row0 * rowB, (uint32_t)(rows * rowB));
    __amdgpu_buffer_rsrc_t rr = rc;
    if constexpr (kSignRes<F>) rr = make_rsrc(p.resid + (int64_t)row0 * K, (uint32_t)(rows * K));
    if constexpr (F == F_Q4) rr = make_rsrc(p.resid + (int64_t)row0 * (K / 16), (uint32_t)(rows * (K / 16)));
    __amdgpu_buffer_rsrc_t rz = rc;  // zero-points of this workgroup's rows (SIGN1_RES8Z)
    if constexpr (F == F_SRZ) rz = make_rsrc(p.zero + row0, (uint32_t)rows);
    // with the dynamic groups the row scales are prefetched with each item
    // (read in the epilogue, their loads would be vector loads that wait for
    // the prefetched item too); the fixed share reads them there (scalar loads)
    constexpr bool kRowScale = kDynItems;
    constexpr bool kTensorScale = (F == F_TERN || F == F_TERN3);
    const __amdgpu_buffer_rsrc_t rs1 = make_rsrc(p.scale + (kTensorScale ? 0 : row0), kTensorScale ? 4u : (uint32_t)(rows * 4));
    const __amdgpu_buffer_rsrc_t rs2 = make_rsrc(kSignRes<F> ? p.scale2 + row0 : p.scale, kSignRes<F> ? (uint32_t)(rows * 4) : 0u);
    const uint32_t oob_c = (uint32_t)(rows * rowB);
    const uint32_t oob_r = (uint32_t)(rows * (F == F_Q4 ? K / 16 : K));

    // Row groups (U rows).  Waves w and w + 4 share a SIMD and the older
    // issues first: with a fixed share the younger waves of a sign + residual
    // launch finished up to a quarter of the kernel later (per-wave
    // timestamps on MI355X), streaming alone at the end.  For those formats
    // the groups are handed out dynamically: a wave takes groups w and w + 8
    // (known before any LDS access, which lets the prologue issue two items
    // at once) and then the next free group from an LDS counter, fetched one
    // group ahead of its use.  The other formats keep the fixed share (w,
    // w + 8, ...): at their decode shapes the counter's atomic made the
    // compiler wait for the prefetched item, which cost more than it saved.
    const int ngroups = (rows + U - 1) / U;
    const int my_groups = ngroups > wave ? (ngroups - wave + kQWaves - 1) / kQWaves : 0;
    const int nit = my_groups * nseg;  // fixed share: items of this wave
    __shared__ int next_group;
    if (kDynamic && tid == 0) next_group = 2 * kQWaves;  // read only after the prologue's barrier
    struct Item {
        int g, seg;  // row group, segment of the row (wave-uniform)
    };
    // Pairs (int8 weights, float x).  Waves w and w + 4 (one SIMD) share the
    // groups g = w % 4 + 4 i, i < npool: the older wave takes i = 0, 1, ...
    // from the front and owns [0, own_front); the younger takes
    // i = npool - 1, npool - 2, ... from the back and owns [own_back, npool).
    // Before taking its next index a wave reads the other's published bound
    // and takes the index only if the other does not own it; after taking it
    // the wave publishes its new bound.  Both accesses are plain LDS words
    // written and read by the whole wave (no atomic, no branch); a race can
    // only let both waves take the last index, which then is computed twice
    // with identical results, never skipped.
    __shared__ int pair_bound[kQWaves];  // [w]: own_front of front wave w, [w + 4]: own_back of back wave w + 4
    const int pair = wave & 3;
    const bool front = wave < 4;
    const int npool = ngroups > pair ? (ngroups - pair + 3) / 4 : 0;
    int own = front ? (npool >= 1 ? 1 : 0) : (npool >= 2 ? npool - 1 : npool);  // this wave's bound
    if constexpr (kPaired) pair_bound[wave] = own;  // (whole wave, one value) read only after the prologue's barrier
    auto next_pair_group = [&]() -> int {
        const int other = __builtin_amdgcn_readfirstlane(pair_bound[front ? wave + 4 : wave - 4]);
        int g = ngroups;  // past the last group: the item reads zeros and stores nothing
        if (front) {
            const int i = own;
            if (i < other) { g = pair + 4 * i; own = i + 1; }
        } else {
            const int j = own - 1;
            if (j >= other && j >= 0) { g = pair + 4 * j; own = j; }
        }
        pair_bound[wave] = own;
        return g;
    };
    int started = 1;  // groups this wave has started
    int g_pend = 0;   // lane 0: the group after the current one (LDS atomic in flight)
    typedef __attribute__((address_space(3))) int lds_int;
    lds_int* const ctr = (lds_int*)(&next_group);
    auto fetch_group = [&]() {
        if (lane == 0) g_pend = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    auto next_item = [&](const Item& x) -> Item {
        if (x.seg + 1 < nseg) return Item{x.g, x.seg + 1};
        int g;
        if constexpr (kPaired) {
            g = next_pair_group();
        } else if (!kDynamic || started == 1) {
            g = wave + kQWaves;
        } else {
            g = __builtin_amdgcn_readfirstlane(g_pend);
            fetch_group();
        }
        ++started;
        return Item{g, 0};
    };

    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (uint32_t)(K * (XT == 0 ? 4 : 2)));
    // Every issue is unconditional (no load sits behind a branch after a
    // load that is waited on: the waitcnt pass would otherwise merge paths
    // and wait for the prefetched item too).  Groups past the last, ragged
    // rows and chunks read zeros through out-of-range offsets.
    // an item is named by its index in the wave's fixed share (int) or, with
    // dynamic groups, by its Item
    auto group_of = [&](const auto& x) -> int {
        if constexpr (std::is_integral_v<std::decay_t<decltype(x)>>) return wave + kQWaves * ((int)x / nseg);
        else return x.g;
    };
    auto seg_of = [&](const auto& x) -> int {
        if constexpr (std::is_integral_v<std::decay_t<decltype(x)>>) return (int)x % nseg;
        else return x.seg;
    };
    auto issue = [&](const auto& x, Frag (&fr)[U][JS], float (&sc)[U][2]) {
        const bool live = true;
        const int g = group_of(x);
        const int seg = seg_of(x);
        if constexpr (kRowScale) {  // every item (no load behind a branch)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = g * U + u;
                const uint32_t o = kTensorScale ? 0u : (r < rows ? (uint32_t)(4 * r) : (uint32_t)(4 * rows));
                sc[u][0] = __uint_as_float(load4(rs1, o));
                if constexpr (kSignRes<F>) sc[u][1] = __uint_as_float(load4(rs2, o));
            }
        }
#pragma unroll
        for (int j = 0; j < JS; ++j) {  // issue in the order consume() uses the data
            const int c = lane + 64 * (seg * JS + j);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = g * U + u;
                const bool ok = live && (r < rows) && (c < C);
                if constexpr (kSignRes<F>) {
                    const uint32_t orr = ok ? (uint32_t)(r * K + 32 * c) : oob_r;
                    fr[u][j].r0 = load16(rr, orr);  // r0 / r1 split each line: normal loads
                    fr[u][j].r1 = load16(rr, ok ? orr + 16 : oob_r);
                    fr[u][j].s = load4_nt(rc, ok ? (uint32_t)(r * rowB + 4 * c) : oob_c);
                    if constexpr (F == F_SRZ) {
                        if (j == 0) fr[u][0].z = load1(rz, r < rows ? (uint32_t)r : (uint32_t)rows);
                    }
                } else if constexpr (F == F_Q4) {
                    // the group's 32 activations (bf16, shared by the U rows; not
                    // with XREG), then its super-block record, then its codes
                    if (!XREG && u == 0) {
                        const uint32_t xo = (c < C) ? (uint32_t)(64 * c) : (uint32_t)(K * 2);
#pragma unroll
                        for (int h = 0; h < 4; ++h) fr[0][j].x[h] = load16(rx, xo + 16 * h);
                    }
                    fr[u][j].meta = load16_nt(rr, ok ? (uint32_t)(r * (K / 16) + 16 * (c >> 3)) : oob_r);
                    fr[u][j].w = load16_nt(rc, ok ? (uint32_t)(r * rowB + 16 * c) : oob_c);
                } else {
                    if constexpr (F == F_INT8F) {
                        // the 16 activations of this chunk, requested just ahead of the
                        // chunk's weights and shared by the U rows of the item
                        // (with XREG they are in registers already)
                        if (!XREG && u == 0) {
                            constexpr int kXB = (XT == 0) ? 64 : 32;  // bytes of x per chunk
                            const uint32_t xo = (c < C) ? (uint32_t)(kXB * c) : (uint32_t)(K * (XT == 0 ? 4 : 2));
#pragma unroll
                            for (int h = 0; h < kXB / 16; ++h) fr[0][j].x[h] = load16(rx, xo + 16 * h);
                        }
                    }
                    fr[u][j].w = load16_nt(rc, ok ? (uint32_t)(r * rowB + 16 * c) : oob_c);
                }
            }
        }
    };

    // ------------------------------------------------------------ stage x
    // vmcnt retires loads in issue order, so x must be requested BEFORE the
    // first weights: then staging waits only for x while the weights stream
    // in.  Each thread loads kXL pieces of 16 B (8 bf16 or 4 fp32) into
    // registers through a buffer resource (pieces past K read as zeros).
    constexpr int kElems = (XT == 0) ? 4 : 8;  // elements per 16 B piece
    const int npieces = K / kElems;
    // (unconditional loads: pieces past K read zeros through the range check;
    // a branch around a load would make the compiler wait for all loads at
    // the join, the weights included)
    static_assert(F != F_Q4 || XT == 1, "4-bit groups take bf16 activations");
    static_assert(!XREG || F == F_Q4 || F == F_INT8F, "register-resident x: 4-bit groups and int8 weights");
    // XREG, int8 weights: this lane's raw x (16 B pieces) is requested here,
    // ahead of the first item's weights, and converted to fp32 after that
    // item is issued (so the conversion waits for x only)
    constexpr bool kXRegI8 = XREG && F == F_INT8F;
    constexpr int kXPc = (XT == 0) ? 4 : 2;  // 16-byte pieces of x per chunk
    u32x4 xraw[kXRegI8 ? JS : 1][kXRegI8 ? kXPc : 1];
    float xf[kXRegI8 ? JS : 1][kXRegI8 ? 16 : 1];
    if constexpr (kXRegI8) {
        const uint32_t xend = (uint32_t)(K * (XT == 0 ? 4 : 2));
#pragma unroll
        for (int j = 0; j < JS; ++j) {
            const int c = lane + 64 * j;
#pragma unroll
            for (int q = 0; q < kXPc; ++q) xraw[j][q] = load16(rx, c < C ? (uint32_t)(16 * kXPc * c + 16 * q) : xend);
        }
        __builtin_amdgcn_sched_barrier(0);  // x goes out ahead of the first weights
    }
    // XREG, 4-bit groups: this lane's x (fp32) and the sums of its groups, for every row
    constexpr bool kXRegQ4 = XREG && F == F_Q4;
    uint32_t xq4[kXRegQ4 ? JS : 1][kXRegQ4 ? 16 : 1];  // bf16 pairs
    float xsq4[kXRegQ4 ? JS : 1];
    if constexpr (kXRegQ4) {
        const uint32_t xend = (uint32_t)(K * 2);
#pragma unroll
        for (int j = 0; j < JS; ++j) {
            const int c = lane + 64 * j;
            u32x4 h[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) h[q] = load16(rx, c < C ? (uint32_t)(64 * c + 16 * q) : xend);
            float xs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const uint32_t d = h[t >> 2][t & 3];
                xq4[j][t] = d;
                xs[(2 * t) & 3] += bf16_to_f32(d & 0xFFFFu);
                xs[(2 * t + 1) & 3] += __uint_as_float(d & 0xFFFF0000u);
            }
            xsq4[j] = (xs[0] + xs[1]) + (xs[2] + xs[3]);
        }
    }
    constexpr bool kXPerItem = (F == F_INT8F || F == F_Q4);  // x travels with the items (or sits in registers): nothing staged
    // ternary 2-bit: a thread owns whole 16-column groups m = tid + 512 r
    // (r < kGW in registers), so that it can write each group's codes to LDS
    // as one 16-byte store in the byte-plane order
    constexpr bool kGroups16 = (F == F_TERN);
    constexpr int kPG = 16 / kElems;  // 16-byte pieces per 16-column group
    constexpr int kGW = 2;            // groups per thread in registers (K <= 16384)
    constexpr int kXW = kGroups16 ? kGW * kPG : kXL;
    u32x4 xr[kXW];
    if constexpr (!kXPerItem) {
        const uint32_t xend = (uint32_t)(K * (XT == 0 ? 4 : 2));
#pragma unroll
        for (int l = 0; l < kXW; ++l) {
            const int pi = kGroups16 ? kPG * (tid + kQThreads * (l / kPG)) + l % kPG : tid + kQThreads * l;
            xr[l] = load16(rx, pi < npieces ? (uint32_t)(16 * pi) : xend);
        }
        __builtin_amdgcn_sched_barrier(0);  // x goes out ahead of the first weights
    }
    Frag fa[U][JS], fb[U][JS];
    float sa[U][2] = {}, sb[U][2] = {};  // the items' row scales
    constexpr int kNP = NPF > 0 ? NPF : 1;
    Frag fp[kNP][U][JS];   // NPF: every item of the wave
    float sp[kNP][U][2] = {};
    // unconditional, like the x loads: a wave without rows reads zeros (its
    // offsets are out of range) and never consumes them.  For the ternary
    // formats, whose x prologue is a quantization with a workgroup max, the
    // second item goes out before it too: at the decode shapes a wave owns
    // only one or two items, which then all stream while x is prepared
    // (measured faster there, and slower for the other staged formats).
    constexpr bool kTwoAhead = (F == F_TERN || F == F_TERN3 || F == F_INT8L);
    Item ia{wave, 0}, ib{0, 0};
    if constexpr (NPF > 0) {
        static_assert(!kDynItems, "prefetch-all takes the fixed share");
#pragma unroll
        for (int i = 0; i < NPF; ++i) issue(i, fp[i], sp[i]);  // items past nit read zeros
    } else if constexpr (kPaired) {  // the first index of each end (taken without a check)
        ia.g = front ? (npool >= 1 ? pair : ngroups) : (npool >= 2 ? pair + 4 * (npool - 1) : ngroups);
        issue(ia, fa, sa);
    } else if constexpr (kDynamic) {
        issue(ia, fa, sa);
    } else {
        issue(0, fa, sa);
        if constexpr (kTwoAhead) issue(1, fb, sb);
    }
    if constexpr (kXRegI8) {
        __builtin_amdgcn_sched_barrier(0);  // the first item is in flight before x is converted
#pragma unroll
        for (int j = 0; j < JS; ++j) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                if constexpr (XT == 0) {
                    xf[j][q] = __uint_as_float(xraw[j][q >> 2][q & 3]);
                } else {
                    const uint32_t d = xraw[j][q >> 3][(q >> 1) & 3];
                    xf[j][q] = (q & 1) ? __uint_as_float(d & 0xFFFF0000u) : bf16_to_f32(d & 0xFFFFu);
                }
            }
        }
    }

    // piece -> fp32 values
    auto piece_vals = [&](const u32x4& r, float v[kElems]) {
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
    // visit every real piece of x once: f(piece index, values); pieces past
    // the register window (K > kXL * 256 pieces) are loaded here, after the
    // weights, and so wait for them
    // (guarded = false: the register window is visited unconditionally --
    // its pieces past K hold zeros -- so no branch sits between the x loads
    // and their use)
    auto for_pieces = [&](auto&& f, bool guarded = true) {
#pragma unroll
        for (int l = 0; l < kXL; ++l) {
            const int pi = tid + kQThreads * l;
            if (!guarded || pi < npieces) {
                float v[kElems];
                piece_vals(xr[l], v);
                f(pi, v);
            }
        }
        for (int pi = tid + kQThreads * kXL; pi < npieces; pi += kQThreads) {
            float v[kElems];
            piece_vals(load16(rx, (uint32_t)(16 * pi)), v);
            f(pi, v);
        }
    };

    float sx = 1.0f;  // activation scale (integer modes)
    int sum_xq = 0;   // sum of int8 activations (ternary offset correction)
    if constexpr (kXPerItem) {
        // nothing to stage: every item carries its own slice of x
    } else if constexpr (kGroups16) {
        // 16-column groups m: codes of columns 16 m + 4 b + f go to byte b of
        // dword f of slot (m % 4, m / 4), i.e. chunk m / 4, plane m % 4 (the
        // byte-plane order of the 2-bit decode); one 16-byte LDS store each
        const int ngr = K / 16;  // K % 64 == 0
        auto group_vals = [&](const u32x4* pc, float v[16]) {
#pragma unroll
            for (int q = 0; q < kPG; ++q) piece_vals(pc[q], v + q * kElems);
        };
        auto load_group = [&](int mg, u32x4* pc) {
#pragma unroll
            for (int q = 0; q < kPG; ++q) pc[q] = load16(rx, (uint32_t)(16 * (kPG * mg + q)));
        };
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < kGW; ++r) {  // unconditional: groups past K hold zeros
            float v[16];
            group_vals(xr + r * kPG, v);
#pragma unroll
            for (int e = 0; e < 16; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e]));
        }
        for (int mg = tid + kQThreads * kGW; mg < ngr; mg += kQThreads) {  // past the register window
            u32x4 pc[kPG];
            load_group(mg, pc);
            float v[16];
            group_vals(pc, v);
#pragma unroll
            for (int e = 0; e < 16; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e]));
        }
        m = wave_max_to_lane63(m);
        if (lane == 63) redf[wave] = m;
        lds_barrier();
#pragma unroll
        for (int i = 0; i < kQWaves; ++i) m = __builtin_fmaxf(m, redf[i]);
        sx = absmax_scale(m);
        auto put_group = [&](int mg, const float* v) {
            u32x4 d;
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                uint32_t w = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int q = qcode(v[4 * b + f], sx);
                    sum_xq += q;
                    w |= (uint32_t)(q & 0xFF) << (8 * b);
                }
                d[f] = w;
            }
            reinterpret_cast<u32x4*>(xs)[(mg & 3) * NC + (mg >> 2)] = d;
        };
#pragma unroll
        for (int r = 0; r < kGW; ++r) {
            const int mg = tid + kQThreads * r;
            if (mg < ngr) {
                float v[16];
                group_vals(xr + r * kPG, v);
                put_group(mg, v);
            }
        }
        for (int mg = tid + kQThreads * kGW; mg < ngr; mg += kQThreads) {
            u32x4 pc[kPG];
            load_group(mg, pc);
            float v[16];
            group_vals(pc, v);
            put_group(mg, v);
        }
        {  // whole padding chunks (K % 64 == 0), in all four planes
            const int c0 = K / 64, npad = NC - c0;
            for (int i = tid; i < 4 * npad; i += kQThreads)
                reinterpret_cast<u32x4*>(xs)[(i / npad) * NC + c0 + i % npad] = u32x4{0u, 0u, 0u, 0u};
        }
        sum_xq = wave_sum_to_lane63(sum_xq);  // per-wave partials, summed after the staging barrier
        if (lane == 63) redi[wave] = sum_xq;
    } else if constexpr (F == F_INT8I || F == F_TERN || F == F_TERN3) {
        float m = 0.0f;
        for_pieces(
            [&](int, const float* v) {
#pragma unroll
                for (int e = 0; e < kElems; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e]));
            },
            false);
        // max over the workgroup with a single barrier (redf is not reused);
        // DPP within the wave, no LDS round trips
        m = wave_max_to_lane63(m);
        if (lane == 63) redf[wave] = m;
        lds_barrier();
#pragma unroll
        for (int i = 0; i < kQWaves; ++i) m = __builtin_fmaxf(m, redf[i]);
        sx = absmax_scale(m);
        for_pieces([&](int pi, const float* v) {
#pragma unroll
            for (int e = 0; e < kElems; ++e) {
                const int q = qcode(v[e], sx);
                sum_xq += q;
                const int c = pi * kElems + e;
                if constexpr (F == F_INT8I) {
                    xs[c] = (uint8_t)(q & 0xFF);
                } else if constexpr (F == F_TERN3) {
                    xs[tern3_slot(c)] = (uint8_t)(q & 0xFF);
                } else {  // column 64 ch + 16 d + 4 b + f: plane d, chunk ch, byte 4 f + b (byte-plane order)
                    const int l = c & 15;
                    xs[(((c >> 4) & 3) * NC + (c >> 6)) * 16 + 4 * (l & 3) + (l >> 2)] = (uint8_t)(q & 0xFF);
                }
            }
        });
        if constexpr (F == F_TERN3) {  // padding columns sit inside the last chunk's permutation
            for (int c = K + tid; c < padded_cols; c += kQThreads) xs[tern3_slot(c)] = 0;
        } else if constexpr (F == F_TERN) {  // whole padding chunks (K % 64 == 0), in all four planes
            const int c0 = K / 64, npad = NC - c0;
            for (int i = tid; i < 4 * npad; i += kQThreads)
                reinterpret_cast<u32x4*>(xs)[(i / npad) * NC + c0 + i % npad] = u32x4{0u, 0u, 0u, 0u};
        } else {
            for (int i = K / 4 + tid; i < padded_cols / 4; i += kQThreads) reinterpret_cast<uint32_t*>(xs)[i] = 0u;
        }
        if constexpr (F == F_TERN || F == F_TERN3) {  // per-wave partials, summed after the staging barrier
            sum_xq = wave_sum_to_lane63(sum_xq);
            if (lane == 63) redi[wave] = sum_xq;
        }
    } else if constexpr (F == F_INT8L) {  // column 16 ch + 4 pc + e: plane pc, chunk ch, dword e (fp32)
        float* xfl = reinterpret_cast<float*>(xs);
        for_pieces([&](int pi, const float* v) {
#pragma unroll
            for (int e = 0; e < kElems; ++e) {
                const int c = pi * kElems + e;
                xfl[4 * (((c >> 2) & 3) * NC + (c >> 4)) + (c & 3)] = v[e];
            }
        });
        const int c0 = K / 16, npad = NC - c0;  // whole padding chunks (K % 16 == 0), in all four planes
        for (int i = tid; i < 4 * npad; i += kQThreads)
            reinterpret_cast<u32x4*>(xs)[(i / npad) * NC + c0 + i % npad] = u32x4{0u, 0u, 0u, 0u};
    } else {  // sign + residual: pair p = q & 15 of unit u is bf16 x[32u+q] | bf16 x[32u+q+16] << 16,
              // in plane p / 4, slot u, dword p % 4
        uint16_t* xh = reinterpret_cast<uint16_t*>(xs);
        for_pieces([&](int pi, const float* v) {
#pragma unroll
            for (int e = 0; e < kElems; ++e) {
                const int c = pi * kElems + e;
                const int u = c >> 5, q = c & 31, pr = q & 15;
                xh[2 * (4 * ((pr >> 2) * NC + u) + (pr & 3)) + (q >> 4)] = (uint16_t)(__float_as_uint(v[e]) >> 16);
            }
        });
        const int c0 = K / 32, npad = NC - c0;  // whole padding units (K % 32 == 0), in all four planes
        for (int i = tid; i < 4 * npad; i += kQThreads)
            reinterpret_cast<u32x4*>(xs)[(i / npad) * NC + c0 + i % npad] = u32x4{0u, 0u, 0u, 0u};
    }
    // x staged (and the group counter set); the prefetched weights stay in flight
    if constexpr (kDynItems || !kXPerItem) lds_barrier();
    if constexpr (kDynamic) fetch_group();
    if constexpr (F == F_TERN || F == F_TERN3) {
        sum_xq = 0;
#pragma unroll
        for (int i = 0; i < kQWaves; ++i) sum_xq += redi[i];
    }

    // ternary 2-bit with every item in flight: each row's int32 total is
    // kept (wave-uniform) and the rows of the wave are rescaled and stored
    // together after the last item, one row per lane
    constexpr bool kBatchRows = (NPF > 0 && F == F_TERN);
    int rsum[kBatchRows ? NPF : 1][U];
    float accf[U], accf2[U];
    int acc1[U], acc4[U], acc16[U];
#pragma unroll
    for (int u = 0; u < U; ++u) { accf[u] = 0.f; accf2[u] = 0.f; acc1[u] = 0; acc4[u] = 0; acc16[u] = 0; }

    auto consume = [&](const auto& x, Frag (&fr)[U][JS], const float (&sc)[U][2]) {
        const int g = group_of(x);
        const int seg = seg_of(x);
        if (seg == 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) { accf[u] = 0.f; accf2[u] = 0.f; acc1[u] = 0; acc4[u] = 0; acc16[u] = 0; }
        }
#pragma unroll
        for (int j = 0; j < JS; ++j) {
            const int c = lane + 64 * (seg * JS + j);  // < nseg * JS * 64: inside the padded LDS copy
            if constexpr (F == F_INT8F || F == F_INT8L) {
                float xv[16];
                if constexpr (F == F_INT8L) {
                    const u32x4* xp = reinterpret_cast<const u32x4*>(xs) + c;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const u32x4 t = xp[q * NC];
#pragma unroll
                        for (int e = 0; e < 4; ++e) xv[4 * q + e] = __uint_as_float(t[e]);
                    }
                } else if constexpr (XREG) {
#pragma unroll
                    for (int q = 0; q < 16; ++q) xv[q] = xf[j][q];
                } else if constexpr (XT == 0) {
#pragma unroll
                    for (int q = 0; q < 16; ++q) xv[q] = __uint_as_float(fr[0][j].x[q >> 2][q & 3]);
                } else {
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const uint32_t d = fr[0][j].x[q >> 2][q & 3];
                        xv[2 * q] = bf16_to_f32(d & 0xFFFFu);
                        xv[2 * q + 1] = __uint_as_float(d & 0xFFFF0000u);
                    }
                }
#pragma unroll
                for (int b = 0; b < 16; ++b) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const uint32_t wd = fr[u][j].w[b >> 2];
                        const float wv = (float)(int8_t)(wd >> (8 * (b & 3)));
                        accf[u] = __builtin_fmaf(wv, xv[b], accf[u]);
                    }
                }
            } else if constexpr (F == F_Q4) {
                // x as bf16 pairs (element 2t low, 2t + 1 high) and the group's sum
                uint32_t xp[16];
                float xsum;
                if constexpr (XREG) {
#pragma unroll
                    for (int t = 0; t < 16; ++t) xp[t] = xq4[j][t];
                    xsum = xsq4[j];
                } else {
                    float xs[4] = {0.f, 0.f, 0.f, 0.f};  // sum of the group's x, four chains
#pragma unroll
                    for (int t = 0; t < 16; ++t) {
                        xp[t] = fr[0][j].x[t >> 2][t & 3];
                        xs[(2 * t) & 3] += bf16_to_f32(xp[t] & 0xFFFFu);
                        xs[(2 * t + 1) & 3] += __uint_as_float(xp[t] & 0xFFFF0000u);
                    }
                    xsum = (xs[0] + xs[1]) + (xs[2] + xs[3]);
                }
                const int grp = c & 7;  // group inside its super-block (= lane & 7)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    // S = d * sc and M = dmin * m from the super-block record
                    const u32x4 m = fr[u][j].meta;
                    const uint64_t lo64 = (uint64_t)m[0] | ((uint64_t)m[1] << 32);  // bits 0..63
                    const uint64_t hi64 = (uint64_t)m[1] | ((uint64_t)m[2] << 32);  // bits 32..95
                    const float sc = (float)((uint32_t)(lo64 >> (6 * grp)) & 63u);
                    const float mq = (float)((int)((uint32_t)(hi64 >> (16 + 6 * grp)) & 63u) - 32);
                    const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(m[3] & 0xFFFFu));
                    const float dm = (float)__builtin_bit_cast(_Float16, (uint16_t)(m[3] >> 16));
                    const float S = d * sc, M = dm * mq;
                    // code q as the bf16 value 128 + q (exact): a byte's two codes
                    // become one bf16 pair for v_dot2 against the matching x pair,
                    // and the 128 * sum(x) that this adds is taken off below
                    float a0 = 0.f, a1 = 0.f;  // sum_k (128 + q) x, two chains
#pragma unroll
                    for (int dw = 0; dw < 4; ++dw) {
                        const uint32_t wd = fr[u][j].w[dw];
                        const uint32_t lo = wd & 0x0F0F0F0Fu, hi = (wd >> 4) & 0x0F0F0F0Fu;  // even, odd codes
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            const uint32_t sel = (uint32_t)b | 0x0C00u | ((uint32_t)(4 + b) << 16) | 0x0C000000u;
                            const uint32_t wp = __builtin_amdgcn_perm(hi, lo, sel) | 0x43004300u;
                            if (b & 1) a1 = dot2bf(wp, xp[4 * dw + b], a1);
                            else a0 = dot2bf(wp, xp[4 * dw + b], a0);
                        }
                    }
                    accf[u] += S * (a0 + a1) + (M - 128.0f * S) * xsum;
                }
            } else if constexpr (F == F_INT8I) {
                const u32x4 xq = reinterpret_cast<const u32x4*>(xs)[c];
#pragma unroll
                for (int u = 0; u < U; ++u) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) acc1[u] = sdot4(fr[u][j].w[d], xq[d], acc1[u]);
                }
            } else if constexpr (F == F_TERN3) {
                // x of the chunk: dword 5 d + i holds the activations of digit i
                // of the four bytes of weight dword d
                const u32x4* xp = reinterpret_cast<const u32x4*>(xs) + 5 * c;
                uint32_t xv[20];
#pragma unroll
                for (int q = 0; q < 5; ++q) {
                    const u32x4 t = xp[q];
                    xv[4 * q] = t[0]; xv[4 * q + 1] = t[1]; xv[4 * q + 2] = t[2]; xv[4 * q + 3] = t[3];
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t w = fr[u][j].w[d];
                        // the four bytes in four 16-bit lanes: bytes 0, 2 low, 1, 3 high
                        uint64_t m = (uint64_t)__builtin_amdgcn_perm(0u, w, 0x0C020C00u) |
                                     ((uint64_t)__builtin_amdgcn_perm(0u, w, 0x0C030C01u) << 32);
#pragma unroll
                        for (int i = 0; i < 5; ++i) {
                            // x3 in every lane (< 2^10: no carry between lanes) as one
                            // 64-bit shift-add; the compiler's own form is two 32-bit
                            // multiplies, measured slower on MI355X
                            asm("v_lshl_add_u64 %0, %1, 1, %1" : "=v"(m) : "v"(m));
                            // digit i of each byte is now bits 8-9 of its lane: gather bytes 1 and 3
                            const uint32_t dg = __builtin_amdgcn_perm((uint32_t)(m >> 32), (uint32_t)m, 0x07030501u);
                            acc1[u] = sdot4(dg, xv[5 * d + i], acc1[u]);
                            if (i < 4) m &= 0x00FF00FF00FF00FFull;  // keep the fraction
                        }
                    }
                }
            } else if constexpr (F == F_TERN) {
                const u32x4* xp = reinterpret_cast<const u32x4*>(xs) + c;
                u32x4 xq[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) xq[d] = xp[d * NC];
#pragma unroll
                for (int u = 0; u < U; ++u) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t w = fr[u][j].w[d];
                        acc1[u] = sdot4(w & 0x03030303u, xq[d][0], acc1[u]);
                        acc4[u] = sdot4(w & 0x0C0C0C0Cu, xq[d][1], acc4[u]);
                        acc16[u] = sdot4(w & 0x30303030u, xq[d][2], acc16[u]);
                        acc16[u] = sdot4((w >> 2) & 0x30303030u, xq[d][3], acc16[u]);
                    }
                }
            } else {  // F_SR
                const u32x4* xp = reinterpret_cast<const u32x4*>(xs) + c;
                uint32_t xv[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4 t = xp[q * NC];
                    xv[4 * q] = t[0]; xv[4 * q + 1] = t[1]; xv[4 * q + 2] = t[2]; xv[4 * q + 3] = t[3];
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t ns = ~fr[u][j].s;
                    uint32_t zz = 0;  // bf16 pair (-z, -z): exact, |z| <= 128
                    if constexpr (F == F_SRZ) {
                        const uint32_t h = __float_as_uint(-(float)(int8_t)fr[u][0].z) >> 16;
                        zz = h | (h << 16);
                    }
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        const float lo = (float)(int8_t)(fr[u][j].r0[q >> 2] >> (8 * (q & 3)));
                        const float hi = (float)(int8_t)(fr[u][j].r1[q >> 2] >> (8 * (q & 3)));
                        const uint32_t rp = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
                        accf2[u] = dot2bf(rp, xv[q], accf2[u]);
                        if constexpr (F == F_SRZ) accf2[u] = dot2bf(zz, xv[q], accf2[u]);
                        const uint32_t sp = ((ns << (15 - q)) & 0x80008000u) | 0x3F803F80u;
                        accf[u] = dot2bf(sp, xv[q], accf[u]);
                    }
                }
            }
        }
        if (seg == nseg - 1) {
            // reduce every row of the group at once (independent DPP chains);
            // lane 63 holds the sums and writes the outputs
            if constexpr (F == F_INT8F || F == F_INT8L || kSignRes<F> || F == F_Q4) {
                float v[U], v2[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    v[u] = wave_sum_to_lane63(accf[u]);
                    if constexpr (kSignRes<F>) v2[u] = wave_sum_to_lane63(accf2[u]);
                }
                if (lane == 63) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int r = g * U + u;
                        if (r < rows) {
                            const int row = row0 + r;
                            float o;
                            if constexpr (kSignRes<F>) o = sc[u][0] * v[u] + v2[u] / sc[u][1];
                            else if constexpr (F == F_Q4) o = v[u];  // group scales already applied
                            else if constexpr (kRowScale) o = v[u] / sc[u][0];
                            else o = v[u] / p.scale[row];
                            if constexpr (YT == 0) static_cast<float*>(p.y)[row] = o;
                            else static_cast<uint16_t*>(p.y)[row] = (uint16_t)f32_to_bf16(o);
                        }
                    }
                }
            } else {
                int v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if constexpr (F == F_TERN) v[u] = wave_sum_to_lane63(acc1[u] + (acc4[u] >> 2) + (acc16[u] >> 4));
                    else v[u] = wave_sum_to_lane63(acc1[u]);
                }
                if constexpr (kBatchRows) {
                    static_assert(std::is_integral_v<std::decay_t<decltype(x)>>, "fixed share");
#pragma unroll
                    for (int u = 0; u < U; ++u) rsum[(int)x][u] = __builtin_amdgcn_readlane(v[u], 63);
                } else if (lane == 63) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int r = g * U + u;
                        if (r < rows) {
                            const int row = row0 + r;
                            const int a = (F == F_TERN || F == F_TERN3) ? v[u] - sum_xq : v[u];
                            float o;
                            if constexpr (F == F_TERN || F == F_TERN3) o = (float)a * (p.scale[0] / sx);
                            else o = (float)a / (p.scale[row] * sx);
                            if (p.acc_out) p.acc_out[row] = a;
                            if constexpr (YT == 0) static_cast<float*>(p.y)[row] = o;
                            else static_cast<uint16_t*>(p.y)[row] = (uint16_t)f32_to_bf16(o);
                        }
                    }
                }
            }
        }
    };

    if constexpr (NPF > 0) {
#pragma unroll
        for (int i = 0; i < NPF; ++i)
            if (i < nit) consume(i, fp[i], sp[i]);
        if constexpr (kBatchRows) {
            // lane j = U * (group ordinal) + u takes that row's total
            int a = 0;
#pragma unroll
            for (int i = 0; i < NPF; ++i) {
                if (i < nit && i % nseg == nseg - 1) {
#pragma unroll
                    for (int u = 0; u < U; ++u) a = (lane == U * (i / nseg) + u) ? rsum[i][u] : a;
                }
            }
            const float gs = p.scale[0] / sx;  // gamma / s_x
            const int gi = lane / U, u = lane % U;
            const int r = (wave + kQWaves * gi) * U + u;
            if (gi < my_groups && r < rows) {
                const int t = a - sum_xq;
                const int row = row0 + r;
                if (p.acc_out) p.acc_out[row] = t;
                const float o = (float)t * gs;
                if constexpr (YT == 0) static_cast<float*>(p.y)[row] = o;
                else static_cast<uint16_t*>(p.y)[row] = (uint16_t)f32_to_bf16(o);
            }
        }
    } else if constexpr (kDynItems) {
        // The loop ends after the first item past the wave's last group
        // (the LDS counter's groups increase; a pair's ends stop once they
        // meet).  Every issued item is consumed on every
        // path (such an item reads zeros and stores nothing): a load left
        // unused on the exit path would be sunk below the exit test by the
        // compiler, past the consumption of the item before it, which would
        // then wait for both.  Item ia is in flight in fa at the top of
        // every trip.
        while (true) {
            ib = next_item(ia);
            issue(ib, fb, sb);
            consume(ia, fa, sa);
            if (ib.g >= ngroups) {
                consume(ib, fb, sb);
                break;
            }
            ia = next_item(ib);
            issue(ia, fa, sa);
            consume(ib, fb, sb);
            if (ia.g >= ngroups) {
                consume(ia, fa, sa);
                break;
            }
        }
    } else if constexpr (kTwoAhead) {
        // fixed share, peeled so that no load is conditional behind a load
        // that is waited on.  Items it (fa) and it + 1 (fb) are in flight at
        // the top of every trip; issues past nit read zeros and are never
        // consumed
        int it = 0;
        for (; it + 2 < nit; it += 2) {
            consume(it, fa, sa);
            issue(it + 2, fa, sa);
            consume(it + 1, fb, sb);
            issue(it + 3, fb, sb);
        }
        if (it + 2 == nit) {  // two items left
            consume(it, fa, sa);
            consume(it + 1, fb, sb);
        } else if (it + 1 == nit) {  // one item left
            consume(it, fa, sa);
        }
    } else {
        // fixed share: item it is in flight in fa at the top of every trip
        int it = 0;
        for (; it + 2 < nit; it += 2) {
            issue(it + 1, fb, sb);
            consume(it, fa, sa);
            issue(it + 2, fa, sa);
            consume(it + 1, fb, sb);
        }
        if (it + 2 == nit) {  // two items left
            issue(it + 1, fb, sb);
            consume(it, fa, sa);
            consume(it + 1, fb, sb);
        } else if (it + 1 == nit) {  // one item left
            consume(it, fa, sa);
        }
    }
}

// ------------------------------------------------------------------ host side
int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) cu = 256;
        cached[dev] = cu;
    }
    return cached[dev];
}

// Rows per workgroup of matrix m of a launch: workgroups are handed out per
// matrix in proportion to its rows (about one per CU in all), each owning a
// contiguous block of rows; `cap` keeps buffer ranges below 2 GiB.
static int64_t rows_per_wg(const QgemvArgs* a, int count, int m, int64_t cap) {
    const int cus = device_cu_count();
    int64_t total_rows = 0;
    for (int i = 0; i < count; ++i) total_rows += a[i].n;
    const int64_t N = a[m].n;
    int64_t share = (cus * N + total_rows / 2) / total_rows;  // workgroups for this matrix
    if (share < 1) share = 1;
    int64_t rpw = (N + share - 1) / share;
    if (rpw > cap) rpw = cap;
    if (rpw < 1) rpw = 1;
    return rpw;
}

template <int F, int XT, int YT, int U, int JS, bool XREG = false, int NPF = 0>
static hipError_t run(const QgemvArgs* a, int count, hipStream_t st) {
    constexpr int kCols = Fmt<F>::kColsPerChunk;
    const int K = (int)a[0].k;
    const int C = (K + kCols - 1) / kCols;
    const int J = (C + 63) / 64;
    const int nseg = (J + JS - 1) / JS;
    if (XREG && nseg != 1) return hipErrorInvalidValue;  // register-resident x needs items spanning the row
    const size_t lds = (size_t)nseg * JS * 64 * kCols * Fmt<F>::kLdsBytesPerCol;
    const int64_t rowB = (F == F_TERN) ? K / 4 : kSignRes<F> ? K / 8 : (F == F_Q4) ? K / 2 : (F == F_TERN3) ? 16 * C : K;
    const int64_t resB = kSignRes<F> ? K : (F == F_Q4) ? K / 16 : 0;
    const int64_t cap = ((int64_t)1 << 31) / (rowB > resB ? rowB : resB);  // buffer ranges stay below 2 GiB
    auto launch = [&](auto slots) -> hipError_t {
        constexpr int MG = decltype(slots)::value;
        KGroup<MG> g;
        int wgx = 1;  // grid: (workgroups of the largest matrix) x (matrices)
        for (int m = 0; m < count; ++m) {
            const int64_t N = a[m].n;
            const int64_t rpw = rows_per_wg(a, count, m, cap);
            if (NPF > 0) {  // every item of every wave must fit the prefetch
                const int64_t groups = (rpw + U - 1) / U;
                if (((groups + kQWaves - 1) / kQWaves) * nseg > NPF) return hipErrorInvalidValue;
            }
            KParams& p = g.mats[m];
            p.codes = static_cast<const uint8_t*>(a[m].codes);
            p.resid = a[m].resid;
            p.scale = a[m].scale;
            p.scale2 = a[m].scale2;
            p.zero = a[m].zero;
            p.x = a[m].x;
            p.y = a[m].y;
            p.acc_out = a[m].acc_out;
            p.n = (int32_t)N;
            p.k = K;
            p.rows_per_wg = (int32_t)rpw;
            const int nwg = (int)((N + rpw - 1) / rpw);
            if (nwg > wgx) wgx = nwg;
        }
        auto kern = qgemv_kernel<F, XT, YT, U, JS, XREG, NPF, MG>;
        if (lds > 64 * 1024) {
            static bool attr_set = false;  // per instantiation
            if (!attr_set) {
                hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                if (e != hipSuccess) return e;
                attr_set = true;
            }
        }
        kern<<<dim3(wgx, count), kQThreads, lds, st>>>(g);
        return hipGetLastError();
    };
    if (count == 1) return launch(std::integral_constant<int, 1>{});
    if (count <= 3) return launch(std::integral_constant<int, 3>{});
    return launch(std::integral_constant<int, kMaxGroup>{});
}

template <int F, int U, int JS, bool XREG = false, int NPF = 0>
static hipError_t run_xy(const QgemvArgs* a, int count, hipStream_t st) {
    if (a[0].xt == 0 && a[0].yt == 0) return run<F, 0, 0, U, JS, XREG, NPF>(a, count, st);
    if (a[0].xt == 0 && a[0].yt == 1) return run<F, 0, 1, U, JS, XREG, NPF>(a, count, st);
    if (a[0].xt == 1 && a[0].yt == 0) return run<F, 1, 0, U, JS, XREG, NPF>(a, count, st);
    return run<F, 1, 1, U, JS, XREG, NPF>(a, count, st);
}

// int8 weights with float x.  The per-weight work is one conversion and one
// FMA; x is converted once per launch, not per row:
//   * rows of up to 4 chunk iterations (K <= 4096): one item spans the row,
//     and each lane keeps the 16 fp32 activations of each of its chunks in
//     registers (XREG), loaded before the first item;
//   * rows of up to 12 chunk iterations (K <= 12288): x staged once per
//     workgroup in LDS as fp32, items of 4 chunk iterations (measured on
//     MI355X at 4096 x 11008: 10.6 us, against 11.3 us with x carried by
//     each item and 12.2 us with one item per row), the first two out
//     before the staging;
//   * longer rows: each item carries its activations (bf16 or fp32) with it.
// One row per item at the decode shapes (16-86 rows per workgroup); two rows
// per item once a workgroup owns hundreds of rows, where the longer items
// stream faster (measured on MI355X).
static hipError_t run_int8_float_x(const QgemvArgs* a, int count, hipStream_t st) {
    const int J = (int)((a[0].k / 16 + 63) / 64);  // chunk iterations per row
    int64_t total_rows = 0;
    for (int m = 0; m < count; ++m) total_rows += a[m].n;
    const bool tall = total_rows >= (int64_t)256 * device_cu_count();
    if (J <= 1) return run_xy<F_INT8F, 1, 1, true>(a, count, st);
    if (J <= 2) return run_xy<F_INT8F, 1, 2, true>(a, count, st);
    if (J <= 4) return tall ? run_xy<F_INT8F, 2, 4, true>(a, count, st) : run_xy<F_INT8F, 1, 4, true>(a, count, st);
    if (J <= 12) return run_xy<F_INT8L, 1, 4>(a, count, st);
    return tall ? run_xy<F_INT8F, 2, 4>(a, count, st) : run_xy<F_INT8F, 1, 4>(a, count, st);
}

// All entries share fmt, amode, xt, yt and k (validated by the caller).
hipError_t launch_qgemv_group(const QgemvArgs* a, int count, hipStream_t st) {
    // Rows per item U and chunk iterations per item JS, per format, are the
    // fastest measured on MI355X at the decode shapes (16-112 rows per
    // workgroup; two items in flight per wave).
    const QgemvArgs& h = a[0];
    if (h.fmt == 0 && h.amode == 1) return run_int8_float_x(a, count, st);
    if (h.fmt == 0 && h.amode == 0) return run_xy<F_INT8I, 2, 4>(a, count, st);
    if (h.fmt == 1) {
        // short packed rows (K / 4 bytes): one or two rows per item, every item
        // of a wave out in the prologue when each wave has at most 8; else
        // four-row items, two in flight
        const int64_t J = (h.k / 64 + 63) / 64;  // chunk iterations per row
        int64_t rpw = 1;
        for (int m = 0; m < count; ++m) {
            const int64_t r = rows_per_wg(a, count, m, (int64_t)1 << 40);
            if (r > rpw) rpw = r;
        }
        auto per_wave = [&](int64_t u) { return ((rpw + u - 1) / u + kQWaves - 1) / kQWaves * J; };
        if (per_wave(1) <= 8) return run_xy<F_TERN, 1, 1, false, 8>(a, count, st);
        if (per_wave(2) <= 8) return run_xy<F_TERN, 2, 1, false, 8>(a, count, st);
        return run_xy<F_TERN, 4, 1>(a, count, st);
    }
    if (h.fmt == 5) return run_xy<F_TERN3, 4, 1>(a, count, st);
    if (h.fmt == 3) {  // bf16 activations only
        // rows of at most 2 chunk iterations: items of two rows (a row is only
        // 2 KB of codes; with one-row items too few bytes were in flight:
        // 11008 x 4096 measured 8.53 us with one row, 7.8 us with two, 8.9 us
        // with four on MI355X)
        const bool spans = (h.k / 32 + 63) / 64 <= 2;  // one item of 2 chunk iterations covers the row
        if (h.yt == 0) return spans ? run<F_Q4, 1, 0, 2, 2, true>(a, count, st) : run<F_Q4, 1, 0, 4, 1>(a, count, st);
        return spans ? run<F_Q4, 1, 1, 2, 2, true>(a, count, st) : run<F_Q4, 1, 1, 4, 1>(a, count, st);
    }
    if (h.fmt == 4) {  // sign + zero-point residual
        if (h.yt == 0) return run<F_SRZ, 1, 0, 1, 2>(a, count, st);
        return run<F_SRZ, 1, 1, 1, 2>(a, count, st);
    }
    if (h.yt == 0) return run<F_SR, 1, 0, 1, 2>(a, count, st);
    return run<F_SR, 1, 1, 1, 2>(a, count, st);
}

hipError_t launch_qgemv(const QgemvArgs& a, hipStream_t st) { return launch_qgemv_group(&a, 1, st); }

}  // namespace qg
