// chain.hip -- the weight-only int8 products (W8A16) of a batch-1 decode
// step, with the data dependencies between them, as ONE persistent launch.
//
// A decode step is a sequence of stages; a stage is one to eight products
// y_m = W_m x that read the same activation vector (q, k and v; gate and
// up), and its x is the output of an earlier stage.  Launched one stage at a
// time, each launch pays its start-up and drain (dispatch, first-load
// latency, the last rows' tail): on MI355X about 2.6 us per launch, a fifth of
// the whole step at the 7B shapes.  Here one launch runs every stage, and the
// weights of a stage stream in while the stage before it is still finishing;
// only x waits for its producer.
//
// Work: every stage is cut into slots of up to 128 consecutive rows of one
// matrix, about one slot per workgroup (a table of slot records in the
// plan).  Workgroups (one per CU)
// take slots in a single global order from a ticket counter, so a slot is
// only ever taken after every slot of every earlier stage has been taken by
// a running workgroup.  Each workgroup is
//   * 8 worker waves: each takes the rows w, w + 8, ... of the workgroup's
//     slots, in order, as items of one row x 4096 columns (64 lanes x 4 x
//     16 B), 6 items in flight in registers.  Their loads are issued as soon
//     as the slot is known, whatever its stage; a worker waits only before
//     it multiplies an item, for the slot's x in LDS.  Workers touch global
//     memory only through those weight loads: x comes from LDS and row sums
//     go to LDS, so no wait of theirs ever covers the weights in flight.
//   * a claim/release wave: takes slots (one ticket per atomic while it
//     holds fewer than 3, then one load of the slot's record) and posts them
//     to the workers; when all 8 workers are done with a slot, writes its bf16
//     outputs and then increments the stage's completion counter.
//   * a staging wave: once the stage a slot depends on is complete, copies
//     the slot's x into LDS (fp32, four planes, two stage buffers) and flags
//     it ready.  The two roles are separate waves so that a dependency seen
//     complete is staged at once, never behind a release or a claim.
// Visibility across XCDs: outputs are written with agent-coherent stores
// (sc1, written through to the memory side), their completion is waited for
// (vmcnt) before the counter increment (an atomic add); the counter is read
// with an atomic add of 0 (atomics are coherent with one another across
// XCDs), and x with agent-coherent loads once the counter shows the
// producing stage complete.  No L2 writeback or invalidate of the whole
// cache is needed on either side.
// Completion counters exist in 8 copies (each workgroup polls the one of its
// XCD, blockIdx % 8), so that 256 pollers do not all read one address.
//
// Every wait is bounded by a deadline (s_memrealtime): a wait that passes it
// sets the plan's error word, tells every wave of the workgroup to stop, and
// the launch ends normally (its outputs are then unspecified and the plan's
// control words must be restored from the host image before the next call).
// On success, the last workgroup to finish resets the ticket, the exit count
// and the completion counters, so consecutive launches (and graph replays)
// need no reset of their own.
//
// Deadlock freedom: a workgroup processes its slots in ticket order, and a
// slot's stage depends only on earlier stages.  The lowest unfinished slot
// belongs to a running workgroup (tickets are handed out only to running
// workgroups) whose earlier slots are finished, and whose dependency is a
// stage all of whose slots have lower tickets, hence finished: it makes
// progress.  Inside a workgroup, workers never block on a slot's descriptor
// (an unknown slot leaves a hole in the ring), only on x of their oldest
// item; the sync waves never block at all.  No co-residency of the grid is
// assumed.
#include <climits>

#include "qg_chain.h"
#include "qg_device.h"
#include "qg_launch.h"

namespace qg {
namespace chain {

constexpr int kThreadsC = (kWorkers + 2) * kWave;  // + the claim/release and staging waves
constexpr int kWaveRel = kWorkers;      // claim/release wave
constexpr int kWaveStage = kWorkers + 1;  // staging wave
constexpr int kCPolSC1 = 16;            // cache policy: agent-scope coherent (sc1)
constexpr int kJS = kItemChunks / kWave;  // chunk iterations per item
constexpr int kNB = 6;                     // items in flight per worker
constexpr int kRing = 8;                   // slots a workgroup holds at once

typedef uint32_t g_u32;  // global (the kernel argument it derives from is global)

struct SlotL {  // a claimed slot, as the sync wave posts it
    uint64_t codes, scale, y;  // the slot's first row
    int32_t rows, k, nseg, stage, end, pad;
};

struct Lds {
    SlotL desc[kRing];
    int32_t seq[kRing];     // local slot index posted in desc[e]
    int32_t xready[kRing];  // 2 * (local slot) + x buffer, once the slot's x is staged
    int32_t fin[kRing];     // workers done with the slot in entry e
    int32_t abort_flag;
    int32_t claimed;   // local slots posted (the END slot included)
    int32_t released;  // local slots released
    int32_t q_end;     // local index of the END slot (INT_MAX until claimed)
    int32_t zero;      // always 0: an operand the compiler cannot see through
    float y[kRing][kMaxRows];  // row sums (fp32) of the slot in entry e
    float sc[kRing][kMaxRows];  // row scales s_w of the slot in entry e
};

struct Args {
    uint8_t* plan;
    uint64_t stages_off, slots_off;
    uint64_t timeout;
    int32_t nstages, total_slots, stride, nc;
};

__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t rfl64(uint64_t v) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
__device__ __forceinline__ int lds_ld(int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(int32_t* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// completes this wave's LDS operations and keeps the compiler from moving
// memory accesses across (no wait on vector memory: the weights in flight)
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ uint64_t now() { return __builtin_amdgcn_s_memrealtime(); }

__global__ __launch_bounds__(kThreadsC) void chain_kernel(Args a) {
    __shared__ Lds L;
    extern __shared__ __attribute__((aligned(16))) float4 xsm[];  // [2 buffers][4 planes][nc chunks]

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = rfl(tid >> 6);
    const uint64_t deadline = now() + a.timeout;
    const int nc = a.nc;
    g_u32* const err = reinterpret_cast<g_u32*>(a.plan + kOffError);

    if (wave == kWaveRel) {
        if (lane < kRing) {
            L.seq[lane] = -1;
            L.xready[lane] = -1;
            L.fin[lane] = 0;
        }
        if (lane == 0) {
            L.abort_flag = 0;
            L.claimed = 0;
            L.released = 0;
            L.q_end = INT_MAX;
            L.zero = 0;
        }
    }
    lds_barrier();

    // a wait ran past the deadline: flag the plan and stop the workgroup
    auto give_up = [&]() {
        if (lane == 0) {
            __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            lds_st(&L.abort_flag, 1);
        }
    };

    if (wave < kWorkers) {
        // ============================================================ worker
        u32x4 wr[kNB][kJS];  // the items' weights (16 B per lane per chunk iteration)
        int iq[kNB], ir[kNB], isg[kNB];  // local slot (-1: no item), row in the slot, segment
        int nq = 0, nr = wave, ns = 0;   // the next item to issue
        bool ended = false, stop = false;
        float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
        int xq = -1, xoff = 0;  // slot whose x is current, its buffer (float4 index)

        auto ack = [&](int e) {  // this worker is done with the slot in entry e
            lds_fence();          // its row results are in LDS first
            if (lane == 63) __hip_atomic_fetch_add(&L.fin[e], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        };
        // Next item into ring entry b: the weights only (the row scales come
        // through LDS).  The number of loads is the same on every path (no item: empty buffer resources, which read zeros), so
        // the compiler's waits stay in issue order.
        auto issue = [&](int b) {
            iq[b] = -1;
            uint64_t base = 0;
            uint32_t bytes = 0;
            int seg = 0;
            for (int guard = 0; guard <= kRing && !ended && !stop; ++guard) {
                const int e = nq & (kRing - 1);
                if (rfl(lds_ld(&L.seq[e])) != nq) break;  // not posted yet: try again later
                asm volatile("" ::: "memory");
                if (rfl(L.desc[e].end)) {
                    ended = true;
                    break;
                }
                const int rows = rfl(L.desc[e].rows);
                if (nr < rows) {
                    const int k = rfl(L.desc[e].k);
                    base = rfl64(L.desc[e].codes) + (uint64_t)nr * (uint64_t)k;
                    bytes = (uint32_t)k;
                    iq[b] = nq;
                    ir[b] = nr;
                    isg[b] = ns;
                    seg = ns;
                    if (++ns == rfl(L.desc[e].nseg)) {
                        ns = 0;
                        nr += kWorkers;
                    }
                    break;
                }
                if (wave >= rows) ack(e);  // no row of this slot is ours
                ++nq;
                nr = wave;
                ns = 0;
            }
            const __amdgpu_buffer_rsrc_t rw = make_rsrc(reinterpret_cast<const void*>(base), bytes);
#pragma unroll
            for (int j = 0; j < kJS; ++j) wr[b][j] = load16_nt(rw, 16u * (uint32_t)(lane + kWave * (seg * kJS + j)));
        };
        auto consume = [&](int b) {
            const int q = stop ? -1 : iq[b];
            if (q < 0) {
                // an empty entry still waits for its (zero) loads, in issue
                // order: otherwise its registers stay pending on this path and
                // their next writer would have to wait for every later load
#pragma unroll
                for (int j = 0; j < kJS; ++j) asm volatile("" ::"v"(wr[b][j]));
                return;
            }
            const int e = q & (kRing - 1);
            if (q != xq) {  // first item of a slot: wait until its x is staged
                int v;
                while (true) {
                    v = rfl(lds_ld(&L.xready[e]));
                    if ((v >> 1) == q) break;
                    if (rfl(lds_ld(&L.abort_flag))) {
                        stop = true;
                        return;
                    }
                    if (now() > deadline) {
                        give_up();
                        stop = true;
                        return;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                asm volatile("" ::: "memory");
                xq = q;
                xoff = (v & 1) * 4 * nc;
            }
            const int seg = isg[b], r = ir[b];
            if (seg == 0) {
                acc0 = 0.f;
                acc1 = 0.f;
                acc2 = 0.f;
                acc3 = 0.f;
            }
#pragma unroll
            for (int j = 0; j < kJS; ++j) {
                const int c = lane + kWave * (seg * kJS + j);
                // plane d holds columns 4d..4d+3 of the chunk: the bytes of weight dword d
                const float4 x0 = xsm[xoff + c];
                const float4 x1 = xsm[xoff + nc + c];
                const float4 x2 = xsm[xoff + 2 * nc + c];
                const float4 x3 = xsm[xoff + 3 * nc + c];
                const u32x4 w = wr[b][j];
                acc0 = __builtin_fmaf((float)(int8_t)(w[0]), x0.x, acc0);
                acc0 = __builtin_fmaf((float)(int8_t)(w[0] >> 8), x0.y, acc0);
                acc0 = __builtin_fmaf((float)(int8_t)(w[0] >> 16), x0.z, acc0);
                acc0 = __builtin_fmaf((float)(int8_t)(w[0] >> 24), x0.w, acc0);
                acc1 = __builtin_fmaf((float)(int8_t)(w[1]), x1.x, acc1);
                acc1 = __builtin_fmaf((float)(int8_t)(w[1] >> 8), x1.y, acc1);
                acc1 = __builtin_fmaf((float)(int8_t)(w[1] >> 16), x1.z, acc1);
                acc1 = __builtin_fmaf((float)(int8_t)(w[1] >> 24), x1.w, acc1);
                acc2 = __builtin_fmaf((float)(int8_t)(w[2]), x2.x, acc2);
                acc2 = __builtin_fmaf((float)(int8_t)(w[2] >> 8), x2.y, acc2);
                acc2 = __builtin_fmaf((float)(int8_t)(w[2] >> 16), x2.z, acc2);
                acc2 = __builtin_fmaf((float)(int8_t)(w[2] >> 24), x2.w, acc2);
                acc3 = __builtin_fmaf((float)(int8_t)(w[3]), x3.x, acc3);
                acc3 = __builtin_fmaf((float)(int8_t)(w[3] >> 8), x3.y, acc3);
                acc3 = __builtin_fmaf((float)(int8_t)(w[3] >> 16), x3.z, acc3);
                acc3 = __builtin_fmaf((float)(int8_t)(w[3] >> 24), x3.w, acc3);
            }
            if (seg == rfl(L.desc[e].nseg) - 1) {
                const float v = wave_sum_to_lane63((acc0 + acc1) + (acc2 + acc3));
                if (lane == 63) L.y[e][r] = v;
                if (r + kWorkers >= rfl(L.desc[e].rows)) ack(e);  // this worker's last row of the slot
            }
        };

#pragma unroll
        for (int b = 0; b < kNB; ++b) issue(b);
        // One exit, at the end of the unrolled body: a path that left the body
        // in the middle would reach the loop head with another count of loads
        // in flight, and the compiler's waits would then have to assume it.
        while (true) {
#pragma unroll
            for (int b = 0; b < kNB; ++b) {
                consume(b);  // once stopped: a no-op
                issue(b);    // once stopped or ended: empty loads
            }
            if (stop) break;
            bool any = false;
#pragma unroll
            for (int b = 0; b < kNB; ++b) any = any || iq[b] >= 0;
            if (!any) {
                if (ended) break;
                if (rfl(lds_ld(&L.abort_flag))) break;
                if (now() > deadline) {
                    give_up();
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        return;
    }

    g_u32* const ticket = reinterpret_cast<g_u32*>(a.plan + kOffTicket);
    g_u32* const exited = reinterpret_cast<g_u32*>(a.plan + kOffExited);
    g_u32* const done = reinterpret_cast<g_u32*>(a.plan + kOffDone);
    const StageD* const stages = reinterpret_cast<const StageD*>(a.plan + a.stages_off);

    if (wave == kWaveStage) {
        // ============================================================ staging wave
        const int rep = (int)(blockIdx.x % kRep);
        int q_stage = 0;
        int xb_stage0 = -1, xb_stage1 = -1;  // stage whose x each buffer holds
        int xb_last0 = -1, xb_last1 = -1;    // last local slot that reads each buffer
        // x of stage s into buffer b: fp32, chunk c's 16 columns as four
        // planes of 4, zero-padded to whole item segments; agent-coherent
        // loads (x was written by other workgroups during this launch)
        auto stage_x = [&](int s, int b) {
            const int K = stages[s].k;
            const int pieces = K / 8;  // 16 B = 8 bf16 each
            const __amdgpu_buffer_rsrc_t rx = make_rsrc(reinterpret_cast<const void*>(stages[s].x), (uint32_t)(2 * K));
            constexpr int kPL = 16;  // pieces per lane per round (K <= 8192 in one round)
            float4* const xb = xsm + b * 4 * nc;
            for (int p0 = 0; p0 < pieces; p0 += kPL * kWave) {
                u32x4 v[kPL];
#pragma unroll
                for (int i = 0; i < kPL; ++i) {
                    const int pi = p0 + lane + kWave * i;
                    v[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, pi < pieces ? 16u * (uint32_t)pi : (uint32_t)(2 * K),
                                                                 0, kCPolSC1);
                }
#pragma unroll
                for (int i = 0; i < kPL; ++i) {
                    const int pi = p0 + lane + kWave * i;
                    if (pi < pieces) {
                        const int c = pi >> 1, h = pi & 1;
                        const u32x4 t = v[i];
                        xb[(2 * h) * nc + c] = make_float4(bf16_to_f32(t[0] & 0xFFFFu), __uint_as_float(t[0] & 0xFFFF0000u),
                                                           bf16_to_f32(t[1] & 0xFFFFu), __uint_as_float(t[1] & 0xFFFF0000u));
                        xb[(2 * h + 1) * nc + c] = make_float4(bf16_to_f32(t[2] & 0xFFFFu), __uint_as_float(t[2] & 0xFFFF0000u),
                                                               bf16_to_f32(t[3] & 0xFFFFu), __uint_as_float(t[3] & 0xFFFF0000u));
                    }
                }
            }
            const int cend = stages[s].nseg * kItemChunks;
            for (int c = K / 16 + lane; c < cend; c += kWave) {
#pragma unroll
                for (int p = 0; p < 4; ++p) xb[p * nc + c] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        };
        while (true) {
            if (rfl(lds_ld(&L.abort_flag))) break;
            if (q_stage == rfl(lds_ld(&L.q_end))) break;  // every real slot staged
            bool progress = false;
            if (q_stage < rfl(lds_ld(&L.claimed))) {
                asm volatile("" ::: "memory");
                const int e = q_stage & (kRing - 1);
                // the END entry is posted like a slot (its other fields are
                // stale): q_end may have been read before it was set
                if (rfl(L.desc[e].end)) break;
                const int s = rfl(L.desc[e].stage);
                if (s < 0 || s >= a.nstages) {  // a descriptor the plan cannot have written
                    give_up();
                    break;
                }
                int b = (xb_stage0 == s) ? 0 : (xb_stage1 == s) ? 1 : -1;
                if (b < 0) {
                    // a buffer that no unreleased slot reads
                    const int q_rel = rfl(lds_ld(&L.released));
                    const int fb = (xb_last0 < q_rel) ? 0 : (xb_last1 < q_rel) ? 1 : -1;
                    if (fb >= 0) {
                        const int dep = stages[s].dep;
                        bool ready = true;
                        if (dep >= 0) {
                            // read the count with a read-modify-write (adding 0):
                            // agent-scope atomics are coherent with one another
                            // across XCDs, while the value they leave in the
                            // issuing XCD's L2 would reach a plain load only
                            // after an L2 writeback.  The 0 comes from LDS so
                            // that the compiler keeps the atomic.
                            const uint32_t z = (uint32_t)rfl(lds_ld(&L.zero));
                            uint32_t v = 0;
                            if (lane == 0)
                                v = __hip_atomic_fetch_add(done + rep * a.stride + dep, z, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                            ready = (uint32_t)rfl((int)v) >= (uint32_t)stages[dep].nslots;
                        }
                        asm volatile("" ::: "memory");
                        if (ready) {
                            stage_x(s, fb);
                            if (fb == 0) xb_stage0 = s;
                            else xb_stage1 = s;
                            b = fb;
                        }
                    }
                }
                if (b >= 0) {
                    if (b == 0) xb_last0 = q_stage;
                    else xb_last1 = q_stage;
                    lds_fence();  // x before the flag
                    if (lane == 0) lds_st(&L.xready[e], 2 * q_stage + b);
                    ++q_stage;
                    progress = true;
                }
            }
            if (!progress) {
                if (now() > deadline) {
                    give_up();
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        return;
    }

    // ================================================================ claim/release wave
    const int total = a.total_slots;
    const __amdgpu_buffer_rsrc_t rslots = make_rsrc(a.plan + a.slots_off, (uint32_t)((uint64_t)total * sizeof(SlotD)));
    // One ticket per claim, while the workgroup holds fewer than kHold
    // slots: the tickets of a stage then spread over all workgroups (claiming
    // several consecutive tickets at once gave a few workgroups most of a
    // stage, whose completion every later stage waits for).
    constexpr int kHold = 3;
    int q_claim = 0, q_rel = 0, q_end = INT_MAX;
    bool aborted = false;
    while (true) {
        bool progress = false;
        if (rfl(lds_ld(&L.abort_flag))) {
            aborted = true;
            break;
        }
        // ---- release the slots every worker is done with, in order
        while (q_rel < q_claim && q_rel != q_end) {
            const int e = q_rel & (kRing - 1);
            if (rfl(lds_ld(&L.fin[e])) < kWorkers) break;
            asm volatile("" ::: "memory");
            const int rows = rfl(L.desc[e].rows);
            const int s = rfl(L.desc[e].stage);
            const __amdgpu_buffer_rsrc_t ry = make_rsrc(reinterpret_cast<const void*>(rfl64(L.desc[e].y)), (uint32_t)(2 * rows));
#pragma unroll
            for (int h = 0; h < kMaxRows / kWave; ++h) {
                const int r = lane + kWave * h;
                if (r < rows) {
                    const uint32_t o = f32_to_bf16(L.y[e][r] / L.sc[e][r]);
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)o, ry, 2u * (uint32_t)r, 0, kCPolSC1);
                }
            }
            if (lane == 0) lds_st(&L.fin[e], 0);
            // the outputs are at the coherence point before the count says so
            __builtin_amdgcn_s_waitcnt(0);
            asm volatile("" ::: "memory");
            if (lane < kRep) __hip_atomic_fetch_add(done + lane * a.stride + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ++q_rel;
            lds_fence();
            if (lane == 0) lds_st(&L.released, q_rel);
            progress = true;
        }
        if (q_rel == q_end) break;
        // ---- claim the free entries with one atomic (consecutive tickets)
        const int nfree = (q_claim - q_rel < kHold) ? 1 : 0;
        if (q_end == INT_MAX && nfree > 0) {
            uint32_t t0 = 0;
            if (lane == 0) t0 = __hip_atomic_fetch_add(ticket, (uint32_t)nfree, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            t0 = (uint32_t)rfl((int)t0);
            // lane i < nfree: the record of ticket t0 + i (past the last slot: zeros)
            const int64_t t = (int64_t)t0 + lane;
            const uint32_t ro = (lane < nfree && t < total) ? (uint32_t)(t * (int64_t)sizeof(SlotD)) : 0xFFFFFF00u;
            const u32x4 r0 = load16(rslots, ro);
            const u32x4 r1 = load16(rslots, ro + 16u);
            const u32x4 r2 = load16(rslots, ro + 32u);
            const uint64_t rc = (uint64_t)r0[0] | ((uint64_t)r0[1] << 32);
            const uint64_t rsc = (uint64_t)r0[2] | ((uint64_t)r0[3] << 32);
            const uint64_t ryy = (uint64_t)r1[0] | ((uint64_t)r1[1] << 32);
            const int rrows = (int)r1[2], rk = (int)r1[3], rnseg = (int)r2[0], rstage = (int)r2[1];
            const int nreal = (int)min((int64_t)nfree, max((int64_t)0, (int64_t)total - (int64_t)t0));
            if (lane < nfree) {
                const int e = (q_claim + lane) & (kRing - 1);
                if (lane < nreal) {
                    L.desc[e].codes = rc;
                    L.desc[e].scale = rsc;
                    L.desc[e].y = ryy;
                    L.desc[e].rows = rrows;
                    L.desc[e].k = rk;
                    L.desc[e].nseg = rnseg;
                    L.desc[e].stage = rstage;
                    L.desc[e].end = 0;
                } else if (lane == nreal) {
                    L.desc[e].end = 1;
                }
            }
            // the new slots' row scales (for the release), one load per lane each
            for (int i = 0; i < nreal; ++i) {
                const int e = (q_claim + i) & (kRing - 1);
                const int rows_i = __builtin_amdgcn_readlane(rrows, i);
                const uint64_t sc_i = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(rsc >> 32), i) << 32) |
                                      (uint32_t)__builtin_amdgcn_readlane((int)rsc, i);
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<const void*>(sc_i), (uint32_t)(4 * rows_i));
#pragma unroll
                for (int h = 0; h < kMaxRows / kWave; ++h)  // rows past the slot read 0
                    L.sc[e][lane + kWave * h] = __uint_as_float(load4(rs, 4u * (uint32_t)(lane + kWave * h)));
            }
            const int nposted = (nreal < nfree) ? nreal + 1 : nfree;  // with the END slot, if reached
            lds_fence();  // descriptors before their sequence numbers
            if (lane < nposted) lds_st(&L.seq[(q_claim + lane) & (kRing - 1)], q_claim + lane);
            if (nreal < nfree) q_end = q_claim + nreal;
            q_claim += nposted;
            lds_fence();
            if (lane == 0) {
                if (q_end != INT_MAX) lds_st(&L.q_end, q_end);
                lds_st(&L.claimed, q_claim);
            }
            progress = true;
        }
        if (!progress) {
            if (now() > deadline) {
                give_up();
                aborted = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    if (!aborted) {
        // every count this workgroup added is performed before it checks out
        __builtin_amdgcn_s_waitcnt(0);
        asm volatile("" ::: "memory");
        uint32_t old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(exited, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = (uint32_t)rfl((int)old);
        if (old == gridDim.x - 1) {
            // the last workgroup out: every other one has released all its
            // slots; reset the control words for the next launch, with
            // atomics like every other access to them
            for (int i = lane; i < kRep * a.stride; i += kWave)
                __hip_atomic_exchange(done + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (lane == 0) {
                __hip_atomic_exchange(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_exchange(exited, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

}  // namespace chain

// ------------------------------------------------------------------ host side
hipError_t launch_chain(const void* image, void* plan, hipStream_t st) {
    using namespace chain;
    const Header& h = *static_cast<const Header*>(image);
    Args a;
    a.plan = static_cast<uint8_t*>(plan);
    a.stages_off = h.stages_off;
    a.slots_off = h.slots_off;
    a.timeout = h.timeout_ticks;
    a.nstages = h.nstages;
    a.total_slots = h.total_slots;
    a.stride = h.stride;
    a.nc = h.nc;
    const size_t lds = (size_t)2 * 4 * (size_t)h.nc * 16;
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(chain_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)(2 * 4 * ((kMaxK / 16 + kItemChunks - 1) / kItemChunks * kItemChunks) * 16));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    chain_kernel<<<dim3(h.grid), dim3(kThreadsC), lds, st>>>(a);
    return hipGetLastError();
}

}  // namespace qg
