// qg_chain.h -- the plan of a chained decode step (chain.hip): the byte image
// that the host builds once (qg_chain_plan) and the kernel reads from device
// memory, with the control words the launch updates and leaves reset.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {
namespace chain {

constexpr uint32_t kMagic = 0x48434751u;  // "QGCH"
constexpr uint32_t kVersion = 1;
constexpr int kMaxStages = 4096;
constexpr int kMaxMatsPerStage = 8;
constexpr int kMinK = 128;
constexpr int kMaxK = 16384;   // two staged copies of x (fp32) fit the LDS with room to spare
constexpr int kRep = 8;        // copies of each stage's completion counter (one per XCD)
constexpr int kWorkers = 8;    // worker waves per workgroup (plus one sync wave)
constexpr int kMaxRows = 128;  // rows of one slot
constexpr int kItemChunks = 256;  // 16-column chunks of one item segment (64 lanes x 4)

// byte offsets in the image
constexpr int kOffError = 64;    // uint32: bit 0 set when a wait ran past the time bound
constexpr int kOffTicket = 128;  // uint32 slot ticket, its own 128-byte line
constexpr int kOffExited = 256;  // uint32 workgroups finished, its own line
constexpr int kOffDone = 384;    // kRep copies of uint32[nstages], each copy on its own lines

struct Header {                  // at offset 0 (64 bytes)
    uint32_t magic, version;
    int32_t nstages, total_slots;
    int32_t max_k;
    int32_t stride;              // uint32 words between the counter copies (a multiple of 32)
    int32_t nc;                  // 16-column chunks per staged plane of x
    int32_t grid;                // workgroups of the launch
    uint64_t stages_off, slots_off;  // byte offsets of the tables
    uint64_t timeout_ticks;      // bound on every wait, in s_memrealtime ticks
    uint64_t bytes;              // size of the image
};
static_assert(sizeof(Header) == 64, "header size");

struct StageD {                  // 32 bytes
    uint64_t x;                  // bf16 [k]
    int32_t k, dep;              // dep: stage whose outputs x holds, or -1
    int32_t slot0, nslots;       // the stage's slots in the ticket order
    int32_t nseg, pad;           // nseg: item segments per row (kItemChunks chunks each)
};
static_assert(sizeof(StageD) == 32, "stage size");

struct SlotD {                   // 48 bytes: up to kMaxRows consecutive rows of one matrix
    uint64_t codes, scale, y;    // the slot's first row: int8 [rows][k], fp32 [rows], bf16 [rows]
    int32_t rows, k, nseg, stage;
    int32_t pad[2];
};
static_assert(sizeof(SlotD) == 48, "slot size");

inline int32_t done_stride(int32_t nstages) { return (nstages + 31) / 32 * 32; }

inline uint64_t plan_bytes(int32_t nstages, int64_t total_slots) {
    const uint64_t stages_off = (uint64_t)kOffDone + (uint64_t)kRep * done_stride(nstages) * 4;
    const uint64_t slots_off = (stages_off + (uint64_t)nstages * sizeof(StageD) + 63) / 64 * 64;
    return slots_off + (uint64_t)total_slots * sizeof(SlotD);
}

}  // namespace chain

// The chained decode step: `image` is the host copy of the plan built by
// qg_chain_plan, `plan` its device copy (control words included).
hipError_t launch_chain(const void* image, void* plan, hipStream_t st);

}  // namespace qg
