// Internal interface between the host-side C ABI (rtopk_host.cpp) and the
// gfx950 kernels (rtopk_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace rtopk {

constexpr int kThreads = 256;       // threads per workgroup (4 wave64s)
constexpr int kMaxChunkLimit = 256; // candidate slots of one piece (LDS stage and workspace)
constexpr int kSortKeys = 1024;     // LDS keys the per-batch selection sorts in one pass
constexpr int kMaxPieces = 2048;    // pieces (beam * chunks) of one batch element
constexpr int kMaxBeam = 512;       // per-beam LDS tables of the per-batch selection
constexpr int kMaxK = 64;
constexpr int kTicketCap = 65536;   // batch elements the ticket region holds (B limit)

// Everything one launch needs, passed by value as the kernel argument.
struct StepArgs {
    const uint8_t *logits_aligned; // logits base rounded down to 16 bytes
    const float *alive;            // [B][beam]
    const uint8_t *finished;       // [B][beam] or nullptr
    int B, beam, V, k, eos_id;
    int align_elems;               // logits base misalignment, elements
    int chunks;                    // pieces per row
    int vecs_per_chunk;            // 16-byte vectors per piece
    int ngroups;                   // groups of the threshold pass (power of two >= k)
    int chunk_limit;               // >= k, <= kMaxChunkLimit: candidates a piece stages in LDS
    int queue_cap;                 // candidate slots per batch element = beam*chunks*k
    // workspace; only the ticket region must be zero when a call starts
    uint32_t *ticket;              // [kTicketCap] arrivals, first B used
    uint64_t *head;                // [B*beam*chunks][2]: (max2 | sum << 32), (threshold | count << 32)
    uint64_t *slots;               // [B*beam*chunks][k] each piece's top-k sort keys by logit
    // outputs
    int32_t *out_beam, *out_token;
    float *out_score;
    // debug (nullable)
    float *dbg_T;
    uint32_t *dbg_hits;
    float *dbg_lse;
    uint32_t *dbg_count;
    uint64_t *dbg_queue;
};

struct Plan {
    int elem_bytes, epv;
    int chunks, vecs_per_thread, vecs_per_chunk;
    int ngroups, chunk_limit, queue_cap, align_elems;
    long long grid;
    size_t ws_ticket_off, ws_head_off, ws_slots_off, ws_bytes;
};

// Enqueue the fused select + sort kernel. Returns a hipError_t.
hipError_t launch_step(const StepArgs &a, int dtype, int vecs_per_thread, hipStream_t stream);

// Enqueue a zero fill of `bytes` (multiple of 4) at `p` (no hipMemsetAsync).
hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream);

// Templates instantiated for vecs_per_thread.
bool supported_vecs_per_thread(int nv);

} // namespace rtopk
