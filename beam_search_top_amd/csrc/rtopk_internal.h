// Internal interface between the host-side C ABI (rtopk_host.cpp) and the
// gfx950 kernels (rtopk_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace rtopk {

constexpr int kLanes = 64;          // one wave64 per piece
constexpr int kMaxWaves = 16;       // pieces (waves) per workgroup, at most
constexpr int kMaxChunkLimit = 128; // candidates a piece stages in LDS (up to two per lane)
constexpr int kMaxSortKeys = 512;   // LDS sort keys of the per-batch selection
constexpr int kMaxPieces = 3072;    // pieces (beam * chunks) of one batch element (LDS tables)
constexpr int kMaxK = 64;
constexpr int kTicketCap = 65536;   // batch elements the ticket region holds (B limit)
constexpr int kMaxShards = 8;       // vocabulary shards of one sharded call
// Row-local workgroups hand their lists over through a mailbox of 64-bit
// slots that is all zero between calls; a shape whose lists do not fit it
// takes the per-piece publication path.
constexpr int kMailboxSlots = 1 << 17;
constexpr uint64_t kEmptySlot = 1;  // a published slot without a key (below every real key)
constexpr int kStatusWords = 64;    // error words of the workspace (word 0: a wait gave up)
constexpr unsigned kDefaultSpinLimit = 1u << 22; // polls of the mailbox before a wait gives up

// The part of every workspace that must be zero when a call starts and that
// every completed call leaves zero: tickets, status words, mailbox.
constexpr size_t kWsTicketOff = 0;
constexpr size_t kWsStatusOff = kWsTicketOff + 4 * (size_t)kTicketCap;
constexpr size_t kWsMailboxOff = kWsStatusOff + 4 * (size_t)kStatusWords;
constexpr size_t kWsFixedBytes = kWsMailboxOff + 8 * (size_t)kMailboxSlots;

// Division by a launch constant d >= 1 for dividends n < 2^31:
// floor(n / d) = (n * mul) >> shr with shr = 31 + ceil(log2 d) and
// mul = floor(2^shr / d) + 1 < 2^32 (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994, Theorem 4.2 with N = 31).
struct Magic {
    uint32_t mul, shr;
};

inline Magic make_magic(uint32_t d)
{
    uint32_t l = 0;
    while ((1ull << l) < d)
        ++l;
    const uint32_t shr = 31 + l;
    return Magic{(uint32_t)((1ull << shr) / d + 1), shr};
}

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
    int sort_keys;                 // LDS sort keys of the per-batch selection (power of two)
    int waves;                     // pieces (waves) per workgroup, <= kMaxWaves
    int rowlocal;                  // workgroups hold whole rows (chunks divides waves)
    int split;                     // per-piece path: pieces only publish; rtopk_select selects
    int maxl;                      // row-local: workgroup lists per batch element, at most
    unsigned spin_limit;           // row-local: polls of the mailbox before the merge gives up
    Magic mc, mb, mp, mw, mv;      // division by chunks, beam, beam*chunks, waves, V
    // Vocabulary shards: a row's pieces g*cps .. g*cps + cps - 1 lie in shard g,
    // whose [B][beam][vshard] tensor starts at shard[g] (one shard: shard[0] is
    // logits_aligned, vshard = V, cps = chunks). Token t of shard g is g*vshard + t.
    int vshard, cps;
    Magic ms;                      // division by cps
    const uint8_t *shard[kMaxShards];
    // workspace; only the fixed region (tickets, status, mailbox) must be zero when a call starts
    uint32_t *ticket;              // [kTicketCap] arrivals, first B used
    uint32_t *status;              // [kStatusWords] sticky error words
    uint64_t *mailbox;             // row-local lists [B][maxl][k] (kEmptySlot pads a short list)
    uint64_t *head;                // [B*beam*chunks][2]: (max2 | sum << 32), (threshold | count << 32)
    uint64_t *slots;               // [B*beam*chunks][k] each piece's top-k sort keys by logit
    // outputs
    int32_t *out_beam, *out_token;
    float *out_score;
    // top-k sampling drawn by row-local kernels built for k > 8 (nullable;
    // beam 1, zero running scores): one token and log-probability per row
    int32_t *smp_token;
    float *smp_logprob;
    float smp_tau;
    uint64_t smp_seed, smp_step;
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
    int ngroups, chunk_limit, queue_cap, align_elems, sort_keys, waves, rowlocal, maxl;
    int split; // per-piece publication in rounds: the per-batch selection is a second launch
    size_t select_lds; // LDS bytes of that launch
    int nshards, vshard, cps; // vocabulary shards, logits per shard row, pieces per shard row
    long long grid;
    size_t lds_bytes;
    size_t ws_head_off, ws_slots_off, ws_bytes;
};

// Enqueue the fused select + sort kernel for logits of type DT (0 float32,
// 1 float16, 2 bfloat16). Returns a hipError_t.
template <int DT>
hipError_t launch_dtype(const StepArgs &a, int vecs_per_thread, size_t lds_bytes, hipStream_t stream);
// Enqueue the per-batch selection of a split step (one workgroup of a.waves
// waves per batch element over the pieces the step kernel published).
hipError_t launch_select(const StepArgs &a, size_t lds_bytes, hipStream_t stream);

// The LM head fused with pass 1 (rtopk_kernels.hip, bfloat16 unit).
struct LmArgs {
    const uint16_t *x;   // [M][H] hidden states, bfloat16 bits
    const uint16_t *w;   // [V][H] output projection, bfloat16 bits
    const float *alive;  // [B][beam] running scores
    const uint8_t *finished; // [B][beam], nonzero = finished; may be null
    int B, M, V, H;      // batch, rows (B * beam), vocabulary, hidden size (a multiple of 64)
    int beam, k, ngroups, eos_id;
    int C, mtiles;       // 320-wide vocabulary tiles (pieces per row), 256-row tiles
    Magic mb, mv;        // division by beam, by V
    uint64_t *ms;        // [M*C] piece log-sum-exp partials: sum bits << 32 | max bits (base 2)
    uint64_t *slots;     // [M*C][k] piece top-k keys by logit, descending, 0 = empty
    int32_t *out_beam, *out_token;
    float *out_score;
};
constexpr int kLmTileV = 320;  // vocabulary columns per tile (one piece of a row)
constexpr int kLmTileM = 256;  // rows per tile
constexpr int kLmMaxK = 8;     // the epilogue keeps its group maxima in registers
constexpr int kLmMaxBeam = 512; // rows of a batch element the selection holds in LDS
// Enqueue the tile kernel and the per-batch selection.
hipError_t launch_lmhead(const LmArgs &a, hipStream_t stream);

// Enqueue a zero fill of `bytes` (multiple of 4) at `p` (no hipMemsetAsync).
hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream);
// top-k sampling (rtopk_sample.hip)
hipError_t launch_topk_sample(const int32_t *tok, const float *sc, int R, int k, float tau, uint64_t seed,
                              uint64_t step, int32_t *out_tok, float *out_lp, hipStream_t stream);
// cache refresh (rtopk_reorder.hip)
long long reorder_chunk_bytes();
hipError_t launch_beam_reorder(const void *src, void *dst, long long nslabs, int B, int beam, long long row_bytes,
                               const int32_t *ids, int ld, hipStream_t stream);
hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t marker, uint32_t *out, hipStream_t stream);
hipError_t launch_read_probe_shape(const void *src, size_t bytes, int vecs, int threads, uint32_t marker,
                                   uint32_t *out, hipStream_t stream);

// The status and thread-local message of the C ABI's last error (rtopk_last_error).
int set_error(int status, const char *fmt, ...);
// rtopk_noalloc.hip: the static scratch of device `dev` if a call has used it.
void *noalloc_scratch_if_used(int dev);

// Templates instantiated for vecs_per_thread.
bool supported_vecs_per_thread(int nv);

// Dynamic LDS of a workgroup of `waves` pieces whose per-batch selection
// needs sort_bytes (and, row-local, keys for the workgroup's own selection).
size_t group_lds_bytes(int waves, size_t sort_bytes, bool rowlocal, int k, int maxl);
// LDS of rtopk_select (kMaxWaves waves) for a selection of sort_bytes.
size_t select_lds_bytes(size_t sort_bytes);

// Row-local workgroups: LDS keys of the workgroup's own selection (every
// candidate of its pieces plus one per finished row) followed, in the
// workgroup that merges, by the other workgroups' lists.
__host__ __device__ constexpr int rowlocal_keys(int waves, int k, int maxl)
{
    return waves * (k + 1) + maxl * k;
}

} // namespace rtopk
