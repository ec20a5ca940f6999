// Host side of the C ABI declared in include/rtopk.h: argument validation,
// the decomposition of a call into workgroups, the workspace cache and the
// launch. All argument checks run before any HIP call, so a rejected call
// touches neither the GPU nor its outputs.
//
// The per-stream workspace follows the memory-reuse idea of the LightSeq
// inference article (its memory-reuse passage): buffers are sized once and
// reused on every request instead of being allocated per step.
#include "rtopk.h"
#include "rtopk_internal.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <utility>

static_assert(rtopk::kWsFixedBytes == RTOPK_WS_FIXED_BYTES, "the header states the fixed region's size");

namespace {

thread_local std::string g_err;

int vfail(int status, const char *fmt, va_list ap)
{
    char buf[512];
    vsnprintf(buf, sizeof buf, fmt, ap);
    g_err = buf;
    return status;
}

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    const int st = vfail(status, fmt, ap);
    va_end(ap);
    return st;
}

std::atomic<int> g_override_nv{0};
std::atomic<int> g_override_limit{0};
std::atomic<int> g_override_waves{0};
std::atomic<int> g_rowlocal{1};
std::atomic<int> g_split{1};
std::atomic<unsigned> g_spin_limit{rtopk::kDefaultSpinLimit};

const int kVecsPerThread[] = {1, 2, 3, 4, 6, 8, 10, 12};
// Most 16-byte vectors a lane holds without register spills and with >= 4
// waves per SIMD; rows that share vectors with their neighbours need the
// element-wise masking code and get fewer.
int max_vecs_per_thread(bool aligned_rows) { return aligned_rows ? 12 : 8; }
// Waves (one per piece) wanted per launch before pieces are made smaller:
// 16 per CU on 256 CUs.
constexpr long long kTargetGrid = 4096;
constexpr int kMinVecs = 8;
// Pieces the GPU runs at once: one 16-wave workgroup per CU on 256 CUs.
constexpr long long kResidentPieces = 4096;
constexpr long long kCUs = 256;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workgroups of 16 pieces while the grid fits the GPU at once (one per CU),
// of 8 when workgroups run in rounds and CUs must refill as they go
// (measured on 64 x 8 x 250000 bf16: 4 waves 87.7 us, 8 waves 82.5, 16 waves 92.1).
int waves_for(long long pieces) { return pieces <= kResidentPieces ? rtopk::kMaxWaves : 8; }

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

int pow2_ceil(int x)
{
    int p = 1;
    while (p < x)
        p <<= 1;
    return p;
}

// Validates the scalar arguments and computes the decomposition. With G
// vocabulary shards each row is G shard rows of V / G logits: pieces are cut
// per shard row (cps of them) and a row has chunks = G * cps pieces.
int make_plan(const void *logits, int B, int beam, int V, int k, int dtype, rtopk::Plan *p, int G = 1)
{
    if (dtype != RTOPK_F32 && dtype != RTOPK_F16 && dtype != RTOPK_BF16)
        return fail(RTOPK_EINVAL, "unknown dtype %d", dtype);
    if (B < 1 || beam < 1 || V < 1 || k < 1)
        return fail(RTOPK_EINVAL, "sizes must be >= 1 (B=%d beam=%d V=%d k=%d)", B, beam, V, k);
    if ((long long)beam * V > INT_MAX)
        return fail(RTOPK_EINVAL, "beam*V = %lld exceeds 2^31-1", (long long)beam * V);
    if ((long long)k > (long long)beam * V)
        return fail(RTOPK_EINVAL, "k=%d exceeds beam*V=%lld", k, (long long)beam * V);
    if (k > RTOPK_MAX_K)
        return fail(RTOPK_ENOTSUP, "k=%d exceeds the implementation limit %d", k, RTOPK_MAX_K);
    if (beam > RTOPK_MAX_BEAM)
        return fail(RTOPK_ENOTSUP, "beam=%d exceeds the implementation limit %d", beam, RTOPK_MAX_BEAM);

    p->elem_bytes = dtype == RTOPK_F32 ? 4 : 2;
    p->epv = 16 / p->elem_bytes;
    const uintptr_t mis = logits ? (uintptr_t)logits % 16 : 0;
    if (mis % p->elem_bytes)
        return fail(RTOPK_EINVAL, "logits pointer is not aligned to its element size");
    p->align_elems = (int)(mis / p->elem_bytes);
    const int Vs = V / G; // logits of one shard row
    const bool aligned_rows = p->align_elems == 0 && Vs % p->epv == 0;
    // 16-byte vectors one shard row touches at most
    const long long span = aligned_rows ? Vs / p->epv : ceil_div(Vs, p->epv) + 1;
    const long long rows = (long long)B * beam;
    const long long srows = rows * G; // shard rows

    int nv = g_override_nv.load();
    long long C;
    if (nv > 0) {
        C = ceil_div(span, (long long)rtopk::kLanes * nv);
    } else {
        const int nvmax = max_vecs_per_thread(aligned_rows);
        const long long c0 = ceil_div(span, (long long)rtopk::kLanes * nvmax);
        C = c0;
        if (srows * c0 < kTargetGrid) {
            long long want = ceil_div(kTargetGrid, srows);
            // no smaller than kMinVecs vectors per lane: past that, more pieces
            // add per-piece overhead faster than they add memory parallelism
            long long cmax = ceil_div(span, (long long)rtopk::kLanes * kMinVecs);
            C = want < cmax ? want : cmax;
            if (C < c0)
                C = c0;
        }
        const long long need = ceil_div(span, (long long)rtopk::kLanes * C);
        nv = nvmax;
        for (int v : kVecsPerThread)
            if (v >= need && v <= nvmax) {
                nv = v;
                break;
            }
        C = ceil_div(span, (long long)rtopk::kLanes * nv);
        // Prefer somewhat larger pieces when they make a row's pieces divide
        // the workgroup: its rows are then selected inside it (row-local),
        // which saves a cross-workgroup round trip per piece; at most half of
        // the pieces are given up for it.
        if (g_rowlocal.load() && waves_for(srows * C) % (G * C) != 0) {
            for (int v : kVecsPerThread) {
                if (v <= nv || v > nvmax)
                    continue;
                const long long c2 = ceil_div(span, (long long)rtopk::kLanes * v);
                if (2 * c2 < C)
                    break;
                if (waves_for(srows * c2) % (G * c2) == 0) {
                    nv = v;
                    C = c2;
                    break;
                }
            }
        }
    }
    p->vecs_per_thread = nv;
    p->nshards = G;
    p->vshard = Vs;
    p->cps = (int)C;
    C *= G; // pieces per row
    p->chunks = (int)C;
    // pieces hold exactly lanes*nv vectors (so the kernel's unmasked path
    // covers them), except a row's last piece, which holds the remainder
    p->vecs_per_chunk = rtopk::kLanes * nv;
    p->ngroups = pow2_ceil(k);
    int lim = g_override_limit.load();
    p->chunk_limit = lim > 0 ? lim : rtopk::kMaxChunkLimit;
    if (p->chunk_limit < k)
        p->chunk_limit = k; // a piece always may emit its own top-k
    p->waves = waves_for(rows * C);
    // Large k: a row-local workgroup selects the rows of each batch element it
    // holds one after the other on one wave, and a top-k of many keys is the
    // slow part of that tail. When a workgroup would hold several batch
    // elements, it holds one instead, so their selections run on different
    // workgroups (measured: 512 rows x 40000 fp16, k = 40, 57 -> 39 us).
    if (g_rowlocal.load() && k >= 16 && p->waves % C == 0 && (long long)beam * C < p->waves)
        p->waves = (int)(beam * C);
    // A small row-local grid (fewer workgroups than CUs) takes smaller
    // workgroups: the smallest that holds whole batch elements when one fits
    // (no handoff between workgroups), else one row per workgroup, which
    // spreads the stream over more CUs (measured: 32 x 4 x 40000 fp16 12.4 ->
    // 10.1 us with 8-wave workgroups; 2 x 2 x 8 fp32 5.4 -> 4.1 us with 2).
    else if (g_rowlocal.load() && p->waves % C == 0 && ceil_div(rows * C, p->waves) < kCUs) {
        const long long whole = (long long)beam * C;
        int w = (int)C;
        if (whole <= p->waves)
            while (w < whole)
                w <<= 1;
        p->waves = w;
    }
    // Row-local: when a row's pieces divide the workgroup, workgroups hold
    // whole rows and select them themselves; a batch element's rows then span
    // at most maxl workgroups, which exchange one list of k keys each.
    const int ow = g_override_waves.load();
    if (ow > 0)
        p->waves = ow;
    p->grid = ceil_div(rows * C, p->waves);
    p->rowlocal = p->waves % C == 0 && g_rowlocal.load() ? 1 : 0;
    p->maxl = (int)ceil_div((long long)beam * C, p->waves) + 1;
    // row-local lists go through the mailbox of the workspace's fixed region
    if (p->rowlocal && (long long)B * p->maxl * k > rtopk::kMailboxSlots)
        p->rowlocal = 0;
    // Per-piece publication in rounds (more pieces than the GPU holds at once):
    // the per-batch selection becomes a second launch (measured on 64 x 8 x
    // 250000 bf16, see rtopk_select)
    p->split = !p->rowlocal && rows * C > kResidentPieces && g_split.load() ? 1 : 0;
    if (rows * C >= (1ll << 31)) // piece indices are 31-bit in the kernel
        return fail(RTOPK_ENOTSUP, "%lld pieces are too many", rows * C);
    if ((long long)beam * C > rtopk::kMaxPieces)
        return fail(RTOPK_ENOTSUP, "beam*chunks = %lld exceeds the implementation limit %d (vocabulary too large "
                    "for this beam count)", (long long)beam * C, rtopk::kMaxPieces);
    const long long qcap = (long long)beam * C * k; // every piece publishes at most its top-k
    if (qcap > INT_MAX)
        return fail(RTOPK_ENOTSUP, "candidate queue of %lld entries is too large", qcap);
    p->queue_cap = (int)qcap;
    // LDS of the per-batch selection: sort keys for every published candidate
    // plus one per finished beam (capped; more survivors take the argmax path),
    // three float tables per beam, one count byte per piece
    const long long want_keys = qcap + beam;
    p->sort_keys = pow2_ceil(want_keys < rtopk::kMaxSortKeys ? (int)want_keys : rtopk::kMaxSortKeys);
    // sort keys, three floats and a count byte per piece, three floats and a
    // flag byte per beam
    const size_t pieces = (size_t)beam * (size_t)C;
    const size_t sort_lds = 8 * (size_t)p->sort_keys + 13 * pieces + 13 * (size_t)beam;
    p->lds_bytes = (rtopk::group_lds_bytes(p->waves, sort_lds, p->rowlocal != 0, k, p->maxl) + 15) & ~size_t(15);
    p->select_lds = (rtopk::select_lds_bytes(sort_lds) + 15) & ~size_t(15);

    if (B > rtopk::kTicketCap)
        return fail(RTOPK_ENOTSUP, "B=%d exceeds the implementation limit %d", B, rtopk::kTicketCap);
    // tickets, status words and the mailbox first, in a region of fixed size:
    // no shape ever stores other data there, so it stays zero between calls
    // whatever the shapes are; then the per-piece headers and slots
    size_t off = align256(rtopk::kWsFixedBytes);
    p->ws_head_off = off;
    if (!p->rowlocal) {
        off = align256(off + sizeof(uint64_t) * 2 * (size_t)rows * (size_t)C); // piece headers, two words each
        p->ws_slots_off = off;
        off = align256(off + sizeof(uint64_t) * (size_t)B * (size_t)p->queue_cap); // every piece's top-k
    } else {
        p->ws_slots_off = off;
    }
    p->ws_bytes = off;
    return RTOPK_OK;
}

int check_pointers(const void *logits, const float *alive, const int32_t *ob, const int32_t *ot,
                   const float *os)
{
    if (!logits)
        return fail(RTOPK_EINVAL, "logits is NULL");
    if (!alive)
        return fail(RTOPK_EINVAL, "alive_scores is NULL");
    if (!ob || !ot || !os)
        return fail(RTOPK_EINVAL, "an output pointer is NULL");
    return RTOPK_OK;
}

struct Debug {
    float *T = nullptr;
    uint32_t *hits = nullptr;
    float *lse = nullptr;
    uint32_t *count = nullptr;
    uint64_t *queue = nullptr;
};

struct SampleArgs { // a top-k draw fused into the selection (row-local kernels built for k > 8)
    int32_t *token = nullptr;
    float *logprob = nullptr;
    float tau = 1.f;
    uint64_t seed = 0, step = 0;
};

// Whether the selection kernel of this plan draws the sample itself.
bool fused_draw(const rtopk::Plan &p, int k) { return p.rowlocal != 0 && k > 8; }

int enqueue(const rtopk::Plan &p, const void *logits, int dtype, const float *alive,
            const uint8_t *finished, int B, int beam, int V, int k, int eos_id, int32_t *ob,
            int32_t *ot, float *os, void *ws, const Debug &dbg, hipStream_t stream,
            const void *const *shards = nullptr, const SampleArgs &smp = SampleArgs{})
{
    rtopk::StepArgs a{};
    a.logits_aligned = (const uint8_t *)logits - (size_t)p.align_elems * p.elem_bytes;
    a.vshard = p.vshard;
    a.cps = p.cps;
    a.ms = rtopk::make_magic((uint32_t)p.cps);
    for (int g = 0; g < rtopk::kMaxShards; ++g)
        a.shard[g] = shards && g < p.nshards ? (const uint8_t *)shards[g] : a.logits_aligned;
    a.alive = alive;
    a.finished = finished;
    a.B = B;
    a.beam = beam;
    a.V = V;
    a.k = k;
    a.eos_id = eos_id;
    a.align_elems = p.align_elems;
    a.chunks = p.chunks;
    a.vecs_per_chunk = p.vecs_per_chunk;
    a.ngroups = p.ngroups;
    a.chunk_limit = p.chunk_limit;
    a.queue_cap = p.queue_cap;
    a.sort_keys = p.sort_keys;
    a.waves = p.waves;
    a.rowlocal = p.rowlocal;
    a.split = p.split;
    a.maxl = p.maxl;
    a.mc = rtopk::make_magic((uint32_t)p.chunks);
    a.mb = rtopk::make_magic((uint32_t)beam);
    a.mp = rtopk::make_magic((uint32_t)beam * (uint32_t)p.chunks);
    a.mw = rtopk::make_magic((uint32_t)p.waves);
    a.mv = rtopk::make_magic((uint32_t)V);
    a.spin_limit = g_spin_limit.load();
    uint8_t *w = (uint8_t *)ws;
    a.ticket = (uint32_t *)(w + rtopk::kWsTicketOff);
    a.status = (uint32_t *)(w + rtopk::kWsStatusOff);
    a.mailbox = (uint64_t *)(w + rtopk::kWsMailboxOff);
    a.head = (uint64_t *)(w + p.ws_head_off);
    a.slots = (uint64_t *)(w + p.ws_slots_off);
    a.out_beam = ob;
    a.out_token = ot;
    a.out_score = os;
    a.smp_token = smp.token;
    a.smp_logprob = smp.logprob;
    a.smp_tau = smp.tau;
    a.smp_seed = smp.seed;
    a.smp_step = smp.step;
    a.dbg_T = dbg.T;
    a.dbg_hits = dbg.hits;
    a.dbg_lse = dbg.lse;
    a.dbg_count = dbg.count;
    a.dbg_queue = dbg.queue;
    hipError_t e = dtype == RTOPK_F32   ? rtopk::launch_dtype<0>(a, p.vecs_per_thread, p.lds_bytes, stream)
                   : dtype == RTOPK_F16 ? rtopk::launch_dtype<1>(a, p.vecs_per_thread, p.lds_bytes, stream)
                                        : rtopk::launch_dtype<2>(a, p.vecs_per_thread, p.lds_bytes, stream);
    if (e == hipSuccess && p.split)
        e = rtopk::launch_select(a, p.select_lds, stream);
    if (e != hipSuccess)
        return fail(RTOPK_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return RTOPK_OK;
}

// ---------------------------------------------------------------- workspace cache
struct WsEntry {
    void *ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, void *>, WsEntry> g_ws;

int acquire_workspace(size_t need, hipStream_t stream, void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(RTOPK_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_ws_mu);
    WsEntry &w = g_ws[{dev, (void *)stream}];
    if (w.bytes < need) {
        if (w.ptr) {
            // earlier calls on this stream may still use the old buffer
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess)
                return fail(RTOPK_EHIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
            (void)hipFree(w.ptr);
            w.ptr = nullptr;
            w.bytes = 0;
        }
        size_t bytes = align256(need + need / 2);
        void *p = nullptr;
        e = hipMalloc(&p, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(RTOPK_ENOMEM, "hipMalloc(%zu) for the workspace: %s", bytes, hipGetErrorString(e));
        }
        e = rtopk::launch_zero(p, bytes, stream);
        if (e != hipSuccess) {
            (void)hipFree(p);
            return fail(RTOPK_EHIP, "zero-filling the workspace: %s", hipGetErrorString(e));
        }
        w.ptr = p;
        w.bytes = bytes;
    }
    *out = w.ptr;
    return RTOPK_OK;
}

// A device buffer of zeros per device (the running scores of sampling rows),
// zero-filled once and never written after; grown when a call needs more.
std::map<int, WsEntry> g_zeros;

int acquire_zeros(size_t n, hipStream_t stream, const float **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(RTOPK_EHIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lock(g_ws_mu);
    WsEntry &z = g_zeros[dev];
    const size_t bytes = n * sizeof(float);
    if (z.bytes < bytes) {
        const size_t grow = bytes > 2 * z.bytes ? bytes : 2 * z.bytes;
        void *p = nullptr;
        hipError_t e = hipMalloc(&p, grow);
        if (e != hipSuccess)
            return fail(RTOPK_ENOMEM, "hipMalloc(%zu) for the zero scores: %s", grow, hipGetErrorString(e));
        if ((e = rtopk::launch_zero(p, grow, stream)) != hipSuccess || (e = hipStreamSynchronize(stream)) != hipSuccess) {
            (void)hipFree(p);
            return fail(RTOPK_EHIP, "zero-filling the zero scores: %s", hipGetErrorString(e));
        }
        if (z.ptr) { // an earlier, smaller buffer may still be read by enqueued work
            (void)hipDeviceSynchronize();
            (void)hipFree(z.ptr);
        }
        z.ptr = p;
        z.bytes = grow;
    }
    *out = (const float *)z.ptr;
    return RTOPK_OK;
}

} // namespace

int rtopk::set_error(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    const int st = vfail(status, fmt, ap);
    va_end(ap);
    return st;
}

extern "C" {

int rtopk_beam_step(const void *logits, int dtype, const float *alive_scores,
                    const uint8_t *finished_mask, int B, int beam, int V, int k, int eos_id,
                    int32_t *out_beam_ids, int32_t *out_token_ids, float *out_scores, void *stream)
{
    int st = check_pointers(logits, alive_scores, out_beam_ids, out_token_ids, out_scores);
    if (st != RTOPK_OK)
        return st;
    rtopk::Plan p;
    if ((st = make_plan(logits, B, beam, V, k, dtype, &p)) != RTOPK_OK)
        return st;
    if (eos_id < 0 || eos_id >= V)
        return fail(RTOPK_EINVAL, "eos_id=%d outside [0, %d)", eos_id, V);
    void *ws = nullptr;
    if ((st = acquire_workspace(p.ws_bytes, (hipStream_t)stream, &ws)) != RTOPK_OK)
        return st;
    return enqueue(p, logits, dtype, alive_scores, finished_mask, B, beam, V, k, eos_id, out_beam_ids,
                   out_token_ids, out_scores, ws, Debug{}, (hipStream_t)stream);
}

int rtopk_beam_step_sharded(const void *const *shards, int nshards, int dtype, const float *alive_scores,
                            const uint8_t *finished_mask, int B, int beam, int V_shard, int k, int eos_id,
                            int32_t *out_beam_ids, int32_t *out_token_ids, float *out_scores, void *stream)
{
    if (!shards)
        return fail(RTOPK_EINVAL, "shards is NULL");
    if (nshards < 1 || nshards > rtopk::kMaxShards)
        return fail(RTOPK_EINVAL, "nshards=%d outside [1, %d]", nshards, rtopk::kMaxShards);
    for (int g = 0; g < nshards; ++g) {
        if (!shards[g])
            return fail(RTOPK_EINVAL, "shard %d is NULL", g);
        if ((uintptr_t)shards[g] % 16)
            return fail(RTOPK_EINVAL, "shard %d is not 16-byte aligned", g);
    }
    int st = check_pointers(shards[0], alive_scores, out_beam_ids, out_token_ids, out_scores);
    if (st != RTOPK_OK)
        return st;
    if (V_shard < 1)
        return fail(RTOPK_EINVAL, "V_shard=%d must be >= 1", V_shard);
    const int esz = dtype == RTOPK_F32 ? 4 : 2;
    if ((long long)V_shard * esz % 16)
        return fail(RTOPK_EINVAL, "V_shard=%d: a shard row of %lld bytes is not a multiple of 16", V_shard,
                    (long long)V_shard * esz);
    if ((long long)V_shard * nshards > INT_MAX)
        return fail(RTOPK_EINVAL, "V_shard*nshards exceeds 2^31-1");
    const int V = V_shard * nshards;
    rtopk::Plan p;
    if ((st = make_plan(shards[0], B, beam, V, k, dtype, &p, nshards)) != RTOPK_OK)
        return st;
    if (eos_id < 0 || eos_id >= V)
        return fail(RTOPK_EINVAL, "eos_id=%d outside [0, %d)", eos_id, V);
    void *ws = nullptr;
    if ((st = acquire_workspace(p.ws_bytes, (hipStream_t)stream, &ws)) != RTOPK_OK)
        return st;
    return enqueue(p, shards[0], dtype, alive_scores, finished_mask, B, beam, V, k, eos_id, out_beam_ids,
                   out_token_ids, out_scores, ws, Debug{}, (hipStream_t)stream, shards);
}

size_t rtopk_workspace_bytes(int B, int beam, int V, int k, int dtype)
{
    rtopk::Plan p;
    if (make_plan(nullptr, B, beam, V, k, dtype, &p) != RTOPK_OK)
        return 0;
    // the largest misalignment can add one vector per row; size for it
    rtopk::Plan q;
    if (make_plan((const void *)(uintptr_t)(16 - (dtype == RTOPK_F32 ? 4 : 2)), B, beam, V, k, dtype, &q) !=
        RTOPK_OK)
        return p.ws_bytes;
    return p.ws_bytes > q.ws_bytes ? p.ws_bytes : q.ws_bytes;
}

static int step_ws(const void *logits, int dtype, const float *alive_scores, const uint8_t *finished_mask,
                   int B, int beam, int V, int k, int eos_id, int32_t *ob, int32_t *ot, float *os,
                   void *workspace, size_t ws_bytes, const Debug &dbg, void *stream)
{
    int st = check_pointers(logits, alive_scores, ob, ot, os);
    if (st != RTOPK_OK)
        return st;
    rtopk::Plan p;
    if ((st = make_plan(logits, B, beam, V, k, dtype, &p)) != RTOPK_OK)
        return st;
    if (eos_id < 0 || eos_id >= V)
        return fail(RTOPK_EINVAL, "eos_id=%d outside [0, %d)", eos_id, V);
    if (!workspace)
        return fail(RTOPK_EINVAL, "workspace is NULL");
    if ((uintptr_t)workspace % 256)
        return fail(RTOPK_EINVAL, "workspace is not 256-byte aligned");
    if (ws_bytes < p.ws_bytes)
        return fail(RTOPK_ENOMEM, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, p.ws_bytes);
    return enqueue(p, logits, dtype, alive_scores, finished_mask, B, beam, V, k, eos_id, ob, ot, os,
                   workspace, dbg, (hipStream_t)stream);
}

int rtopk_beam_step_ws(const void *logits, int dtype, const float *alive_scores,
                       const uint8_t *finished_mask, int B, int beam, int V, int k, int eos_id,
                       int32_t *out_beam_ids, int32_t *out_token_ids, float *out_scores, void *workspace,
                       size_t ws_bytes, void *stream)
{
    return step_ws(logits, dtype, alive_scores, finished_mask, B, beam, V, k, eos_id, out_beam_ids,
                   out_token_ids, out_scores, workspace, ws_bytes, Debug{}, stream);
}

int rtopk_debug_step(const void *logits, int dtype, const float *alive_scores,
                     const uint8_t *finished_mask, int B, int beam, int V, int k, int eos_id,
                     int32_t *out_beam_ids, int32_t *out_token_ids, float *out_scores, void *workspace,
                     size_t ws_bytes, float *dbg_T, uint32_t *dbg_hits, float *dbg_lse,
                     uint32_t *dbg_count, uint64_t *dbg_queue, void *stream)
{
    Debug d;
    d.T = dbg_T;
    d.hits = dbg_hits;
    d.lse = dbg_lse;
    d.count = dbg_count;
    d.queue = dbg_queue;
    return step_ws(logits, dtype, alive_scores, finished_mask, B, beam, V, k, eos_id, out_beam_ids,
                   out_token_ids, out_scores, workspace, ws_bytes, d, stream);
}

int rtopk_plan(const void *logits, int B, int beam, int V, int k, int dtype, rtopk_plan_t *out)
{
    if (!out)
        return fail(RTOPK_EINVAL, "out is NULL");
    rtopk::Plan p;
    int st = make_plan(logits, B, beam, V, k, dtype, &p);
    if (st != RTOPK_OK)
        return st;
    out->chunks = p.chunks;
    out->threads = rtopk::kLanes;
    out->pieces_per_group = p.waves;
    out->row_local = p.rowlocal;
    out->vecs_per_thread = p.vecs_per_thread;
    out->vecs_per_chunk = p.vecs_per_chunk;
    out->elems_per_vec = p.epv;
    out->ngroups = p.ngroups;
    out->chunk_limit = p.chunk_limit;
    out->queue_cap = p.queue_cap;
    out->align_elems = p.align_elems;
    out->grid = (int)p.grid;
    out->sort_keys = p.sort_keys;
    out->lds_bytes = (int)p.lds_bytes;
    return RTOPK_OK;
}

int rtopk_set_override(int vecs_per_thread, int chunk_limit)
{
    if (vecs_per_thread != 0 && !rtopk::supported_vecs_per_thread(vecs_per_thread))
        return fail(RTOPK_EINVAL, "vecs_per_thread=%d is not one of the built variants", vecs_per_thread);
    if (chunk_limit < 0 || chunk_limit > rtopk::kMaxChunkLimit)
        return fail(RTOPK_EINVAL, "chunk_limit=%d outside [0, %d]", chunk_limit, rtopk::kMaxChunkLimit);
    g_override_nv.store(vecs_per_thread);
    g_override_limit.store(chunk_limit);
    return RTOPK_OK;
}

int rtopk_set_row_local(int enable)
{
    g_rowlocal.store(enable != 0 ? 1 : 0);
    return RTOPK_OK;
}

int rtopk_set_split(int enable)
{
    g_split.store(enable != 0 ? 1 : 0);
    return RTOPK_OK;
}

int rtopk_set_waves(int waves)
{
    if (waves < 0 || waves > rtopk::kMaxWaves)
        return fail(RTOPK_EINVAL, "waves=%d outside [0, %d]", waves, rtopk::kMaxWaves);
    g_override_waves.store(waves);
    return RTOPK_OK;
}

int rtopk_set_spin_limit(unsigned polls)
{
    g_spin_limit.store(polls);
    return RTOPK_OK;
}

// Reads the status word of workspace `ws`; if a wait gave up, clears the
// fixed region (late lists may have landed in the mailbox after the call).
int check_workspace(void *ws, hipStream_t stream)
{
    uint32_t status = 0;
    hipError_t e = hipMemcpy(&status, (uint8_t *)ws + rtopk::kWsStatusOff, sizeof status, hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return fail(RTOPK_EHIP, "reading the workspace status: %s", hipGetErrorString(e));
    if (status == 0)
        return RTOPK_OK;
    if ((e = rtopk::launch_zero(ws, rtopk::kWsFixedBytes, stream)) != hipSuccess ||
        (e = hipStreamSynchronize(stream)) != hipSuccess)
        return fail(RTOPK_EHIP, "clearing the workspace after a failed wait: %s", hipGetErrorString(e));
    return fail(RTOPK_ETIMEOUT, "a row-local merge gave up waiting for another workgroup's list (status 0x%x); "
                "its batch elements were written as padding; the workspace has been cleared", status);
}

int rtopk_check(void *workspace, void *stream)
{
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess)
        return fail(RTOPK_EHIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
    if (workspace)
        return check_workspace(workspace, (hipStream_t)stream);
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess)
        return fail(RTOPK_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    void *lib = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_ws_mu);
        auto it = g_ws.find({dev, stream});
        if (it != g_ws.end())
            lib = it->second.ptr;
    }
    int st = RTOPK_OK;
    if (lib)
        st = check_workspace(lib, (hipStream_t)stream);
    if (void *scr = rtopk::noalloc_scratch_if_used(dev)) { // the static scratch of rtopk_beam_step_noalloc
        const int st2 = check_workspace(scr, (hipStream_t)stream);
        if (st == RTOPK_OK)
            st = st2;
    }
    return st;
}

int rtopk_sample_step(const void *logits, int dtype, int R, int V, int k, float temperature, uint64_t seed,
                      uint64_t step, int32_t *out_token, float *out_logprob, void *stream)
{
    if (!logits || !out_token || !out_logprob)
        return fail(RTOPK_EINVAL, "sample step: NULL pointer");
    if (!(temperature > 0.f) || !std::isfinite(temperature))
        return fail(RTOPK_EINVAL, "sample step: temperature must be finite and > 0");
    rtopk::Plan p;
    int st = make_plan(logits, R, 1, V, k, dtype, &p);
    if (st != RTOPK_OK)
        return st;
    // the selection's outputs follow its workspace; a zero running score per row
    const size_t off = align256(p.ws_bytes);
    const size_t rk = (size_t)R * (size_t)k;
    const size_t need = off + 3 * align256(4 * rk);
    void *ws = nullptr;
    if ((st = acquire_workspace(need, (hipStream_t)stream, &ws)) != RTOPK_OK)
        return st;
    const float *zeros = nullptr;
    if ((st = acquire_zeros((size_t)R, (hipStream_t)stream, &zeros)) != RTOPK_OK)
        return st;
    uint8_t *w = (uint8_t *)ws;
    int32_t *ob = (int32_t *)(w + off);
    int32_t *ot = (int32_t *)(w + off + align256(4 * rk));
    float *os = (float *)(w + off + 2 * align256(4 * rk));
    // row-local kernels built for k > 8 draw right after each row's top-k;
    // the others leave the lists to the draw kernel
    SampleArgs smp;
    const bool fused = fused_draw(p, k);
    if (fused) {
        smp.token = out_token;
        smp.logprob = out_logprob;
        smp.tau = temperature;
        smp.seed = seed;
        smp.step = step;
    }
    if ((st = enqueue(p, logits, dtype, zeros, nullptr, R, 1, V, k, 0, ob, ot, os, ws, Debug{},
                      (hipStream_t)stream, nullptr, smp)) != RTOPK_OK)
        return st;
    if (fused)
        return RTOPK_OK;
    const hipError_t e = rtopk::launch_topk_sample(ot, os, R, k, temperature, seed, step, out_token, out_logprob,
                                                   (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(RTOPK_EHIP, "sample launch: %s", hipGetErrorString(e));
    return RTOPK_OK;
}

int rtopk_lmhead_step(const void *hidden, const void *weight, const float *alive_scores,
                      const uint8_t *finished_mask, int B, int beam, int H, int V, int k, int eos_id,
                      int32_t *out_beam_ids, int32_t *out_token_ids, float *out_scores, void *stream)
{
    if (!hidden || !weight || !alive_scores || !out_beam_ids || !out_token_ids || !out_scores)
        return fail(RTOPK_EINVAL, "lmhead step: NULL pointer");
    if (B < 1 || beam < 1 || H < 1 || V < 1 || k < 1)
        return fail(RTOPK_EINVAL, "lmhead step: sizes must be >= 1 (B=%d beam=%d H=%d V=%d k=%d)", B, beam, H, V, k);
    if ((long long)k > (long long)beam * V)
        return fail(RTOPK_EINVAL, "lmhead step: k=%d exceeds beam*V", k);
    if (eos_id < 0 || eos_id >= V)
        return fail(RTOPK_EINVAL, "lmhead step: eos_id=%d outside [0, %d)", eos_id, V);
    if ((uintptr_t)hidden % 16 || (uintptr_t)weight % 16)
        return fail(RTOPK_EINVAL, "lmhead step: hidden and weight must be 16-byte aligned");
    if (H % 64)
        return fail(RTOPK_ENOTSUP, "lmhead step: H=%d is not a multiple of 64", H);
    if (k > rtopk::kLmMaxK)
        return fail(RTOPK_ENOTSUP, "lmhead step: k=%d exceeds the fused path's limit %d", k, rtopk::kLmMaxK);
    if (beam > rtopk::kLmMaxBeam)
        return fail(RTOPK_ENOTSUP, "lmhead step: beam=%d beyond the implementation limit %d", beam, rtopk::kLmMaxBeam);
    const long long M = (long long)B * beam;
    // buffer offsets are 32-bit, up to the end of the last (partial) tile
    if ((M + rtopk::kLmTileM) * H * 2 >= (1ll << 31) || ((long long)V + rtopk::kLmTileV) * H * 2 >= (1ll << 31))
        return fail(RTOPK_ENOTSUP, "lmhead step: hidden or weight of 2 GiB or more");
    if ((long long)beam * V > INT_MAX)
        return fail(RTOPK_EINVAL, "lmhead step: beam*V exceeds 2^31-1");
    const long long C = (V + rtopk::kLmTileV - 1) / rtopk::kLmTileV; // pieces per row
    const long long npieces = M * C;
    // workspace: the fixed region (left to the step kernels, which share the
    // cached workspace), then the piece partials and slots
    const size_t ms_off = align256(rtopk::kWsFixedBytes);
    const size_t slots_off = align256(ms_off + 8 * (size_t)npieces);
    const size_t need = align256(slots_off + 8 * (size_t)npieces * k);
    void *ws = nullptr;
    int st = acquire_workspace(need, (hipStream_t)stream, &ws);
    if (st != RTOPK_OK)
        return st;
    uint8_t *w8 = (uint8_t *)ws;
    rtopk::LmArgs la{};
    la.x = (const uint16_t *)hidden;
    la.w = (const uint16_t *)weight;
    la.alive = alive_scores;
    la.finished = finished_mask;
    la.B = B;
    la.M = (int)M;
    la.V = V;
    la.H = H;
    la.beam = beam;
    la.k = k;
    la.ngroups = pow2_ceil(k);
    la.eos_id = eos_id;
    la.C = (int)C;
    la.mtiles = (int)((M + rtopk::kLmTileM - 1) / rtopk::kLmTileM);
    la.mb = rtopk::make_magic((uint32_t)beam);
    la.mv = rtopk::make_magic((uint32_t)V);
    la.ms = (uint64_t *)(w8 + ms_off);
    la.slots = (uint64_t *)(w8 + slots_off);
    la.out_beam = out_beam_ids;
    la.out_token = out_token_ids;
    la.out_score = out_scores;
    const hipError_t e = rtopk::launch_lmhead(la, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(RTOPK_EHIP, "lmhead step launch: %s", hipGetErrorString(e));
    return RTOPK_OK;
}

int rtopk_beam_reorder(const void *src, void *dst, long long nslabs, int B, int beam, long long row_bytes,
                       const int32_t *beam_ids, int ld, void *stream)
{
    if (src == nullptr || dst == nullptr || beam_ids == nullptr)
        return fail(RTOPK_EINVAL, "beam reorder: NULL pointer");
    if (nslabs < 1 || B < 1 || beam < 1 || row_bytes < 1)
        return fail(RTOPK_EINVAL, "beam reorder: sizes must be >= 1 (nslabs=%lld B=%d beam=%d row_bytes=%lld)",
                    nslabs, B, beam, row_bytes);
    if (ld < beam)
        return fail(RTOPK_EINVAL, "beam reorder: ld=%d is below beam=%d", ld, beam);
    const long long rows = (long long)B * beam;
    if (rows > (1ll << 40) / nslabs || nslabs * rows > (1ll << 50) / row_bytes)
        return fail(RTOPK_EINVAL, "beam reorder: cache size overflows");
    const long long bytes = nslabs * rows * row_bytes;
    const long long cpr = (row_bytes + rtopk::reorder_chunk_bytes() - 1) / rtopk::reorder_chunk_bytes();
    if (nslabs * rows * cpr > 0x7fffffffLL)
        return fail(RTOPK_EINVAL, "beam reorder: %lld chunks exceed one launch", nslabs * rows * cpr);
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
    if (s0 < d0 + (uintptr_t)bytes && d0 < s0 + (uintptr_t)bytes)
        return fail(RTOPK_EINVAL, "beam reorder: source and destination overlap");
    const hipError_t e = rtopk::launch_beam_reorder(src, dst, nslabs, B, beam, row_bytes, beam_ids, ld,
                                                    (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(RTOPK_EHIP, "beam reorder launch: %s", hipGetErrorString(e));
    return RTOPK_OK;
}

int rtopk_read_probe(const void *src, size_t bytes, uint32_t marker, uint32_t *out, void *stream)
{
    if (src == nullptr || out == nullptr)
        return fail(RTOPK_EINVAL, "read probe: NULL pointer");
    if ((uintptr_t)src % 16 != 0 || bytes % 16 != 0)
        return fail(RTOPK_EINVAL, "read probe: src must be 16-byte aligned and bytes a multiple of 16");
    const hipError_t e = rtopk::launch_read_probe(src, bytes, marker, out, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(RTOPK_EHIP, "read probe launch: %s", hipGetErrorString(e));
    return RTOPK_OK;
}

int rtopk_read_probe_shape(const void *src, size_t bytes, int vecs_per_lane, int threads, uint32_t marker,
                           uint32_t *out, void *stream)
{
    if (src == nullptr || out == nullptr)
        return fail(RTOPK_EINVAL, "read probe: NULL pointer");
    if ((uintptr_t)src % 16 != 0 || bytes % 16 != 0)
        return fail(RTOPK_EINVAL, "read probe: src must be 16-byte aligned and bytes a multiple of 16");
    const int v = vecs_per_lane;
    if (!(v == 1 || v == 2 || v == 4 || v == 8 || v == 10 || v == 16))
        return fail(RTOPK_EINVAL, "read probe: vecs_per_lane=%d is not 1, 2, 4, 8, 10 or 16", v);
    if (threads < 64 || threads > 1024 || threads % 64 != 0)
        return fail(RTOPK_EINVAL, "read probe: threads=%d is not a multiple of 64 in [64, 1024]", threads);
    const hipError_t e = rtopk::launch_read_probe_shape(src, bytes, v, threads, marker, out, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(RTOPK_EHIP, "read probe launch: %s", hipGetErrorString(e));
    return RTOPK_OK;
}

const char *rtopk_last_error(void) { return g_err.c_str(); }

void rtopk_release(void)
{
    std::lock_guard<std::mutex> lock(g_ws_mu);
    int cur = -1;
    if (!g_ws.empty() && hipGetDevice(&cur) != hipSuccess)
        cur = -1;
    for (auto &kv : g_ws) {
        if (kv.second.ptr) {
            (void)hipSetDevice(kv.first.first);
            (void)hipDeviceSynchronize();
            (void)hipFree(kv.second.ptr);
        }
    }
    g_ws.clear();
    for (auto &kv : g_zeros) {
        if (kv.second.ptr) {
            (void)hipSetDevice(kv.first);
            (void)hipDeviceSynchronize();
            (void)hipFree(kv.second.ptr);
        }
    }
    g_zeros.clear();
    if (cur >= 0)
        (void)hipSetDevice(cur);
}

} // extern "C"
