/*
 * rtopk.h -- C ABI of the MI355X (gfx950) hierarchical beam-search selection step.
 *
 * One decode step of beam search, as stated by the LightSeq inference
 * article (hierarchical-decoding passage): from a [batch_size, beam_size,
 * vocab_size] logit matrix pick, for every batch element, the k best
 * (beam, token) continuations, where the score of a continuation is the
 * beam's running score plus the token's log-softmax:
 *
 *     score(b, j, t) = alive_scores[b][j] + logits[b][j][t] - lse(b, j),
 *     lse(b, j)      = log(sum_t exp(logits[b][j][t])).
 *
 * The article's rewrite -- a first pass that splits each beam's logits into k
 * groups, takes the minimum of the k group maxima as a lower bound (the
 * "R-top-k") of the k-th largest logit and computes log_sum_exp in the same
 * traversal, a second pass that keeps only logits >= R-top-k in a per-batch
 * candidate queue, and one small sort of that queue -- gives exactly this
 * result without a softmax or a sort over all beam*vocab elements.
 *
 * Conventions for every entry point below:
 *  - Pointers marked "device" are HIP device memory owned by the caller; the
 *    library never frees or retains them. They must stay valid until the work
 *    enqueued on `stream` has completed.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls
 *    are asynchronous: they validate, enqueue and return. Results are valid
 *    once the stream reaches them.
 *  - Validation is synchronous and happens before anything is enqueued; on a
 *    non-OK status nothing was launched and no output was written.
 *    rtopk_last_error() then describes the problem.
 *  - Layouts are C-contiguous row-major. Logits may have any base alignment
 *    that is a multiple of the element size.
 *  - Output order per batch element: score descending, equal scores by the
 *    lower flat index j*V + t. When fewer than k candidates exist (possible
 *    only when finished beams leave fewer than k), the tail is padded with
 *    beam = token = -1 and score = -inf.
 *  - A finished beam (finished_mask != 0) offers the single continuation
 *    (j, eos_id) at its unchanged running score; its logits are never read
 *    (the flag sizes the row's loads to zero bytes).
 *  - Scores are computed in float32: alive + (logit - lse), lse accumulated in
 *    float32 in a fixed order, so results are bit-reproducible across calls.
 *  - NaN or +inf logits, and alive beams whose logits are all -inf, are
 *    outside the contract (unspecified output, no error). Individual -inf
 *    logits are fine.
 */
#ifndef RTOPK_H
#define RTOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Logit storage types. */
typedef enum { RTOPK_F32 = 0, RTOPK_F16 = 1, RTOPK_BF16 = 2 } rtopk_dtype;

/* Status codes returned by the entry points. */
typedef enum {
    RTOPK_OK = 0,
    RTOPK_EINVAL = -1,  /* bad argument: NULL pointer, size < 1, k > beam*V, eos outside [0,V), ... */
    RTOPK_ENOTSUP = -2, /* valid but beyond the implementation limits: k > 64, beam > 512,
                           B > 65536, beam * pieces-per-row > 3072 */
    RTOPK_ENOMEM = -3,  /* device allocation failed, or a caller workspace is too small */
    RTOPK_EHIP = -4,    /* a HIP runtime call or kernel launch failed */
    RTOPK_ETIMEOUT = -5 /* reported by rtopk_check: a cross-workgroup wait of an earlier call gave up */
} rtopk_status;

/* Implementation limits. */
#define RTOPK_MAX_K 64
#define RTOPK_MAX_BEAM 512

/*
 * How one call is decomposed (reported by rtopk_plan; the kernel uses it).
 * Each beam's row is split into `chunks` contiguous pieces of at most
 * `vecs_per_chunk` 16-byte vectors, one wave64 (`threads` lanes) per piece,
 * each lane holding `vecs_per_thread` vectors in registers; a workgroup holds
 * `pieces_per_group` consecutive pieces and `grid` workgroups are launched. Within
 * a piece, element e (counted from the 16-byte-aligned address at or below the
 * logits base pointer) belongs to group e mod `ngroups`; ngroups is k rounded
 * up to a power of two and the piece's threshold is the k-th largest group
 * maximum (the minimum when ngroups == k). Each piece publishes only its own
 * exact top-k by (logit desc, flat index asc) among the logits at or above its
 * threshold; up to `chunk_limit` of those are ranked in LDS, a piece with more
 * finds its top-k by k rounds of argmax. `queue_cap` = beam * chunks * k is the
 * candidate count per batch element. The last piece of a batch element to
 * finish selects its k outputs, ranking up to `sort_keys` survivors in LDS;
 * `lds_bytes` is the dynamic LDS of one workgroup. When `row_local` is set
 * (chunks divides pieces_per_group), workgroups hold whole rows: each selects
 * the exact top-k of the rows it holds in LDS, and only those lists of k
 * keys are exchanged between the workgroups that share a batch element (the
 * last of them to finish its pieces merges; the others leave their lists in
 * the workspace's mailbox).
 */
typedef struct {
    int chunks;          /* pieces per beam row (C) */
    int threads;         /* threads per piece (one wave64) */
    int vecs_per_thread; /* 16-byte vectors held per thread */
    int vecs_per_chunk;  /* 16-byte vectors per piece */
    int elems_per_vec;   /* 4 for float32, 8 for float16/bfloat16 */
    int ngroups;         /* groups of the threshold pass */
    int chunk_limit;     /* candidates a piece ranks in LDS before switching to k argmax rounds */
    int queue_cap;       /* candidate slots per batch element (beam * chunks * k) */
    int align_elems;     /* misalignment of the logits base, in elements */
    int grid;            /* workgroups launched: ceil(B * beam * chunks / pieces_per_group) */
    int sort_keys;       /* survivors the per-batch selection ranks in LDS */
    int lds_bytes;       /* dynamic LDS per workgroup */
    int pieces_per_group; /* pieces (waves) per workgroup */
    int row_local;       /* 1: workgroups hold whole rows and select them in LDS */
} rtopk_plan_t;

/*
 * One beam-search selection step.
 *   logits         device [B][beam][V], element type `dtype`
 *   alive_scores   device [B][beam] float32 running log-probability scores
 *   finished_mask  device [B][beam] uint8, nonzero = finished; NULL = none finished
 *   B, beam, V, k  batch size, beams per batch element, vocabulary size, outputs per
 *                  batch element; 1 <= k <= min(64, beam*V), beam <= 512, beam*V < 2^31
 *   eos_id         token offered by a finished beam, in [0, V)
 *   out_beam_ids   device [B][k] int32, in [0, beam) or -1
 *   out_token_ids  device [B][k] int32, in [0, V) or -1
 *   out_scores     device [B][k] float32
 * Uses a workspace owned by the library, cached per (device, stream): the first
 * call for a given stream (or for a larger shape) allocates and zero-fills it,
 * later calls allocate nothing. Calls on one stream are serialised by the
 * stream; concurrent calls on different streams use different workspaces.
 */
int rtopk_beam_step(const void *logits, int dtype, const float *alive_scores,
                    const uint8_t *finished_mask, int B, int beam, int V, int k, int eos_id,
                    int32_t *out_beam_ids, int32_t *out_token_ids, float *out_scores,
                    void *stream);

/*
 * rtopk_beam_step on a vocabulary split into nshards shards, as a
 * vocabulary-parallel LM head leaves it: shard g is its own device tensor
 * [B][beam][V_shard] holding vocabulary indices g*V_shard .. (g+1)*V_shard - 1.
 * Each shard row is processed on its own (its pieces' R-top-k thresholds, exact
 * per-piece candidates and log-sum-exp partials) and only those are merged per
 * beam and batch element -- the exchange a multi-GPU vocabulary split needs
 * (the article's rough-select kernel and candidate queue, applied per shard),
 * here inside one launch on one GPU. Results equal rtopk_beam_step on the
 * concatenated [B][beam][nshards*V_shard] logits (token ids are vocabulary
 * indices), up to the fp32 rounding of the log-sum-exp merge order.
 *   shards    HOST array of nshards device pointers, each 16-byte aligned
 *   nshards   1..8
 *   V_shard   logits per shard row; V_shard * element size must be a multiple of 16
 * Everything else as rtopk_beam_step (library-owned workspace, eos_id < nshards*V_shard).
 */
int rtopk_beam_step_sharded(const void *const *shards, int nshards, int dtype, const float *alive_scores,
                            const uint8_t *finished_mask, int B, int beam, int V_shard, int k, int eos_id,
                            int32_t *out_beam_ids, int32_t *out_token_ids, float *out_scores, void *stream);

/* Bytes of caller workspace rtopk_beam_step_ws needs for this shape (0 on bad arguments). */
size_t rtopk_workspace_bytes(int B, int beam, int V, int k, int dtype);

/*
 * rtopk_beam_step with a caller-owned device workspace of ws_bytes >=
 * rtopk_workspace_bytes(...) bytes, 256-byte aligned. It must be zero-filled
 * before its first use; every completed call leaves it ready for any later
 * call whose shape fits (its first RTOPK_WS_FIXED_BYTES bytes -- arrival
 * counters, status words and the mailbox through which workgroups hand over
 * their lists -- are zero again after each call; the rest holds scratch
 * data). Calls sharing one workspace must be ordered (same stream).
 * Allocates nothing. RTOPK_ENOMEM when ws_bytes is too small.
 */
#define RTOPK_WS_FIXED_BYTES 1310976
int rtopk_beam_step_ws(const void *logits, int dtype, const float *alive_scores,
                       const uint8_t *finished_mask, int B, int beam, int V, int k, int eos_id,
                       int32_t *out_beam_ids, int32_t *out_token_ids, float *out_scores,
                       void *workspace, size_t ws_bytes, void *stream);

/*
 * rtopk_beam_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, the same kernels and results, and no allocation of any
 * kind (no hipMalloc, no library routine that allocates). Its workspace is a
 * file-scope device array of RTOPK_NOALLOC_SCRATCH_BYTES (8 MiB) that every
 * GPU the library runs on holds until the process ends; it is zero when the
 * library is loaded and every completed call leaves its fixed region zero
 * again. Every call on one GPU shares that GPU's array: calls that overlap on
 * one GPU (on different streams) race and must not be made; calls ordered on
 * one stream are fine. RTOPK_ENOMEM, with nothing launched, when the shape
 * needs more workspace than the array holds (rtopk_workspace_bytes > 8 MiB);
 * RTOPK_EHIP when the array's device address cannot be looked up.
 * rtopk_check(NULL, stream) also reports a give-up of a wait on this array.
 */
#define RTOPK_NOALLOC_SCRATCH_BYTES 8388608
int rtopk_beam_step_noalloc(const void *logits, int dtype, const float *alive_scores,
                            const uint8_t *finished_mask, int B, int beam, int V, int k, int eos_id,
                            int32_t *out_beam_ids, int32_t *out_token_ids, float *out_scores,
                            void *stream);

/*
 * rtopk_beam_step_ws that also copies out intermediate values (for tests):
 *   dbg_T       device [B*beam*chunks] float32: each piece's threshold (-inf if empty)
 *   dbg_hits    device [B*beam*chunks] uint32: logits >= threshold in the piece (its
 *               R-top-k survivors, of which it publishes the best min(hits, k))
 *   dbg_lse     device [B*beam] float32: merged log-sum-exp (NaN for finished beams)
 *   dbg_count   device [B] uint32, zero-filled by the caller: candidates the pieces of
 *               each batch element emitted
 *   dbg_queue   device [B*queue_cap] uint64: those candidates, entry = (float32 bits of
 *               the logit << 32) | (j*V + t), in no particular order; only the first
 *               dbg_count[b] of each batch element are defined
 * Any debug pointer may be NULL. Finished beams leave their dbg_T/dbg_hits unset.
 */
int rtopk_debug_step(const void *logits, int dtype, const float *alive_scores,
                     const uint8_t *finished_mask, int B, int beam, int V, int k, int eos_id,
                     int32_t *out_beam_ids, int32_t *out_token_ids, float *out_scores,
                     void *workspace, size_t ws_bytes, float *dbg_T, uint32_t *dbg_hits,
                     float *dbg_lse, uint32_t *dbg_count, uint64_t *dbg_queue, void *stream);

/*
 * The decomposition a call with these arguments would use. `logits` is only
 * inspected for its alignment (may be NULL = 16-byte aligned). Host only.
 */
int rtopk_plan(const void *logits, int B, int beam, int V, int k, int dtype, rtopk_plan_t *out);

/*
 * Process-wide tuning overrides for experiments and tests (0 = automatic):
 * vecs_per_thread forces the 16-byte vectors each thread holds (one of
 * 1,2,3,4,6,8,10,12; others are rejected with RTOPK_EINVAL);
 * chunk_limit forces the per-piece LDS candidate limit (1..128, raised to k),
 * which makes the argmax-rounds top-k path run whenever a piece has more
 * candidates.
 */
int rtopk_set_override(int vecs_per_thread, int chunk_limit);

/*
 * Process-wide tuning override for experiments and tests: the pieces (waves)
 * per workgroup, 1..16, or 0 for the planner's choice (RTOPK_EINVAL outside
 * 0..16). Shapes whose pieces per row do not divide it take the per-piece
 * publication path.
 */
int rtopk_set_waves(int waves);

/*
 * Process-wide bound of the one wait in the selection kernel: the workgroup
 * that merges a batch element whose rows span several workgroups polls the
 * others' lists at most `polls` times (default 4194304, each poll followed
 * by a short sleep) before it gives up. The other workgroups are running
 * when the wait starts (they counted their arrival before it), so the bound
 * is only reached if the GPU stops running them, e.g. under preemption. On
 * give-up the batch element's outputs are written as padding (-1, -1, -inf)
 * and the workspace's status word is set; rtopk_check reports it. 0 gives up
 * without polling (tests use it to exercise that path). Always RTOPK_OK.
 */
int rtopk_set_spin_limit(unsigned polls);

/*
 * Synchronises `stream` and reports whether a wait of an earlier call on
 * `workspace` (a caller workspace of rtopk_beam_step_ws / rtopk_debug_step,
 * or NULL for the library-owned workspace of `stream` and the static scratch
 * of rtopk_beam_step_noalloc on the current device) gave up:
 * RTOPK_ETIMEOUT, after clearing the workspace's fixed region so that later
 * calls are exact again (those batch elements were written as padding).
 * RTOPK_OK when no wait gave up, RTOPK_EHIP when a HIP call fails.
 */
int rtopk_check(void *workspace, void *stream);

/*
 * Process-wide switch for tests and experiments: 0 turns the row-local
 * workgroup selection off (every shape then takes the per-piece publication
 * path), nonzero (the default) uses it wherever chunks divides the
 * workgroup's pieces. Always RTOPK_OK.
 */
int rtopk_set_row_local(int enable);

/*
 * Process-wide switch for tests and experiments: with per-piece publication
 * in a grid that runs in rounds (more pieces than the GPU holds at once), the
 * per-batch selection is by default a second launch over the published
 * pieces (one workgroup per batch element, after every piece is done); 0
 * selects each batch element inside the step kernel instead, by the
 * workgroup that completes it. The results are the same. Always RTOPK_OK.
 */
int rtopk_set_split(int enable);

/*
 * Top-k sampling with the same hierarchical selection. The LightSeq inference
 * article reports sampling-decode speedups next to its beam-search ones (its
 * results passage). Every row r < R of logits [R][V] is selected as a batch
 * element with one beam and a zero running score, which gives its k best
 * tokens with scores s_i = x_i - lse(row), best first (ties: lower token).
 * One of them is then drawn from the top-k distribution at `temperature`:
 *     w_i = exp((s_i - s_1) / temperature),   S = w_1 + ... + w_k (rank order, fp32),
 *     u   = (word 0 of Philox4x64-10 with counter (r, step, 0, 0) and key
 *            (seed, 0)) >> 40, times 2^-24,
 *     i   = the first rank with u*S < w_1 + ... + w_i (the last rank if none).
 *   out_token    device [R] int32: the token of rank i
 *   out_logprob  device [R] float32: log(w_i / S), its log-probability under the
 *                top-k distribution
 * 1 <= k <= min(64, V); temperature finite and > 0. The same (seed, step) draws
 * the same tokens. When the rows are selected row-locally and k > 8, the
 * selection kernel draws right after each row's top-k (one launch); else a
 * draw kernel follows it. Uses the library-owned workspace of `stream` (allocated on
 * the first call for a shape, like rtopk_beam_step) and a library-owned buffer
 * of zero scores per device.
 */
int rtopk_sample_step(const void *logits, int dtype, int R, int V, int k, float temperature, uint64_t seed,
                      uint64_t step, int32_t *out_token, float *out_logprob, void *stream);

/*
 * The step fused into the LM head in front of it. The LightSeq inference
 * article computes the logits with a GEMM ahead of the decoding step and
 * fuses the work around its GEMMs into them (kernel-fusion passage). Here
 *     logits[b*beam + j][t] = sum_h hidden[b*beam + j][h] * weight[t][h]
 * (bfloat16 inputs, float32 accumulation on the matrix cores) are computed
 * in 256-row x 320-column tiles whose epilogue runs pass 1 and the per-piece
 * top-k of the selection (a piece = one row of one 320-wide vocabulary tile;
 * its groups are the vocabulary indices mod ngroups), so the [B*beam][V]
 * logits never reach HBM; a second launch merges each row's pieces (its
 * log-sum-exp and its k best logits) and selects each batch element with the
 * scores, order, finished-beam rule and padding of rtopk_beam_step. Results
 * are those of rtopk_beam_step on the float32 logits of that GEMM.
 *   hidden   device [B*beam][H] bfloat16 (row b*beam + j is beam j of batch element b)
 *   weight   device [V][H] bfloat16, one row per vocabulary entry (the output
 *            projection as a [V][H] matrix); both 16-byte aligned
 *   H        a multiple of 64 (else RTOPK_ENOTSUP)
 *   k        1 <= k <= min(8, beam*V) (k > 8: RTOPK_ENOTSUP)
 * Everything else as rtopk_beam_step (library-owned workspace of `stream`,
 * 8 * B*beam * ceil(V/320) * (k + 1) bytes past its fixed region).
 * RTOPK_ENOTSUP also when beam > 512 or hidden or weight spans about 2 GiB
 * or more (32-bit buffer offsets, counted to the end of the last tile).
 */
int rtopk_lmhead_step(const void *hidden, const void *weight, const float *alive_scores,
                      const uint8_t *finished_mask, int B, int beam, int H, int V, int k, int eos_id,
                      int32_t *out_beam_ids, int32_t *out_token_ids, float *out_scores, void *stream);

/*
 * Cache refresh after a selection step. The LightSeq inference article's
 * hierarchical-decoding passage ends the step with a cache update once the
 * top-k are known (its profile: 10% of latency in fp32, 6% in fp16). For a
 * beam-major cache of nslabs slabs (e.g. layers x {keys, values}) of B*beam
 * rows of row_bytes bytes, new beam j of batch element b takes the row of old
 * beam beam_ids[b*ld + j]:
 *     dst[s][b*beam + j][0..row_bytes) = src[s][b*beam + beam_ids[b*ld + j]][0..row_bytes)
 * for every s < nslabs, b < B, j < beam.
 *   src, dst   device, [nslabs][B*beam][row_bytes] bytes each, not overlapping
 *              (caller-owned; a double-buffered cache swaps them each step)
 *   beam_ids   device [B][ld] int32, ld >= beam: rtopk_beam_step's out_beam_ids
 *              with k = beam is [B][k]; an id outside [0, beam) (the -1 padding of
 *              a batch element with fewer than k candidates) leaves that
 *              destination row as it was
 * Rows move as 16-byte vectors when src, dst and row_bytes are multiples of
 * 16, else byte by byte. Asynchronous on `stream`; allocates nothing.
 * RTOPK_EINVAL: NULL pointer, a size < 1, ld < beam, overlapping buffers, a
 * cache too large to address or to launch in one grid.
 */
int rtopk_beam_reorder(const void *src, void *dst, long long nslabs, int B, int beam, long long row_bytes,
                       const int32_t *beam_ids, int ld, void *stream);

/*
 * Measurement aid, not part of the selection: a plain streaming read that
 * gives the practical HBM ceiling the selection kernel is compared with. It
 * reads `bytes` bytes at `src` once with 16-byte non-temporal loads (ten per
 * lane, 256-lane workgroups, one launch) and sets out[0] = 1 if any aligned
 * 32-bit word equals `marker`; otherwise it writes nothing.
 *   src     device, 16-byte aligned; bytes a multiple of 16 (else RTOPK_EINVAL)
 *   out     device uint32[1], caller-owned
 * Asynchronous on `stream`; allocates nothing.
 */
int rtopk_read_probe(const void *src, size_t bytes, uint32_t marker, uint32_t *out, void *stream);

/*
 * The same measurement aid with the launch shape chosen by the caller:
 * vecs_per_lane 16-byte loads per lane (1, 2, 4, 8, 10 or 16) and `threads`
 * lanes per workgroup (a multiple of 64 in [64, 1024]); else as
 * rtopk_read_probe. RTOPK_EINVAL also for another vecs_per_lane or threads.
 */
int rtopk_read_probe_shape(const void *src, size_t bytes, int vecs_per_lane, int threads, uint32_t marker,
                           uint32_t *out, void *stream);

/* Thread-local description of the last non-OK status ("" if none). */
const char *rtopk_last_error(void);

/* Frees every cached library-owned workspace (synchronises their streams). */
void rtopk_release(void);

#ifdef __cplusplus
}
#endif

#endif /* RTOPK_H */
