// gfx950 (CDNA4) kernel of the hierarchical beam-search selection step.
//
// The method is the LightSeq inference article's hierarchical decoding
// (its passage on the logit rough-select kernel and the candidate queue):
//  pass 1  per beam, split the logits into k groups, take each group's
//          maximum and the minimum of those maxima -- the "R-top-k", never
//          above the k-th largest logit -- and compute log_sum_exp in the
//          same traversal;
//  pass 2  keep every logit >= R-top-k as a candidate of its batch element;
//  sort    one small sort of each batch element's candidates gives its exact
//          top-k.
//
// MI355X design (one launch per step, kernel `rtopk_step`):
//  * A beam row is cut into `chunks` contiguous pieces of 64 x NV 16-byte
//    vectors. One wave64 owns a piece: every lane loads its NV vectors from
//    HBM with 16-byte loads straight into registers, where they stay for both
//    passes, so HBM is read exactly once. Pieces are independent: a wave
//    never waits for another wave after its loads are issued, and the only
//    cross-lane traffic is DPP, readlane and ballots inside the wave. A
//    workgroup holds `waves` consecutive pieces: 16 when the whole grid is
//    resident at once, 8 when workgroups run in rounds (a workgroup frees its
//    CU only when its slowest wave is done).
//  * Pass 1 keeps one running maximum per element slot (packed v_pk_max_f16
//    for fp16) and accumulates the log-sum-exp online in fp32, base 2,
//    rescaled once per block of 4 vectors so that the work follows the
//    arriving data. Group g holds the elements e = g mod ngroups, so a slot's
//    maximum is a group maximum of the lane; DPP row reductions plus
//    readlanes make the piece's group maxima. Its threshold is the k-th
//    largest of the ngroups (k rounded up to a power of two) group maxima:
//    the R-top-k itself when k is a power of two.
//  * A piece may treat its own threshold as the row's: any logit among the
//    row's top-k that lies in the piece is among the piece's top-k, and those
//    are all >= the piece's threshold. So each piece publishes just its own
//    exact top-k (by logit desc, flat index asc) among its logits >= T.
//  * Pass 2 tests each vector with one packed maximum; a vector where some
//    lane has a hit is examined element by element, hits are ranked by ballot
//    + mbcnt into 64 LDS entries (one per lane) and the piece's top-k is found
//    by rank counting (k rounds of wave argmax if more than `chunk_limit`).
//  * Cross-workgroup data moves only through device-coherent (sc1) atomic
//    stores and loads, so no L2 writeback or invalidate is ever needed.
//    Device-scope atomics on one address serialise at the memory side, so
//    they are issued per workgroup and batch element, never per wave.
//  * Row-local workgroups (a row's pieces divide the workgroup, e.g. 4 x
//    40000-logit fp16 batch elements: 8 pieces per row, 2 rows per
//    workgroup) keep every piece's results in LDS and select their rows
//    there: merge each row's (max, sum) partials by DPP butterflies, apply
//    the row threshold max_c T_c and the bound S = max_j (alive_j + T_j -
//    lse_j) (at least k candidates score >= S), keep the k best. The
//    workgroups sharing a batch element count their arrival at its ticket
//    before selecting (low 16 bits); all but the last publish their k keys
//    and then count the publication (high 16 bits); the last waits for those
//    counts, merges the lists and writes the outputs.
//  * Other workgroups publish each piece's top-k and partials; wave 0 adds
//    the workgroup's piece count to the ticket of each batch element it
//    touched, and the workgroup that completes a ticket merges every piece
//    of that batch element in the same way.
//  * A ticket is put back to zero by the workgroup that finishes its batch
//    element; tickets live in a region of the workspace that no shape uses
//    for anything else.
// Compiled once per logit type (-DRTOPK_DTYPE=0 float32, 1 float16,
// 2 bfloat16) so the instantiations build in parallel; the float32 unit also
// holds the type-independent host helpers.
#ifndef RTOPK_DTYPE
#error "define RTOPK_DTYPE (0, 1 or 2)"
#endif
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rtopk_draw.h"
#include "rtopk_internal.h"

// No implicit a*b+c contraction: a score and the bound it is compared with
// must round identically (explicit fmaf calls still map to FMA instructions).
#pragma clang fp contract(off)

namespace rtopk {
namespace {

constexpr int kBlock = 4; // vectors per online log-sum-exp rescale
// LDS of a workgroup: arrival counter, the shared group maxima of each of its
// (at most `waves`) rows as order-preserving bits, then the waves' selection
// LDS or, for the wave that completes a ticket, the sorter's.
constexpr int kLdsShare = 256; // GroupLds (counters, reduction scratch) first
__host__ __device__ constexpr size_t lds_header(int waves) { return kLdsShare + 4 * (size_t)waves * kMaxK; }
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t word(const uint4 &d, int i)
{
    return i == 0 ? d.x : i == 1 ? d.y : i == 2 ? d.z : d.w;
}

__device__ __forceinline__ void set_word(uint4 &d, int i, uint32_t w)
{
    if (i == 0)
        d.x = w;
    else if (i == 1)
        d.y = w;
    else if (i == 2)
        d.z = w;
    else
        d.w = w;
}

// Order-preserving map of a float to uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t ord_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ord(uint32_t o)
{
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Sort key: higher score first, then lower flat index. -0 is folded into +0.
__device__ __forceinline__ uint64_t score_key(float score, uint32_t flat)
{
    return ((uint64_t)ord_bits(score + 0.0f) << 32) | (uint64_t)(0xffffffffu - flat);
}

// A published candidate is its sort key by logit, score_key(x, flat).
__device__ __forceinline__ float entry_x(uint64_t e) { return from_ord((uint32_t)(e >> 32)); }
__device__ __forceinline__ uint32_t entry_flat(uint64_t e) { return 0xffffffffu - (uint32_t)e; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Merge of two base-2 log-sum-exp partials (m = max in log2 units, s = sum of
// 2^(x - m)).
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2)
{
    float M = fmaxf(m, m2);
    if (M == -INFINITY) {
        m = M;
        s = 0.f;
        return;
    }
    s = s * fast_exp2(m - M) + s2 * fast_exp2(m2 - M);
    m = M;
}

// Cross-workgroup data (candidates, partials, counters) moves only through
// agent-scope atomic stores and loads, which gfx950 issues with sc1: they are
// performed at the device coherence point, past the per-XCD L2s, so no L2
// writeback (buffer_wbl2) or invalidate (buffer_inv) is ever needed. A writer
// drains its own stores (s_waitcnt vmcnt(0)) before it takes its ticket; the
// compiler barriers keep the stores on their side of the wait.
__device__ __forceinline__ void put64(uint64_t *p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get64(const uint64_t *p)
{
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put32(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void drain_stores()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0); // vmcnt(0) expcnt(0) lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// q / d for 0 <= q < 2^22 and 1 <= d < 2^22, via one float multiply: the
// quotient's error is below 1/(2d) of a unit, so (q + 0.5) * (1/d) never
// crosses an integer boundary before the truncation.
__device__ __forceinline__ int small_div(int q, float inv_d) { return (int)(((float)q + 0.5f) * inv_d); }

// ---------------------------------------------------------------- XCD grouping
// Workgroups are dispatched to the 8 XCDs round robin (workgroup w on XCD
// w mod 8), and each XCD has its own L2 and address translation caches.
// Workgroup w takes the pieces of logical workgroup L(w), which gives every
// XCD one contiguous eighth of the tensor (the last G mod 8 workgroups keep
// their index). A bijection on [0, G); nothing relies on it for correctness.
constexpr int kXcds = 8;
__device__ __forceinline__ int logical_group(int w, int G)
{
    const uint32_t uw = (uint32_t)w, G8 = (uint32_t)G & ~(uint32_t)(kXcds - 1);
    return uw < G8 ? (int)((uw % kXcds) * (G8 / kXcds) + uw / kXcds) : w;
}

// floor(n / d) for n < 2^31, d given by its multiplier and shift (host-made)
__device__ __forceinline__ uint32_t mdiv(uint32_t n, Magic m)
{
    return (uint32_t)(((uint64_t)n * m.mul) >> m.shr);
}
// ---------------------------------------------------------------- wave primitives
__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lane_prefix(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Wave-wide reductions with DPP row operations (VALU only, no LDS): swap
// neighbours (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1), mirror
// within 8 lanes, mirror within 16 lanes -- after which every lane of a
// 16-lane row holds the row's total -- then the four row totals are combined
// in a fixed order from readlanes. Each step combines the same two values on
// both partner lanes, so the result is identical on every lane and from run
// to run. Every lane must be active.
template <int CTRL> __device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_f(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ float wave_max_f(float v)
{
    v = fmaxf(v, dpp_f<0xb1>(v));
    v = fmaxf(v, dpp_f<0x4e>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float row16_max_f(float v) // every lane: the maximum over its 16-lane row
{
    v = fmaxf(v, dpp_f<0xb1>(v));
    v = fmaxf(v, dpp_f<0x4e>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    return fmaxf(v, dpp_f<0x140>(v));
}
__device__ __forceinline__ float wave_min_f(float v)
{
    v = fminf(v, dpp_f<0xb1>(v));
    v = fminf(v, dpp_f<0x4e>(v));
    v = fminf(v, dpp_f<0x141>(v));
    v = fminf(v, dpp_f<0x140>(v));
    return fminf(fminf(lane_f(v, 0), lane_f(v, 16)), fminf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum_f(float v)
{
    v = v + dpp_f<0xb1>(v);
    v = v + dpp_f<0x4e>(v);
    v = v + dpp_f<0x141>(v);
    v = v + dpp_f<0x140>(v);
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
template <int CTRL> __device__ __forceinline__ uint32_t dpp_u(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u<0xb1>(v));
    v = max(v, dpp_u<0x4e>(v));
    v = max(v, dpp_u<0x141>(v));
    v = max(v, dpp_u<0x140>(v));
    return max(max((uint32_t)__builtin_amdgcn_readlane(v, 0), (uint32_t)__builtin_amdgcn_readlane(v, 16)),
               max((uint32_t)__builtin_amdgcn_readlane(v, 32), (uint32_t)__builtin_amdgcn_readlane(v, 48)));
}
// Wave maximum of 64-bit keys with DPP only: the largest high word, then the
// largest low word among the lanes that hold it. Every lane must be active.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v)
{
    const uint32_t hi = wave_max_u32((uint32_t)(v >> 32));
    const uint32_t lo = wave_max_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, d);
        const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), d);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}
__device__ __forceinline__ uint32_t first_u32(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        v += __shfl_xor(v, d);
    return v;
}
// Sum of v over the lanes below this one.
__device__ __forceinline__ uint32_t wave_excl_scan_u32(uint32_t v, int lane)
{
    uint32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t t = __shfl_up(x, d);
        x += lane >= d ? t : 0u;
    }
    return x - v;
}

// Workgroup barrier that waits only for this wave's LDS (and scalar)
// operations, s_waitcnt lgkmcnt(0) with vmcnt and expcnt at their maxima:
// __syncthreads would also wait for every global load and store in flight,
// and here barriers only ever order LDS accesses.
__device__ __forceinline__ void lds_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Orders one wave's LDS accesses across its lanes (the wave runs in lockstep
// and LDS executes its instructions in order, so compiler fences suffice).
// Sibling waves are not waited for: code that only one wave runs uses this
// instead of a workgroup barrier.
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------- dtype traits
template <int DT> struct Traits;

template <> struct Traits<0> { // float32
    static constexpr int epv = 4;
    struct Acc {
        float v[4];
    };
    __device__ static uint4 neg_inf() { return make_uint4(0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u); }
    __device__ static float elem(const uint4 &d, int i) { return __uint_as_float(word(d, i)); }
    __device__ static float elem_rt(const uint4 &d, int i) { return __uint_as_float(word(d, i)); }
    __device__ static void mask_if(uint4 &d, int i, bool m) { set_word(d, i, m ? 0xff800000u : word(d, i)); }
    __device__ static void init(Acc &a)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a.v[i] = -INFINITY;
    }
    __device__ static void update(Acc &a, const uint4 &d)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a.v[i] = fmaxf(a.v[i], elem(d, i));
    }
    __device__ static float amax(const Acc &a) { return fmaxf(fmaxf(a.v[0], a.v[1]), fmaxf(a.v[2], a.v[3])); }
    __device__ static void order_after(Acc &a, float x, float y)
    {
        asm volatile("" : "+v"(a.v[0]), "+v"(a.v[1]), "+v"(a.v[2]), "+v"(a.v[3]) : "v"(x), "v"(y));
    }
    __device__ static void slots(const Acc &a, float *s)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s[i] = a.v[i];
    }
    __device__ static bool any_ge(const uint4 &d, float T)
    {
        return fmaxf(fmaxf(elem(d, 0), elem(d, 1)), fmaxf(elem(d, 2), elem(d, 3))) >= T;
    }
    // element 0, and the vector moved down by one element (rolled loops)
    __device__ static float first(const uint4 &d) { return __uint_as_float(d.x); }
    __device__ static void shift(uint4 &d)
    {
        d.x = d.y;
        d.y = d.z;
        d.z = d.w;
    }
};

// Moves a vector of 16-bit elements down by one element.
__device__ __forceinline__ void shift16(uint4 &d)
{
    d.x = __builtin_amdgcn_alignbit(d.y, d.x, 16);
    d.y = __builtin_amdgcn_alignbit(d.z, d.y, 16);
    d.z = __builtin_amdgcn_alignbit(d.w, d.z, 16);
    d.w >>= 16;
}

template <> struct Traits<1> { // float16, max kept on packed pairs
    static constexpr int epv = 8;
    struct Acc {
        half2v h[4];
    };
    __device__ static half2v pair(const uint4 &d, int p) { return __builtin_bit_cast(half2v, word(d, p)); }
    __device__ static uint4 neg_inf() { return make_uint4(0xfc00fc00u, 0xfc00fc00u, 0xfc00fc00u, 0xfc00fc00u); }
    __device__ static float elem(const uint4 &d, int i)
    {
        half2v h = pair(d, i >> 1);
        return (i & 1) ? (float)h.y : (float)h.x;
    }
    __device__ static float elem_rt(const uint4 &d, int i)
    {
        const uint32_t w = word(d, i >> 1) >> ((i & 1) * 16);
        return (float)__builtin_bit_cast(_Float16, (uint16_t)w);
    }
    __device__ static void mask_if(uint4 &d, int i, bool m)
    {
        const uint32_t w = word(d, i >> 1);
        const uint32_t mw = (i & 1) ? ((w & 0x0000ffffu) | 0xfc000000u) : ((w & 0xffff0000u) | 0x0000fc00u);
        set_word(d, i >> 1, m ? mw : w);
    }
    __device__ static void init(Acc &a)
    {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            a.h[p] = __builtin_bit_cast(half2v, 0xfc00fc00u);
    }
    __device__ static void update(Acc &a, const uint4 &d)
    {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            a.h[p] = __builtin_elementwise_max(a.h[p], pair(d, p));
    }
    __device__ static float amax(const Acc &a)
    {
        half2v t = __builtin_elementwise_max(__builtin_elementwise_max(a.h[0], a.h[1]),
                                             __builtin_elementwise_max(a.h[2], a.h[3]));
        return fmaxf((float)t.x, (float)t.y);
    }
    __device__ static void order_after(Acc &a, float x, float y)
    {
        asm volatile("" : "+v"(a.h[0]), "+v"(a.h[1]), "+v"(a.h[2]), "+v"(a.h[3]) : "v"(x), "v"(y));
    }
    __device__ static void slots(const Acc &a, float *s)
    {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            s[2 * p] = (float)a.h[p].x;
            s[2 * p + 1] = (float)a.h[p].y;
        }
    }
    // T is an fp16 value widened (or -inf), so the comparison can stay in fp16
    __device__ static bool any_ge(const uint4 &d, float T)
    {
        half2v t = __builtin_elementwise_max(__builtin_elementwise_max(pair(d, 0), pair(d, 1)),
                                             __builtin_elementwise_max(pair(d, 2), pair(d, 3)));
        const _Float16 th = (_Float16)T;
        return __builtin_fmaxf16(t.x, t.y) >= th; // one compare: its lane mask is the ballot
    }
    __device__ static float first(const uint4 &d) { return (float)__builtin_bit_cast(_Float16, (uint16_t)d.x); }
    __device__ static void shift(uint4 &d) { shift16(d); }
};

template <> struct Traits<2> { // bfloat16: widened to fp32 by a shift or a mask
    static constexpr int epv = 8;
    struct Acc {
        float v[8];
    };
    __device__ static uint4 neg_inf() { return make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u); }
    __device__ static float elem(const uint4 &d, int i)
    {
        uint32_t w = word(d, i >> 1);
        return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    __device__ static float elem_rt(const uint4 &d, int i) { return elem(d, i); }
    __device__ static void mask_if(uint4 &d, int i, bool m)
    {
        const uint32_t w = word(d, i >> 1);
        const uint32_t mw = (i & 1) ? ((w & 0x0000ffffu) | 0xff800000u) : ((w & 0xffff0000u) | 0x0000ff80u);
        set_word(d, i >> 1, m ? mw : w);
    }
    __device__ static void init(Acc &a)
    {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            a.v[i] = -INFINITY;
    }
    __device__ static void update(Acc &a, const uint4 &d)
    {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            a.v[i] = fmaxf(a.v[i], elem(d, i));
    }
    __device__ static float amax(const Acc &a)
    {
        float m = a.v[0];
#pragma unroll
        for (int i = 1; i < 8; ++i)
            m = fmaxf(m, a.v[i]);
        return m;
    }
    __device__ static void order_after(Acc &a, float x, float y)
    {
        asm volatile("" : "+v"(a.v[0]), "+v"(a.v[1]), "+v"(a.v[2]), "+v"(a.v[3]), "+v"(a.v[4]), "+v"(a.v[5]),
                     "+v"(a.v[6]), "+v"(a.v[7]) : "v"(x), "v"(y));
    }
    __device__ static void slots(const Acc &a, float *s)
    {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            s[i] = a.v[i];
    }
    __device__ static bool any_ge(const uint4 &d, float T)
    {
        float m = elem(d, 0);
#pragma unroll
        for (int i = 1; i < 8; ++i)
            m = fmaxf(m, elem(d, i));
        return m >= T;
    }
    __device__ static float first(const uint4 &d) { return __uint_as_float(d.x << 16); }
    __device__ static void shift(uint4 &d) { shift16(d); }
};

// d[r] for a wave-uniform r, by selects (no indexing of the register array).
template <int NV> __device__ __forceinline__ uint4 pick(const uint4 (&d)[NV], int r)
{
    uint4 v = d[0];
#pragma unroll
    for (int i = 1; i < NV; ++i) {
        const bool s = r == i;
        v.x = s ? d[i].x : v.x;
        v.y = s ? d[i].y : v.y;
        v.z = s ? d[i].z : v.z;
        v.w = s ? d[i].w : v.w;
    }
    return v;
}

// ------------------------------------------------------------ passes 1 and 2
// Read in place of the finished mask when there is none (0), or in place of a
// piece past the end of the grid (1), so that the flag load needs no branch.
__device__ uint8_t kFlagConst[2] = {0, 1}; // global memory, like the mask: a global (not flat) load

// Hides the staged vectors' values from the optimiser, so that pass 2
// re-derives what it needs from the packed data instead of keeping every
// converted element of pass 1 alive in registers.
__device__ __forceinline__ void opaque(uint4 &v)
{
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// Rows that start on a 16-byte boundary (kAligned): only slots past a
// piece's end need masking. Rows that share their first/last 16-byte vector
// with a neighbour row (kGeneral) are masked element by element.
enum PieceMode { kAligned = 0, kGeneral = 1 };

// LDS of the selection phase: the piece's candidates, one entry per lane;

// Cache policy of the logit loads: non-temporal (the NT bit of gfx950's
// buffer instructions).
constexpr int kBufNT = 2;

// The arrival counter of batch element b. Counters of consecutive batch
// elements lie in different 64-byte lines (16 counters per line, b mod 4096
// picks the line): their atomics then never queue behind each other's at the
// memory side. A bijection on [0, kTicketCap).
__device__ __forceinline__ uint32_t *ticket_of(const StepArgs &a, int b)
{
    static_assert(kTicketCap == 65536, "4096 lines of 16 counters");
    return a.ticket + ((((uint32_t)b & 4095u) << 4) | ((uint32_t)b >> 12));
}

// in row-local workgroups also the piece's published top-k and header.
struct SelectLds {
    uint64_t stage[2 * kLanes]; // a piece's staged candidates (up to kMaxChunkLimit)
    uint64_t top[kMaxK];
    float hm, hs, ht; // lse partial (max2, sum) and threshold
    uint32_t hemit;   // keys in top
    float ha;         // the row's running score
    uint32_t hf;      // the row's finished flag
    uint32_t pad[2];
};
static_assert(sizeof(SelectLds) % 16 == 0, "per-wave LDS regions stay 16-byte aligned");

// One wave's piece between its loads and its computation: the 16-byte vectors
// in flight and the wave-uniform facts about the piece.
template <int NV> struct Piece {
    uint4 d[NV];
    uint32_t fin;     // the row's finished flag (1 past the last piece)
    float alv;        // the row's running score (row-local kernels)
    uint32_t row, flat0;
    int lead, pbeg, pend;
    uint32_t *gshare; // the row's shared group maxima
};

// Issues the loads of piece u (wave-uniform); row0: the first row of the
// workgroup.
template <int DT, int NV, bool RL>
__device__ __forceinline__ void piece_load(const StepArgs &a, Piece<NV> &P, uint32_t *gshare_rows, uint32_t u,
                                           bool valid, uint32_t row0, int lane)
{
    using Tr = Traits<DT>;
    constexpr int EPV = Tr::epv;
    // Everything about the piece is wave-uniform scalar work, divisions by
    // multiplication: the loads issue after a few instructions.
    const uint32_t uu = valid ? u : row0 * (uint32_t)a.chunks;
    const uint32_t row = mdiv(uu, a.mc);
    const int cr = (int)(uu - row * (uint32_t)a.chunks); // piece of the row
    const int g = (int)mdiv((uint32_t)cr, a.ms);          // its vocabulary shard
    const int c = cr - g * a.cps;                         // piece of the shard's row
    const int j = (int)(row - mdiv(row, a.mb) * (uint32_t)a.beam);
    P.row = row;
    // this row's shared group maxima (rows are counted from the workgroup's first)
    P.gshare = gshare_rows + (row - row0) * kMaxK;
    // Vectors are counted in the 16-byte-aligned frame of the tensor; a row
    // starts `lead` elements into its first vector v0 and spans `span` vectors.
    // Everything per lane is 32-bit and relative to the row.
    const int VS = a.vshard; // logits of this row in its shard (V when unsharded)
    const uint64_t e0 = (uint64_t)row * (uint32_t)VS + (uint32_t)a.align_elems;
    const uint64_t v0 = e0 / EPV;
    const int lead = (int)(e0 - v0 * EPV);
    const int span = (lead + VS + EPV - 1) / EPV;
    const int pbeg = c * a.vecs_per_chunk; // piece start, vectors from v0
    const int pend = pbeg + a.vecs_per_chunk < span ? pbeg + a.vecs_per_chunk : span;
    P.lead = lead;
    P.pbeg = pbeg;
    P.pend = pend;
    // flat index j*V + vocabulary index of slot 0 of vector 0
    P.flat0 = (uint32_t)j * (uint32_t)a.V + (uint32_t)g * (uint32_t)VS - (uint32_t)lead;

    // The finished flag is loaded first and sizes the piece's descriptor: a
    // finished row's loads read nothing (its logits never leave HBM), at the
    // price of waiting for the flag before the stream starts. Measured on the
    // 128 x 4 x 40000 step: the same time as loading first and testing later,
    // with 2.1 MB less traffic per launch.
    const uint8_t *finp = !valid ? &kFlagConst[1] : a.finished != nullptr ? &a.finished[row] : &kFlagConst[0];
    P.fin = *finp;
    // row-local workgroups select their rows themselves: the row's score is
    // loaded here too, its latency hidden under the stream like the flag's
    P.alv = 0.f;
    if constexpr (RL)
        P.alv = a.alive[row];
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // Buffer loads through a descriptor that spans exactly the piece: a slot
    // past its end reads 0 without touching memory, so the loads need no
    // clamp and no 64-bit address per lane, and stay unconditional (each
    // load's distance to its use visible to the waitcnt pass); such slots are
    // overwritten with -inf at their use. A wave past the last piece gets an
    // empty descriptor. The loads are non-temporal: the stream is read once,
    // and without the hint it evicts from the L2s the code and workspace
    // lines the end of the step needs.
    const uint32_t nbytes = valid && pend > pbeg && P.fin == 0 ? (uint32_t)(pend - pbeg) * 16u : 0u;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.shard[g]) + (v0 + (uint64_t)pbeg) * 16u, 0, nbytes, 0x00020000);
#pragma unroll
    for (int r = 0; r < NV; ++r) {
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane * 16, r * kLanes * 16, kBufNT);
        P.d[r] = make_uint4(w.x, w.y, w.z, w.w);
    }
}

// Passes 1 and 2 of piece u over the vectors piece_load issued, and its top-k.
template <int DT, int NV, int MODE, bool RL>
__device__ __forceinline__ void piece_compute(const StepArgs &a, SelectLds &sm, Piece<NV> &P, uint32_t u, int lane)
{
    using Tr = Traits<DT>;
    constexpr int EPV = Tr::epv;
    uint4 (&d)[NV] = P.d;
    const uint32_t row = P.row;
    const int lead = P.lead, pbeg = P.pbeg, pend = P.pend, VS = a.vshard;
    const uint32_t flat0 = P.flat0;
    uint32_t *gshare = P.gshare;
    const float alv = P.alv;
    uint32_t fin = P.fin;
    asm volatile("" : "+v"(fin)); // the test waits for the flag here, past the loads
    if (fin != 0) {
        if (RL && lane == 0) { // an empty piece for the workgroup's own selection
            sm.hm = -INFINITY;
            sm.hs = 0.f;
            sm.ht = -INFINITY;
            sm.hemit = 0;
            sm.ha = alv;
            sm.hf = 1;
        }
        return;
    }
    // slots r < nfull hold valid vectors in every lane
    const int nfull = pend > pbeg ? (pend - pbeg) / kLanes : 0;

    // ---- pass 1: slot maxima + online log-sum-exp (base 2), one block of
    // kBlock vectors at a time so that the work follows the arriving data
    typename Tr::Acc acc;
    Tr::init(acc);
    float m2 = -INFINITY, s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int r0 = 0; r0 < NV; r0 += kBlock) {
        // The previous block's sums become inputs of this block's maxima: the
        // compiler cannot hoist every block's max ahead of all exponentials,
        // so each block is finished while later vectors are still in flight.
        Tr::order_after(acc, s0, s1);
#pragma unroll
        for (int r = r0; r < r0 + kBlock && r < NV; ++r) {
            const int q = pbeg + lane + r * kLanes;
            if (MODE == kAligned) {
                if (r >= nfull) { // uniform: never taken in a piece that fills its slots
                    const bool ok = q < pend;
                    const uint4 ni = Tr::neg_inf();
                    d[r].x = ok ? d[r].x : ni.x;
                    d[r].y = ok ? d[r].y : ni.y;
                    d[r].z = ok ? d[r].z : ni.z;
                    d[r].w = ok ? d[r].w : ni.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < EPV; ++i) {
                    const int t = q * EPV + i - lead;
                    Tr::mask_if(d[r], i, q >= pend || t < 0 || t >= VS);
                }
            }
            Tr::update(acc, d[r]);
        }
        const float nb = Tr::amax(acc) * kLog2e;
        const float f = (nb == m2) ? 1.f : fast_exp2(m2 - nb);
        s0 *= f;
        s1 *= f;
        m2 = nb;
        const float base = nb == -INFINITY ? 0.f : nb;
#pragma unroll
        for (int r = r0; r < r0 + kBlock && r < NV; ++r) {
#pragma unroll
            for (int i = 0; i < EPV; i += 2) {
                s0 += fast_exp2(fmaf(Tr::elem(d[r], i), kLog2e, -base));
                s1 += fast_exp2(fmaf(Tr::elem(d[r], i + 1), kLog2e, -base));
            }
        }
    }
    const float tmax = Tr::amax(acc);

    // ---- the piece's log-sum-exp partial: wave maximum, one rescale per lane, a sum
    const float pm = wave_max_f(m2);
    const float ps = wave_sum_f((pm == -INFINITY) ? 0.f : (s0 + s1) * fast_exp2(m2 - pm));

    // ---- threshold. Slot i of a lane holds elements e = i mod EPV; folding
    // slots i and i + h for h >= F = min(ngroups, EPV) leaves slot f with
    // group f of this lane (ngroups <= EPV), or with group f of the lane's
    // class lane mod D, D = ngroups / EPV (ngroups > EPV): pieces start on
    // multiples of 64 vectors, so a vector's first element is lane mod D
    // groups of EPV away from a multiple of ngroups.
    float slot[EPV];
    Tr::slots(acc, slot);
    const int ng = a.ngroups;
    const int F = ng < EPV ? ng : EPV;
    const int D = ng / F;
#pragma unroll
    for (int h = EPV / 2; h >= 1; h >>= 1) {
        if (h >= F) {
#pragma unroll
            for (int i = 0; i < h; ++i)
                slot[i] = fmaxf(slot[i], slot[i + h]);
        }
    }
    // The R-top-k bound holds for any set of a row's logits: the k-th
    // largest of its group maxima is at most its own k-th largest logit, so at
    // most the row's. So the waves of a row share their group maxima in LDS
    // (atomic max on order-preserving bits) and each takes the threshold of
    // everything its row has published so far, itself included: the later
    // waves of a row filter with nearly the whole row's R-top-k.
    if (D == 1) {
#pragma unroll
        for (int f = 0; f < EPV; ++f) {
            if (f < F) {
                const float v = row16_max_f(slot[f]); // each 16-lane row's maximum
                if ((lane & 15) == 0)
                    atomicMax(&gshare[f], ord_bits(v));
            }
        }
    } else {
        // lanes l and l' hold the same groups iff l = l' mod D: butterflies over
        // distances >= D leave lane l < D with groups l*F .. l*F + F - 1
#pragma unroll
        for (int f = 0; f < EPV; ++f) {
            for (int dd = 32; dd >= D; dd >>= 1)
                slot[f] = fmaxf(slot[f], __shfl_xor(slot[f], dd));
            if (lane < D)
                atomicMax(&gshare[lane * F + f], ord_bits(slot[f]));
        }
    }
    wave_sync();
    // One read per lane is the snapshot; each value is a group maximum over a
    // subset of the row that contains this piece, which keeps the threshold
    // below the row's k-th largest logit whatever the other waves do meanwhile.
    const float cur = lane < ng ? from_ord(gshare[lane]) : INFINITY;
    float T;
    if (ng == a.k) { // the R-top-k: the least group maximum
        T = wave_min_f(cur);
    } else { // k below a power of two: the k-th largest of the ngroups maxima,
        // the largest t (order-preserving bits) that at least k of them reach,
        // found bit by bit from the top with one compare and ballot per bit
        const uint32_t o = lane < ng ? ord_bits(cur) : 0u;
        uint32_t t = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t c = t | (1u << bit);
            if (__builtin_popcountll(ballot(o >= c)) >= a.k)
                t = c;
        }
        T = from_ord(t);
    }

    // ---- pass 2: stage the sort key of every valid logit >= T. The wave
    // tests each of its vectors with one packed maximum; only a vector in
    // which some lane holds a hit (a wave-uniform branch, usually taken once
    // or twice per piece) is examined element by element: one compare per
    // element straight into a lane mask, and only the elements that hit
    // somewhere are staged. Hits are ranked by ballot + mbcnt, so the count is
    // wave-uniform and no atomics are needed. With T finite, slots outside
    // the row or piece (set to -inf in pass 1) cannot reach it. T = -inf (a
    // piece without k finite logits) is rare and takes a compact rolled loop
    // that checks each element's position.
    const uint32_t cap = (uint32_t)a.chunk_limit;
    auto in_piece = [&](int q, int e) { // vector q (from v0), element e of the aligned frame
        const int t = e - lead;
        return q < pend && (MODE != kGeneral || (t >= 0 && t < VS));
    };
    uint32_t wn = 0;
    if (ballot(tmax >= T) != 0) {
        int qb0 = pbeg + lane; // opaque: keeps per-element index math inside this block
        asm volatile("" : "+v"(qb0));
        if (T > -INFINITY) {
            // per vector, the lanes holding a hit: in row-local kernels all the
            // (independent) compares first; the others, whose tail already fills
            // the registers, test each vector as they go
            uint64_t vm[NV];
            if constexpr (RL) {
#pragma unroll
                for (int r = 0; r < NV; ++r) {
                    opaque(d[r]);
                    vm[r] = ballot(Tr::any_ge(d[r], T));
                }
            }
#pragma unroll
            for (int r = 0; r < NV; ++r) {
                if constexpr (!RL) {
                    opaque(d[r]);
                    vm[r] = ballot(Tr::any_ge(d[r], T));
                }
                if (vm[r] != 0) {
                    const int q = qb0 + r * kLanes;
                    uint64_t mk[EPV];
#pragma unroll
                    for (int i = 0; i < EPV; ++i)
                        mk[i] = ballot(Tr::elem(d[r], i) >= T);
#pragma unroll
                    for (int i = 0; i < EPV; ++i) {
                        if (mk[i] != 0) {
                            const uint32_t pos = wn + lane_prefix(mk[i]);
                            if (((mk[i] >> lane) & 1u) && pos < cap)
                                sm.stage[pos] = score_key(Tr::elem(d[r], i), flat0 + (uint32_t)(q * EPV + i));
                            wn += (uint32_t)__builtin_popcountll(mk[i]);
                        }
                    }
                }
            }
        } else {
#pragma unroll 1
            for (int r = 0; r < NV; ++r) {
                uint4 w = pick(d, r);
                const int q = qb0 + r * kLanes;
#pragma unroll 1
                for (int i = 0, e = q * EPV; i < EPV; ++i, ++e) {
                    const float x = Tr::first(w);
                    Tr::shift(w);
                    const bool h = x >= T && in_piece(q, e);
                    const uint64_t m = ballot(h);
                    if (m != 0) {
                        const uint32_t pos = wn + lane_prefix(m);
                        if (h && pos < cap)
                            sm.stage[pos] = score_key(x, flat0 + (uint32_t)e);
                        wn += (uint32_t)__builtin_popcountll(m);
                    }
                }
            }
        }
    }
    wave_sync();

    // ---- more hits than the stage holds (heavy ties): find v, the piece's
    // k-th largest logit counted with multiplicity, by walking its distinct
    // values down from the top (one round when the top value repeats k
    // times); then stage every logit > v and the first k - #(> v) logits == v
    // in flat order (vectors, then lanes, then elements). That is exactly the
    // piece's top-k by (logit desc, flat asc). A rare path: rolled loops.
    uint32_t nst = wn; // staged keys
    if (wn > cap) {
        float prev = INFINITY, v = -INFINITY;
        uint32_t above = 0;
        for (int round = 0; round < a.k; ++round) { // wn > cap >= k valid logits are >= T
            float mx = -INFINITY;
#pragma unroll 1
            for (int r = 0; r < NV; ++r) {
                uint4 w = pick(d, r);
                const int q = pbeg + lane + r * kLanes;
#pragma unroll 1
                for (int i = 0, e = q * EPV; i < EPV; ++i, ++e) {
                    const float x = Tr::first(w);
                    Tr::shift(w);
                    mx = in_piece(q, e) && x < prev ? fmaxf(mx, x) : mx;
                }
            }
            v = wave_max_f(mx);
            uint32_t c = 0;
#pragma unroll 1
            for (int r = 0; r < NV; ++r) {
                uint4 w = pick(d, r);
                const int q = pbeg + lane + r * kLanes;
#pragma unroll 1
                for (int i = 0, e = q * EPV; i < EPV; ++i, ++e) {
                    c += in_piece(q, e) && Tr::first(w) == v;
                    Tr::shift(w);
                }
            }
            c = wave_sum_u32(c);
            if (above + c >= (uint32_t)a.k)
                break;
            above += c;
            prev = v;
        }
        nst = 0;
#pragma unroll 1
        for (int r = 0; r < NV; ++r) { // the logits > v (fewer than k)
            uint4 w = pick(d, r);
            const int q = pbeg + lane + r * kLanes;
#pragma unroll 1
            for (int i = 0, e = q * EPV; i < EPV; ++i, ++e) {
                const float x = Tr::first(w);
                Tr::shift(w);
                const bool h = in_piece(q, e) && x > v;
                const uint64_t m = ballot(h);
                if (m != 0) {
                    if (h)
                        sm.stage[nst + lane_prefix(m)] = score_key(x, flat0 + (uint32_t)e);
                    nst += (uint32_t)__builtin_popcountll(m);
                }
            }
        }
        uint32_t need = (uint32_t)a.k - above;
#pragma unroll 1
        for (int r = 0; r < NV && need != 0; ++r) { // the first `need` logits == v
            const uint4 w0 = pick(d, r);
            const int q = pbeg + lane + r * kLanes;
            uint4 w = w0;
            uint32_t bits = 0;
#pragma unroll 1
            for (int i = 0, e = q * EPV; i < EPV; ++i, ++e) {
                bits |= (uint32_t)(in_piece(q, e) && Tr::first(w) == v) << i;
                Tr::shift(w);
            }
            const uint32_t cnt = (uint32_t)__builtin_popcount(bits);
            const uint32_t before = wave_excl_scan_u32(cnt, lane);
            const uint32_t total = first_u32(__builtin_amdgcn_readlane(before + cnt, 63));
            w = w0;
#pragma unroll 1
            for (int i = 0, e = q * EPV; i < EPV; ++i, ++e) {
                const uint32_t rank = before + (uint32_t)__builtin_popcount(bits & ((1u << i) - 1u));
                if (((bits >> i) & 1u) && rank < need)
                    sm.stage[nst + rank] = score_key(Tr::first(w), flat0 + (uint32_t)e);
                Tr::shift(w);
            }
            const uint32_t took = total < need ? total : need;
            nst += took;
            need -= took;
        }
        wave_sync();
    }

    // ---- publish this piece's own top-min(hits, k) by (logit desc, flat
    // asc), in no particular slot order: only those can be among the batch
    // element's top-k. Keys are distinct, so ranks are unique.
    uint64_t *mine = a.slots + (long long)u * a.k;
    const uint32_t emit = nst < (uint32_t)a.k ? nst : (uint32_t)a.k;
    // up to two staged keys per lane (lane, lane + 64), ranked among all nst
    uint64_t key = 0, key2 = 0;
    uint32_t rank = ~0u, rank2 = ~0u;
    if ((uint32_t)lane < nst) {
        key = sm.stage[lane];
        rank = lane;
    }
    if ((uint32_t)lane + kLanes < nst) {
        key2 = sm.stage[lane + kLanes];
        rank2 = lane + kLanes;
    }
    if (nst > (uint32_t)kLanes) { // uniform: the second half of the stage is in use
        uint32_t r1 = 0, r2 = 0;
#pragma unroll 8
        for (uint32_t i = 0; i < nst; ++i) {
            const uint64_t x = sm.stage[i];
            r1 += x > key;
            r2 += x > key2;
        }
        rank = (uint32_t)lane < nst ? r1 : ~0u;
        rank2 = (uint32_t)lane + kLanes < nst ? r2 : ~0u;
    } else if (nst > (uint32_t)a.k && (uint32_t)lane < nst) {
        rank = 0;
#pragma unroll 8
        for (uint32_t i = 0; i < nst; ++i)
            rank += sm.stage[i] > key;
    }
    if (RL) {
        // The workgroup holds whole rows and selects them itself: the piece's
        // top-k and header stay in LDS; nothing to store or drain.
        if (rank < (uint32_t)a.k)
            sm.top[rank] = key;
        if (rank2 < (uint32_t)a.k)
            sm.top[rank2] = key2;
        if (lane == 0) {
            sm.hm = pm;
            sm.hs = ps;
            sm.ht = T;
            sm.hemit = emit;
            sm.ha = alv;
            sm.hf = 0;
            if (a.dbg_T)
                a.dbg_T[u] = T;
            if (a.dbg_hits)
                a.dbg_hits[u] = wn;
        }
        if (a.dbg_count) { // debug: append to the batch element's queue
            const int b = row / a.beam;
            if (rank < (uint32_t)a.k) {
                const uint32_t pos = atomicAdd(&a.dbg_count[b], 1u);
                if (a.dbg_queue)
                    a.dbg_queue[(long long)b * a.queue_cap + pos] =
                        ((uint64_t)__float_as_uint(entry_x(key)) << 32) | entry_flat(key);
            }
            if (rank2 < (uint32_t)a.k) {
                const uint32_t pos = atomicAdd(&a.dbg_count[b], 1u);
                if (a.dbg_queue)
                    a.dbg_queue[(long long)b * a.queue_cap + pos] =
                        ((uint64_t)__float_as_uint(entry_x(key2)) << 32) | entry_flat(key2);
            }
        }
        return;
    }
    if (rank < (uint32_t)a.k)
        put64(&mine[rank], key);
    if (rank2 < (uint32_t)a.k)
        put64(&mine[rank2], key2);
    if (lane == 0) {
        put64(&a.head[2 * (long long)u], ((uint64_t)__float_as_uint(ps) << 32) | __float_as_uint(pm));
        put64(&a.head[2 * (long long)u + 1], ((uint64_t)emit << 32) | __float_as_uint(T));
        if (a.dbg_T)
            a.dbg_T[u] = T;
        if (a.dbg_hits)
            a.dbg_hits[u] = wn;
    }
    // every store of this wave is performed before it takes its ticket
    drain_stores();
}

// ------------------------------------------------------------ per-batch selection
// LDS of the selection of batch element b, laid out by the host: sort keys,
// per-piece partials, per-beam tables, per-piece candidate counts.
struct SortLds {
    uint64_t *keys;           // [sort_keys]
    float *pm, *ps, *pt;      // [pieces] max2, sum, threshold of each piece
    float *lse, *thr, *alive; // [beam]
    uint8_t *pn;              // [pieces] candidates each piece published
    uint8_t *fin;             // [beam] finished flags
};

// Counters and reduction scratch of a workgroup, in front of its LDS.
struct GroupLds {
    uint32_t todo[2]; // batch elements whose ticket this workgroup completed
    uint32_t ns, ndbg;
    float fred[kMaxWaves];
    uint64_t kred[kMaxWaves];
};

static_assert(sizeof(GroupLds) <= kLdsShare, "GroupLds fits in front of the shared group maxima");

// The selection runs on the whole workgroup (W waves) or on wave 0 alone (W
// = 1, its siblings gone): a workgroup barrier or just the wave's own order.
__device__ __forceinline__ void group_sync(int W)
{
    if (W == 1)
        wave_sync();
    else
        lds_barrier();
}

__device__ __forceinline__ SortLds sort_lds(uint8_t *base, const StepArgs &a)
{
    const int P = a.beam * a.chunks;
    SortLds sm;
    sm.keys = reinterpret_cast<uint64_t *>(base);
    sm.pm = reinterpret_cast<float *>(base + 8 * (size_t)a.sort_keys);
    sm.ps = sm.pm + P;
    sm.pt = sm.ps + P;
    sm.lse = sm.pt + P;
    sm.thr = sm.lse + a.beam;
    sm.alive = sm.thr + a.beam;
    sm.pn = reinterpret_cast<uint8_t *>(sm.alive + a.beam);
    sm.fin = sm.pn + P;
    return sm;
}

// Workgroup-wide maxima (every wave of the workgroup takes part).
__device__ __forceinline__ float block_max_f(float v, GroupLds &g, int lane, int wave, int W)
{
    v = wave_max_f(v);
    if (lane == 0)
        g.fred[wave] = v;
    group_sync(W);
    float r = g.fred[0];
    for (int w = 1; w < W; ++w)
        r = fmaxf(r, g.fred[w]);
    group_sync(W);
    return r;
}
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, GroupLds &g, int lane, int wave, int W)
{
    v = wave_max_u64(v);
    if (lane == 0)
        g.kred[wave] = v;
    group_sync(W);
    uint64_t r = g.kred[0];
    for (int w = 1; w < W; ++w)
        r = g.kred[w] > r ? g.kred[w] : r;
    group_sync(W);
    return r;
}

// Descending bitonic sort of keys[0..P), P a power of two, whole workgroup.
__device__ __forceinline__ void bitonic_desc(uint64_t *keys, int P, int tid, int nth)
{
    const int W = nth / kLanes;
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < (P >> 1); i += nth) {
                int lo = 2 * i - (i & (stride - 1));
                int hi = lo + stride;
                bool desc = (lo & size) == 0;
                uint64_t x = keys[lo], y = keys[hi];
                if ((x < y) == desc) {
                    keys[lo] = y;
                    keys[hi] = x;
                }
            }
            group_sync(W);
        }
    }
}

// Run by the whole workgroup that completed the ticket of batch element b. One
// round trip loads every piece header, the beams' flags and scores and the
// first kSpec*threads published candidates; each beam's partials are merged
// by a fixed binary tree over its pieces; candidates are filtered by the
// per-beam threshold and the batch bound and ranked into LDS by ballot; the k
// best survivors are found by rank counting (a bitonic sort when many).
__device__ __forceinline__ void sort_batch(const StepArgs &a, const SortLds &sm, GroupLds &g, int b, int tid, int W)
{
    const int lane = tid & (kLanes - 1), wave = tid / kLanes, nth = W * kLanes;
    const int beam = a.beam, C = a.chunks, L = a.k;
    const int P = beam * C, NS = P * L; // pieces and published slots of b
    const uint64_t *slots = a.slots + (long long)b * NS;
    const uint64_t *head = a.head + 2 * (long long)b * P;
    const uint32_t K = (uint32_t)a.sort_keys;
    const bool has_fin = a.finished != nullptr;
    const uint8_t *finb = has_fin ? a.finished + (long long)b * beam : nullptr;
    const float invC = 1.f / (float)C, invL = 1.f / (float)L;

    // ---- A: speculative slot loads, every header, the beams' flags and
    // scores, all in flight at once. A finished beam published nothing this
    // call: its stale partials are merged and ignored, its counts zeroed.
    constexpr int kSpec = 4;
    uint64_t spec[kSpec];
#pragma unroll
    for (int r = 0; r < kSpec; ++r) {
        const int gi = tid + r * nth;
        spec[r] = gi < NS ? get64(&slots[gi]) : 0ull;
    }
    if (tid == 0) {
        g.ns = 0;
        g.ndbg = 0;
    }
    for (int jj = tid; jj < beam; jj += nth) {
        sm.alive[jj] = a.alive[b * beam + jj];
        sm.fin[jj] = has_fin ? finb[jj] : 0;
    }
    for (int p0 = 0; p0 < P; p0 += 2 * nth) {
        uint64_t hb[4];
        uint32_t fb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int p = p0 + tid + i * nth;
            hb[2 * i] = p < P ? get64(&head[2 * p]) : 0ull;
            hb[2 * i + 1] = p < P ? get64(&head[2 * p + 1]) : 0ull;
            fb[i] = p < P && has_fin ? finb[small_div(p, invC)] : 0u;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int p = p0 + tid + i * nth;
            if (p < P) {
                sm.pm[p] = __uint_as_float((uint32_t)hb[2 * i]);
                sm.ps[p] = __uint_as_float((uint32_t)(hb[2 * i] >> 32));
                sm.pt[p] = __uint_as_float((uint32_t)hb[2 * i + 1]);
                sm.pn[p] = fb[i] ? 0 : (uint8_t)(hb[2 * i + 1] >> 32);
            }
        }
    }
    // each beam's pieces merged pairwise at doubling distances: a fixed tree,
    // so the result does not depend on arrival order
    for (int stride = 1; stride < C; stride <<= 1) {
        group_sync(W);
        for (int p = tid; p < P; p += nth) {
            const int c = p - small_div(p, invC) * C;
            if ((c & (2 * stride - 1)) == 0 && c + stride < C) {
                float m = sm.pm[p], sum = sm.ps[p];
                lse_merge(m, sum, sm.pm[p + stride], sm.ps[p + stride]);
                sm.pm[p] = m;
                sm.ps[p] = sum;
                sm.pt[p] = fmaxf(sm.pt[p], sm.pt[p + stride]);
            }
        }
    }
    group_sync(W);
    float bound = -INFINITY;
    for (int jj = tid; jj < beam; jj += nth) {
        const float alv = sm.alive[jj];
        float lse = 0.f, thr = INFINITY; // a finished beam's thr keeps its slots out
        if (!sm.fin[jj]) {
            lse = (sm.pm[jj * C] + fast_log2(sm.ps[jj * C])) * kLn2;
            thr = sm.pt[jj * C];
            // at least k logits of this beam are >= thr, so at least k
            // candidates score >= alive + (thr - lse)
            bound = fmaxf(bound, alv + (thr - lse));
        }
        sm.lse[jj] = lse;
        sm.thr[jj] = thr;
        if (a.dbg_lse) // NaN bits mark a finished beam
            reinterpret_cast<uint32_t *>(a.dbg_lse)[b * beam + jj] = sm.fin[jj] ? 0x7fc00000u : __float_as_uint(lse);
    }
    bound = block_max_f(bound, g, lane, wave, W); // its barriers also publish the tables

    // ---- B: survivors -> sort keys, ranked into LDS by ballot, one LDS atomic per wave
    auto offer = [&](bool ok, uint64_t key) {
        const uint64_t m = ballot(ok);
        if (m != 0) {
            uint32_t base = 0;
            if (lane == 0)
                base = atomicAdd(&g.ns, (uint32_t)__builtin_popcountll(m));
            const uint32_t pos = first_u32(base) + lane_prefix(m);
            if (ok && pos < K)
                sm.keys[pos] = key;
        }
    };
    auto survivor = [&](int gi, uint64_t ent, uint64_t &key) {
        const int p = small_div(gi, invL);
        if (gi - p * L >= (int)sm.pn[p]) // slots past a piece's count hold stale data
            return false;
        const int jj = small_div(p, invC);
        const float x = entry_x(ent);
        if (!(x >= sm.thr[jj]))
            return false;
        const float sc = sm.alive[jj] + (x - sm.lse[jj]);
        key = score_key(sc, entry_flat(ent));
        return sc >= bound;
    };
#pragma unroll
    for (int r = 0; r < kSpec; ++r) {
        const int gi = tid + r * nth;
        uint64_t key = 0;
        const bool ok = gi < NS && survivor(gi, spec[r], key);
        offer(ok, key);
    }
    for (int g0 = kSpec * nth; g0 < NS; g0 += 4 * nth) { // 4 loads per thread in flight
        uint64_t eb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int gi = g0 + tid + i * nth;
            eb[i] = gi < NS ? get64(&slots[gi]) : 0ull;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int gi = g0 + tid + i * nth;
            uint64_t key = 0;
            const bool ok = gi < NS && survivor(gi, eb[i], key);
            offer(ok, key);
        }
    }
    if (has_fin) {
        for (int j0 = 0; j0 < beam; j0 += nth) {
            const int jj = j0 + tid;
            const bool ok = jj < beam && sm.fin[jj] && sm.alive[jj] >= bound;
            const uint64_t key = ok ? score_key(sm.alive[jj], (uint32_t)jj * (uint32_t)a.V + (uint32_t)a.eos_id) : 0ull;
            offer(ok, key);
        }
    }
    group_sync(W);
    const uint32_t ns = g.ns;

    // ---- D: the k best keys, in order
    auto emit_out = [&](int p, uint64_t key) {
        const long long o = (long long)b * a.k + p;
        const uint32_t flat = 0xffffffffu - (uint32_t)key;
        const uint32_t jj = flat / (uint32_t)a.V;
        a.out_beam[o] = (int32_t)jj;
        a.out_token[o] = (int32_t)(flat - jj * (uint32_t)a.V);
        a.out_score[o] = from_ord((uint32_t)(key >> 32));
    };
    if (ns <= (uint32_t)nth && ns <= K) {
        // rank counting: keys are distinct (flat indices are), so ranks are a permutation
        // (only keys that fit the LDS were staged: more survivors take the argmax rounds)
        if ((uint32_t)tid < ns) {
            const uint64_t mine = sm.keys[tid];
            uint32_t rank = 0;
#pragma unroll 8
            for (uint32_t i = 0; i < ns; ++i)
                rank += sm.keys[i] > mine;
            if (rank < (uint32_t)a.k)
                emit_out((int)rank, mine);
        }
    } else if (ns <= K) {
        int Pw = 2;
        while ((uint32_t)Pw < ns)
            Pw <<= 1;
        for (int i = (int)ns + tid; i < Pw; i += nth)
            sm.keys[i] = 0ull; // below every real key
        group_sync(W);
        bitonic_desc(sm.keys, Pw, tid, nth);
        for (int p = tid; p < a.k && (uint32_t)p < ns; p += nth)
            emit_out(p, sm.keys[p]);
    } else {
        // more survivors than the LDS holds: k rounds of workgroup argmax over every candidate
        uint64_t prev = ~0ull;
        for (int round = 0; round < a.k; ++round) {
            uint64_t best = 0;
            for (int gi = tid; gi < NS; gi += nth) {
                uint64_t key = 0;
                if (survivor(gi, get64(&slots[gi]), key) && key < prev && key > best)
                    best = key;
            }
            if (has_fin) {
                for (int jj = tid; jj < beam; jj += nth) {
                    if (sm.fin[jj] && sm.alive[jj] >= bound) {
                        const uint64_t key =
                            score_key(sm.alive[jj], (uint32_t)jj * (uint32_t)a.V + (uint32_t)a.eos_id);
                        if (key < prev && key > best)
                            best = key;
                    }
                }
            }
            best = block_max_u64(best, g, lane, wave, W);
            prev = best;
            if (tid == 0 && best != 0ull)
                emit_out(round, best);
        }
    }
    // padding when fewer than k candidates exist at all
    for (int p = (int)ns + tid; p < a.k; p += nth) {
        const long long o = (long long)b * a.k + p;
        a.out_beam[o] = -1;
        a.out_token[o] = -1;
        a.out_score[o] = -INFINITY;
    }

    // ---- E: debug copies; the ticket goes back to zero for the next call. Headers
    // and slots need no clearing: every piece of an alive beam rewrites its
    // header before its arrival is counted, and slots are read only below a count.
    if (a.dbg_queue || a.dbg_count) {
        group_sync(W);
        uint64_t *dq = a.dbg_queue ? a.dbg_queue + (long long)b * a.queue_cap : nullptr;
        for (int p = tid; p < P; p += nth) {
            const int n = (int)sm.pn[p];
            const uint32_t base = atomicAdd(&g.ndbg, (uint32_t)n);
            if (dq)
                for (int e = 0; e < n; ++e) {
                    const uint64_t ent = get64(&slots[(long long)p * L + e]);
                    dq[base + e] = ((uint64_t)__float_as_uint(entry_x(ent)) << 32) | entry_flat(ent);
                }
        }
        group_sync(W);
        if (tid == 0 && a.dbg_count)
            a.dbg_count[b] = g.ndbg;
    }
    if (tid == 0)
        put32(ticket_of(a, b), 0u);
}

// DPP partner exchange for the in-register merge tree of the wave selection:
// level 0 pairs lanes i ^ 1, level 1 pairs i ^ 2 (quad permutes), level 2
// mirrors 8-lane halves, level 3 mirrors 16-lane rows. After levels 0..L-1
// every lane of an aligned 2^L-lane segment has combined the whole segment.
template <int LEVEL> __device__ __forceinline__ uint32_t dpp_partner(uint32_t v)
{
    constexpr int ctrl = LEVEL == 0 ? 0xb1 : LEVEL == 1 ? 0x4e : LEVEL == 2 ? 0x141 : 0x140;
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, 0xf, 0xf, false);
}
template <int LEVEL> __device__ __forceinline__ void merge_level(float &m, float &s, float &t)
{
    const float m2 = __uint_as_float(dpp_partner<LEVEL>(__float_as_uint(m)));
    const float s2 = __uint_as_float(dpp_partner<LEVEL>(__float_as_uint(s)));
    const float t2 = __uint_as_float(dpp_partner<LEVEL>(__float_as_uint(t)));
    lse_merge(m, s, m2, s2); // symmetric: both partners get the same bits
    t = fmaxf(t, t2);
}

// The selection of batch element b by one wave, when its P <= 64 pieces fit
// the lanes and its P*k <= 256 published slots fit 4 per lane: lane p owns
// piece p and loads, with everything else, its beam's score and flag; each
// beam's partials are merged by DPP butterflies over its lanes (C a power of
// two <= 16) or by a fixed tree in LDS; survivors are ranked by ballot with
// the count in a scalar register. No barriers, no LDS atomics.
__device__ __forceinline__ void sort_batch_wave(const StepArgs &a, const SortLds &sm, int b, int lane)
{
    const int beam = a.beam, C = a.chunks, L = a.k;
    const int P = beam * C, NS = P * L;
    const uint64_t *slots = a.slots + (long long)b * NS;
    const uint64_t *head = a.head + 2 * (long long)b * P;
    const uint32_t K = (uint32_t)a.sort_keys;
    const bool has_fin = a.finished != nullptr;
    const uint8_t *finb = has_fin ? a.finished + (long long)b * beam : nullptr;
    const float invC = 1.f / (float)C, invL = 1.f / (float)L;

    // ---- one round trip: 4 slots per lane, this lane's piece header, its beam's
    // flag and score (device-coherent loads)
    uint64_t spec[4];
    const bool own = lane < P;
    const int jp = own ? small_div(lane, invC) : 0; // this lane's beam
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int gi = lane + r * kLanes;
        spec[r] = gi < NS ? get64(&slots[gi]) : 0ull;
    }
    const uint64_t h0 = own ? get64(&head[2 * lane]) : 0ull;
    const uint64_t h1 = own ? get64(&head[2 * lane + 1]) : 0ull;
    const float alv = own ? a.alive[b * beam + jp] : 0.f;
    const bool fin = own && has_fin && finb[jp] != 0;
    float m = own ? __uint_as_float((uint32_t)h0) : -INFINITY;
    float sum = own ? __uint_as_float((uint32_t)(h0 >> 32)) : 0.f;
    float t = own ? __uint_as_float((uint32_t)h1) : -INFINITY;
    const uint32_t pn = own && !fin ? (uint32_t)(h1 >> 32) : 0u;

    // ---- each beam's partials, merged over its C lanes by a fixed tree
    if ((C & (C - 1)) == 0 && C <= 16) {
        if (C >= 2)
            merge_level<0>(m, sum, t);
        if (C >= 4)
            merge_level<1>(m, sum, t);
        if (C >= 8)
            merge_level<2>(m, sum, t);
        if (C >= 16)
            merge_level<3>(m, sum, t);
    } else {
        if (own) {
            sm.pm[lane] = m;
            sm.ps[lane] = sum;
            sm.pt[lane] = t;
        }
        for (int stride = 1; stride < C; stride <<= 1) {
            wave_sync();
            const int c = lane - jp * C;
            if (own && (c & (2 * stride - 1)) == 0 && c + stride < C) {
                float mm = sm.pm[lane], ss = sm.ps[lane];
                lse_merge(mm, ss, sm.pm[lane + stride], sm.ps[lane + stride]);
                sm.pm[lane] = mm;
                sm.ps[lane] = ss;
                sm.pt[lane] = fmaxf(sm.pt[lane], sm.pt[lane + stride]);
            }
        }
        wave_sync();
        if (own) {
            m = sm.pm[jp * C];
            sum = sm.ps[jp * C];
            t = sm.pt[jp * C];
        }
        wave_sync(); // every lane has read before the tables below are rewritten
    }
    const float lse = fin ? 0.f : (m + fast_log2(sum)) * kLn2; // unused for a finished beam
    const float thr = fin ? INFINITY : t;
    // at least k logits of a beam are >= thr, so at least k candidates score >= alive + (thr - lse)
    const float bound = wave_max_f(own && !fin ? alv + (thr - lse) : -INFINITY);
    // per-piece copies of the beam values, read by slot below (the per-piece
    // arrays pm, ps, pt hold lse, thr, alive here); one finished flag per beam
    float *plse = sm.pm, *pthr = sm.ps, *palive = sm.pt;
    if (own) {
        plse[lane] = lse;
        pthr[lane] = thr;
        palive[lane] = alv;
        sm.pn[lane] = (uint8_t)pn;
        if (lane == jp * C) {
            sm.fin[jp] = (uint8_t)fin;
            if (a.dbg_lse) // NaN bits mark a finished beam
                reinterpret_cast<uint32_t *>(a.dbg_lse)[b * beam + jp] = fin ? 0x7fc00000u : __float_as_uint(lse);
        }
    }
    wave_sync();

    // ---- survivors -> sort keys, ranked by ballot; ns is wave-uniform
    uint32_t ns = 0;
    auto offer = [&](bool ok, uint64_t key) {
        const uint64_t mk = ballot(ok);
        if (mk != 0) {
            const uint32_t pos = ns + lane_prefix(mk);
            if (ok && pos < K)
                sm.keys[pos] = key;
            ns += (uint32_t)__builtin_popcountll(mk);
        }
    };
    // the four table reads of every slot are independent (no nested tests),
    // so their LDS latencies overlap
    bool ok4[4];
    uint64_t key4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int gi = lane + r * kLanes;
        const int p = gi < NS ? small_div(gi, invL) : 0;
        const uint32_t n = sm.pn[p];
        const float th = pthr[p], al = palive[p], ls = plse[p];
        const float x = entry_x(spec[r]);
        const float sc = al + (x - ls);
        key4[r] = score_key(sc, entry_flat(spec[r]));
        // slots past a piece's count hold stale data
        ok4[r] = gi < NS && (uint32_t)(gi - p * L) < n && x >= th && sc >= bound;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
        offer(ok4[r], key4[r]);
    if (has_fin) { // a finished beam offers its end token at its running score
        const int pj = lane * C; // the first piece of beam `lane`
        const bool ok = lane < beam && sm.fin[lane] && palive[pj] >= bound;
        offer(ok, ok ? score_key(palive[pj], (uint32_t)lane * (uint32_t)a.V + (uint32_t)a.eos_id) : 0ull);
    }
    wave_sync();

    // ---- the k best keys, in order (ns <= P*k + beam <= 320)
    const bool small_flat = (long long)beam * a.V < (1 << 22);
    const float invV = 1.f / (float)a.V;
    auto emit_out = [&](int p, uint64_t key) {
        const long long o = (long long)b * a.k + p;
        const uint32_t flat = 0xffffffffu - (uint32_t)key;
        const uint32_t jj = small_flat ? (uint32_t)small_div((int)flat, invV) : flat / (uint32_t)a.V;
        a.out_beam[o] = (int32_t)jj;
        a.out_token[o] = (int32_t)(flat - jj * (uint32_t)a.V);
        a.out_score[o] = from_ord((uint32_t)(key >> 32));
    };
    if (ns <= (uint32_t)kLanes) {
        if ((uint32_t)lane < ns) {
            const uint64_t mine = sm.keys[lane];
            uint32_t rank = 0;
#pragma unroll 8
            for (uint32_t i = 0; i < ns; ++i)
                rank += sm.keys[i] > mine;
            if (rank < (uint32_t)a.k)
                emit_out((int)rank, mine);
        }
    } else {
        int Pw = 2;
        while ((uint32_t)Pw < ns)
            Pw <<= 1;
        for (int i = (int)ns + lane; i < Pw; i += kLanes)
            sm.keys[i] = 0ull; // below every real key
        wave_sync();
        bitonic_desc(sm.keys, Pw, lane, kLanes);
        for (int p = lane; p < a.k && (uint32_t)p < ns; p += kLanes)
            emit_out(p, sm.keys[p]);
    }
    for (int p = (int)ns + lane; p < a.k; p += kLanes) { // padding: fewer than k candidates at all
        const long long o = (long long)b * a.k + p;
        a.out_beam[o] = -1;
        a.out_token[o] = -1;
        a.out_score[o] = -INFINITY;
    }
    if (a.dbg_queue || a.dbg_count) { // debug copies of every published candidate
        const uint32_t before = wave_excl_scan_u32(pn, lane);
        const uint32_t total = __builtin_amdgcn_readlane(before + pn, 63);
        if (a.dbg_queue) {
            uint64_t *dq = a.dbg_queue + (long long)b * a.queue_cap;
            for (uint32_t e = 0; e < pn; ++e) {
                const uint64_t ent = get64(&slots[(long long)lane * L + e]);
                dq[before + e] = ((uint64_t)__float_as_uint(entry_x(ent)) << 32) | entry_flat(ent);
            }
        }
        if (lane == 0 && a.dbg_count)
            a.dbg_count[b] = total;
    }
    if (lane == 0)
        put32(ticket_of(a, b), 0u);
}

// ------------------------------------------------------------ row-local workgroups
// When a row's pieces divide a workgroup, every workgroup holds whole rows and
// can score them itself: wave 0 merges each row's partials (DPP over the C
// lanes of its pieces), forms the workgroup's exact top-k of each batch
// element it holds (candidates scored with the rows' own lse, filtered by the
// rows' thresholds and the workgroup's bound), and either writes the outputs
// (it held every row) or publishes that list of k keys. The batch element's
// top-k restricted to one workgroup's rows lies in that workgroup's list, so
// the last list to arrive merges exactly: one round trip of a few keys.

// The kept (<= 64) best of keys[0..n), 64 < n <= 512, into best_out by rank:
// up to 8 keys per lane, held in registers. t, the kept-th largest key, by a
// search over its bits from the top: a candidate prefix stays when at least
// `kept` keys are >= it (one ballot per register and bit), and the search
// stops once exactly `kept` keys are >= t (keys are distinct). Those are
// compacted to keys[0..kept) and ranked by counting.
__device__ __forceinline__ void wave_topk_bits(uint64_t *keys, uint32_t n, uint32_t kept, int lane, uint64_t *best_out)
{
    uint64_t mine[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t i = (uint32_t)lane + (uint32_t)j * kLanes;
        mine[j] = i < n ? keys[i] : 0ull; // 0: below every real key
    }
    uint64_t t = 0;
    uint32_t cnt_t = n;
    for (int bit = 63; bit >= 0 && cnt_t != kept; --bit) { // uniform
        const uint64_t c = t | (1ull << bit);
        uint32_t cnt = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            cnt += (uint32_t)__builtin_popcountll(ballot(mine[j] >= c));
        if (cnt >= kept) {
            t = c;
            cnt_t = cnt;
        }
    }
    wave_sync(); // every lane has read keys[] before it is rewritten
    uint32_t pos = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const bool sel = (uint32_t)lane + (uint32_t)j * kLanes < n && mine[j] >= t;
        const uint64_t m = ballot(sel);
        const uint32_t q = pos + lane_prefix(m);
        if (sel && q < kept)
            keys[q] = mine[j];
        pos += (uint32_t)__builtin_popcountll(m);
    }
    wave_sync();
    if ((uint32_t)lane < kept) { // kept <= k <= 64
        const uint64_t x = keys[lane];
        uint32_t rank = 0;
#pragma unroll 8
        for (uint32_t i = 0; i < kept; ++i)
            rank += keys[i] > x;
        best_out[rank] = x;
    }
}

// Keys of this workgroup's selection: the k best of keys[0..n), then either
// the outputs or the published list. `rank` of lane entries by counting when
// n <= 64; up to 512 keys, a search for the k-th largest key's bits in the
// kernels built for k > 8 (BIGK), else k rounds of wave argmax; more, k rounds
// over LDS. Returns the number kept; keys[] may be overwritten.
template <bool BIGK>
__device__ __forceinline__ uint32_t wave_topk(uint64_t *keys, uint32_t n, int k, int lane, uint64_t *best_out)
{
    const uint32_t kept = n < (uint32_t)k ? n : (uint32_t)k;
    if (n <= (uint32_t)kLanes) {
        if ((uint32_t)lane < n) {
            const uint64_t mine = keys[lane];
            uint32_t rank = 0;
#pragma unroll 8
            for (uint32_t i = 0; i < n; ++i)
                rank += keys[i] > mine;
            if (rank < (uint32_t)k)
                best_out[rank] = mine;
        }
    } else if (BIGK && n <= 8u * kLanes) {
        wave_topk_bits(keys, n, kept, lane, best_out);
    } else if (n <= 8u * kLanes) {
        // up to 8 keys per lane, held in registers; k rounds of a DPP wave
        // maximum of the keys below the previous round's (keys are distinct)
        uint64_t mine[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t i = (uint32_t)lane + (uint32_t)j * kLanes;
            mine[j] = i < n ? keys[i] : 0ull;
        }
        uint64_t prev = ~0ull;
        for (uint32_t round = 0; round < kept; ++round) {
            uint64_t best = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                best = mine[j] < prev && mine[j] > best ? mine[j] : best;
            best = wave_max_key(best);
            if (lane == 0)
                best_out[round] = best;
            prev = best;
        }
    } else {
        uint64_t prev = ~0ull;
        for (uint32_t round = 0; round < kept; ++round) {
            uint64_t best = 0;
            for (uint32_t i = lane; i < n; i += kLanes) {
                const uint64_t x = keys[i];
                best = x < prev && x > best ? x : best;
            }
            best = wave_max_key(best);
            if (lane == 0)
                best_out[round] = best;
            prev = best;
        }
    }
    wave_sync();
    return kept;
}

__device__ __forceinline__ void emit_outputs(const StepArgs &a, int b, const uint64_t *best, uint32_t kept, int lane)
{
    for (int p = lane; p < a.k; p += kLanes) {
        const long long o = (long long)b * a.k + p;
        if ((uint32_t)p < kept) {
            const uint64_t key = best[p];
            const uint32_t flat = 0xffffffffu - (uint32_t)key;
            const uint32_t jj = mdiv(flat, a.mv);
            a.out_beam[o] = (int32_t)jj;
            a.out_token[o] = (int32_t)(flat - jj * (uint32_t)a.V);
            a.out_score[o] = from_ord((uint32_t)(key >> 32));
        } else { // fewer than k candidates at all
            a.out_beam[o] = -1;
            a.out_token[o] = -1;
            a.out_score[o] = -INFINITY;
        }
    }
}

// The outputs of batch element b from its k best keys; kernels built for
// k > 8 also draw the top-k sample of the row when asked (one beam, zero
// running score: the keys' scores are s_i = x_i - lse).
template <bool BIGK>
__device__ __forceinline__ void finish_outputs(const StepArgs &a, int b, const uint64_t *best, uint32_t kept, int lane)
{
    emit_outputs(a, b, best, kept, lane);
    if constexpr (BIGK) {
        if (a.smp_token) {
            const bool has = (uint32_t)lane < kept;
            const uint64_t key = has ? best[lane] : 0ull;
            const float s = has ? from_ord((uint32_t)(key >> 32)) : -INFINITY;
            const uint32_t flat = 0xffffffffu - (uint32_t)key;
            const int32_t t = has ? (int32_t)(flat - mdiv(flat, a.mv) * (uint32_t)a.V) : -1;
            draw_topk_row(s, t, a.k, lane, b, a.smp_tau, a.smp_seed, a.smp_step, a.smp_token, a.smp_logprob);
        }
    }
}

// Wave 0 of a row-local workgroup: its rows j0..j1 of batch element b (all
// their pieces, np = (j1 - j0 + 1) * C <= W <= 16 of them, one per lane).
// Merges each row's partials, and puts into keys[0..n) the sort keys of its
// candidates that can be among b's top-k: at least k of them score >= the
// bound S = max over its alive rows of alive + (threshold - lse), so no
// candidate below S can. Returns n.
__device__ __forceinline__ uint32_t row_candidates(const StepArgs &a, const SelectLds *wl, uint64_t *keys,
                                                   uint32_t ufirst, int b, int j0, int j1, int lane)
{
    const int C = a.chunks, beam = a.beam, k = a.k;
    const int nrows = j1 - j0 + 1, np = nrows * C;
    const long long p0 = ((long long)b * beam + j0) * C; // first piece
    const bool own = lane < np;
    const int w = own ? (int)(p0 + lane - ufirst) : 0; // the wave that ran piece `lane`
    const int jl = lane / C, j = j0 + jl;              // C is a power of two here
    const float alv = own ? wl[w].ha : 0.f;
    const bool fin = own && wl[w].hf != 0;
    float m = own ? wl[w].hm : -INFINITY, sum = own ? wl[w].hs : 0.f, t = own ? wl[w].ht : -INFINITY;
    const uint32_t emit = own && !fin ? wl[w].hemit : 0u;
    if (C >= 2)
        merge_level<0>(m, sum, t);
    if (C >= 4)
        merge_level<1>(m, sum, t);
    if (C >= 8)
        merge_level<2>(m, sum, t);
    if (C >= 16)
        merge_level<3>(m, sum, t);
    const float lse = fin ? 0.f : (m + fast_log2(sum)) * kLn2; // unused for a finished row
    const float thr = fin ? INFINITY : t;
    const float bound = wave_max_f(own && !fin ? alv + (thr - lse) : -INFINITY);
    if (a.dbg_lse && own && lane == jl * C) // NaN bits mark a finished row
        reinterpret_cast<uint32_t *>(a.dbg_lse)[(long long)b * beam + j] = fin ? 0x7fc00000u : __float_as_uint(lse);

    // survivors -> keys, by ballot (ns is wave-uniform)
    uint32_t ns = 0;
    auto offer = [&](bool ok, uint64_t key) {
        const uint64_t mk = ballot(ok);
        if (mk != 0) {
            if (ok)
                keys[ns + lane_prefix(mk)] = key;
            ns += (uint32_t)__builtin_popcountll(mk);
        }
    };
    const float invk = 1.f / (float)k;
    for (int g0 = 0; g0 < np * k; g0 += kLanes) {
        const int gi = g0 + lane;
        const int p = gi < np * k ? small_div(gi, invk) : 0;
        const int e = gi - p * k;
        // the row values of piece p live in every lane of its row, e.g. lane p
        const float plse = __shfl(lse, p), pthr = __shfl(thr, p), palv = __shfl(alv, p);
        const uint32_t pe = (uint32_t)__shfl((int)emit, p);
        const uint64_t ent = gi < np * k ? wl[p0 + p - ufirst].top[e] : 0ull;
        const float x = entry_x(ent);
        const float sc = palv + (x - plse);
        const bool ok = gi < np * k && (uint32_t)e < pe && x >= pthr && sc >= bound;
        offer(ok, score_key(sc, entry_flat(ent)));
    }
    if (a.finished != nullptr) { // a finished row offers its end token at its running score
        const bool first = own && lane == jl * C;
        const bool ok = first && fin && alv >= bound;
        offer(ok, ok ? score_key(alv, (uint32_t)j * (uint32_t)a.V + (uint32_t)a.eos_id) : 0ull);
    }
    return ns;
}

// The workgroup of batch element b that arrived last at its ticket appends
// to keys[0..n) the lists the others put in the mailbox. Each of them arrived
// earlier and fills all k of its slots (kEmptySlot past its list) once its
// rows are selected; a slot still zero is not there yet, and is read again.
// A wait that exceeds the poll limit gives up (`failed`). Returns the new
// count.
__device__ __forceinline__ uint32_t take_lists(const StepArgs &a, uint64_t *keys, uint32_t n, int b, int nl,
                                               int self, int lane, bool &failed)
{
    const int k = a.k, nslot = nl * k;
    const uint64_t *box = a.mailbox + (long long)b * a.maxl * k;
    const float invk = 1.f / (float)k;
    for (int g0 = 0; g0 < nslot && !failed; g0 += kLanes) {
        const int gi = g0 + lane;
        const bool rd = gi < nslot && small_div(gi, invk) != self;
        uint64_t ent = kEmptySlot;
        for (unsigned spin = 0;; ++spin) { // uniform
            if (spin >= a.spin_limit) {
                failed = true;
                break;
            }
            ent = rd ? get64(&box[gi]) : kEmptySlot;
            if (ballot(ent == 0) == 0)
                break;
            __builtin_amdgcn_s_sleep(2);
        }
        const bool ok = !failed && ent != kEmptySlot;
        const uint64_t mk = ballot(ok);
        if (ok)
            keys[n + lane_prefix(mk)] = ent;
        n += (uint32_t)__builtin_popcountll(mk);
    }
    return n;
}

// Wave 0 of a row-local workgroup, once every piece of it is done, for each
// batch element b of its rows: the candidates of its rows; if b has rows in
// other workgroups, either this workgroup arrived last at b's ticket and
// appends the others' lists, or it leaves its own k best in the mailbox; then
// the k best of the keys, and the outputs of b from the one that merges.
// Every mailbox slot read and the ticket go back to zero. A merge whose wait
// gave up writes padding and sets status word 0 (the fixed region must then
// be cleared before the next call).
template <bool BIGK>
__device__ __forceinline__ void rl_tail(const StepArgs &a, const SelectLds *wl, uint64_t *keys, uint64_t *best,
                                        uint32_t ufirst, int LG, int bfirst, int blast, int rfirst, int rlast,
                                        int lane)
{
    const int PB = a.beam * a.chunks; // pieces of a batch element
    // The arrival at the ticket of each batch element that also has rows in
    // other workgroups (lane i for bfirst + i), counted once every piece of
    // this workgroup is done: the last workgroup to arrive merges, and every
    // other one has its list ready by then or soon. The round trip overlaps
    // the candidate selection below.
    uint32_t arrived = 0;
    {
        const int bb = bfirst + lane;
        if (bb <= blast && (bb * a.beam < rfirst || (bb + 1) * a.beam - 1 > rlast))
            arrived = __hip_atomic_fetch_add(ticket_of(a, bb), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int b = bfirst; b <= blast; ++b) {
        const int j0 = rfirst > b * a.beam ? rfirst - b * a.beam : 0;
        const int j1 = rlast < (b + 1) * a.beam - 1 ? rlast - b * a.beam : a.beam - 1;
        const bool whole = j0 == 0 && j1 == a.beam - 1; // every row of b is here
        int nl = 1, self = 0;
        bool merge = true;
        if (!whole) {
            const int Lf = (int)mdiv((uint32_t)b * (uint32_t)PB, a.mw);
            const int Ll = (int)mdiv(((uint32_t)b + 1) * (uint32_t)PB - 1, a.mw);
            nl = Ll - Lf + 1; // workgroups holding rows of b
            self = LG - Lf;
        }
        uint32_t n = row_candidates(a, wl, keys, ufirst, b, j0, j1, lane);
        if (!whole)
            merge = first_u32(__builtin_amdgcn_readlane(arrived, b - bfirst)) + 1 >= (uint32_t)nl;
        bool failed = false;
        if (!whole && merge)
            n = take_lists(a, keys, n, b, nl, self, lane, failed);
        wave_sync();
        const uint32_t kept = failed ? 0u : wave_topk<BIGK>(keys, n, a.k, lane, best);
        if (merge) {
            finish_outputs<BIGK>(a, b, best, kept, lane);
            if (failed) {
                if (lane == 0)
                    __hip_atomic_fetch_or(&a.status[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else if (!whole) {
                uint64_t *box = a.mailbox + (long long)b * a.maxl * a.k;
                const float invk = 1.f / (float)a.k;
                for (int gi = lane; gi < nl * a.k; gi += kLanes)
                    if (small_div(gi, invk) != self)
                        put64(&box[gi], 0ull);
                if (lane == 0)
                    put32(ticket_of(a, b), 0u);
            }
        } else { // hand the list over (all k slots, kEmptySlot past it)
            uint64_t *box = a.mailbox + ((long long)b * a.maxl + self) * a.k;
            for (int p = lane; p < a.k; p += kLanes)
                put64(&box[p], (uint32_t)p < kept ? best[p] : kEmptySlot);
        }
        wave_sync();
    }
}

// Per-piece publication: tickets count the pieces; the workgroup that
// completes a batch element selects its outputs from every published list.
__device__ __forceinline__ void rtopk_step_tail(const StepArgs &a, GroupLds &g, uint8_t *lds, size_t hdr, int tid,
                                                int lane, int wave, int W, uint32_t ufirst, uint32_t ulast)
{
    const int P = a.beam * a.chunks;
    const int bfirst = (int)mdiv(ufirst, a.mp), blast = (int)mdiv(ulast, a.mp); // at most W batch elements
    if (wave == 0) {
        const int bb = bfirst + lane;
        bool done = false;
        if (bb <= blast) {
            const long long lo = (long long)bb * P > ufirst ? (long long)bb * P : ufirst;
            const long long hi = (long long)(bb + 1) * P - 1 < ulast ? (long long)(bb + 1) * P - 1 : ulast;
            const uint32_t n = (uint32_t)(hi - lo + 1);
            const uint32_t now =
                __hip_atomic_fetch_add(ticket_of(a, bb), n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + n;
            done = now == (uint32_t)P; // every piece of bb has published
        }
        const uint64_t m = ballot(done);
        if (lane == 0) {
            g.todo[0] = (uint32_t)m;
            g.todo[1] = (uint32_t)(m >> 32);
        }
    }
    lds_barrier();
    uint64_t todo = ((uint64_t)g.todo[1] << 32) | g.todo[0];
    if (todo == 0)
        return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // A batch element whose pieces and published slots fit one wave's lanes
    // (up to 4 slots per lane) is selected by wave 0 alone, with no workgroup
    // barriers in the way; larger ones by the whole workgroup.
    int SW = W;
    if (P <= kLanes && P * a.k <= 4 * kLanes) {
        if (wave != 0)
            return;
        SW = 1;
    }
    const SortLds sm = sort_lds(lds + hdr, a); // the waves' selection LDS is free now
    bool again = false;
    while (todo != 0) {
        const int i = __builtin_ctzll(todo);
        todo &= todo - 1;
        if (again)
            group_sync(SW); // the previous batch element's LDS readers are done
        again = true;
        if (SW == 1)
            sort_batch_wave(a, sm, bfirst + i, lane);
        else
            sort_batch(a, sm, g, bfirst + i, tid, SW);
    }
}

// RL: row-local workgroups (chunks divides waves), a separate instantiation so
// that neither tail's register needs weigh on the other.
template <int DT, int NV, bool ALIGNED, int RL> // RL: 0 per-piece publication, 1 row-local, 2 row-local, k > 8
__global__ __launch_bounds__(kLanes *kMaxWaves) void rtopk_step(const StepArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    GroupLds &g = *reinterpret_cast<GroupLds *>(lds);
    const int tid = threadIdx.x, lane = tid & (kLanes - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kLanes); // uniform: piece math stays scalar
    const int W = a.waves;
    const size_t hdr = lds_header(W);
    const uint32_t total = (uint32_t)a.B * (uint32_t)a.beam * (uint32_t)a.chunks; // pieces, < 2^31
    const int LG = logical_group((int)blockIdx.x, (int)gridDim.x);
    const uint32_t ufirst = (uint32_t)LG * (uint32_t)W;
    const uint32_t u = ufirst + (uint32_t)wave;
    const uint32_t ulast = (ufirst + W < total ? ufirst + W : total) - 1;
    const uint32_t row0 = mdiv(ufirst, a.mc);
    uint32_t *gshare = reinterpret_cast<uint32_t *>(lds + kLdsShare);
    // The barrier before the loads orders the clearing of the shared group
    // maxima before any wave's use; after the loads it would hold every wave
    // until the last of the workgroup's loads could issue.
    for (int i = tid; i < W * kMaxK; i += kLanes * W)
        gshare[i] = 0x007fffffu; // ord_bits(-inf)
    lds_barrier();

    const int rfirst = (int)row0, rlast = (int)mdiv(ulast, a.mc);
    Piece<NV> P;
    piece_load<DT, NV, (RL > 0)>(a, P, gshare, u, u < total, row0, lane);
    SelectLds &sm = *reinterpret_cast<SelectLds *>(lds + hdr + wave * sizeof(SelectLds));
    constexpr int MODE = ALIGNED ? kAligned : kGeneral;
    if constexpr (RL > 0) {
        piece_compute<DT, NV, MODE, true>(a, sm, P, u, lane);
        // Every wave is done with its piece. A workgroup's resources are
        // released only when its last wave ends, so the others wait here for
        // free; then wave 0 selects what the workgroup holds.
        lds_barrier();
        if (wave != 0)
            return;
        const SelectLds *wl = reinterpret_cast<const SelectLds *>(lds + hdr);
        uint64_t *keys = reinterpret_cast<uint64_t *>(lds + hdr + (size_t)W * sizeof(SelectLds));
        uint64_t *best = keys + rowlocal_keys(W, a.k, a.maxl);
        rl_tail<(RL > 1)>(a, wl, keys, best, ufirst, LG, (int)mdiv((uint32_t)rfirst, a.mb),
                          (int)mdiv((uint32_t)rlast, a.mb), rfirst, rlast, lane);
    } else {
        piece_compute<DT, NV, MODE, false>(a, sm, P, u, lane);
        if (a.split) // the selection is a second launch, once every piece has published
            return;
        lds_barrier();
        rtopk_step_tail(a, g, lds, hdr, tid, lane, wave, W, ufirst, ulast);
    }
}

#if RTOPK_DTYPE == 0
// The per-batch selection of a split step: when the step's workgroups run in
// rounds, a workgroup that completed a batch element would hold its CU for the
// selection while later workgroups wait to stream, and the last round's
// selections would all come after the stream. Instead the step kernel only
// publishes, and this launch selects every batch element at once (one
// workgroup each) from the same published pieces, with the same code as the
// in-kernel tail. The kernel boundary orders the pieces' stores before these
// reads; no ticket is counted.
// It runs kMaxWaves waves whatever the step's workgroup size, so that the
// speculative loads of sort_batch cover every published slot at once.
__global__ __launch_bounds__(kLanes *kMaxWaves) void rtopk_select(const StepArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    GroupLds &g = *reinterpret_cast<GroupLds *>(lds);
    const int tid = threadIdx.x, lane = tid & (kLanes - 1);
    const int W = (int)blockDim.x / kLanes;
    const SortLds sm = sort_lds(lds + lds_header(W), a);
    const int P = a.beam * a.chunks;
    if (P <= kLanes && P * a.k <= 4 * kLanes) {
        if (tid < kLanes)
            sort_batch_wave(a, sm, (int)blockIdx.x, lane);
    } else {
        sort_batch(a, sm, g, (int)blockIdx.x, tid, W);
    }
}

// Plain streaming read (measurement aid): kReadVecs 16-byte vectors per lane,
// consecutive lanes on consecutive vectors, all loads issued before any use.
constexpr int kReadVecs = 10;
constexpr int kReadThreads = 256;
__global__ __launch_bounds__(kReadThreads) void read_probe(const u32x4 *src, size_t n16, uint32_t marker,
                                                           uint32_t *out)
{
    const size_t base = (size_t)blockIdx.x * kReadThreads * kReadVecs + threadIdx.x;
    u32x4 v[kReadVecs];
#pragma unroll
    for (int i = 0; i < kReadVecs; ++i) {
        const size_t idx = base + (size_t)i * kReadThreads;
        v[i] = idx < n16 ? __builtin_nontemporal_load(src + idx) : u32x4{0u, 0u, 0u, 0u};
    }
    bool hit = false;
#pragma unroll
    for (int i = 0; i < kReadVecs; ++i) {
        const size_t idx = base + (size_t)i * kReadThreads;
        hit |= idx < n16 && (v[i].x == marker || v[i].y == marker || v[i].z == marker || v[i].w == marker);
    }
    if (hit)
        out[0] = 1u;
}

// The same read for another launch shape: VECS vectors per lane, any
// multiple of 64 lanes per workgroup (measurement of the read ceiling's
// dependence on the launch shape).
template <int VECS>
__global__ __launch_bounds__(1024) void read_probe_shape(const u32x4 *src, size_t n16, uint32_t marker, uint32_t *out)
{
    const size_t T = blockDim.x;
    const size_t base = (size_t)blockIdx.x * T * VECS + threadIdx.x;
    u32x4 v[VECS];
#pragma unroll
    for (int i = 0; i < VECS; ++i) {
        const size_t idx = base + (size_t)i * T;
        v[i] = idx < n16 ? __builtin_nontemporal_load(src + idx) : u32x4{0u, 0u, 0u, 0u};
    }
    bool hit = false;
#pragma unroll
    for (int i = 0; i < VECS; ++i) {
        const size_t idx = base + (size_t)i * T;
        hit |= idx < n16 && (v[i].x == marker || v[i].y == marker || v[i].z == marker || v[i].w == marker);
    }
    if (hit)
        out[0] = 1u;
}

__global__ void zero_fill(uint32_t *p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}
#endif

#if RTOPK_DTYPE == 2
// ------------------------------------------------- LM head fused with pass 1
// The logits of a decode step come from the LM head, a GEMM:
// logits[m][v] = sum_h x[m][h] * w[v][h] (hidden states [M][H], output
// projection [V][H], bfloat16; fp32 accumulation). The LightSeq inference
// article fuses the work around its GEMMs into them (kernel-fusion passage);
// here pass 1 and the per-piece top-k of the selection run in the GEMM's
// epilogue, so the [M][V] logits never reach HBM.
//
// lmhead_tiles: one workgroup of 8 waves per 256 x 320 tile (rows of x by
// vocabulary columns). Wave (wm, wn) computes rows 128 wm .. + 127 and
// columns 80 wn .. + 79 of it as 8 x 5 blocks of v_mfma_f32_16x16x32_bf16
// (160 accumulator registers). Tall wave tiles keep the LDS bytes read per
// multiply low, and 256 x 320 tiles cover B*beam = 512 and V = 40000 in 250
// workgroups, one round on 256 CUs, each reading 256 rows of x and 320 rows
// of w once. The operands stream through two LDS stages filled by
// direct-to-LDS buffer loads (no registers in between), 64 steps of H
// (whole 128-byte lines of every row) per stage, one stage in flight while
// the other is multiplied. The 8 lanes of a row slice in a load fetch its
// 16-byte chunks permuted by the row (chunk c of row r at slot c ^ swz(r)),
// so the fragment reads, 16 rows at one chunk, fall in distinct LDS banks
// whether the LDS serves 8 or 16 lanes of a 16-byte read per clock. The
// epilogue then takes the tile 64 rows at a time through LDS, 8 threads per
// row: every row of the tile is a piece of the per-piece path, whose group
// maxima (group = vocabulary index mod ngroups), R-top-k threshold, base-2
// log-sum-exp partial and exact top-k by (logit desc, flat asc) go to the
// workspace; lmhead_select reduces the pieces of each batch element.
constexpr int kLM = kLmTileM, kLN = kLmTileV, kLThreads = 512;
constexpr int kLWaves = kLThreads / kLanes;
constexpr int kLWM = 128, kLWN = 80;           // rows and columns per wave
constexpr int kLBI = kLWM / 16, kLBJ = kLWN / 16; // 16 x 16 blocks per wave: 8 x 5
constexpr int kLK = 64;                        // steps of H per stage
constexpr int kLStages = 2;
constexpr int kLRow = kLK * 2;                 // bytes of a row slice (128: one line)
constexpr int kLRowsLoad = kLanes / (kLRow / 16); // rows per direct load (8)
constexpr int kLStageA = kLM * kLRow;          // bytes of x in a stage: [256 rows][128 bytes]
constexpr int kLStage = (kLM + kLN) * kLRow;   // x, then w as [320 rows][128 bytes]
constexpr int kLSmem = kLStages * kLStage;     // 144 KiB
constexpr int kLLoadsA = kLM / kLRowsLoad / kLWaves; // x loads per wave per stage (4)
constexpr int kLLoadsB = kLN / kLRowsLoad / kLWaves; // w loads per wave per stage (5)
constexpr int kLEQ = 40;                       // columns per epilogue thread
constexpr int kLERows = kLThreads / (kLN / kLEQ); // rows per epilogue round (64)
constexpr int kLEStride = 352;                 // floats per epilogue row: 8 blocks of 40 columns, 44 apart
// epilogue LDS index of (row, column): the 40-column blocks sit 44 floats apart and
// every 4 rows 16 floats further on, so the threads' b128 reads (8 per row, 2 rows
// per 16 lanes) and the accumulator stores (16 columns x 4 rows 4 apart) spread
// over the banks
__device__ __forceinline__ int lm_eidx(int r, int c) { return r * kLEStride + (r >> 2) * 16 + 44 * (c / kLEQ) + c % kLEQ; }
static_assert(kLM == 2 * kLWM && kLN == 4 * kLWN && kLWaves == 8, "the wave layout the tile assumes");
static_assert(kLLoadsA * kLRowsLoad * kLWaves == kLM && kLLoadsB * kLRowsLoad * kLWaves == kLN, "whole loads per wave");
static_assert((kLERows * kLEStride + kLERows / 4 * 16) * 4 <= kLSmem, "an epilogue round fits the ring");
static_assert(kLEQ % kLmMaxK == 0 && kLN % kLmMaxK == 0, "tiles and thread columns start at multiples of ngroups");
static_assert(kLWM / 16 % 2 == 0 && kLERows == 2 * 16 * (kLM / kLWM), "a round is two block-rows of every wave row");

// Chunk slot permutation of row r (its residue mod 16 decides): 8 consecutive
// rows at one chunk cover 128 distinct bytes of the bank space, 16 rows 256.
__device__ __forceinline__ int lm_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// The N best keys seen, descending (0 = empty): insertion by compare-exchange.
template <int N> __device__ __forceinline__ void topn_insert(uint64_t (&t)[N], uint64_t key)
{
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const uint64_t hi = key > t[i] ? key : t[i];
        key = key > t[i] ? t[i] : key;
        t[i] = hi;
    }
}

// Reductions over the 8 aligned lanes of this lane's octet: lane i meets 7 - i
// (row_half_mirror), then its quad partners (quad_perm 1,0,3,2 and 2,3,0,1).
__device__ __forceinline__ float octet_max(float v)
{
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0xb1>(v));
    return fmaxf(v, dpp_f<0x4e>(v));
}
__device__ __forceinline__ float octet_sum(float v)
{
    v = v + dpp_f<0x141>(v);
    v = v + dpp_f<0xb1>(v);
    return v + dpp_f<0x4e>(v);
}
template <int CTRL> __device__ __forceinline__ uint64_t dpp_u64(uint64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t octet_max_u64(uint64_t v)
{
    uint64_t o = dpp_u64<0x141>(v);
    v = o > v ? o : v;
    o = dpp_u64<0xb1>(v);
    v = o > v ? o : v;
    o = dpp_u64<0x4e>(v);
    return o > v ? o : v;
}

// Wait until at most N of this wave's vector memory loads are in flight, then
// meet the other waves. A direct-to-LDS load counts as done once its data is
// in LDS, so after this every wave's loads issued before its last N are
// visible. (A plain __syncthreads would wait for every load in flight.)
template <int N> __device__ __forceinline__ void ring_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14)); // vmcnt(N), expcnt and lgkmcnt at their maxima
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int NG>
__global__ __launch_bounds__(kLThreads) void lmhead_tiles(const LmArgs a)
{
    __shared__ __align__(16) uint8_t smem[kLSmem];
    const int tid = threadIdx.x, lane = tid & (kLanes - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kLanes);
    const int wm = wave >> 2, wn = wave & 3;
    // the two row tiles of one vocabulary slice are consecutive logical
    // workgroups, hence on one XCD at about the same time: w comes from HBM once
    const int L = logical_group((int)blockIdx.x, (int)gridDim.x);
    const int nt = L / a.mtiles, mt = L - nt * a.mtiles;
    const int m0 = mt * kLM, n0 = nt * kLN;
    // buffer descriptors spanning exactly x and w: rows past M or V read 0
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.x), 0, (uint32_t)(a.M * a.H * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.w), 0, (uint32_t)(a.V * a.H * 2), 0x00020000);
    // wave w loads x rows 8 (w + 8 q) + lane / 8 (q < 4) and w rows 8 (w + 8 q) + lane / 8
    // (q < 5); lane mod 8 is the slot, holding chunk slot ^ swz(row)
    const int lr = lane >> 3, lslot = lane & 7;
    uint32_t gx[kLLoadsA], gw[kLLoadsB];
#pragma unroll
    for (int q = 0; q < kLLoadsA; ++q) {
        const int r = (wave + q * kLWaves) * kLRowsLoad + lr;
        gx[q] = (uint32_t)(((m0 + r) * a.H + (lslot ^ lm_swz(r)) * 8) * 2);
    }
#pragma unroll
    for (int q = 0; q < kLLoadsB; ++q) {
        const int r = (wave + q * kLWaves) * kLRowsLoad + lr;
        gw[q] = (uint32_t)(((n0 + r) * a.H + (lslot ^ lm_swz(r)) * 8) * 2);
    }
    auto issue = [&](int buf, int kt) {
        uint8_t *st = smem + buf * kLStage;
        const int soff = kt * kLRow;
#pragma unroll
        for (int q = 0; q < kLLoadsA; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (lds_void *)(st + (wave + q * kLWaves) * kLRowsLoad * kLRow), 16, gx[q], soff, 0, 0);
#pragma unroll
        for (int q = 0; q < kLLoadsB; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rw, (lds_void *)(st + kLStageA + (wave + q * kLWaves) * kLRowsLoad * kLRow), 16, gw[q], soff, 0, 0);
    };
    f32x4v acc[kLBI][kLBJ];
#pragma unroll
    for (int i = 0; i < kLBI; ++i)
#pragma unroll
        for (int j = 0; j < kLBJ; ++j)
            acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};
    const int KT = a.H / kLK;
    issue(0, 0);
    // operands of this lane: A row (B column) lane mod 16 of each 16-block, k values
    // 32 ks + 8 (lane / 16) .. + 7 of step ks, i.e. chunk 4 ks + lane / 16, at slot
    // chunk ^ swz(row) (rows 16-aligned plus lane mod 16)
    const int swz = lm_swz(lane & 15);
    const int arow = (wm * kLWM + (lane & 15)) * kLRow, brow = kLStageA + (wn * kLWN + (lane & 15)) * kLRow;
    int slot[kLK / 32];
#pragma unroll
    for (int ks = 0; ks < kLK / 32; ++ks)
        slot[ks] = ((4 * ks + (lane >> 4)) ^ swz) * 16;
    for (int kt = 0; kt < KT; ++kt) {
        // stage kt is in LDS; after the barrier every wave is also done with the
        // other buffer, which the next stage refills while this one is multiplied
        ring_barrier<0>();
        if (kt + 1 < KT)
            issue((kt + 1) & 1, kt + 1);
        const uint8_t *st = smem + (kt & 1) * kLStage;
#pragma unroll
        for (int ks = 0; ks < kLK / 32; ++ks) {
            bf16x8 af[kLBI], bf[kLBJ];
#pragma unroll
            for (int i = 0; i < kLBI; ++i)
                af[i] = *reinterpret_cast<const bf16x8 *>(st + arow + i * 16 * kLRow + slot[ks]);
#pragma unroll
            for (int j = 0; j < kLBJ; ++j)
                bf[j] = *reinterpret_cast<const bf16x8 *>(st + brow + j * 16 * kLRow + slot[ks]);
#pragma unroll
            for (int i = 0; i < kLBI; ++i)
#pragma unroll
                for (int j = 0; j < kLBJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }

    // ---- epilogue, in 4 rounds: round rd takes block-rows 2 rd and 2 rd + 1 of
    // every wave, 64 rows in LDS at lm_eidx; accumulator e of lane l in block
    // (i, j) is row 16 i + 4 (l / 16) + e, column 16 j + l mod 16 of the wave's block
    float *E = reinterpret_cast<float *>(smem);
    const int r = tid >> 3, o = tid & 7;           // this thread: epilogue row r, columns 40 o .. + 39
    const int cbase = n0 + o * kLEQ;               // vocabulary index of its first column
    const int nvalid = a.V - cbase;                // its columns inside the vocabulary (may be <= 0)
    const float *er = E + lm_eidx(r, o * kLEQ);   // its 40 columns, contiguous
#pragma unroll
    for (int rd = 0; rd < kLBI / 2; ++rd) {
        lds_barrier(); // the ring (first round) or the previous round's rows are done with
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
            for (int j = 0; j < kLBJ; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = wm * 32 + i2 * 16 + (lane >> 4) * 4 + e;
                    const int c = wn * kLWN + j * 16 + (lane & 15);
                    E[lm_eidx(row, c)] = acc[2 * rd + i2][j][e];
                }
        lds_barrier();
        const int gm = m0 + (r >> 5) * kLWM + rd * 32 + (r & 31); // the row of logits (b * beam + j)
        // this thread's 40 logits; columns past the vocabulary read as -inf (a
        // wave-uniform branch: only the waves of the last vocabulary tile take it)
        float v[kLEQ];
#pragma unroll
        for (int q = 0; q < kLEQ / 4; ++q) {
            const float4 f = *reinterpret_cast<const float4 *>(er + 4 * q);
            v[4 * q] = f.x;
            v[4 * q + 1] = f.y;
            v[4 * q + 2] = f.z;
            v[4 * q + 3] = f.w;
        }
        if (ballot(nvalid < kLEQ) != 0) {
#pragma unroll
            for (int c = 0; c < kLEQ; ++c)
                v[c] = c < nvalid ? v[c] : -INFINITY;
        }
        // pass A: group maxima (group = column mod NG; 40 o and n0 are multiples of NG),
        // over the row's 8 threads
        float gmx[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g)
            gmx[g] = v[g];
#pragma unroll
        for (int c = NG; c < kLEQ; ++c)
            gmx[c % NG] = fmaxf(gmx[c % NG], v[c]);
        float rmax = -INFINITY;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            gmx[g] = octet_max(gmx[g]);
            rmax = fmaxf(rmax, gmx[g]);
        }
        // the threshold: the k-th largest of the NG group maxima (the least when k == NG)
        float srt[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g)
            srt[g] = gmx[g];
#pragma unroll
        for (int x = 0; x < NG; ++x) // descending by exchanges (NG <= 8)
#pragma unroll
            for (int y = NG - 1; y > x; --y) {
                const float hi = fmaxf(srt[y - 1], srt[y]), lo = fminf(srt[y - 1], srt[y]);
                srt[y - 1] = hi;
                srt[y] = lo;
            }
        float T = srt[0];
#pragma unroll
        for (int g = 1; g < NG; ++g)
            T = g == a.k - 1 ? srt[g] : T;
        // pass B: the log-sum-exp partial in base 2 around the row maximum, and the
        // candidates (a -inf threshold, fewer than k groups in the vocabulary, takes
        // every column inside it)
        const float pm = rmax * kLog2e;
        const float base = rmax == -INFINITY ? 0.f : pm;
        float ssum = 0.f;
        uint64_t cm = 0; // bit c: column c is a candidate
#pragma unroll
        for (int c = 0; c < kLEQ; ++c) {
            ssum += fast_exp2(fmaf(v[c], kLog2e, -base));
            cm |= (uint64_t)(v[c] >= T) << c;
        }
        cm &= nvalid >= kLEQ ? ~0ull : nvalid <= 0 ? 0ull : (1ull << nvalid) - 1ull;
        ssum = octet_sum(ssum); // every lane of the octet holds a sum; the first one's is published
        // this thread's NG best candidates by (logit desc, flat asc), then the row's
        // k best by k rounds of an octet maximum
        const int beamj = gm - (int)mdiv((uint32_t)gm, a.mb) * a.beam;
        const uint32_t flat0 = (uint32_t)beamj * (uint32_t)a.V + (uint32_t)cbase;
        uint64_t t[NG];
#pragma unroll
        for (int x = 0; x < NG; ++x)
            t[x] = 0ull;
        while (cm != 0) {
            const int c = __builtin_ctzll(cm);
            cm &= cm - 1;
            topn_insert<NG>(t, score_key(er[c], flat0 + (uint32_t)c));
        }
        const long long u = (long long)gm * a.C + nt; // the piece (row, tile)
        uint64_t *sl = a.slots + u * a.k;
        const bool own = gm < a.M && o == 0;          // a row inside the batch, written by its first thread
        for (int x = 0; x < a.k; ++x) {
            const uint64_t best = octet_max_u64(t[0]);
            if (best != 0ull && t[0] == best) { // keys are unique: one thread of the octet owns it
#pragma unroll
                for (int y = 0; y + 1 < NG; ++y)
                    t[y] = t[y + 1];
                t[NG - 1] = 0ull;
            }
            if (own)
                sl[x] = best; // 0: fewer candidates than k, the rest is empty
        }
        if (own)
            a.ms[u] = ((uint64_t)__float_as_uint(ssum) << 32) | __float_as_uint(pm);
    }
}

// lmhead_select: one workgroup per batch element, one wave per beam row.
// A row's log-sum-exp merges its C partials (each lane its pieces in order,
// then DPP reductions in a fixed order), its k best logits come from the union of its
// pieces' top-k lists (exact by the chunk lemma), and each becomes the score
// alive + (logit - lse) in fp32. A finished row offers (eos_id, alive) alone.
// Wave 0 then takes the k best of the beam * k scores, ties to the lower flat
// index, and pads with (-1, -1, -inf).
constexpr int kLSelWaves = 16;
constexpr int kLSelBatch = 4; // partials per lane per batch of loads (slot keys: 4x that)
template <int NG>
__global__ __launch_bounds__(kLanes *kLSelWaves) void lmhead_select(const LmArgs a)
{
    __shared__ uint64_t cand[kLmMaxBeam * kLmMaxK];
    const int tid = threadIdx.x, lane = tid & (kLanes - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kLanes), W = (int)blockDim.x / kLanes;
    const int b = (int)blockIdx.x;
    for (int j = wave; j < a.beam; j += W) {
        const long long row = (long long)b * a.beam + j;
        uint64_t *cj = cand + j * a.k;
        // the first batch of partials and keys, the running score and the finished
        // flag all load at once (a finished row's pieces are read and ignored)
        const uint64_t *ms = a.ms + row * a.C;
        const uint64_t *sl = a.slots + row * a.C * a.k;
        const int nkeys = a.C * a.k;
        uint64_t vm[kLSelBatch], vk[4 * kLSelBatch];
#pragma unroll
        for (int q = 0; q < kLSelBatch; ++q) {
            const int p = q * kLanes + lane;
            vm[q] = p < a.C ? ms[p] : 0ull;
        }
#pragma unroll
        for (int q = 0; q < 4 * kLSelBatch; ++q) {
            const int i = q * kLanes + lane;
            vk[q] = i < nkeys ? sl[i] : 0ull;
        }
        const float alive = a.alive[row];
        if (a.finished != nullptr && a.finished[row] != 0) {
            if (lane < a.k)
                cj[lane] = lane == 0 ? score_key(alive, (uint32_t)j * (uint32_t)a.V + (uint32_t)a.eos_id) : 0ull;
            continue;
        }
        float m = -INFINITY, s = 0.f;
        uint64_t t[NG];
#pragma unroll
        for (int i = 0; i < NG; ++i)
            t[i] = 0ull;
        for (int p0 = 0;;) { // each lane its partials in order of p
#pragma unroll
            for (int q = 0; q < kLSelBatch; ++q)
                if (p0 + q * kLanes + lane < a.C)
                    lse_merge(m, s, __uint_as_float((uint32_t)vm[q]), __uint_as_float((uint32_t)(vm[q] >> 32)));
            p0 += kLSelBatch * kLanes;
            if (p0 >= a.C)
                break;
#pragma unroll
            for (int q = 0; q < kLSelBatch; ++q) {
                const int p = p0 + q * kLanes + lane;
                vm[q] = p < a.C ? ms[p] : 0ull;
            }
        }
        for (int q0 = 0;;) {
#pragma unroll
            for (int q = 0; q < 4 * kLSelBatch; ++q)
                topn_insert<NG>(t, vk[q]);
            q0 += 4 * kLSelBatch * kLanes;
            if (q0 >= nkeys)
                break;
#pragma unroll
            for (int q = 0; q < 4 * kLSelBatch; ++q) {
                const int i = q0 + q * kLanes + lane;
                vk[q] = i < nkeys ? sl[i] : 0ull;
            }
        }
        // the wave's maximum, then the sum of the lanes' sums rescaled to it (DPP, fixed order)
        const float M = wave_max_f(m);
        const float S = wave_sum_f(m == -INFINITY ? 0.f : s * fast_exp2(m - M));
        const float lse = (M + fast_log2(S)) * kLn2;
        for (int i = 0; i < a.k; ++i) {
            const uint64_t best = wave_max_key(t[0]);
            if (best != 0ull && t[0] == best) { // keys are unique: one lane owns it
#pragma unroll
                for (int q = 0; q + 1 < NG; ++q)
                    t[q] = t[q + 1];
                t[NG - 1] = 0ull;
            }
            if (lane == 0)
                cj[i] = best == 0ull ? 0ull : score_key(alive + (entry_x(best) - lse), entry_flat(best));
        }
    }
    __syncthreads();
    if (wave != 0)
        return;
    uint64_t t[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i)
        t[i] = 0ull;
    for (int q = lane; q < a.beam * a.k; q += kLanes)
        topn_insert<NG>(t, cand[q]);
    for (int p = 0; p < a.k; ++p) {
        const uint64_t best = wave_max_key(t[0]);
        if (best != 0ull && t[0] == best) {
#pragma unroll
            for (int q = 0; q + 1 < NG; ++q)
                t[q] = t[q + 1];
            t[NG - 1] = 0ull;
        }
        if (lane == 0) {
            const long long o = (long long)b * a.k + p;
            if (best != 0ull) {
                const uint32_t flat = entry_flat(best), jj = mdiv(flat, a.mv);
                a.out_beam[o] = (int32_t)jj;
                a.out_token[o] = (int32_t)(flat - jj * (uint32_t)a.V);
                a.out_score[o] = entry_x(best);
            } else { // fewer than k candidates at all
                a.out_beam[o] = -1;
                a.out_token[o] = -1;
                a.out_score[o] = -INFINITY;
            }
        }
    }
}
#endif

} // namespace

#if RTOPK_DTYPE == 0

size_t select_lds_bytes(size_t sort_bytes) { return lds_header(kMaxWaves) + sort_bytes; }

size_t group_lds_bytes(int waves, size_t sort_bytes, bool rowlocal, int k, int maxl)
{
    const size_t sel = (size_t)waves * sizeof(SelectLds);
    if (rowlocal) // the waves' regions stay; then the selection's keys and its top-k
        return lds_header(waves) + sel + 8 * ((size_t)rowlocal_keys(waves, k, maxl) + k);
    return lds_header(waves) + (sel > sort_bytes ? sel : sort_bytes);
}

bool supported_vecs_per_thread(int nv)
{
    switch (nv) {
    case 1: case 2: case 3: case 4: case 6: case 8: case 10: case 12:
        return true;
    default:
        return false;
    }
}

hipError_t launch_select(const StepArgs &a, size_t lds_bytes, hipStream_t stream)
{
    hipLaunchKernelGGL(rtopk_select, dim3((unsigned)a.B), dim3(kLanes * kMaxWaves), lds_bytes, stream, a);
    return hipGetLastError();
}

hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t marker, uint32_t *out, hipStream_t stream)
{
    const size_t n16 = bytes / 16;
    const size_t per = (size_t)kReadThreads * kReadVecs;
    const size_t blocks = (n16 + per - 1) / per;
    if (blocks == 0)
        return hipSuccess;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(read_probe, dim3((unsigned)blocks), dim3(kReadThreads), 0, stream,
                       static_cast<const u32x4 *>(src), n16, marker, out);
    return hipGetLastError();
}

hipError_t launch_read_probe_shape(const void *src, size_t bytes, int vecs, int threads, uint32_t marker,
                                   uint32_t *out, hipStream_t stream)
{
    const size_t n16 = bytes / 16;
    const size_t per = (size_t)threads * (size_t)vecs;
    const size_t blocks = (n16 + per - 1) / per;
    if (blocks == 0)
        return hipSuccess;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    const u32x4 *s16 = static_cast<const u32x4 *>(src);
    const dim3 g((unsigned)blocks), b((unsigned)threads);
    switch (vecs) {
    case 1: hipLaunchKernelGGL(read_probe_shape<1>, g, b, 0, stream, s16, n16, marker, out); break;
    case 2: hipLaunchKernelGGL(read_probe_shape<2>, g, b, 0, stream, s16, n16, marker, out); break;
    case 4: hipLaunchKernelGGL(read_probe_shape<4>, g, b, 0, stream, s16, n16, marker, out); break;
    case 8: hipLaunchKernelGGL(read_probe_shape<8>, g, b, 0, stream, s16, n16, marker, out); break;
    case 10: hipLaunchKernelGGL(read_probe_shape<10>, g, b, 0, stream, s16, n16, marker, out); break;
    case 16: hipLaunchKernelGGL(read_probe_shape<16>, g, b, 0, stream, s16, n16, marker, out); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream)
{
    const size_t n = bytes / 4;
    unsigned blocks = (unsigned)((n + 255) / 256);
    if (blocks > 1024)
        blocks = 1024;
    if (blocks == 0)
        blocks = 1;
    hipLaunchKernelGGL(zero_fill, dim3(blocks), dim3(256), 0, stream, (uint32_t *)p, n);
    return hipGetLastError();
}
#endif

#if RTOPK_DTYPE == 2
hipError_t launch_lmhead(const LmArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)(a.mtiles * a.C)), block(kLThreads);
    const dim3 sgrid((unsigned)a.B), sblock(kLanes * (a.beam < kLSelWaves ? a.beam : kLSelWaves));
    switch (a.ngroups) {
    case 1: hipLaunchKernelGGL(lmhead_tiles<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(lmhead_tiles<2>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(lmhead_tiles<4>, grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL(lmhead_tiles<8>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    switch (a.ngroups) {
    case 1: hipLaunchKernelGGL(lmhead_select<1>, sgrid, sblock, 0, s, a); break;
    case 2: hipLaunchKernelGGL(lmhead_select<2>, sgrid, sblock, 0, s, a); break;
    case 4: hipLaunchKernelGGL(lmhead_select<4>, sgrid, sblock, 0, s, a); break;
    default: hipLaunchKernelGGL(lmhead_select<8>, sgrid, sblock, 0, s, a); break;
    }
    return hipGetLastError();
}
#endif

template <>
hipError_t launch_dtype<RTOPK_DTYPE>(const StepArgs &a, int nv, size_t lds, hipStream_t s)
{
    constexpr int DT = RTOPK_DTYPE;
    const long long pieces = (long long)a.B * a.beam * a.chunks;
    const dim3 grid((unsigned)((pieces + a.waves - 1) / a.waves)), block(kLanes * a.waves);
    const bool aligned = a.align_elems == 0 && a.vshard % Traits<DT>::epv == 0;
    const int rl = a.rowlocal == 0 ? 0 : a.k > 8 ? 2 : 1;
    switch (nv) {
#define RTOPK_CASE(N)                                                                      \
    case N:                                                                                \
        if (aligned && rl == 2)                                                            \
            hipLaunchKernelGGL((rtopk_step<DT, N, true, 2>), grid, block, lds, s, a);      \
        else if (aligned && rl == 1)                                                       \
            hipLaunchKernelGGL((rtopk_step<DT, N, true, 1>), grid, block, lds, s, a);      \
        else if (aligned)                                                                  \
            hipLaunchKernelGGL((rtopk_step<DT, N, true, 0>), grid, block, lds, s, a);      \
        else if (rl == 2)                                                                  \
            hipLaunchKernelGGL((rtopk_step<DT, N, false, 2>), grid, block, lds, s, a);     \
        else if (rl == 1)                                                                  \
            hipLaunchKernelGGL((rtopk_step<DT, N, false, 1>), grid, block, lds, s, a);     \
        else                                                                               \
            hipLaunchKernelGGL((rtopk_step<DT, N, false, 0>), grid, block, lds, s, a);     \
        break;
        RTOPK_CASE(1) RTOPK_CASE(2) RTOPK_CASE(3) RTOPK_CASE(4) RTOPK_CASE(6) RTOPK_CASE(8)
        RTOPK_CASE(10) RTOPK_CASE(12)
#undef RTOPK_CASE
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace rtopk
