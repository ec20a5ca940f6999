// gfx950 (CDNA4) kernels of the hierarchical beam-search selection step.
//
// The method is the LightSeq inference article's hierarchical decoding
// (its passage on the logit rough-select kernel and the candidate queue):
//  pass 1  per beam, split the logits into k groups, take each group's
//          maximum and the minimum of those maxima -- the "R-top-k", never
//          above the k-th largest logit -- and compute log_sum_exp in the
//          same traversal;
//  pass 2  keep every logit >= R-top-k in a device-memory candidate queue,
//          written concurrently by many threads, one segment per batch
//          element;
//  sort    one small sort of each batch element's queue gives its exact top-k.
//
// MI355X design (one launch per step, kernel `rtopk_step`):
//  * A beam row is cut into `chunks` pieces; one 256-thread workgroup owns a
//    piece and streams it once from HBM with 16-byte loads straight into
//    registers (up to 12 x 16 B per thread), where it stays for both passes:
//    HBM is read exactly once. Registers instead of LDS: the 512 KB VGPR file
//    per CU holds more than the 160 KB LDS, and pass 2 compares straight from
//    registers without an LDS round trip.
//  * Pass 1 keeps one running maximum per element slot (packed v_pk_max_f16
//    for fp16), which yields the group maxima, with groups = element index
//    mod ngroups; the log-sum-exp is accumulated online in fp32 in base 2,
//    rescaled once per block of 4 vectors, with v_fma_mix/v_exp_f32.
//  * Groups are combined by wave butterflies and LDS; the piece threshold is
//    the k-th largest of the ngroups (k rounded up to a power of two) group
//    maxima, i.e. the R-top-k itself when k is a power of two.
//  * Pass 2 skips every thread whose maximum is below the threshold; hits are
//    appended to an LDS stage with a wave ballot, mbcnt prefix and one LDS
//    atomic per wave, then reserved in the batch element's global queue with
//    one atomic per workgroup. A piece with more than `chunk_limit` hits
//    emits only its own exact top-k (k rounds of block argmax), which keeps
//    the result exact: a beam's top-k within any piece is inside that
//    piece's own top-k.
//  * The last workgroup of a batch element (device-scope ticket) merges the
//    per-piece (max, sum) pairs in piece order, applies the tighter per-beam
//    threshold max_c T_c and the batch bound S = max_j (alive_j + T_j -
//    lse_j) (at least k candidates score >= S), and sorts the survivors with
//    an LDS bitonic network on 64-bit keys (score desc, flat index asc).
//    It then puts its ticket back to zero; tickets live in a region of the
//    workspace that no shape uses for anything else.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rtopk_internal.h"

// No implicit a*b+c contraction: a score and the bound it is compared with
// must round identically (explicit fmaf calls still map to FMA instructions).
#pragma clang fp contract(off)

namespace rtopk {
namespace {

constexpr int kWaves = kThreads / 64;
constexpr int kBlock = 4; // vectors per online log-sum-exp rescale
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Merge of two base-2 log-sum-exp partials (m = max in log2 units, s = sum of
// 2^(x - m)). Symmetric in its arguments, so butterfly lanes agree bit for bit.
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

// Cross-workgroup data (queue entries, partials, counters) moves only through
// agent-scope atomic stores and loads, which gfx950 issues with sc1: they are
// performed at the device coherence point, past the per-XCD L2s, so no L2
// writeback (buffer_wbl2) or invalidate (buffer_inv) is ever needed. A writer
// drains its own stores (s_waitcnt vmcnt(0)) before its workgroup takes the
// ticket; the compiler barriers keep the stores on their side of the wait.
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
__device__ __forceinline__ uint32_t get32(const uint32_t *p)
{
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void drain_stores()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0); // vmcnt(0) expcnt(0) lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int d)
{
    uint32_t lo = __shfl_xor((uint32_t)v, d);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), d);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t lane_prefix(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
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
    __device__ static float vmax(const uint4 &d)
    {
        return fmaxf(fmaxf(elem(d, 0), elem(d, 1)), fmaxf(elem(d, 2), elem(d, 3)));
    }
};

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
    __device__ static float vmax(const uint4 &d)
    {
        half2v t = __builtin_elementwise_max(__builtin_elementwise_max(pair(d, 0), pair(d, 1)),
                                             __builtin_elementwise_max(pair(d, 2), pair(d, 3)));
        return fmaxf((float)t.x, (float)t.y);
    }
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
    __device__ static float vmax(const uint4 &d)
    {
        float m = elem(d, 0);
#pragma unroll
        for (int i = 1; i < 8; ++i)
            m = fmaxf(m, elem(d, i));
        return m;
    }
};

// ---------------------------------------------------------------- shared memory
struct SelectSmem {
    float gslot[kWaves][64]; // per-wave group maxima
    float gm[64];            // group maxima of the piece
    float wm[kWaves], ws[kWaves];
    uint64_t stage[kMaxChunkLimit];
    uint64_t kred[kWaves];
    uint32_t nc;
    float T;
};

struct SortSmem {
    uint64_t keys[kSortKeys]; // survivors' sort keys
    uint16_t pn[kMaxPieces];  // candidates per piece
    float lse[kMaxBeam], thr[kMaxBeam], alive[kMaxBeam];
    float fred[kWaves];
    uint64_t kred[kWaves];
    uint32_t ns, ndbg;
};

union Smem {
    SelectSmem s;
    SortSmem t;
};

// Wave-wide reductions with DPP row operations (VALU only, no LDS): swap
// neighbours (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1), mirror
// within 8 lanes, mirror within 16 lanes -- after which every lane of a
// 16-lane row holds the row's total -- then the four row totals are combined
// in a fixed order from readlanes. Each step combines the same two values on
// both partner lanes, so the result is identical on every lane and from run
// to run.
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
__device__ __forceinline__ float wave_sum_f(float v)
{
    v = v + dpp_f<0xb1>(v);
    v = v + dpp_f<0x4e>(v);
    v = v + dpp_f<0x141>(v);
    v = v + dpp_f<0x140>(v);
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ float block_max_f(float v, float *red, int tid)
{
    v = wave_max_f(v);
    if ((tid & 63) == 0)
        red[tid >> 6] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
        r = fmaxf(r, red[w]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t *red, int tid)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        uint64_t o = shfl_xor_u64(v, d);
        v = o > v ? o : v;
    }
    if ((tid & 63) == 0)
        red[tid >> 6] = v;
    __syncthreads();
    uint64_t r = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
        r = red[w] > r ? red[w] : r;
    __syncthreads();
    return r;
}

// Descending bitonic sort of keys[0..P), P a power of two, whole workgroup.
__device__ void bitonic_desc(uint64_t *keys, int P, int tid)
{
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < (P >> 1); i += kThreads) {
                int lo = 2 * i - (i & (stride - 1));
                int hi = lo + stride;
                bool desc = (lo & size) == 0;
                uint64_t x = keys[lo], y = keys[hi];
                if ((x < y) == desc) {
                    keys[lo] = y;
                    keys[hi] = x;
                }
            }
            __syncthreads();
        }
    }
}

// A candidate slot holds the candidate's sort key by logit, score_key(x, flat):
// the order-preserving bits of the logit above 0xffffffff - flat.
__device__ __forceinline__ float entry_x(uint64_t e) { return from_ord((uint32_t)(e >> 32)); }
__device__ __forceinline__ uint32_t entry_flat(uint64_t e) { return 0xffffffffu - (uint32_t)e; }

// ------------------------------------------------------------ passes 1 and 2
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

template <int DT, int NV, int MODE>
__device__ void select_piece(const StepArgs &a, SelectSmem &sm, int row, int j, int c, int tid)
{
    using Tr = Traits<DT>;
    constexpr int EPV = Tr::epv;
    const int lane = tid & 63, wave = tid >> 6;
    // Vectors are counted in the 16-byte-aligned frame of the tensor; a row
    // starts `lead` elements into its first vector v0 and spans `span` vectors.
    // Everything per thread is 32-bit and relative to the row.
    const long long e0 = (long long)row * a.V + a.align_elems;
    const long long v0 = e0 / EPV;
    const int lead = (int)(e0 - v0 * EPV);
    const int span = (lead + a.V + EPV - 1) / EPV;
    const int pbeg = c * a.vecs_per_chunk;                          // piece start, vectors from v0
    const int pend = pbeg + a.vecs_per_chunk < span ? pbeg + a.vecs_per_chunk : span;
    const uint4 *src = reinterpret_cast<const uint4 *>(a.logits_aligned) + v0;
    const uint32_t flat0 = (uint32_t)j * (uint32_t)a.V - (uint32_t)lead; // flat index of slot 0 of vector 0

    // Unconditional loads (index clamped into the piece) keep each load's
    // distance to its use visible to the waitcnt pass; empty or out-of-row
    // slots are overwritten with -inf at their use, by selects.
    uint4 d[NV];
    const int qlast = pend - 1;
#pragma unroll
    for (int r = 0; r < NV; ++r) {
        const int q = pbeg + tid + r * kThreads;
        d[r] = src[q < qlast ? q : qlast];
    }
    // slots r < nfull hold valid vectors in every thread of the workgroup
    const int nfull = pend > pbeg ? (pend - pbeg) / kThreads : 0;

    // ---- pass 1: group maxima + online log-sum-exp (base 2), one block of
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
            const int q = pbeg + tid + r * kThreads;
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
                    Tr::mask_if(d[r], i, q >= pend || t < 0 || t >= a.V);
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
    float s = s0 + s1;
    const float tmax = Tr::amax(acc);

    // ---- groups: fold slots to F = min(ngroups, EPV), reduce lanes that share groups
    float slot[EPV];
    Tr::slots(acc, slot);
    const int ng = a.ngroups;
    const int F = ng < EPV ? ng : EPV;
    const int D = ng / F; // lanes l and l' hold the same groups iff l = l' mod D
#pragma unroll
    for (int h = EPV / 2; h >= 1; h >>= 1) {
        if (h >= F) {
#pragma unroll
            for (int i = 0; i < h; ++i)
                slot[i] = fmaxf(slot[i], slot[i + h]);
        }
    }
    if (D == 1) { // every lane holds the same groups: plain wave maxima
#pragma unroll
        for (int f = 0; f < EPV; ++f) {
            if (f < F) {
                const float g = wave_max_f(slot[f]);
                if (lane == 0)
                    sm.gslot[wave][f] = g;
            }
        }
    } else { // lanes l and l' share groups iff l = l' mod D: butterflies over distances >= D
#pragma unroll
        for (int f = 0; f < EPV; ++f) {
            if (f < F) {
                for (int dd = 32; dd >= D; dd >>= 1)
                    slot[f] = fmaxf(slot[f], __shfl_xor(slot[f], dd));
                if (lane < D)
                    sm.gslot[wave][lane * F + f] = slot[f];
            }
        }
    }
    // wave log-sum-exp: the wave maximum first, then one rescale per lane and a sum
    const float wm = wave_max_f(m2);
    s = (wm == -INFINITY) ? 0.f : s * fast_exp2(m2 - wm);
    s = wave_sum_f(s);
    if (lane == 0) {
        sm.wm[wave] = wm;
        sm.ws[wave] = s;
    }
    if (tid == 0)
        sm.nc = 0;
    __syncthreads();
    float pm = 0.f, ps = 0.f;
    if (tid == 0) { // fixed merge order: waves 0..3
        pm = sm.wm[0];
        ps = sm.ws[0];
        for (int w = 1; w < kWaves; ++w)
            lse_merge(pm, ps, sm.wm[w], sm.ws[w]);
    }
    float T;
    if (ng == a.k) {
        // the R-top-k: minimum over the groups of the group maxima (each thread reads them all)
        T = INFINITY;
        for (int g = 0; g < ng; ++g) {
            float v = sm.gslot[0][g];
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                v = fmaxf(v, sm.gslot[w][g]);
            T = fminf(T, v);
        }
    } else {
        // k below a power of two: the k-th largest of the ngroups maxima
        if (tid < ng) {
            float g = sm.gslot[0][tid];
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                g = fmaxf(g, sm.gslot[w][tid]);
            sm.gm[tid] = g;
        }
        __syncthreads();
        if (tid < ng) {
            const float v = sm.gm[tid];
            int gt = 0, ge = 0;
            for (int u = 0; u < ng; ++u) {
                const float w = sm.gm[u];
                gt += w > v;
                ge += w >= v;
            }
            if (gt < a.k && a.k <= ge)
                sm.T = v;
        }
        __syncthreads();
        T = sm.T;
    }

    // ---- pass 2: stage the sort key of every valid logit >= T. A lane only
    // examines the element positions (slots) whose running maximum reaches T
    // -- usually none, rarely more than one -- across its vectors: it counts
    // the hits, reserves them with one LDS atomic add (aggregated per wave by
    // the compiler), and writes them.
    if (tmax >= T) {
        int qb0 = pbeg + tid; // opaque: keeps per-element index math inside this cold block
        asm volatile("" : "+v"(qb0));
        float sl[EPV];
        Tr::slots(acc, sl);
        auto hit = [&](int r, int i, float x) {
            const int q = qb0 + r * kThreads;
            const int t = q * EPV + i - lead;
            return x >= T && q < pend && (MODE != kGeneral || (t >= 0 && t < a.V));
        };
        uint32_t cnt = 0;
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
            if (sl[i] >= T) {
#pragma unroll
                for (int r = 0; r < NV; ++r) {
                    opaque(d[r]);
                    cnt += hit(r, i, Tr::elem(d[r], i));
                }
            }
        }
        uint32_t pos = atomicAdd(&sm.nc, cnt);
#pragma unroll
        for (int i = 0; i < EPV; ++i) {
            if (sl[i] >= T) {
#pragma unroll
                for (int r = 0; r < NV; ++r) {
                    opaque(d[r]);
                    const float x = Tr::elem(d[r], i);
                    if (hit(r, i, x)) {
                        if (pos < (uint32_t)a.chunk_limit)
                            sm.stage[pos] = score_key(x, flat0 + (uint32_t)((qb0 + r * kThreads) * EPV + i));
                        ++pos;
                    }
                }
            }
        }
    }
    __syncthreads();
    const uint32_t nc = sm.nc;
    const long long u = (long long)row * a.chunks + c;
    uint64_t *mine = a.slots + u * a.k; // this piece's k candidate slots
    uint32_t emit;
    if (nc <= (uint32_t)a.chunk_limit) {
        // The piece's own top-k by (logit desc, flat asc): only those can be
        // among the batch element's top-k. Keys are distinct, so ranks are
        // unique; slot r receives the key of rank r.
        emit = nc < (uint32_t)a.k ? nc : (uint32_t)a.k;
        if ((uint32_t)tid < nc) {
            const uint64_t key = sm.stage[tid];
            uint32_t rank = tid;
            if (nc > (uint32_t)a.k) {
                rank = 0;
                for (uint32_t i = 0; i < nc; ++i)
                    rank += sm.stage[i] > key;
            }
            if (rank < (uint32_t)a.k)
                put64(&mine[rank], key);
        }
    } else {
        // more candidates than the stage holds: k rounds of block argmax over the registers
        emit = (uint32_t)a.k;
        uint64_t prev = ~0ull;
        for (int round = 0; round < a.k; ++round) {
            uint64_t best = 0;
            int qb0 = pbeg + tid; // opaque per round: no key hoisted out of the round loop
            asm volatile("" : "+v"(qb0));
#pragma unroll
            for (int r = 0; r < NV; ++r) {
                const int q = qb0 + r * kThreads;
                opaque(d[r]);
                if (q < pend) {
#pragma unroll 1
                    for (int i = 0; i < EPV; ++i) {
                        const int t = q * EPV + i - lead;
                        if (MODE != kGeneral || (t >= 0 && t < a.V)) {
                            const uint64_t key = score_key(Tr::elem_rt(d[r], i), flat0 + (uint32_t)(q * EPV + i));
                            if (key < prev && key > best)
                                best = key;
                        }
                    }
                }
            }
            best = block_max_u64(best, sm.kred, tid);
            if (tid == 0)
                put64(&mine[round], best);
            prev = best;
        }
    }
    if (tid == 0) {
        put64(&a.head[2 * u], ((uint64_t)__float_as_uint(ps) << 32) | __float_as_uint(pm));
        put64(&a.head[2 * u + 1], ((uint64_t)emit << 32) | __float_as_uint(T));
        if (a.dbg_T)
            a.dbg_T[u] = T;
        if (a.dbg_hits)
            a.dbg_hits[u] = nc;
    }
    // every store of this workgroup is performed before it takes its ticket
    // (the barrier that follows does not wait for memory)
    drain_stores();
}

// ------------------------------------------------------------ per-batch selection
// Run by the last workgroup of batch element b. One round trip loads every
// piece header plus the first S slots of every piece; the beams' log-sum-exp
// are merged in piece order; candidates are filtered by the per-beam
// threshold and by the batch bound; the k best survivors are found by rank
// counting (or a bitonic sort when there are many).
__device__ void sort_batch(const StepArgs &a, SortSmem &sm, int b, int tid)
{
    const int beam = a.beam, C = a.chunks, L = a.k; // k slots per piece
    const int P = beam * C;
    const long long u0 = (long long)b * P;
    // speculative slice: the first S slots of every piece p with (p+1)*S <= kSpec*kThreads
    constexpr int kSpec = 4;
    int S = kSpec * kThreads / P;
    S = S < 1 ? 1 : (S > 32 ? 32 : S);
    S = S < L ? S : L; // never past the piece's own slots
    const int R = (P * S + kThreads - 1) / kThreads < kSpec ? (P * S + kThreads - 1) / kThreads : kSpec;
    const bool has_fin = a.finished != nullptr;

    // ---- A: per-beam merge of the piece headers (fixed piece order) and the
    // speculative slots; all of these loads are independent of each other
    uint64_t spec[kSpec];
#pragma unroll
    for (int r = 0; r < kSpec; ++r) {
        const int g = tid + r * kThreads;
        spec[r] = 0ull;
        if (r < R && g < P * S) {
            const int p = g / S;
            spec[r] = get64(&a.slots[(u0 + p) * L + (g - p * S)]);
        }
    }
    if (tid == 0) {
        sm.ns = 0;
        sm.ndbg = 0;
    }
    float bound = -INFINITY;
    for (int jj = tid; jj < beam; jj += kThreads) {
        const bool fin = has_fin && a.finished[b * beam + jj];
        const float alv = a.alive[b * beam + jj];
        float lse = __uint_as_float(0x7fc00000u), thr = INFINITY; // NaN marks a finished beam
        if (!fin) {
            float M = -INFINITY, Ssum = 0.f, Tm = -INFINITY;
            const uint64_t *h = a.head + 2 * (u0 + (long long)jj * C);
            for (int c0 = 0; c0 < C; c0 += 8) { // headers of 8 pieces in flight at once
                uint64_t hb[16];
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    hb[i] = c0 + (i >> 1) < C ? get64(&h[2 * c0 + i]) : 0ull;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (c0 + i < C) {
                        lse_merge(M, Ssum, __uint_as_float((uint32_t)hb[2 * i]),
                                  __uint_as_float((uint32_t)(hb[2 * i] >> 32)));
                        Tm = fmaxf(Tm, __uint_as_float((uint32_t)hb[2 * i + 1]));
                        sm.pn[jj * C + c0 + i] = (uint16_t)(hb[2 * i + 1] >> 32);
                    }
                }
            }
            lse = (M + fast_log2(Ssum)) * kLn2;
            thr = Tm;
            // at least k logits of this beam are >= thr, so at least k
            // candidates score >= alive + (thr - lse)
            bound = fmaxf(bound, alv + (thr - lse));
        } else {
            for (int cc = 0; cc < C; ++cc)
                sm.pn[jj * C + cc] = 0;
        }
        sm.lse[jj] = lse;
        sm.thr[jj] = thr;
        sm.alive[jj] = alv;
        if (a.dbg_lse)
            a.dbg_lse[b * beam + jj] = lse;
    }
    bound = block_max_f(bound, sm.fred, tid); // its barriers also publish the tables above

    // ---- B: survivors -> sort keys, from the speculative slice and from the
    // slots past it (loaded here, pieces handled one per thread)
    auto consider = [&](uint64_t ent, int jj) {
        const float x = entry_x(ent);
        if (x >= sm.thr[jj]) {
            const float sc = sm.alive[jj] + (x - sm.lse[jj]);
            if (sc >= bound) {
                const uint32_t pos = atomicAdd(&sm.ns, 1u);
                if (pos < (uint32_t)kSortKeys)
                    sm.keys[pos] = score_key(sc, entry_flat(ent));
            }
        }
    };
#pragma unroll
    for (int r = 0; r < kSpec; ++r) {
        const int g = tid + r * kThreads;
        if (r < R && g < P * S) {
            const int p = g / S;
            if (g - p * S < (int)sm.pn[p]) // slots past a piece's count hold stale data
                consider(spec[r], p / C);
        }
    }
    const int covered = R * kThreads / S; // pieces whose first S slots were loaded above
    for (int p = tid; p < P; p += kThreads) {
        const int n = (int)sm.pn[p];
        const int jj = p / C;
        for (int e0 = p < covered ? S : 0; e0 < n; e0 += 8) { // 8 loads in flight
            uint64_t eb[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                eb[i] = e0 + i < n ? get64(&a.slots[(u0 + p) * L + e0 + i]) : 0ull;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (e0 + i < n)
                    consider(eb[i], jj);
        }
    }
    if (has_fin) {
        for (int jj = tid; jj < beam; jj += kThreads) {
            if (a.finished[b * beam + jj] && sm.alive[jj] >= bound) {
                const uint32_t pos = atomicAdd(&sm.ns, 1u);
                if (pos < (uint32_t)kSortKeys)
                    sm.keys[pos] =
                        score_key(sm.alive[jj], (uint32_t)jj * (uint32_t)a.V + (uint32_t)a.eos_id);
            }
        }
    }
    __syncthreads();
    const uint32_t ns = sm.ns;

    // ---- D: the k best keys, in order
    auto emit_out = [&](int p, uint64_t key) {
        const long long o = (long long)b * a.k + p;
        const uint32_t flat = 0xffffffffu - (uint32_t)key;
        const uint32_t jj = flat / (uint32_t)a.V;
        a.out_beam[o] = (int32_t)jj;
        a.out_token[o] = (int32_t)(flat - jj * (uint32_t)a.V);
        a.out_score[o] = from_ord((uint32_t)(key >> 32));
    };
    if (ns <= (uint32_t)kThreads) {
        // rank counting: keys are distinct (flat indices are), so ranks are a permutation
        if ((uint32_t)tid < ns) {
            const uint64_t mine = sm.keys[tid];
            uint32_t rank = 0;
            for (uint32_t i = 0; i < ns; ++i)
                rank += sm.keys[i] > mine;
            if (rank < (uint32_t)a.k)
                emit_out((int)rank, mine);
        }
    } else if (ns <= (uint32_t)kSortKeys) {
        int Pw = 2;
        while ((uint32_t)Pw < ns)
            Pw <<= 1;
        for (int i = (int)ns + tid; i < Pw; i += kThreads)
            sm.keys[i] = 0ull; // below every real key
        __syncthreads();
        bitonic_desc(sm.keys, Pw, tid);
        for (int p = tid; p < a.k && (uint32_t)p < ns; p += kThreads)
            emit_out(p, sm.keys[p]);
    } else {
        // more survivors than the LDS holds: k rounds of block argmax over every entry
        uint64_t prev = ~0ull;
        for (int round = 0; round < a.k; ++round) {
            uint64_t best = 0;
            for (int p = tid; p < P; p += kThreads) {
                const int jj = p / C;
                const int n = (int)sm.pn[p];
                for (int e = 0; e < n; ++e) {
                    const uint64_t ent = get64(&a.slots[(u0 + p) * L + e]);
                    const float x = entry_x(ent);
                    if (x >= sm.thr[jj]) {
                        const float sc = sm.alive[jj] + (x - sm.lse[jj]);
                        const uint64_t key = score_key(sc, entry_flat(ent));
                        if (sc >= bound && key < prev && key > best)
                            best = key;
                    }
                }
            }
            if (has_fin) {
                for (int jj = tid; jj < beam; jj += kThreads) {
                    if (a.finished[b * beam + jj] && sm.alive[jj] >= bound) {
                        const uint64_t key =
                            score_key(sm.alive[jj], (uint32_t)jj * (uint32_t)a.V + (uint32_t)a.eos_id);
                        if (key < prev && key > best)
                            best = key;
                    }
                }
            }
            best = block_max_u64(best, sm.kred, tid);
            prev = best;
            if (tid == 0 && best != 0ull)
                emit_out(round, best);
        }
    }
    // padding when fewer than k candidates exist at all
    for (int p = (int)ns + tid; p < a.k; p += kThreads) {
        const long long o = (long long)b * a.k + p;
        a.out_beam[o] = -1;
        a.out_token[o] = -1;
        a.out_score[o] = -INFINITY;
    }

    // ---- E: debug copies; the ticket goes back to zero for the next call. Headers
    // and slots need no clearing: every piece of an alive beam rewrites its
    // header before taking its ticket, and slots are read only below a count.
    if (a.dbg_queue || a.dbg_count) {
        __syncthreads();
        uint64_t *dq = a.dbg_queue ? a.dbg_queue + (long long)b * a.queue_cap : nullptr;
        for (int p = tid; p < P; p += kThreads) {
            const int n = (int)sm.pn[p];
            const uint32_t base = atomicAdd(&sm.ndbg, (uint32_t)n);
            if (dq)
                for (int e = 0; e < n; ++e) {
                    const uint64_t ent = get64(&a.slots[(u0 + p) * L + e]);
                    dq[base + e] = ((uint64_t)__float_as_uint(entry_x(ent)) << 32) | entry_flat(ent);
                }
        }
        __syncthreads();
        if (tid == 0 && a.dbg_count)
            a.dbg_count[b] = sm.ndbg;
    }
    if (tid == 0)
        put32(&a.ticket[b], 0u);
}

template <int DT, int NV, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void rtopk_step(const StepArgs a)
{
    __shared__ Smem sm;
    __shared__ uint32_t is_last;
    const int tid = threadIdx.x;
    const int u = blockIdx.x;
    const int c = u % a.chunks;
    const int row = u / a.chunks;
    const int b = row / a.beam;
    const int j = row - b * a.beam;
    const bool fin = a.finished && a.finished[row];
    if (!fin)
        select_piece<DT, NV, ALIGNED ? kAligned : kGeneral>(a, sm.s, row, j, c, tid);
    __syncthreads();
    if (tid == 0) {
        const uint32_t old =
            __hip_atomic_fetch_add(&a.ticket[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = old == (uint32_t)(a.beam * a.chunks - 1); // every piece of b has published
    }
    __syncthreads();
    if (!is_last)
        return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    sort_batch(a, sm.t, b, tid);
}

__global__ void zero_fill(uint32_t *p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

} // namespace

bool supported_vecs_per_thread(int nv)
{
    switch (nv) {
    case 1: case 2: case 3: case 4: case 6: case 8: case 10: case 12:
        return true;
    default:
        return false;
    }
}

template <int DT>
static hipError_t launch_dt(const StepArgs &a, int nv, hipStream_t s)
{
    const dim3 grid((unsigned)((long long)a.B * a.beam * a.chunks)), block(kThreads);
    const bool aligned = a.align_elems == 0 && a.V % Traits<DT>::epv == 0;
    switch (nv) {
#define RTOPK_CASE(N)                                                              \
    case N:                                                                        \
        if (aligned)                                                               \
            hipLaunchKernelGGL((rtopk_step<DT, N, true>), grid, block, 0, s, a);   \
        else                                                                       \
            hipLaunchKernelGGL((rtopk_step<DT, N, false>), grid, block, 0, s, a);  \
        break;
        RTOPK_CASE(1) RTOPK_CASE(2) RTOPK_CASE(3) RTOPK_CASE(4) RTOPK_CASE(6) RTOPK_CASE(8)
        RTOPK_CASE(10) RTOPK_CASE(12)
#undef RTOPK_CASE
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_step(const StepArgs &a, int dtype, int vecs_per_thread, hipStream_t stream)
{
    switch (dtype) {
    case 0:
        return launch_dt<0>(a, vecs_per_thread, stream);
    case 1:
        return launch_dt<1>(a, vecs_per_thread, stream);
    case 2:
        return launch_dt<2>(a, vecs_per_thread, stream);
    default:
        return hipErrorInvalidValue;
    }
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

} // namespace rtopk
