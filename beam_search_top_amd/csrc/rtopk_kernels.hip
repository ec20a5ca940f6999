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
//    registers (up to 16 x 16 B per thread), where it stays for both passes:
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
//  * The last workgroup of a batch element (agent-scope ticket) merges the
//    per-piece (max, sum) pairs in piece order, applies the tighter per-beam
//    threshold max_c T_c and the batch bound S = max_j (alive_j + T_j -
//    lse_j) (at least k candidates score >= S), and sorts the survivors with
//    an LDS bitonic network on 64-bit keys (score desc, flat index asc).
//    It then zeroes everything its batch element used in the workspace
//    (queue entries, partials, counter, ticket): between calls the workspace
//    is all-zero, whatever the shapes of the calls that share it.
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
    uint32_t nc, qbase;
    float T;
};

struct SortSmem {
    uint64_t keys[kSortTile];
    float lse[kMaxBeam];
    float thr[kMaxBeam];
    float alive[kMaxBeam];
    float fred[kWaves];
    uint64_t kred[kWaves];
    uint32_t ns;
};

union Smem {
    SelectSmem s;
    SortSmem t;
};

__device__ __forceinline__ float block_max_f(float v, float *red, int tid)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        v = fmaxf(v, __shfl_xor(v, d));
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

// ------------------------------------------------------------ passes 1 and 2
// Processes piece c of row (b, j); leaves the piece's candidates in the batch
// element's queue and its (max, sum, threshold) triple in a.part.
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
__device__ void select_piece(const StepArgs &a, SelectSmem &sm, int row, int b, int j, int c, int tid)
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
    // slots are then overwritten with -inf by selects, without branches.
    uint4 d[NV];
    const int qlast = pend - 1;
#pragma unroll
    for (int r = 0; r < NV; ++r) {
        const int q = pbeg + tid + r * kThreads;
        d[r] = src[q < qlast ? q : qlast];
    }
    // slots r < nfull hold valid vectors in every thread of the workgroup
    const int nfull = pend > pbeg ? (pend - pbeg) / kThreads : 0;
#pragma unroll
    for (int r = 0; r < NV; ++r) {
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
    }

    // ---- pass 1: group maxima + online log-sum-exp (base 2), one block of
    // kBlock vectors at a time so that the work follows the arriving data
    typename Tr::Acc acc;
    Tr::init(acc);
    float m2 = -INFINITY, s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int r0 = 0; r0 < NV; r0 += kBlock) {
#pragma unroll
        for (int r = r0; r < r0 + kBlock && r < NV; ++r)
            Tr::update(acc, d[r]);
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
        __builtin_amdgcn_sched_barrier(0);
    }
    float s = s0 + s1;
    const float tmax = Tr::amax(acc);
#pragma unroll
    for (int r = 0; r < NV; ++r)
        opaque(d[r]);

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
#pragma unroll
    for (int f = 0; f < EPV; ++f) {
        if (f < F) {
            for (int dd = 32; dd >= D; dd >>= 1)
                slot[f] = fmaxf(slot[f], __shfl_xor(slot[f], dd));
            if (lane < D)
                sm.gslot[wave][lane * F + f] = slot[f];
        }
    }
#pragma unroll
    for (int dd = 32; dd >= 1; dd >>= 1) {
        float om = __shfl_xor(m2, dd), os = __shfl_xor(s, dd);
        lse_merge(m2, s, om, os);
    }
    if (lane == 0) {
        sm.wm[wave] = m2;
        sm.ws[wave] = s;
    }
    if (tid == 0) {
        sm.nc = 0;
        sm.T = -INFINITY;
    }
    __syncthreads();
    if (tid < ng) {
        float g = sm.gslot[0][tid];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            g = fmaxf(g, sm.gslot[w][tid]);
        sm.gm[tid] = g;
    }
    float pm = 0.f, ps = 0.f;
    if (tid == 0) { // fixed merge order: waves 0..3
        pm = sm.wm[0];
        ps = sm.ws[0];
        for (int w = 1; w < kWaves; ++w)
            lse_merge(pm, ps, sm.wm[w], sm.ws[w]);
    }
    __syncthreads();
    if (tid < ng) { // the k-th largest group maximum
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
    const float T = sm.T;

    // ---- pass 2: stage every valid logit >= T (ballot + prefix, one LDS atomic per wave)
    const bool maybe = tmax >= T;
    if (__ballot(maybe)) {
        int qb0 = pbeg + tid; // opaque: keeps per-element index math inside this cold block
        asm volatile("" : "+v"(qb0));
#pragma unroll
        for (int r = 0; r < NV; ++r) {
            const int q = qb0 + r * kThreads;
            opaque(d[r]); // nothing derived from d[r] is computed before this point
            const bool hv = maybe && q < pend && Tr::vmax(d[r]) >= T;
            if (__ballot(hv)) {
                opaque(d[r]);
#pragma unroll
                for (int i = 0; i < EPV; ++i) {
                    const int t = q * EPV + i - lead;
                    const float x = Tr::elem(d[r], i);
                    const bool hit = hv && (MODE != kGeneral || (t >= 0 && t < a.V)) && x >= T;
                    const uint64_t m = __ballot(hit);
                    if (m) {
                        const int leader = __ffsll((unsigned long long)m) - 1;
                        uint32_t base = 0;
                        if (lane == leader)
                            base = atomicAdd(&sm.nc, (uint32_t)__popcll(m));
                        base = __shfl(base, leader);
                        if (hit) {
                            const uint32_t pos = base + lane_prefix(m);
                            if (pos < (uint32_t)a.chunk_limit)
                                sm.stage[pos] = ((uint64_t)__float_as_uint(x) << 32) |
                                                (flat0 + (uint32_t)(q * EPV + i));
                        }
                    }
                }
            }
        }
    }
    __syncthreads();
    const uint32_t nc = sm.nc;
    uint32_t emit = nc;
    if (nc > (uint32_t)a.chunk_limit) {
        // overflow: this piece's exact top-k by (logit desc, flat asc)
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
#pragma unroll
                    for (int i = 0; i < EPV; ++i) {
                        const int t = q * EPV + i - lead;
                        if (MODE != kGeneral || (t >= 0 && t < a.V)) {
                            const uint64_t key = score_key(Tr::elem(d[r], i), flat0 + (uint32_t)(q * EPV + i));
                            if (key < prev && key > best)
                                best = key;
                        }
                    }
                }
            }
            best = block_max_u64(best, sm.kred, tid);
            if (tid == 0) {
                const float x = from_ord((uint32_t)(best >> 32));
                const uint32_t flat = 0xffffffffu - (uint32_t)best;
                sm.stage[round] = ((uint64_t)__float_as_uint(x) << 32) | flat;
            }
            prev = best;
        }
    }
    if (tid == 0) {
        sm.qbase = emit ? atomicAdd(&a.count[b], emit) : 0u;
        const long long u = (long long)row * a.chunks + c;
        a.part[u] = make_float4(pm, ps, T, 0.f);
        if (a.dbg_T)
            a.dbg_T[u] = T;
        if (a.dbg_hits)
            a.dbg_hits[u] = nc;
    }
    __syncthreads();
    const uint32_t qb = sm.qbase;
    if ((uint32_t)tid < emit)
        a.queue[(long long)b * a.queue_cap + qb + tid] = sm.stage[tid];
    // waves that stored to global memory make their stores visible device-wide
    // before the workgroup takes its ticket (the barrier does not wait for them)
    if (wave == 0 || (uint32_t)(wave * 64) < emit)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}

// ------------------------------------------------------------ per-batch sort
__device__ void sort_batch(const StepArgs &a, SortSmem &sm, int b, int tid)
{
    const int beam = a.beam, C = a.chunks;
    float bound = -INFINITY;
    for (int jj = tid; jj < beam; jj += kThreads) {
        const int row = b * beam + jj;
        const bool fin = a.finished && a.finished[row];
        const float alv = a.alive[row];
        float lse = __builtin_nanf(""), thr = INFINITY;
        if (!fin) {
            float M = -INFINITY, S = 0.f, Tm = -INFINITY;
            for (int cc = 0; cc < C; ++cc) { // fixed order: pieces 0..C-1
                const float4 p = a.part[(long long)row * C + cc];
                lse_merge(M, S, p.x, p.y);
                Tm = fmaxf(Tm, p.z);
            }
            lse = (M + fast_log2(S)) * kLn2;
            thr = Tm;
            // at least k logits of this beam are >= thr, so at least k
            // candidates score >= alive + (thr - lse)
            bound = fmaxf(bound, alv + (thr - lse));
        }
        sm.lse[jj] = lse;
        sm.thr[jj] = thr;
        sm.alive[jj] = alv;
        if (a.dbg_lse)
            a.dbg_lse[row] = lse;
    }
    if (tid == 0)
        sm.ns = 0;
    bound = block_max_f(bound, sm.fred, tid); // includes barriers
    const uint32_t n = __hip_atomic_load(&a.count[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t *q = a.queue + (long long)b * a.queue_cap;
    for (uint32_t e = tid; e < n; e += kThreads) {
        const uint64_t ent = q[e];
        const float x = __uint_as_float((uint32_t)(ent >> 32));
        const uint32_t flat = (uint32_t)ent;
        const int jj = (int)(flat / (uint32_t)a.V);
        if (x >= sm.thr[jj]) {
            const float sc = sm.alive[jj] + (x - sm.lse[jj]);
            if (sc >= bound) {
                const uint32_t pos = atomicAdd(&sm.ns, 1u);
                if (pos < (uint32_t)kSortTile)
                    sm.keys[pos] = score_key(sc, flat);
            }
        }
    }
    if (a.finished) {
        for (int jj = tid; jj < beam; jj += kThreads) {
            if (a.finished[b * beam + jj]) {
                const float sc = sm.alive[jj];
                if (sc >= bound) {
                    const uint32_t pos = atomicAdd(&sm.ns, 1u);
                    if (pos < (uint32_t)kSortTile)
                        sm.keys[pos] = score_key(sc, (uint32_t)jj * (uint32_t)a.V + (uint32_t)a.eos_id);
                }
            }
        }
    }
    __syncthreads();
    const uint32_t ns = sm.ns;
    if (ns <= (uint32_t)kSortTile) {
        int P = 2;
        while ((uint32_t)P < ns)
            P <<= 1;
        for (int i = (int)ns + tid; i < P; i += kThreads)
            sm.keys[i] = 0ull; // below every real key
        __syncthreads();
        bitonic_desc(sm.keys, P, tid);
    } else {
        // more survivors than one LDS tile: k rounds of block argmax over them
        uint64_t prev = ~0ull;
        for (int round = 0; round < a.k; ++round) {
            uint64_t best = 0;
            for (uint32_t e = tid; e < n; e += kThreads) {
                const uint64_t ent = q[e];
                const float x = __uint_as_float((uint32_t)(ent >> 32));
                const uint32_t flat = (uint32_t)ent;
                const int jj = (int)(flat / (uint32_t)a.V);
                if (x >= sm.thr[jj]) {
                    const float sc = sm.alive[jj] + (x - sm.lse[jj]);
                    if (sc >= bound) {
                        const uint64_t key = score_key(sc, flat);
                        if (key < prev && key > best)
                            best = key;
                    }
                }
            }
            if (a.finished) {
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
            if (tid == 0)
                sm.keys[round] = best;
        }
        __syncthreads();
    }
    for (int p = tid; p < a.k; p += kThreads) {
        const long long o = (long long)b * a.k + p;
        const uint64_t key = sm.keys[p];
        if ((uint32_t)p < ns && key != 0ull) {
            const uint32_t flat = 0xffffffffu - (uint32_t)key;
            const uint32_t jj = flat / (uint32_t)a.V;
            a.out_beam[o] = (int32_t)jj;
            a.out_token[o] = (int32_t)(flat - jj * (uint32_t)a.V);
            a.out_score[o] = from_ord((uint32_t)(key >> 32));
        } else {
            a.out_beam[o] = -1;
            a.out_token[o] = -1;
            a.out_score[o] = -INFINITY;
        }
    }
    if (a.dbg_queue)
        for (uint32_t e = tid; e < n; e += kThreads)
            a.dbg_queue[(long long)b * a.queue_cap + e] = q[e];
    // Leave every workspace byte this batch element used at zero, so the
    // workspace is all-zero between calls whatever shape comes next. Each
    // thread clears only queue entries it read itself; the partials were read
    // before the barriers above.
    uint64_t *qw = a.queue + (long long)b * a.queue_cap;
    for (uint32_t e = tid; e < n; e += kThreads)
        qw[e] = 0ull;
    for (int u = tid; u < beam * C; u += kThreads)
        a.part[(long long)b * beam * C + u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid == 0) {
        if (a.dbg_count)
            a.dbg_count[b] = n;
        a.count[b] = 0u;
        a.ticket[b] = 0u;
    }
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
        select_piece<DT, NV, ALIGNED ? kAligned : kGeneral>(a, sm.s, row, b, j, c, tid);
    __syncthreads();
    if (tid == 0) {
        const uint32_t old =
            __hip_atomic_fetch_add(&a.ticket[b], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        is_last = old == (uint32_t)(a.beam * a.chunks - 1);
    }
    __syncthreads();
    if (!is_last)
        return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
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
    case 1: case 2: case 3: case 4: case 6: case 8: case 10: case 12: case 16:
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
        RTOPK_CASE(10) RTOPK_CASE(12) RTOPK_CASE(16)
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
