// gfx950 (CDNA4) kernel of top-k sampling after the R-top-k selection.
//
// The LightSeq inference article reports sampling-decode speedups next to its
// beam-search ones; its hierarchical decoding (R-top-k filter, candidate
// queue, one small sort) gives the exact top-k of every row either way. For
// sampling, each row r of logits is its own batch element with one beam and a
// zero running score: the selection step then returns its top-k tokens with
// scores x - lse(row), best first. This kernel draws one of them from the
// top-k distribution renormalised at temperature tau:
//     w_i = exp((s_i - s_1) / tau),  S = w_1 + ... + w_k (in rank order),
//     u   = 24 high bits of Philox4x64-10(counter (r, step, 0, 0), key (seed, 0))
//           word 0, times 2^-24,
//     i   = the first rank with u * S < w_1 + ... + w_i (the last rank if none),
// and returns the token of rank i and log(w_i / S). All in fp32, sums in rank
// order. One wave per row; the k <= 64 candidates sit one per lane.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rtopk_internal.h"

namespace rtopk {
namespace {

constexpr int kSampleWaves = 4;

// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC 2011): ten rounds of two 64x64->128 multiplies by the
// round constants, the high halves xored with the other counter words and the
// key, the key bumped by the Weyl constants between rounds. Returns word 0.
__device__ __forceinline__ uint64_t philox4x64_w0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                                                  uint64_t k1)
{
    constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
        const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
        const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += W0;
        k1 += W1;
    }
    return c0;
}

__global__ __launch_bounds__(64 * kSampleWaves) void topk_sample(const int32_t *__restrict__ tok,
                                                                 const float *__restrict__ sc, int R, int k,
                                                                 float tau, uint64_t seed, uint64_t step,
                                                                 int32_t *out_tok, float *out_lp)
{
    const int lane = threadIdx.x & 63;
    const int row = (int)blockIdx.x * kSampleWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    if (row >= R)
        return;
    const bool own = lane < k;
    const float s = own ? sc[(long long)row * k + lane] : 0.f;
    const float s1 = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(s))); // rank 1
    const float w = own ? expf((s - s1) / tau) : 0.f;
    // prefix sums in rank order, one add at a time (the order fixes the rounding)
    float acc = 0.f, c = 0.f;
    for (int i = 0; i < k; ++i) {
        acc += __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(w), i));
        c = lane == i ? acc : c;
    }
    const float S = acc;
    const uint64_t x0 = philox4x64_w0((uint64_t)row, step, 0ull, 0ull, seed, 0ull);
    const float u = (float)(uint32_t)(x0 >> 40) * 0x1p-24f;
    const float t = u * S;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(own && t < c);
    const int i = hit ? __builtin_ctzll(hit) : k - 1;
    if (lane == i) {
        out_tok[row] = tok[(long long)row * k + i];
        out_lp[row] = logf(w / S);
    }
}

} // namespace

hipError_t launch_topk_sample(const int32_t *tok, const float *sc, int R, int k, float tau, uint64_t seed,
                              uint64_t step, int32_t *out_tok, float *out_lp, hipStream_t stream)
{
    const unsigned blocks = (unsigned)((R + kSampleWaves - 1) / kSampleWaves);
    hipLaunchKernelGGL(topk_sample, dim3(blocks), dim3(64 * kSampleWaves), 0, stream, tok, sc, R, k, tau, seed,
                       step, out_tok, out_lp);
    return hipGetLastError();
}

} // namespace rtopk
