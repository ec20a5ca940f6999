// The draw of top-k sampling, shared by the stand-alone draw kernel and the
// row-local selection kernels that draw right after their per-row top-k.
//
// The LightSeq inference article reports sampling-decode speedups next to its
// beam-search ones; its hierarchical decoding gives every row's exact top-k
// either way. Row r's k best tokens, with scores s_i = x_i - lse(row) best
// first, are drawn from the top-k distribution renormalised at temperature
// tau:
//     w_i = exp((s_i - s_1) / tau),  S = w_1 + ... + w_k (in rank order),
//     u   = 24 high bits of Philox4x64-10(counter (r, step, 0, 0), key (seed, 0))
//           word 0, times 2^-24,
//     i   = the first rank with u * S < w_1 + ... + w_i (the last rank if none),
// and the token of rank i is returned with log(w_i / S). All in fp32, sums in
// rank order.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace rtopk {

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

// One wave draws for row `row`: lane i < k holds the score s and token of
// rank i (padding ranks: -inf and -1). Every lane of the wave must be active.
__device__ __forceinline__ void draw_topk_row(float s, int32_t tok, int k, int lane, long long row, float tau,
                                              uint64_t seed, uint64_t step, int32_t *out_tok, float *out_lp)
{
    const bool own = lane < k;
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
        out_tok[row] = tok;
        out_lp[row] = logf(w / S);
    }
}

} // namespace rtopk
