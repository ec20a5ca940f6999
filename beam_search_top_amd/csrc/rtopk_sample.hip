// gfx950 (CDNA4) kernel of top-k sampling after the R-top-k selection, for
// the shapes whose selection does not draw itself: one wave per row reads
// the row's k best tokens and scores (best first, from the selection step
// with one beam and a zero running score) and draws one (rtopk_draw.h).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rtopk_draw.h"
#include "rtopk_internal.h"

namespace rtopk {
namespace {

constexpr int kSampleWaves = 4;

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
    const int32_t t = own ? tok[(long long)row * k + lane] : -1;
    draw_topk_row(s, t, k, lane, row, tau, seed, step, out_tok, out_lp);
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
