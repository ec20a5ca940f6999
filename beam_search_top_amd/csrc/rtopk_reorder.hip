// gfx950 (CDNA4) kernel of the cache refresh that follows a selection step.
//
// The LightSeq inference article's hierarchical-decoding passage ends the
// decode step with a cache update once the top-k are known, and its profile
// puts that update at 10% (fp32) / 6% (fp16) of inference latency. With a
// beam-major cache -- nslabs slabs (layers x {keys, values}) of B*beam rows of
// row_bytes bytes -- the update is a gather: new beam j of batch element b
// takes the row of old beam beam_ids[b][j].
//
// MI355X design: a pure HBM copy (read each selected row once, write each
// destination row once), so no LDS and no MFMA. One workgroup of 256 lanes
// moves one chunk of up to 16 KiB of one source row to every destination row
// that takes it: every lane issues its four 16-byte non-temporal loads before
// its first store, so each wave keeps 4 KiB in flight, and a launch at the
// cache sizes of a decoder step has tens of thousands of workgroups to spread
// over the 256 CUs. The beam ids are scalar loads. Rows that are not 16-byte
// aligned (or whose size is not a multiple of 16) take a byte-wise variant.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rtopk_internal.h"

namespace rtopk {
namespace {

constexpr int kReorderThreads = 256;
constexpr int kReorderVecs = 4; // 16-byte vectors per lane per chunk
constexpr long long kReorderChunk = (long long)kReorderThreads * kReorderVecs * 16;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Workgroup w moves chunk c = w mod cpr of source row r = w / cpr,
// r = (s * B + b) * beam + i, to every destination row of the same slab and
// batch element whose beam continues old beam i: each source byte is read
// from HBM once however many beams continue it, and a beam that no new beam
// continues is not read at all.
template <bool VEC>
__global__ __launch_bounds__(kReorderThreads) void beam_reorder(const uint8_t *__restrict__ src,
                                                                uint8_t *__restrict__ dst, long long row_bytes,
                                                                int beam, long long rows_per_slab,
                                                                const int32_t *__restrict__ ids, int ld,
                                                                long long cpr)
{
    const long long w = blockIdx.x;
    const long long r = w / cpr;
    const long long c = w - r * cpr;
    const long long rb = r % rows_per_slab; // b * beam + i
    const long long b = rb / beam, i = rb - b * beam;
    const int32_t *idb = ids + b * ld;
    int first = -1; // the first destination beam that continues beam i
    for (int j = 0; j < beam; ++j) {
        if (idb[j] == (int32_t)i) {
            first = j;
            break;
        }
    }
    if (first < 0) // no new beam continues old beam i
        return;
    const uint8_t *s = src + r * row_bytes + c * kReorderChunk;
    uint8_t *drow = dst + (r - i) * row_bytes + c * kReorderChunk; // destination row of beam 0
    const long long left = row_bytes - c * kReorderChunk;        // bytes of this row from the chunk start
    if constexpr (VEC) {
        const u32x4 *s4 = reinterpret_cast<const u32x4 *>(s);
        const long long n4 = left / 16;
        u32x4 v[kReorderVecs];
#pragma unroll
        for (int q0 = 0; q0 < kReorderVecs; ++q0) {
            const long long q = (long long)q0 * kReorderThreads + threadIdx.x;
            v[q0] = q < n4 ? __builtin_nontemporal_load(s4 + q) : u32x4{0u, 0u, 0u, 0u};
        }
        for (int j = first; j < beam; ++j) {
            if (idb[j] != (int32_t)i)
                continue;
            u32x4 *d4 = reinterpret_cast<u32x4 *>(drow + (long long)j * row_bytes);
#pragma unroll
            for (int q0 = 0; q0 < kReorderVecs; ++q0) {
                const long long q = (long long)q0 * kReorderThreads + threadIdx.x;
                if (q < n4)
                    __builtin_nontemporal_store(v[q0], d4 + q);
            }
        }
    } else {
        const long long n = left < kReorderChunk ? left : kReorderChunk;
        for (int j = first; j < beam; ++j) {
            if (idb[j] != (int32_t)i)
                continue;
            uint8_t *d = drow + (long long)j * row_bytes;
            for (long long q = threadIdx.x; q < n; q += kReorderThreads)
                d[q] = s[q];
        }
    }
}

} // namespace

long long reorder_chunk_bytes() { return kReorderChunk; }

hipError_t launch_beam_reorder(const void *src, void *dst, long long nslabs, int B, int beam, long long row_bytes,
                               const int32_t *ids, int ld, hipStream_t stream)
{
    const long long cpr = (row_bytes + kReorderChunk - 1) / kReorderChunk;
    const long long rows_per_slab = (long long)B * beam;
    const long long blocks = nslabs * rows_per_slab * cpr;
    if (blocks <= 0 || blocks > 0x7fffffffLL)
        return hipErrorInvalidValue;
    const bool vec = ((uintptr_t)src % 16 == 0) && ((uintptr_t)dst % 16 == 0) && row_bytes % 16 == 0;
    if (vec)
        hipLaunchKernelGGL(beam_reorder<true>, dim3((unsigned)blocks), dim3(kReorderThreads), 0, stream,
                           static_cast<const uint8_t *>(src), static_cast<uint8_t *>(dst), row_bytes, beam,
                           rows_per_slab, ids, ld, cpr);
    else
        hipLaunchKernelGGL(beam_reorder<false>, dim3((unsigned)blocks), dim3(kReorderThreads), 0, stream,
                           static_cast<const uint8_t *>(src), static_cast<uint8_t *>(dst), row_bytes, beam,
                           rows_per_slab, ids, ld, cpr);
    return hipGetLastError();
}

} // namespace rtopk
