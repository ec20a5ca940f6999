// rtopk_beam_step_noalloc: the selection step with its workspace in a
// file-scope device array instead of a library- or caller-allocated buffer,
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array is zero when the code object is loaded, and every completed call
// leaves the part of it that must start at zero (tickets, status words,
// mailbox) zero again. Each GPU holds its own copy until the process ends.
// Its device address is looked up once per device with hipGetSymbolAddress;
// host code never passes the array's name itself to a kernel.
#include "rtopk.h"
#include "rtopk_internal.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>
#include <string>

namespace {

constexpr size_t kScratchBytes = RTOPK_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0 && kScratchBytes >= rtopk::kWsFixedBytes, "scratch holds the fixed region");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices]; // the device address of `scratch` on each device, once looked up

} // namespace

namespace rtopk {

// The device address of the current device's scratch, looked up on first use
// with that device current; nullptr (and the HIP error) if that fails.
void *noalloc_scratch(int dev, hipError_t *err)
{
    *err = hipSuccess;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return nullptr;
        }
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

// The scratch of `dev` if a call has used it, else nullptr (no lookup).
void *noalloc_scratch_if_used(int dev)
{
    if (dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    return g_ptr[dev];
}

} // namespace rtopk

extern "C" int rtopk_beam_step_noalloc(const void *logits, int dtype, const float *alive_scores,
                                       const uint8_t *finished_mask, int B, int beam, int V, int k, int eos_id,
                                       int32_t *out_beam_ids, int32_t *out_token_ids, float *out_scores,
                                       void *stream)
{
    const size_t need = rtopk_workspace_bytes(B, beam, V, k, dtype);
    if (need > kScratchBytes)
        return rtopk::set_error(RTOPK_ENOMEM,
                                "noalloc step: this shape needs %zu bytes of workspace, more than the %zu bytes of "
                                "the static scratch; use rtopk_beam_step_ws with a caller workspace",
                                need, kScratchBytes);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return rtopk::set_error(RTOPK_EHIP, "noalloc step: hipGetDevice: %s", hipGetErrorString(e));
    void *ws = rtopk::noalloc_scratch(dev, &e);
    if (!ws)
        return rtopk::set_error(RTOPK_EHIP, "noalloc step: hipGetSymbolAddress of the scratch on device %d: %s", dev,
                                hipGetErrorString(e));
    // validation (sizes, pointers, dtype, eos) is that of the workspace entry point
    return rtopk_beam_step_ws(logits, dtype, alive_scores, finished_mask, B, beam, V, k, eos_id, out_beam_ids,
                              out_token_ids, out_scores, ws, kScratchBytes, stream);
}
