// Scratch memory of bitlinear_forward_noalloc: a fixed array in this
// library's device code, one copy per GPU, in place of the caller's
// workspace.  For callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The array's name is not a device address in host code: its address on a
// device comes from hipGetSymbolAddress with that device current, looked up
// once per device on the first call there and kept.  Every call on a GPU
// uses that GPU's one copy, so such calls must not overlap in time on one
// GPU (they would race on it).  None of the kernels needs it zeroed: split-K
// partial tiles and expanded rows are written in full before they are read.
#include <mutex>

#include "kernels.hpp"

namespace bl {
namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_mu;
uint8_t *g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, uint8_t **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return e;
        if (sdev != dev) return hipErrorInvalidDevice;   // the stream's device must be current
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = static_cast<uint8_t *>(p);
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace bl
