// noalloc: the static scratch array behind indexer_score_topk_noalloc.
//
// Callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid allocation) get the indexer's
// scratch space from one file-scope device array instead of a caller
// workspace.  The array is a program-scope variable of this code object, so
// every GPU the library runs on holds its own copy, at its own address,
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: the device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels.  Nothing in the array needs to start at zero: the
// kernels ignore the workspace contents on entry.  Every call on one GPU
// shares that GPU's array, so calls that overlap on one GPU (different
// streams, or threads without ordering) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace dsai {
namespace {

constexpr size_t kScratchBytes = size_t(256) << 20;  // 256 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

// The current device must be `device`.
hipError_t noalloc_scratch(int device, void **ptr)
{
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_ptr[device] = p;
    }
    *ptr = g_ptr[device];
    return hipSuccess;
}

}  // namespace dsai
