// moe_layer_noalloc: the whole layer with its workspace in a fixed device
// array of this library, for callers that cannot allocate device memory
// (code under stream capture into a graph, tight serving loops, harnesses
// that forbid allocation). The kernels are moe_layer's; only the workspace
// differs.
//
// The array `scratch` is a file-scope __device__ object: every GPU the library
// runs on holds its own copy, at its own address, from the first use of the
// code object on that GPU until the process ends. In host code its name is
// only a host-side stand-in, so the device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and kept; kernels
// only ever receive that address. Every call on one GPU shares that GPU's
// array: calls that overlap in time on the same GPU race on it, and nothing
// is carried from one call to the next (every intermediate is written before
// it is read).
#include <hip/hip_runtime.h>
#include <mutex>

#include "moe_internal.h"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};

// The device address of this device's copy of `scratch`, looked up on the
// first call on the device. Returns null (and the HIP error in *err) on failure.
void* scratch_for_current_device(hipError_t* err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> hold(g_lock);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess || !p) {
            if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

MOE_EXPORT int32_t moe_layer_noalloc(const moe_layer_args* a, hipStream_t stream) {
    if (!a) return MOE_ERR_NULL;
    const int s = a->shared_w1 ? 1 : 0;
    const size_t need = moe_layer_workspace_size(a->T, a->E_tot, a->k, a->E_loc, a->H, a->I, s, a->flags);
    if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    // everything else moe_layer validates from the scalars alone, before any
    // HIP call; a call that would enqueue nothing needs no workspace
    const int32_t st = moe_layer(a, nullptr, 0, stream);
    if (st != MOE_ERR_WORKSPACE) return st;
    hipError_t err;
    void* ws = scratch_for_current_device(&err);
    if (!ws) return MOE_ERR_HIP;
    return moe_layer(a, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}
