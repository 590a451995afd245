// lattn_fwd_noalloc: the forward pass for callers that cannot allocate device memory.
//
// The forward's workspace (the longest-first order of packed sequences, or the plan
// and the float32 segment states of the intra-sequence split) comes from a device array
// that the library owns: one per device, of kNoallocScratchBytes, held from the
// library's first use on that device until the process ends.  Nothing here allocates;
// the array's device address is looked up once per device and every later call passes
// that address to lattn_fwd as its workspace.  Every call on one device shares the
// array, so calls that overlap in time on one device race on it.  The forward ignores
// the workspace's contents on entry (each call writes what it later reads), so nothing
// has to be cleared between calls.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "lattn.h"

namespace {

constexpr size_t kNoallocScratchBytes = LATTN_NOALLOC_SCRATCH_BYTES;

// The library's scratch array.  In host code this name is only a stand-in for the
// device symbol: its device address comes from hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mutex;

// Device address of `scratch` on the current device (looked up on the first call per
// device, with that device current), or nullptr on failure.
void* scratch_on_current_device(int* status) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
        *status = LATTN_ERR_DEVICE;
        return nullptr;
    }
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr != nullptr) return ptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            *status = LATTN_ERR_DEVICE;
            return nullptr;
        }
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

}  // namespace

extern "C" int lattn_fwd_noalloc(const lattn_problem* p, const void* q, const void* k, const void* v,
                                 const float* g_gamma, float scale, const float* initial_state, int reverse,
                                 const int32_t* cu_seqlens, void* o, float* final_state, void* stream) {
    if (p == nullptr) return LATTN_ERR_INVALID_ARG;
    // Sizes beyond the array are refused before any device call.
    const size_t need = lattn_fwd_workspace_size(p);
    if (need > kNoallocScratchBytes) return LATTN_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        int status = LATTN_OK;
        ws = scratch_on_current_device(&status);
        if (ws == nullptr) return status;
    }
    return lattn_fwd(p, q, k, v, g_gamma, scale, initial_state, reverse, cu_seqlens, o, final_state, ws,
                     need > 0 ? kNoallocScratchBytes : 0, stream);
}
