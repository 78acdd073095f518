// noalloc.hip -- saga_decode_step_noalloc (include/saga.h): the decode step
// for callers that cannot allocate device memory.  Its workspace is a
// file-scope device array of this library, one copy per device, held until
// the process ends; everything else is saga_decode_step's own code path.
//
// Host code never uses the array's name as a device address (on the host it
// names a stand-in): the address comes from hipGetSymbolAddress, looked up
// once per device with that device current, and is what the kernels receive.
#include <mutex>

#include "saga.h"
#include "kernels.hpp"

#define SAGA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

static __device__ __align__(256) unsigned char scratch[SAGA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the current device (looked up on first use).
int scratch_of_current_device(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SAGA_ERR_HIP;
    if (dev < 0 || dev >= kMaxScratchDevices) return SAGA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SAGA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SAGA_OK;
}

}  // namespace

SAGA_EXPORT int saga_decode_step_noalloc(const saga_dims* dims, const void* q_dev,
                                         const void* k_cache_dev, const void* v_cache_dev,
                                         const float* thresholds_dev, void* out_dev,
                                         int32_t* sel_counts_dev, void* stream)
{
    const size_t need = saga::decode_workspace_bytes(dims);
    if (need == 0) {
        // Invalid dims: report the same status the decode step would.
        return saga::decode_step(dims, q_dev, k_cache_dev, v_cache_dev, thresholds_dev, out_dev,
                                 sel_counts_dev, nullptr, 0, stream);
    }
    if (need > (size_t)SAGA_NOALLOC_SCRATCH_BYTES) return SAGA_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    const int st = scratch_of_current_device(&ws);
    if (st != SAGA_OK) return st;
    return saga::decode_step(dims, q_dev, k_cache_dev, v_cache_dev, thresholds_dev, out_dev,
                             sel_counts_dev, ws, (size_t)SAGA_NOALLOC_SCRATCH_BYTES, stream);
}
