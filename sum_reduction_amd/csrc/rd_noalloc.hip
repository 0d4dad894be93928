// rd_noalloc.hip -- rd_sum_dim_noalloc: rd_sum_dim with a fixed device
// scratch buffer as its workspace, for callers that cannot allocate.
//
// The buffer is a file-scope device array.  Its name in host code is only
// the host-side handle the runtime registers for it, not a device address:
// the address is asked for once per device (hipGetSymbolAddress, with that
// device current) and only that address is passed to kernels.  Each device
// holds its own copy of the array, at its own address, from the time the
// library's code is loaded onto it until the process ends.
#include <mutex>

#include <hip/hip_runtime.h>

#include "rd_internal.h"

namespace {

constexpr int64_t kScratchFloats = RD_NOALLOC_SCRATCH_BYTES / int64_t(sizeof(float));
static __device__ __align__(256) float scratch[kScratchFloats];

struct Slot {
    std::once_flag once;
    float* ptr = nullptr;
    hipError_t err = hipSuccess;
};
Slot g_slots[rd::kMaxDevices];

// The device address of `scratch` on device `dev` (the current device),
// looked up on the first call for that device.
rd_status scratch_of(int dev, float** out) {
    if (dev < 0 || dev >= rd::kMaxDevices) return RD_ERR_NO_DEVICE;
    Slot& s = g_slots[dev];
    std::call_once(s.once, [&s] {
        void* p = nullptr;
        s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (s.err == hipSuccess && p == nullptr) s.err = hipErrorInvalidSymbol;
        if (s.err == hipSuccess) s.ptr = static_cast<float*>(p);
    });
    if (s.err != hipSuccess) {
        rd::set_last_hip_error(s.err);
        return RD_ERR_HIP;
    }
    *out = s.ptr;
    return RD_OK;
}

}  // namespace

extern "C" rd_status rd_sum_dim_noalloc(const float* x, int64_t outer, int64_t R,
                                        int64_t inner, float* out, hipStream_t stream) {
    return rd::sum_dim_fixed(x, outer, R, inner, out, scratch_of, RD_NOALLOC_SCRATCH_BYTES,
                             stream);
}
