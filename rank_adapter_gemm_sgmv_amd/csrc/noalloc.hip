// noalloc.hip -- lora_linear_noalloc: lora_linear with the library's own device-resident
// scratch in place of a caller workspace, for callers that cannot allocate (code under HIP
// graph capture, serving loops that forbid hipMalloc).
//
// The scratch is one file-scope device array per GPU (LORA_NOALLOC_SCRATCH_BYTES, held until
// the process ends).  In host code the array's name is only a host-side stand-in, so its
// device address is looked up once per device with hipGetSymbolAddress, with that device
// current, at the entry point's first call on it; every later call passes that address to
// the kernels.  The entry point calls no hipMalloc, hipFree or allocating library routine.
// Every call on one GPU shares the array: calls that overlap in time on one GPU (two streams,
// two host threads) race on it.  Nothing in it must start at zero: every region the kernels
// read in a call is written earlier in the same call.
#include <mutex>

#include "common.h"

namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[LORA_NOALLOC_SCRATCH_BYTES];

std::once_flag g_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices] = {};
hipError_t g_lookup_error[kMaxDevices] = {};

// Device address of this device's scratch (nullptr and the HIP error on failure).
void *scratch_ptr(int dev, hipError_t *err) {
    std::call_once(g_once[dev], [dev] {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_lookup_error[dev] = e;
        g_scratch_ptr[dev] = e == hipSuccess ? p : nullptr;
    });
    *err = g_lookup_error[dev];
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

lora_status_t lora_linear_noalloc(const void *x, const void *W, const void *A, const void *B,
                                  const float *scale, const int32_t *ranks, const int32_t *ids,
                                  int32_t M, int32_t d_in, int32_t d_out, int32_t r_max,
                                  int32_t n_adapters, const lora_segments_t *segs, void *y,
                                  lora_dtype_t y_dtype, lora_mode_t mode, void *stream) {
    const size_t need = lora_workspace_bytes(M, d_in, d_out, r_max, n_adapters);
    if (need == 0)  // M = 0, or sizes lora_linear rejects: its status, nothing enqueued
        return lora::linear_on_workspace(x, W, A, B, scale, ranks, ids, M, d_in, d_out, r_max,
                                         n_adapters, segs, y, y_dtype, mode, nullptr, 0, stream);
    if (need > (size_t)LORA_NOALLOC_SCRATCH_BYTES) return LORA_ERR_WORKSPACE;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
    void *ws = e == hipSuccess ? scratch_ptr(dev, &e) : nullptr;
    if (ws == nullptr) return lora::hip_error_status(e);
    return lora::linear_on_workspace(x, W, A, B, scale, ranks, ids, M, d_in, d_out, r_max,
                                     n_adapters, segs, y, y_dtype, mode, ws,
                                     (size_t)LORA_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
