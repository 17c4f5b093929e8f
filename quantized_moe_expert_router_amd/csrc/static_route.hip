// static_route.hip -- moe_dispatch_static: moe_dispatch with the route's row
// mappings in a fixed device array of the library, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host code
// the name `scratch` is only a host-side stand-in, so it is never passed to a
// kernel or a copy: the device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept in g_scratch_ptr.
// The call binds the caller's route to that address and runs moe_dispatch's
// kernels unchanged.  Nothing is allocated or freed.  The route's arrays need
// no clearing: the dispatch kernels write every entry the consumers read.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.hpp"
#include "moeq.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[MOEQ_STATIC_ROUTE_BYTES];

std::mutex g_init_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call on that device.
moeq_status scratch_on_current_device(void **out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return moeq::report_error(MOEQ_EDEVICE, "hipGetDevice: %s", hipGetErrorString(err));
    if (dev < 0 || dev >= kMaxDevices)
        return moeq::report_error(MOEQ_EUNSUPPORTED, "device %d beyond the %d the static "
                                  "route array is kept for", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_init_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess)
            return moeq::report_error(MOEQ_EDEVICE, "hipGetSymbolAddress(static route): %s",
                                      hipGetErrorString(err));
        if (!ptr || (uintptr_t)ptr % 256 != 0)
            return moeq::report_error(MOEQ_EDEVICE, "static route array is not 256-byte "
                                      "aligned on device %d", dev);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MOEQ_OK;
}

}  // namespace

extern "C" moeq_status moe_dispatch_static(const void *x, moeq_dtype act, int32_t T, int32_t K,
                                           const void *logits, moeq_dtype logit_dtype, int32_t E,
                                           const float *expert_bias, int32_t top_k,
                                           void *values, float *weights, uint32_t *selected,
                                           uint32_t *row_experts, moeq_route *route,
                                           void *stream) {
    if (!route) return moeq::report_error(MOEQ_EINVAL, "route is NULL");
    const size_t need = moeq_route_workspace_bytes(T, E, top_k);
    if (need == 0)
        return moeq::report_error(MOEQ_EINVAL, "invalid route shape T=%d E=%d top_k=%d", T, E,
                                  top_k);
    if (need > (size_t)MOEQ_STATIC_ROUTE_BYTES)
        return moeq::report_error(MOEQ_EWORKSPACE,
                                  "route (T=%d, E=%d, top_k=%d) needs %zu bytes; the static "
                                  "route array holds %zu (use moe_dispatch with a workspace)",
                                  T, E, top_k, need, (size_t)MOEQ_STATIC_ROUTE_BYTES);
    void *ptr = nullptr;
    moeq_status st = scratch_on_current_device(&ptr);
    if (st != MOEQ_OK) return st;
    moeq_route bound;
    if ((st = moeq_route_bind(&bound, ptr, MOEQ_STATIC_ROUTE_BYTES, T, E, top_k)) != MOEQ_OK)
        return st;
    st = moe_dispatch(x, act, T, K, logits, logit_dtype, E, expert_bias, top_k, values, weights,
                      selected, row_experts, &bound, stream);
    if (st == MOEQ_OK) *route = bound;
    return st;
}
