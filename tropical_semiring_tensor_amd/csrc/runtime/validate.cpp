// Pointer and extent checks done on the host before anything is enqueued.
//
// tropical-gemm PR #35 (Key changes, "Summary of Latest Fixes") rejects
// host (pinned) memory, validates that tensors live on the same device and
// guards zero-sized dimensions; the rustytorch index_select / index_add
// commit turns an out-of-range index into a checked failure.  Here every
// pointer must be device memory of the current device, and the furthest
// element a kernel will touch must lie inside the pointer's allocation, so
// a wrong shape or stride is an error code instead of a memory fault.
#include <string>

#include "internal.h"

namespace trop {

bool max_offset(int n, const int64_t* extent, const int64_t* stride, int64_t* out) {
    int64_t acc = 0;
    for (int d = 0; d < n; ++d) {
        if (extent[d] < 1 || stride[d] < 0) return false;
        int64_t t;
        if (__builtin_mul_overflow(extent[d] - 1, stride[d], &t)) return false;
        if (__builtin_add_overflow(acc, t, &acc)) return false;
    }
    *out = acc;
    return true;
}

trop_status check_device_span(const void* p, int dev, int64_t span_elems, size_t elem_bytes,
                              const char* what) {
    if (!p) return fail(TROP_ERR_NOT_DEVICE_MEMORY, std::string(what) + " is NULL");
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(TROP_ERR_NOT_DEVICE_MEMORY,
                    std::string(what) + " is not a HIP allocation (host memory?)");
    }
    if (attr.type != hipMemoryTypeDevice) {
        return fail(TROP_ERR_NOT_DEVICE_MEMORY,
                    std::string(what) + " is not device memory (host or managed allocation)");
    }
    if (attr.device != dev) {
        return fail(TROP_ERR_INVALID_ARGUMENT, std::string(what) + " lives on device " +
                                                   std::to_string(attr.device) + ", current device is " +
                                                   std::to_string(dev));
    }
    if (span_elems > 0) {
        hipDeviceptr_t base = nullptr;
        size_t size = 0;
        e = hipMemGetAddressRange(&base, &size, const_cast<void*>(p));
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(TROP_ERR_NOT_DEVICE_MEMORY, std::string(what) + ": no allocation range");
        }
        const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
        const uintptr_t end = reinterpret_cast<uintptr_t>(base) + size;
        unsigned __int128 need = (unsigned __int128)span_elems * elem_bytes;
        if (lo > end || need > (unsigned __int128)(end - lo)) {
            return fail(TROP_ERR_INVALID_ARGUMENT,
                        std::string(what) + ": shape and strides reach past the end of its allocation");
        }
    }
    return TROP_OK;
}

}  // namespace trop
