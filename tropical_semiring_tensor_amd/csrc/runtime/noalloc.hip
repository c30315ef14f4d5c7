// tropical_contract_pair_noalloc: the pairwise contraction for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  Its intermediates (the operands'
// canonical copies, the product before the output permute, split-K partials,
// reduction winners) live in one file-scope device array instead of a
// caller workspace; everything else is tropical_contract_pair.
//
// The array is a module global of this translation unit: every device the
// library runs on holds its own copy, at its own address, until the process
// ends.  Host code never uses the array's name as an address (on the host it
// is only a stand-in): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.  Calls on one
// device share its array, so calls that overlap on one device (different
// streams, or host threads) race; nothing in it needs to start at zero (every
// kernel writes each element it later reads).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "contract_plan.h"

namespace {

constexpr size_t kScratchBytes = TROP_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
std::atomic<void*> g_scratch[kMaxDevices];

}  // namespace

namespace trop {

// Device address of `scratch` on device `dev`, which must be current.
trop_status noalloc_scratch(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return fail(TROP_ERR_INVALID_ARGUMENT, "device index out of range");
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_mu);
        p = g_scratch[dev].load(std::memory_order_acquire);
        if (!p) {
            hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
            if (!p) return fail(TROP_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return TROP_OK;
}

}  // namespace trop

extern "C" trop_status tropical_contract_pair_noalloc(const char* spec, trop_semiring semiring, trop_dtype dtype,
                                                      const void* A, const int64_t* shapeA,
                                                      const int64_t* stridesA, const void* B,
                                                      const int64_t* shapeB, const int64_t* stridesB, void* C,
                                                      int32_t* argmax, void* stream) {
    using namespace trop;
    int dev = -1;
    trop_status st = current_device(&dev);
    if (st != TROP_OK) return st;
    void* ws = nullptr;
    st = noalloc_scratch(dev, &ws);
    if (st != TROP_OK) return st;
    return contract_pair_call(spec, semiring, dtype, A, shapeA, stridesA, B, shapeB, stridesB, C, argmax, ws,
                              kScratchBytes, true, stream);
}
