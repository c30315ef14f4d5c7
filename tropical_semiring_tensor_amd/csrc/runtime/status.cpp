// Thread-local error text and process-wide counters.
#include <atomic>
#include <cstring>
#include <string>

#include "internal.h"

namespace trop {

static thread_local std::string t_last_error;

std::atomic<uint64_t> g_module_loads{0};
static std::atomic<uint64_t> g_launches_total{0};
static std::atomic<uint64_t> g_launches[TROP_K_FAMILIES];

trop_status fail(trop_status st, const std::string& msg) {
    t_last_error = msg;
    return st;
}

trop_status ok() {
    t_last_error.clear();
    return TROP_OK;
}

trop_status hip_fail(hipError_t e, const char* what) {
    std::string msg = std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
    return fail(TROP_ERR_HIP, msg);
}

void count_launch(trop_kernel_family fam) {
    g_launches_total.fetch_add(1, std::memory_order_relaxed);
    if (fam >= 0 && fam < TROP_K_FAMILIES) g_launches[fam].fetch_add(1, std::memory_order_relaxed);
}

}  // namespace trop

extern "C" const char* tropical_last_error(void) { return trop::t_last_error.c_str(); }

extern "C" trop_status tropical_get_stats(trop_stats* out) {
    if (!out) return trop::fail(TROP_ERR_INVALID_ARGUMENT, "tropical_get_stats: out is NULL");
    std::memset(out, 0, sizeof(*out));
    out->module_loads = trop::g_module_loads.load();
    out->launches_total = trop::g_launches_total.load();
    for (int i = 0; i < TROP_K_FAMILIES; ++i) out->launches[i] = trop::g_launches[i].load();
    return trop::ok();
}

extern "C" void tropical_reset_stats(void) {
    trop::g_launches_total.store(0);
    for (int i = 0; i < TROP_K_FAMILIES; ++i) trop::g_launches[i].store(0);
}
