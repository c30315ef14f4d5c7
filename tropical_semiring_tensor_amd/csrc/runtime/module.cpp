// Per-device cache of the kernel module.
//
// omeinsum-rs issue #52 ("GPU tropical path: keep tensors device-resident +
// device-side permute") traces part of the GPU slowdown to the driver
// context and kernel module being rebuilt for every contraction node
// ("Current state in the code", "Proposed plan" step 1) and asks for them to
// be created once ("Compilation & caching", "Acceptance criteria");
// tropical-gemm PR #35 keeps one context per device (Key changes).  Here the
// gfx950 code object is compiled ahead of time, embedded in this library,
// loaded with hipModuleLoadData at most once per process and device, and
// every entry point is looked up once.  A failed load caches nothing, so a
// later call tries again.
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

// Embedded code object (co_blob.S).
extern "C" const unsigned char trop_code_object[];
extern "C" const unsigned char trop_code_object_end[];

namespace trop {

extern std::atomic<uint64_t> g_module_loads;

namespace {

// Entry-point names, built once: per-semiring families are prefix + ring
// suffix (ring_index order), the rest are listed in KernelId order.
const std::vector<std::string>& kernel_names() {
    static const std::vector<std::string> names = [] {
        static const char* const rings[NRING] = {"maxplus_f32", "minplus_f32", "maxmul_f32",
                                                 "maxplus_i32", "minplus_i32", "maxmul_i32"};
        static const char* const families[] = {"trop_gemm_tiled_",       "trop_gemm_tiled_vo_",
                                               "trop_gemm_tiled_split_", "trop_gemm_tiled_vo_split_",
                                               "trop_gemm_simple_",      "trop_gather_reduce_",
                                               "trop_gemm_splitk_merge_", "trop_gemm_tiled_n_",
                                               "trop_gemm_tiled_g_",     "trop_gather_reduce_vec_",
                                               "trop_gemm_tiled_gkk_",   "trop_gemm_tiled_km_",
                                               "trop_gemm_tiled_kmr_",   "trop_gemm_tiled_vor_",
                                               "trop_gemm_tiled_w1_",    "trop_gemm_tiled_km1_",
                                               "trop_gemm_tiled_vo1_",   "trop_gemm_smallk_"};
        static const char* const singles[] = {
            "trop_fill",                     "trop_gather_copy",
            "trop_gather_tiled",             "trop_gather_naive",
            "trop_gather_tiled_v16_n1",      "trop_gather_tiled_v32_n1",
            "trop_gather_tiled_v64_n1",      "trop_gather_tiled_v16_n2",
            "trop_gather_tiled_v32_n2",      "trop_gather_tiled_v64_n2",
            "trop_gemm_backward_b256",       "trop_gemm_backward_b1024",
            "trop_gemm_backward_b4096",      "trop_gemm_backward_lane_plus",
            "trop_gemm_backward_lane_plus_vec", "trop_gemm_backward_lane_mul",
            "trop_gemm_backward_lane_mul_vec", "trop_gather_runs_v_n1",
            "trop_gather_runs_v_n2",         "trop_gather_runs_s_n1",
            "trop_gather_runs_s_n2",         "trop_argmax_compose",
            "trop_gemm_backward_split_plus", "trop_gemm_backward_split_plus_vec",
            "trop_gemm_backward_split_mul",  "trop_gemm_backward_split_mul_vec",
            "trop_gather_tiled2_v16_n1",     "trop_gather_tiled2_v32_n1",
            "trop_gather_tiled2_v64_n1",     "trop_gather_tiled2_v16_n2",
            "trop_gather_tiled2_v32_n2",     "trop_gather_tiled2_v64_n2",
            "trop_gather_flat_n1",           "trop_gather_flat_n2",
            "trop_gather_flatg_n1",          "trop_gather_flatg_n2",
            "trop_gather_flatb_n1",          "trop_gather_flatb_n2",
            "trop_gather_flatgb_n1",         "trop_gather_flatgb_n2",
            "trop_gemm_backward_range_plus", "trop_gemm_backward_range_mul",
            "trop_gemm_fm_maxplus_i32",      "trop_gemm_fm_minplus_i32",
            "trop_gemm_fmn_maxplus_i32",     "trop_gemm_fmn_minplus_i32",
            "trop_gemm_fmg_maxplus_i32",     "trop_gemm_fmg_minplus_i32",
            "trop_gemm_fmvo_maxplus_i32",    "trop_gemm_fmvo_minplus_i32",
            "trop_gemm_domain_maxplus_i32",  "trop_gemm_domain_minplus_i32",
            "trop_gemm_fmkm_maxplus_i32",    "trop_gemm_fmkm_minplus_i32",
            "trop_gemm_backward_staged_plus_e", "trop_gemm_backward_staged_plus_i",
            "trop_gemm_backward_staged_plus_s", "trop_gemm_backward_staged_mul_e",
            "trop_gemm_backward_staged_mul_i", "trop_gemm_backward_staged_mul_s",
            "trop_gemm_backward_staged2_plus_ee", "trop_gemm_backward_staged2_plus_ei",
            "trop_gemm_backward_staged2_plus_es", "trop_gemm_backward_staged2_plus_ie",
            "trop_gemm_backward_staged2_plus_ii", "trop_gemm_backward_staged2_plus_is",
            "trop_gemm_backward_staged2_plus_se", "trop_gemm_backward_staged2_plus_si",
            "trop_gemm_backward_staged2_plus_ss", "trop_gemm_backward_staged2_mul_ee",
            "trop_gemm_backward_staged2_mul_ei", "trop_gemm_backward_staged2_mul_es",
            "trop_gemm_backward_staged2_mul_ie", "trop_gemm_backward_staged2_mul_ii",
            "trop_gemm_backward_staged2_mul_is", "trop_gemm_backward_staged2_mul_se",
            "trop_gemm_backward_staged2_mul_si", "trop_gemm_backward_staged2_mul_ss"};
        static_assert(sizeof(families) / sizeof(families[0]) * NRING == K_FILL, "families");
        static_assert(K_FILL + sizeof(singles) / sizeof(singles[0]) == K_COUNT, "single kernels");
        std::vector<std::string> v;
        for (const char* f : families)
            for (const char* r : rings) v.push_back(std::string(f) + r);
        for (const char* k : singles) v.push_back(k);
        return v;
    }();
    return names;
}

}  // namespace

const char* kernel_name(KernelId id) { return (id >= 0 && id < K_COUNT) ? kernel_names()[id].c_str() : "?"; }

int ring_index(trop_semiring sr, trop_dtype dt) {
    if (dt == TROP_F32) {
        if (sr == TROP_MAX_PLUS) return 0;
        if (sr == TROP_MIN_PLUS) return 1;
        if (sr == TROP_MAX_MUL) return 2;
    } else if (dt == TROP_I32) {
        if (sr == TROP_MAX_PLUS) return 3;
        if (sr == TROP_MIN_PLUS) return 4;
        if (sr == TROP_MAX_MUL) return 5;
    }
    return -1;
}

namespace {

constexpr int kMaxDevices = 64;

struct DeviceModule {
    hipModule_t module = nullptr;
    hipFunction_t fn[K_COUNT] = {};
    int occupancy[K_COUNT] = {};  // resident workgroups per CU
    int block[K_COUNT] = {};      // threads per workgroup (the kernel's launch bound)
    int cu_count = 0;
};

std::mutex g_mu;
std::atomic<DeviceModule*> g_dev[kMaxDevices];

// The code object to load: the embedded one, or (for testing the failure
// path) the file named by TROPICAL_CODE_OBJECT.
bool code_object_image(std::vector<unsigned char>& storage, const void** image, std::string* err) {
    const char* path = std::getenv("TROPICAL_CODE_OBJECT");
    if (!path || !*path) {
        *image = trop_code_object;
        return true;
    }
    FILE* f = std::fopen(path, "rb");
    if (!f) {
        *err = std::string("cannot open TROPICAL_CODE_OBJECT=") + path;
        return false;
    }
    unsigned char buf[65536];
    size_t got;
    while ((got = std::fread(buf, 1, sizeof(buf), f)) > 0) storage.insert(storage.end(), buf, buf + got);
    std::fclose(f);
    storage.push_back(0);
    *image = storage.data();
    return true;
}

}  // namespace

trop_status current_device(int* dev) {
    hipError_t e = hipGetDevice(dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (*dev < 0 || *dev >= kMaxDevices) return fail(TROP_ERR_INVALID_ARGUMENT, "device index out of range");
    return ensure_module(*dev);
}

trop_status ensure_module(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return fail(TROP_ERR_INVALID_ARGUMENT, "device index out of range");
    if (g_dev[dev].load(std::memory_order_acquire)) return TROP_OK;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_dev[dev].load(std::memory_order_acquire)) return TROP_OK;

    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != dev) {
        e = hipSetDevice(dev);
        if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
    }
    std::vector<unsigned char> storage;
    const void* image = nullptr;
    std::string err;
    trop_status st = TROP_OK;
    DeviceModule* dm = nullptr;
    if (!code_object_image(storage, &image, &err)) {
        st = fail(TROP_ERR_HIP, err);
    } else {
        dm = new DeviceModule;
        e = hipModuleLoadData(&dm->module, image);
        if (e != hipSuccess) {
            st = hip_fail(e, "hipModuleLoadData (gfx950 code object)");
        } else {
            g_module_loads.fetch_add(1);
            for (int i = 0; i < K_COUNT && st == TROP_OK; ++i) {
                e = hipModuleGetFunction(&dm->fn[i], dm->module, kernel_name((KernelId)i));
                if (e != hipSuccess) {
                    st = hip_fail(e, kernel_name((KernelId)i));
                    break;
                }
                e = hipFuncGetAttribute(&dm->block[i], HIP_FUNC_ATTRIBUTE_MAX_THREADS_PER_BLOCK, dm->fn[i]);
                if (e != hipSuccess) {
                    st = hip_fail(e, "hipFuncGetAttribute(max threads per block)");
                    break;
                }
                e = hipModuleOccupancyMaxActiveBlocksPerMultiprocessor(&dm->occupancy[i], dm->fn[i],
                                                                       dm->block[i], 0);
                if (e != hipSuccess) st = hip_fail(e, "hipModuleOccupancyMaxActiveBlocksPerMultiprocessor");
            }
            if (st == TROP_OK) {
                e = hipDeviceGetAttribute(&dm->cu_count, hipDeviceAttributeMultiprocessorCount, dev);
                if (e != hipSuccess) st = hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
            }
            if (st != TROP_OK) (void)hipModuleUnload(dm->module);
        }
    }
    if (cur != dev) (void)hipSetDevice(cur);
    if (st != TROP_OK) {
        delete dm;
        return st;
    }
    g_dev[dev].store(dm, std::memory_order_release);
    return TROP_OK;
}

int device_cu_count(int dev) {
    DeviceModule* dm = g_dev[dev].load(std::memory_order_acquire);
    return dm ? dm->cu_count : 0;
}

int kernel_occupancy(int dev, KernelId id) {
    DeviceModule* dm = g_dev[dev].load(std::memory_order_acquire);
    return (dm && id >= 0 && id < K_COUNT) ? dm->occupancy[id] : 0;
}

int kernel_block(int dev, KernelId id) {
    DeviceModule* dm = g_dev[dev].load(std::memory_order_acquire);
    return (dm && id >= 0 && id < K_COUNT) ? dm->block[id] : 0;
}

trop_status launch(int dev, KernelId id, trop_kernel_family fam, uint32_t grid, uint32_t block,
                   void* params, hipStream_t stream) {
    DeviceModule* dm = g_dev[dev].load(std::memory_order_acquire);
    if (!dm) return fail(TROP_ERR_HIP, "kernel module not loaded on this device");
    if (grid == 0) return TROP_OK;
    void* args[] = {params};
    hipError_t e = hipModuleLaunchKernel(dm->fn[id], grid, 1, 1, block, 1, 1, 0, stream, args, nullptr);
    if (e != hipSuccess) return hip_fail(e, kernel_name(id));
    count_launch(fam);
    return TROP_OK;
}

}  // namespace trop

extern "C" trop_status tropical_init(int device) {
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess) return trop::hip_fail(e, "hipGetDeviceCount");
    if (device < 0 || device >= n)
        return trop::fail(TROP_ERR_INVALID_ARGUMENT, "tropical_init: no device " + std::to_string(device));
    trop_status st = trop::ensure_module(device);
    if (st != TROP_OK) return st;
    // the allocation-free call's scratch: its address on this device, looked
    // up with the device current
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return trop::hip_fail(e, "hipGetDevice");
    if (cur != device) {
        e = hipSetDevice(device);
        if (e != hipSuccess) return trop::hip_fail(e, "hipSetDevice");
    }
    void* scratch = nullptr;
    st = trop::noalloc_scratch(device, &scratch);
    if (cur != device) (void)hipSetDevice(cur);
    return st == TROP_OK ? trop::ok() : st;
}
