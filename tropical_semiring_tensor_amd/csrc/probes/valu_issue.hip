// VALU issue-rate probe for gfx950: the measurements behind the tropical
// GEMM's roofline peak.
//
// Each kernel runs a fixed stream of register-only VALU instructions (16
// independent chains per thread, no memory access but one store per thread
// at the end) and reports lane-instructions per clock per CU at the 2.4 GHz
// peak clock.  Streams:
//   - single instructions: the term operations of the semirings (f32 add /
//     mul, the 32-bit plain and saturating adds), the (+) operations (max3 /
//     min3) and the argmax record pair (compare + select);
//   - the tropical mix, two adds and one max3 per two terms, in two orders:
//     each max3 right after its two adds (dependent pairs back to back), and
//     phased (the adds of all chains, then their max3s),
// at 1, 2, 4 and 8 waves per SIMD (256-thread workgroups, CUs x n of them).
//
// Build and run (repository root):
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//     -o /tmp/valu_issue tropical_semiring_tensor_amd/csrc/probes/valu_issue.hip
//   /tmp/valu_issue
#include <hip/hip_runtime.h>

#include <cstdio>

namespace {

constexpr int NCH = 16;  // independent chains per thread

#define PROBE_KERNEL(NAME, ...)                                                         \
    __global__ __launch_bounds__(256) void NAME(unsigned* out, int iters, unsigned s0,  \
                                                unsigned s1) {                          \
        unsigned a[NCH], m[NCH];                                                        \
        for (int i = 0; i < NCH; ++i) {                                                 \
            a[i] = threadIdx.x + i;                                                     \
            m[i] = 0x3f000000u - i;                                                     \
        }                                                                               \
        for (int it = 0; it < iters; ++it) {                                            \
            _Pragma("unroll") for (int i = 0; i < NCH; ++i) { __VA_ARGS__ }             \
        }                                                                               \
        unsigned r = 0;                                                                 \
        for (int i = 0; i < NCH; ++i) r ^= a[i] ^ m[i];                                 \
        out[blockIdx.x * blockDim.x + threadIdx.x] = r;                                 \
    }

// four dependent instructions per chain and iteration
#define STREAM2(INS)                                                                    \
    asm volatile(INS " %0, %1, %0\n " INS " %0, %2, %0\n " INS " %0, %1, %0\n " INS     \
                     " %0, %2, %0"                                                      \
                 : "+v"(a[i])                                                           \
                 : "v"(s0), "v"(s1));
#define STREAM3(INS)                                                                    \
    asm volatile(INS " %0, %0, %1, %2\n " INS " %0, %0, %2, %1\n " INS                  \
                     " %0, %0, %1, %2\n " INS " %0, %0, %2, %1"                         \
                 : "+v"(a[i])                                                           \
                 : "v"(s0), "v"(s1));

PROBE_KERNEL(p_add_f32, STREAM2("v_add_f32_e32"))
PROBE_KERNEL(p_mul_f32, STREAM2("v_mul_f32_e32"))
PROBE_KERNEL(p_add_u32, STREAM2("v_add_u32_e32"))
PROBE_KERNEL(p_add_i32_clamp, asm volatile("v_add_i32 %0, %1, %0 clamp\n v_add_i32 %0, %2, %0 clamp\n"
                                           " v_add_i32 %0, %1, %0 clamp\n v_add_i32 %0, %2, %0 clamp"
                                           : "+v"(a[i]) : "v"(s0), "v"(s1));)
PROBE_KERNEL(p_max3_f32, STREAM3("v_max3_f32"))
PROBE_KERNEL(p_min3_i32, STREAM3("v_min3_i32"))
PROBE_KERNEL(p_cmp_cndmask, asm volatile("v_cmp_gt_f32_e32 vcc, %0, %1\n v_cndmask_b32_e32 %0, %0, %2, vcc\n"
                                         " v_cmp_gt_f32_e32 vcc, %0, %2\n v_cndmask_b32_e32 %0, %0, %1, vcc"
                                         : "+v"(a[i]) : "v"(s0), "v"(s1) : "vcc");)
// two terms of one chain: two adds, then the max3 that folds them (3 instructions)
PROBE_KERNEL(p_mix_f32, {
    unsigned t0, t1;
    asm volatile("v_add_f32_e32 %1, %4, %3\n v_add_f32_e32 %2, %5, %3\n v_max3_f32 %0, %0, %1, %2"
                 : "+v"(m[i]), "=&v"(t0), "=&v"(t1) : "v"(a[i]), "v"(s0), "v"(s1));
})
PROBE_KERNEL(p_mix_i32_clamp, {
    unsigned t0, t1;
    asm volatile("v_add_i32 %1, %4, %3 clamp\n v_add_i32 %2, %5, %3 clamp\n v_min3_i32 %0, %0, %1, %2"
                 : "+v"(m[i]), "=&v"(t0), "=&v"(t1) : "v"(a[i]), "v"(s0), "v"(s1));
})

// The same 48 instructions per iteration (8 chains, 4 terms each: 32 adds
// and 16 max3) in the two orders.  Operands are fixed registers, so the
// order is exactly the one written.
#define VREGS                                                                                \
    "v0", "v1", "v2", "v3", "v4", "v5", "v6", "v7", "v8", "v9", "v10", "v11", "v12", "v13",  \
        "v14", "v15", "v16", "v17", "v18", "v19", "v20", "v21", "v22", "v23", "v24", "v25",  \
        "v26", "v27", "v28", "v29", "v30", "v31", "v32", "v33", "v34", "v35", "v36", "v37",  \
        "v38", "v39", "v40", "v41", "v42", "v43", "v44", "v45", "v46", "v47", "v48", "v49",  \
        "v50", "v51", "v52", "v53", "v54", "v55", "v56", "v57", "v58", "v59", "v60", "v61",  \
        "v62", "v63"

// chain o (o < 8) reads the A quad v[4 (o / 4)] .. + 3 and the B quad
// v[16 + 4 (o % 4)] .. + 3; its running max is v[48 + o]
__global__ __launch_bounds__(256) void p_order_dependent(unsigned* out, int iters) {
    for (int it = 0; it < iters; ++it) {
        asm volatile(
            ".irp o, 0, 1, 2, 3, 4, 5, 6, 7\n"
            "  v_add_f32_e32 v40, v[(\\o >> 2) * 4], v[16 + (\\o & 3) * 4]\n"
            "  v_add_f32_e32 v41, v[(\\o >> 2) * 4 + 1], v[16 + (\\o & 3) * 4 + 1]\n"
            "  v_max3_f32 v[48 + \\o], v[48 + \\o], v40, v41\n"
            "  v_add_f32_e32 v42, v[(\\o >> 2) * 4 + 2], v[16 + (\\o & 3) * 4 + 2]\n"
            "  v_add_f32_e32 v43, v[(\\o >> 2) * 4 + 3], v[16 + (\\o & 3) * 4 + 3]\n"
            "  v_max3_f32 v[48 + \\o], v[48 + \\o], v42, v43\n"
            ".endr\n" ::: VREGS);
    }
    unsigned r;
    asm volatile("v_mov_b32 %0, v48" : "=v"(r)::VREGS);
    out[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

__global__ __launch_bounds__(256) void p_order_phased(unsigned* out, int iters) {
    for (int it = 0; it < iters; ++it) {
        asm volatile(
            ".irp o, 0, 1, 2, 3, 4, 5, 6, 7\n"
            "  v_add_f32_e32 v[32 + 2 * \\o], v[(\\o >> 2) * 4], v[16 + (\\o & 3) * 4]\n"
            "  v_add_f32_e32 v[33 + 2 * \\o], v[(\\o >> 2) * 4 + 1], v[16 + (\\o & 3) * 4 + 1]\n"
            ".endr\n"
            ".irp o, 0, 1, 2, 3, 4, 5, 6, 7\n"
            "  v_max3_f32 v[48 + \\o], v[48 + \\o], v[32 + 2 * \\o], v[33 + 2 * \\o]\n"
            ".endr\n"
            ".irp o, 0, 1, 2, 3, 4, 5, 6, 7\n"
            "  v_add_f32_e32 v[32 + 2 * \\o], v[(\\o >> 2) * 4 + 2], v[16 + (\\o & 3) * 4 + 2]\n"
            "  v_add_f32_e32 v[33 + 2 * \\o], v[(\\o >> 2) * 4 + 3], v[16 + (\\o & 3) * 4 + 3]\n"
            ".endr\n"
            ".irp o, 0, 1, 2, 3, 4, 5, 6, 7\n"
            "  v_max3_f32 v[48 + \\o], v[48 + \\o], v[32 + 2 * \\o], v[33 + 2 * \\o]\n"
            ".endr\n" ::: VREGS);
    }
    unsigned r;
    asm volatile("v_mov_b32 %0, v48" : "=v"(r)::VREGS);
    out[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

#define CHECK(x)                                                                              \
    do {                                                                                      \
        hipError_t e_ = (x);                                                                  \
        if (e_ != hipSuccess) {                                                               \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);       \
            return 1;                                                                         \
        }                                                                                     \
    } while (0)

}  // namespace

int main() {
    int cus = 0;
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    const int threads = 256, max_wps = 8;
    unsigned* out = nullptr;
    CHECK(hipMalloc(&out, (size_t)cus * max_wps * threads * sizeof(unsigned)));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    const int iters = 2048, reps = 5;
    auto timed = [&](auto launch, int grid, double lane_instr_per_launch, const char* name, int wps) -> int {
        for (int w = 0; w < 2; ++w) launch(grid);
        CHECK(hipDeviceSynchronize());
        CHECK(hipEventRecord(e0));
        for (int r = 0; r < reps; ++r) launch(grid);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float ms = 0;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        const double rate = lane_instr_per_launch * reps / (ms * 1e-3);
        std::printf("%-40s waves/SIMD %d  %6.1f lane-instr / clock / CU at 2.4 GHz\n", name, wps,
                    rate / 2.4e9 / cus);
        std::fflush(stdout);
        return 0;
    };
    struct Stream {
        const char* name;
        void (*k)(unsigned*, int, unsigned, unsigned);
        double per_chain_iter;
    };
    const Stream streams[] = {
        {"v_add_f32", p_add_f32, 4},          {"v_mul_f32", p_mul_f32, 4},
        {"v_add_u32", p_add_u32, 4},          {"v_add_i32 clamp (saturating)", p_add_i32_clamp, 4},
        {"v_max3_f32", p_max3_f32, 4},        {"v_min3_i32", p_min3_i32, 4},
        {"v_cmp_gt_f32 + v_cndmask", p_cmp_cndmask, 4},
        {"mix: 2 v_add_f32 + v_max3_f32", p_mix_f32, 3},
        {"mix: 2 v_add_i32 clamp + v_min3_i32", p_mix_i32_clamp, 3},
    };
    for (const Stream& s : streams) {
        const int wps = 8, grid = cus * wps;
        const double li = (double)grid * threads * iters * NCH * s.per_chain_iter;
        if (timed([&](int g) { hipLaunchKernelGGL(s.k, dim3(g), dim3(threads), 0, 0, out, iters, 1u, 2u); },
                  grid, li, s.name, wps))
            return 1;
    }
    for (int wps : {1, 2, 4, 8}) {
        const int grid = cus * wps;
        const double li = (double)grid * threads * iters * 48.0;
        if (timed([&](int g) { hipLaunchKernelGGL(p_order_dependent, dim3(g), dim3(threads), 0, 0, out, iters); },
                  grid, li, "8 chains: max3 right after its adds", wps))
            return 1;
        if (timed([&](int g) { hipLaunchKernelGGL(p_order_phased, dim3(g), dim3(threads), 0, 0, out, iters); },
                  grid, li, "8 chains: all adds, then the max3s", wps))
            return 1;
    }
    CHECK(hipFree(out));
    std::printf("done\n");
    return 0;
}
