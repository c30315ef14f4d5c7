// Internal interfaces of the host runtime of libtropical.so.
#pragma once
#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../../include/tropical.h"
#include "../kernel_params.h"

namespace trop {

// ---- errors and counters (status.cpp) ------------------------------------
trop_status fail(trop_status st, const std::string& msg);  // records the text
trop_status ok();                                         // clears the text
trop_status hip_fail(hipError_t e, const char* what);
void count_launch(trop_kernel_family fam);

// ---- kernels and the per-device module cache (module.cpp) ----------------
// Kernels.  A per-semiring family has one entry point per (semiring, dtype)
// pair, NRING of them in ring_index order, so that its first id plus
// ring_index(sr, dt) selects the instance.
constexpr int NRING = 6;
enum KernelId : int {
    K_GEMM_TILED_MAXPLUS_F32 = 0,                                          // with argmax
    K_GEMM_TILED_VO_MAXPLUS_F32 = K_GEMM_TILED_MAXPLUS_F32 + NRING,        // value only
    K_GEMM_TILED_SPLIT_MAXPLUS_F32 = K_GEMM_TILED_VO_MAXPLUS_F32 + NRING,  // over (tile, K range)
    K_GEMM_TILED_VO_SPLIT_MAXPLUS_F32 = K_GEMM_TILED_SPLIT_MAXPLUS_F32 + NRING,
    K_GEMM_SIMPLE_MAXPLUS_F32 = K_GEMM_TILED_VO_SPLIT_MAXPLUS_F32 + NRING,
    K_GATHER_REDUCE_MAXPLUS_F32 = K_GEMM_SIMPLE_MAXPLUS_F32 + NRING,
    K_GEMM_SPLITK_MERGE_MAXPLUS_F32 = K_GATHER_REDUCE_MAXPLUS_F32 + NRING,  // merge of split-K partials
    K_GEMM_TILED_N_MAXPLUS_F32 = K_GEMM_SPLITK_MERGE_MAXPLUS_F32 + NRING,  // with argmax, few tiles
    K_GEMM_TILED_G_MAXPLUS_F32 = K_GEMM_TILED_N_MAXPLUS_F32 + NRING,  // with argmax, global resolve (long K)
    K_GATHER_REDUCE_VEC_MAXPLUS_F32 = K_GEMM_TILED_G_MAXPLUS_F32 + NRING,  // reduce, 4 outputs per thread
    K_GEMM_TILED_GKK_MAXPLUS_F32 = K_GATHER_REDUCE_VEC_MAXPLUS_F32 + NRING,  // global resolve, both operands k-vector
    K_GEMM_TILED_KM_MAXPLUS_F32 = K_GEMM_TILED_GKK_MAXPLUS_F32 + NRING,  // wide, A k-vector, B column-vector
    K_GEMM_TILED_KMR_MAXPLUS_F32 = K_GEMM_TILED_KM_MAXPLUS_F32 + NRING,  // the same, with a two-level k
    K_GEMM_TILED_VOR_MAXPLUS_F32 = K_GEMM_TILED_KMR_MAXPLUS_F32 + NRING,  // value only, with a two-level k
    // one 16-column group per thread (products with at most 16 columns):
    // the wide form, its fixed-layout form, the value-only form
    K_GEMM_TILED_W1_MAXPLUS_F32 = K_GEMM_TILED_VOR_MAXPLUS_F32 + NRING,
    K_GEMM_TILED_KM1_MAXPLUS_F32 = K_GEMM_TILED_W1_MAXPLUS_F32 + NRING,
    K_GEMM_TILED_VO1_MAXPLUS_F32 = K_GEMM_TILED_KM1_MAXPLUS_F32 + NRING,
    // short K (at most 16), B held in registers
    K_GEMM_SMALLK_MAXPLUS_F32 = K_GEMM_TILED_VO1_MAXPLUS_F32 + NRING,
    K_FILL = K_GEMM_SMALLK_MAXPLUS_F32 + NRING,
    K_GATHER_COPY,
    K_GATHER_TILED,
    K_GATHER_NAIVE,
    K_GATHER_TILED_V16_N1,
    K_GATHER_TILED_V32_N1,
    K_GATHER_TILED_V64_N1,
    K_GATHER_TILED_V16_N2,
    K_GATHER_TILED_V32_N2,
    K_GATHER_TILED_V64_N2,
    K_GEMM_BACKWARD_B256,  // backward, 256 / 1024 / 4096 bins per LDS chunk
    K_GEMM_BACKWARD_B1024,
    K_GEMM_BACKWARD_B4096,
    K_GEMM_BACKWARD_LANE_PLUS,  // backward, one lane per segment (bins <= 256)
    K_GEMM_BACKWARD_LANE_PLUS_VEC,
    K_GEMM_BACKWARD_LANE_MUL,
    K_GEMM_BACKWARD_LANE_MUL_VEC,
    K_GATHER_RUNS_V_N1,  // runs path: 16-byte / word accesses, 1 or 2 tensors
    K_GATHER_RUNS_V_N2,
    K_GATHER_RUNS_S_N1,
    K_GATHER_RUNS_S_N2,
    K_ARGMAX_COMPOSE,  // argmax through pre-pass reductions
    K_GEMM_BACKWARD_SPLIT_PLUS,  // backward, 16 lanes per segment (bins <= 256)
    K_GEMM_BACKWARD_SPLIT_PLUS_VEC,
    K_GEMM_BACKWARD_SPLIT_MUL,
    K_GEMM_BACKWARD_SPLIT_MUL_VEC,
    K_GATHER_TILED2_V16_N1,  // two tiled gathers in one launch
    K_GATHER_TILED2_V32_N1,
    K_GATHER_TILED2_V64_N1,
    K_GATHER_TILED2_V16_N2,
    K_GATHER_TILED2_V32_N2,
    K_GATHER_TILED2_V64_N2,
    K_GATHER_FLAT_N1,  // flat-tile transpose (short contiguous axes), single-axis sides
    K_GATHER_FLAT_N2,
    K_GATHER_FLATG_N1,  // the same with groups of axes (offset tables)
    K_GATHER_FLATG_N2,
    K_GATHER_FLATB_N1,  // several P x Q blocks per tile, single-axis sides
    K_GATHER_FLATB_N2,
    K_GATHER_FLATGB_N1,  // several blocks per tile, groups of axes
    K_GATHER_FLATGB_N2,
    K_GEMM_BACKWARD_RANGE_PLUS,  // backward, lane form over 64-bin ranges
    K_GEMM_BACKWARD_RANGE_MUL,
    // float mode of int32 max-plus / min-plus: per form, max-plus then
    // min-plus (wide, narrow, global resolve, value only), and the domain
    // pre-pass
    K_GEMM_FM_MAXPLUS,
    K_GEMM_FM_MINPLUS,
    K_GEMM_FMN_MAXPLUS,
    K_GEMM_FMN_MINPLUS,
    K_GEMM_FMG_MAXPLUS,
    K_GEMM_FMG_MINPLUS,
    K_GEMM_FMVO_MAXPLUS,
    K_GEMM_FMVO_MINPLUS,
    K_GEMM_DOMAIN_MAXPLUS,
    K_GEMM_DOMAIN_MINPLUS,
    K_GEMM_FMKM_MAXPLUS,  // float mode, wide, A k-vector, B column-vector
    K_GEMM_FMKM_MINPLUS,
    K_GEMM_BACKWARD_STAGED_PLUS,  // backward, items staged through LDS per 64 segments (bins <= 256);
                                  // + load mode (elements, along items, across segments)
    K_GEMM_BACKWARD_STAGED_MUL = K_GEMM_BACKWARD_STAGED_PLUS + 3,
    K_GEMM_BACKWARD_STAGED2_PLUS = K_GEMM_BACKWARD_STAGED_MUL + 3,  // both gradients: + 3 mode(a) + mode(b)
    K_GEMM_BACKWARD_STAGED2_MUL = K_GEMM_BACKWARD_STAGED2_PLUS + 9,
    K_COUNT = K_GEMM_BACKWARD_STAGED2_MUL + 9
};
const char* kernel_name(KernelId id);

// Index of (semiring, dtype) among the NRING supported pairs, or -1.
int ring_index(trop_semiring sr, trop_dtype dt);

// Current device, with the module loaded on it.  On failure returns an
// error status (message recorded) and caches nothing.
trop_status current_device(int* dev);
trop_status ensure_module(int dev);
// Compute units of a device whose module is loaded.
int device_cu_count(int dev);
// Workgroups of kernel `id` (at its launch bound) that one CU holds at once.
int kernel_occupancy(int dev, KernelId id);
// Threads per workgroup kernel `id` is built for (its launch bound).
int kernel_block(int dev, KernelId id);

// Enqueue kernel `id` (one by-value argument block) on `stream`.
trop_status launch(int dev, KernelId id, trop_kernel_family fam, uint32_t grid, uint32_t block,
                   void* params, hipStream_t stream);

// Magic pair for floor(n / d), n < 2^31, d >= 2: m = floor(2^(31+s) / d) + 1
// with s = ceil(log2 d); then floor(n / d) = umulhi(n, m) >> (s - 1).  The
// error term n * (m * d - 2^(31+s)) / (d * 2^(31+s)) stays below 1/d, so
// the floor is exact.
inline void magic_u31(uint64_t d, uint32_t* m, uint32_t* sh) {
    uint32_t s = 0;
    while ((uint64_t(1) << s) < d) ++s;
    *m = (uint32_t)(((uint64_t(1) << (31 + s)) / d) + 1);
    *sh = s - 1;
}

// ---- the allocation-free call's scratch (noalloc.hip) ---------------------
// Device address of the library's own scratch array on device `dev`, which
// must be current (looked up once per device).
trop_status noalloc_scratch(int dev, void** out);

// ---- argument checks (validate.cpp) --------------------------------------
// `p` must be device memory of `dev` holding at least `span_elems` elements
// of `elem_bytes` from p on (span_elems == 0: only the pointer is checked).
trop_status check_device_span(const void* p, int dev, int64_t span_elems, size_t elem_bytes,
                              const char* what);
// Largest element offset reached by sum_d (extent_d - 1) * stride_d, with
// overflow detection; extents must be >= 1.
bool max_offset(int n, const int64_t* extent, const int64_t* stride, int64_t* out);

// ---- gather planning (gather.cpp) ----------------------------------------
enum GatherPath { GP_NONE = 0, GP_COPY, GP_TILED, GP_NAIVE, GP_REDUCE, GP_RUNS, GP_FLAT };
struct GatherPlan {
    TropGatherParams params;
    GatherPath path;
    int64_t in_span;  // elements of input reached (max offset + 1), 0 if empty
};
// Output axes with extents `oshape` and input strides `ostride`; reduce axes
// likewise.  Builds the normalised plan (size-1 axes dropped, contiguous
// neighbours merged) and picks the kernel path.
trop_status plan_gather(int ndim, const int64_t* oshape, const int64_t* ostride, int nred,
                        const int64_t* rshape, const int64_t* rstride, GatherPlan* plan);
const char* gather_path_name(GatherPath p);
// Enqueue a planned gather (pointers are set here; checks done by caller).
trop_status run_gather(int dev, GatherPlan& plan, int ntensors, const void* const* in,
                       void* const* out, trop_semiring sr, trop_dtype dt, hipStream_t stream);
// Two independent gathers: one launch when both take the same vectorised
// tiled kernel, else run_gather twice.
trop_status run_gather_pair(int dev, GatherPlan& g0, int nt0, const void* const* in0, void* const* out0,
                            GatherPlan& g1, int nt1, const void* const* in1, void* const* out1,
                            trop_semiring sr, trop_dtype dt, hipStream_t stream);

// Label-based diagonal / trace gather into a plan (used by the public call
// and by the contraction driver).
trop_status plan_diag(int in_ndim, const int64_t* in_shape, const int64_t* in_strides,
                      const int32_t* in_labels, int out_ndim, const int32_t* out_labels,
                      GatherPlan* plan);

// ---- GEMM (gemm.cpp) -------------------------------------------------------
// Number of K splits for a product of this shape (1: no split) and the
// workspace the split partials need (0 when not split).  Host-only.
struct SplitK {
    int64_t ksplit = 1, kchunk = 0;
    size_t bytes = 0;
};
SplitK plan_splitk(int64_t m, int64_t n, int64_t k, int64_t batch);
// Workspace a product of this shape can use: the split-K partials when it
// is split, else room for the domain flags of the float mode of int32
// max-plus / min-plus when it is large enough to take it (any dtype: the
// sizing calls know no dtype), else 0.  Host-only.
size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t batch);
// Does a long-K product of this shape gain from reading B along k (k unit
// stride) when A is read along k?  The global-resolve argmax kernel then
// reads both operands in 16-byte quads along k (the value-only kernel is no
// slower).  At least 256 rows, 2^30 terms and K >= 512, K a multiple of 4,
// not split along K (TROPICAL_GEMM_B_TRANSPOSE=0: never, =1: any unsplit
// product with K > 256).
bool kcol_b_pays(int64_t m, int64_t n, int64_t k, int64_t batch);
// The transposed operand copies run_gemm makes in the workspace for a
// product with a long K: a column-major A as (batch, m, k), and with an
// argmax output a row-major B as (batch, n, k) when A is read along k;
// their byte offsets and the workspace bytes they need (0: none).
struct OperandCopies {
    bool a = false, b = false;
    size_t a_off = 0, b_off = 0, bytes = 0;
};
OperandCopies plan_copies(trop_strides sA, trop_strides sB, bool argmax, int64_t m, int64_t n, int64_t k,
                          int64_t batch);
// Two-level k of the GEMM's operands (TropGemmParams a_krun / sa_khi):
// a_run > 0 reads A's k as k = hi a_run + lo, lo at unit stride (sA.col = 1)
// and hi at stride a_hi; a_run is 4, 8 or 16.  Likewise b_run / b_hi with
// sB.row = 1.  0: plain strides.
struct GemmKRuns {
    int32_t a_run = 0, b_run = 0;
    int64_t a_hi = 0, b_hi = 0;
};
inline bool krun_ok(int32_t r) { return r == 4 || r == 8 || r == 16; }

// Enqueue without re-validating pointers (used by the contraction driver).
// `workspace` (may be NULL) holds plan_splitk(...).bytes when a split is
// wanted; without it the product is not split.  `kr` (may be NULL): a
// two-level k, checked by the caller (krun_ok, unit inner stride).
trop_status run_gemm(int dev, trop_semiring sr, trop_dtype dt, const void* A, trop_strides sA,
                     const void* B, trop_strides sB, void* C, trop_strides sC, int32_t* argmax,
                     int64_t m, int64_t n, int64_t k, int64_t batch, hipStream_t stream,
                     void* workspace = nullptr, size_t workspace_bytes = 0, const GemmKRuns* kr = nullptr);
trop_status check_gemm_args(trop_semiring sr, trop_dtype dt, trop_strides sA, trop_strides sB,
                            trop_strides sC, int64_t m, int64_t n, int64_t k, int64_t batch);

}  // namespace trop
