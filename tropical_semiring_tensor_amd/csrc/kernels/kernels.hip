// The one gfx950 code object of libtropical.so: every kernel entry point.
// Built with hipcc --genco and embedded in the library, which loads it once
// per device with hipModuleLoadData and looks the entry points up by name.
#include "backward_kernels.h"
#include "gather_kernels.h"
#include "gemm_kernels.h"

using namespace trop;

// ARGW: the wide argmax kernels' register target (the float ones are held
// to 4 waves per SIMD, i.e. 128 VGPRs; see the float argmax setting in
// gemm_tiled.h).  trop_gemm_tiled_n_*: the narrow setting, for products
// with at most two tiles per CU.
#define TROP_ARGW_F32 __attribute__((amdgpu_waves_per_eu(4)))
#define TROP_ARGW_I32
// the global-resolve argmax kernels (long K): 4 waves per SIMD
#ifndef TROP_GR_WAVES
#define TROP_GR_WAVES 4
#endif
#define TROP_ARGW_GR __attribute__((amdgpu_waves_per_eu(TROP_GR_WAVES)))
#define TROP_GEMM_ENTRIES(NAME, SR, T, ARGW)                                                  \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) ARGW void trop_gemm_tiled_##NAME(    \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, T, true, false>(p);                                                 \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) void trop_gemm_tiled_vo_##NAME(      \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, T, false, false, false, false, T, LAYOUT_ANY, LAYOUT_ANY, false>(p); \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) void trop_gemm_tiled_vor_##NAME(     \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, T, false, false>(p);                                                \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) void trop_gemm_tiled_n_##NAME(       \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, T, true, false, true>(p);                                           \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) TROP_ARGW_GR void trop_gemm_tiled_g_##NAME( \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, T, true, false, false, true>(p);                                    \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) TROP_ARGW_GR void trop_gemm_tiled_gkk_##NAME( \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, T, true, false, false, true, T, LAYOUT_KV, LAYOUT_KV, false>(p);    \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) ARGW void trop_gemm_tiled_km_##NAME(     \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, T, true, false, false, false, T, LAYOUT_KV, LAYOUT_MV, false>(p);   \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) ARGW void trop_gemm_tiled_kmr_##NAME(    \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, T, true, false, false, false, T, LAYOUT_KV, LAYOUT_MV, true>(p);    \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) ARGW void trop_gemm_tiled_w1_##NAME(     \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, T, true, false, false, false, T, LAYOUT_ANY, LAYOUT_ANY, true, 1>(p); \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) ARGW void trop_gemm_tiled_km1_##NAME(    \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, T, true, false, false, false, T, LAYOUT_KV, LAYOUT_MV, true, 1>(p); \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) void trop_gemm_tiled_vo1_##NAME(     \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, T, false, false, false, false, T, LAYOUT_ANY, LAYOUT_ANY, true, 1>(p); \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) void trop_gemm_tiled_split_##NAME(   \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, T, true, true>(p);                                                  \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) void trop_gemm_tiled_vo_split_##NAME( \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, T, false, true>(p);                                                 \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(256) void trop_gemm_simple_##NAME(TropGemmParams p) { \
        gemm_simple_body<SR, T>(p);                                                             \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(256) void trop_gemm_smallk_##NAME(TropGemmParams p) { \
        gemm_smallk_body<SR, T>(p);                                                             \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(256) void trop_gather_reduce_##NAME(                \
        TropGatherParams p) {                                                                   \
        gather_reduce_body<SR, T>(p);                                                           \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(256) void trop_gather_reduce_vec_##NAME(            \
        TropGatherParams p) {                                                                   \
        gather_reduce_vec_body<SR, T>(p);                                                       \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(256) void trop_gemm_splitk_merge_##NAME(            \
        TropSplitMergeParams p) {                                                               \
        splitk_merge_body<SR, T>(p);                                                            \
    }

TROP_GEMM_ENTRIES(maxplus_f32, TROP_SR_MAX_PLUS, float, TROP_ARGW_F32)
TROP_GEMM_ENTRIES(minplus_f32, TROP_SR_MIN_PLUS, float, TROP_ARGW_F32)
TROP_GEMM_ENTRIES(maxmul_f32, TROP_SR_MAX_MUL, float, TROP_ARGW_F32)
TROP_GEMM_ENTRIES(maxplus_i32, TROP_SR_MAX_PLUS, int32_t, TROP_ARGW_I32)
TROP_GEMM_ENTRIES(minplus_i32, TROP_SR_MIN_PLUS, int32_t, TROP_ARGW_I32)
TROP_GEMM_ENTRIES(maxmul_i32, TROP_SR_MAX_MUL, int32_t, TROP_ARGW_I32)

// Float mode of int32 max-plus / min-plus products (the domain pre-pass,
// then the float-mode kernel and the int32 kernel, each gated on its
// flags): wide, narrow, global-resolve and value-only forms.
#define TROP_GEMM_FM_ENTRIES(NAME, SR)                                                          \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) TROP_ARGW_F32 void trop_gemm_fm_##NAME( \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, float, true, false, false, false, int32_t, LAYOUT_ANY, LAYOUT_ANY, false>(p); \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) void trop_gemm_fmn_##NAME(            \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, float, true, false, true, false, int32_t, LAYOUT_ANY, LAYOUT_ANY, false>(p); \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) TROP_ARGW_GR void trop_gemm_fmg_##NAME( \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, float, true, false, false, true, int32_t, LAYOUT_ANY, LAYOUT_ANY, false>(p); \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) void trop_gemm_fmvo_##NAME(           \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, float, false, false, false, false, int32_t, LAYOUT_ANY, LAYOUT_ANY, false>(p); \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GEMM_THREADS) TROP_ARGW_F32 void trop_gemm_fmkm_##NAME( \
        TropGemmParams p) {                                                                     \
        gemm_tiled_body<SR, float, true, false, false, false, int32_t, LAYOUT_KV, LAYOUT_MV, false>(p); \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(256) void trop_gemm_domain_##NAME(TropDomainParams p) { \
        gemm_domain_body<SR>(p);                                                                \
    }
TROP_GEMM_FM_ENTRIES(maxplus_i32, TROP_SR_MAX_PLUS)
TROP_GEMM_FM_ENTRIES(minplus_i32, TROP_SR_MIN_PLUS)

extern "C" __global__ __launch_bounds__(256) void trop_fill(TropFillParams p) { fill_body(p); }

extern "C" __global__ __launch_bounds__(256) void trop_argmax_compose(TropComposeParams p) {
    argmax_compose_body(p);
}

extern "C" __global__ __launch_bounds__(GATHER_THREADS) void trop_gather_copy(TropGatherParams p) {
    gather_copy_body(p);
}

extern "C" __global__ __launch_bounds__(GATHER_THREADS) void trop_gather_tiled(TropGatherParams p) {
    gather_tiled_body(p);
}

#define TROP_TILED_VEC(TPV, NTV)                                                                \
    extern "C" __global__ __launch_bounds__(GATHER_THREADS) void trop_gather_tiled_v##TPV##_n##NTV( \
        TropGatherParams p) {                                                                   \
        gather_tiled_vec_body<TPV, NTV>(p, blockIdx.x, gridDim.x);                              \
    }                                                                                           \
    extern "C" __global__ __launch_bounds__(GATHER_THREADS) void trop_gather_tiled2_v##TPV##_n##NTV( \
        TropGatherPairParams q) {                                                               \
        if ((int)blockIdx.x < q.split)                                                          \
            gather_tiled_vec_body<TPV, NTV>(q.p[0], blockIdx.x, q.split);                       \
        else                                                                                    \
            gather_tiled_vec_body<TPV, NTV>(q.p[1], blockIdx.x - q.split, gridDim.x - q.split); \
    }
TROP_TILED_VEC(16, 1)
TROP_TILED_VEC(32, 1)
TROP_TILED_VEC(64, 1)
TROP_TILED_VEC(16, 2)
TROP_TILED_VEC(32, 2)
TROP_TILED_VEC(64, 2)

#define TROP_RUNS(NAME, VEC, NT)                                                                  \
    extern "C" __global__ __launch_bounds__(GATHER_THREADS) void trop_gather_runs_##NAME(TropGatherParams p) { \
        gather_runs_body<VEC, NT>(p);                                                                \
    }
TROP_RUNS(v_n1, true, 1)
TROP_RUNS(v_n2, true, 2)
TROP_RUNS(s_n1, false, 1)
TROP_RUNS(s_n2, false, 2)

// Waves per SIMD asked of the compiler: 5 (<= 96 VGPRs) where that needs
// no spills; unconstrained the plain forms took 105+.  The block forms
// spill at 5 and get 4.
#define TROP_FLAT(NAME, NT, GROUPS, BLOCKS, WAVES)                                                 \
    extern "C" __global__ __launch_bounds__(GATHER_THREADS) __attribute__((amdgpu_waves_per_eu(WAVES))) \
    void trop_gather_##NAME(TropGatherParams p) {                                                   \
        gather_flat_body<NT, GROUPS, BLOCKS>(p);                                                      \
    }
TROP_FLAT(flat_n1, 1, false, false, 5)
TROP_FLAT(flat_n2, 2, false, false, 5)
TROP_FLAT(flatg_n1, 1, true, false, 5)
TROP_FLAT(flatg_n2, 2, true, false, 5)
TROP_FLAT(flatb_n1, 1, false, true, 4)
TROP_FLAT(flatb_n2, 2, false, true, 4)
TROP_FLAT(flatgb_n1, 1, true, true, 4)
TROP_FLAT(flatgb_n2, 2, true, true, 4)

extern "C" __global__ __launch_bounds__(GATHER_THREADS) void trop_gather_naive(TropGatherParams p) {
    gather_naive_body(p);
}

#define TROP_BACKWARD(NB)                                                                        \
    extern "C" __global__ __launch_bounds__(GBW_THREADS) void trop_gemm_backward_b##NB(          \
        TropBackwardParams p) {                                                                  \
        gemm_backward_body<NB>(p);                                                               \
    }
TROP_BACKWARD(256)
TROP_BACKWARD(1024)
TROP_BACKWARD(4096)

#define TROP_BACKWARD_LANE(NAME, MUL, VEC)                                                       \
    extern "C" __global__ __launch_bounds__(64) void trop_gemm_backward_lane_##NAME(             \
        TropBackwardParams p) {                                                                  \
        gemm_backward_lane_body<MUL, VEC>(p);                                                    \
    }
TROP_BACKWARD_LANE(plus, false, false)
TROP_BACKWARD_LANE(plus_vec, false, true)
TROP_BACKWARD_LANE(mul, true, false)
TROP_BACKWARD_LANE(mul_vec, true, true)

#define TROP_BACKWARD_RANGE(NAME, MUL)                                                           \
    extern "C" __global__ __launch_bounds__(64) void trop_gemm_backward_range_##NAME(            \
        TropBackwardParams p) {                                                                  \
        gemm_backward_lane_body<MUL, false, GBR_BINS>(p);                                        \
    }
TROP_BACKWARD_RANGE(plus, false)
TROP_BACKWARD_RANGE(mul, true)

#define TROP_BACKWARD_SPLIT(NAME, MUL, VEC)                                                      \
    extern "C" __global__ __launch_bounds__(GBS_THREADS) void trop_gemm_backward_split_##NAME(    \
        TropBackwardParams p) {                                                                  \
        gemm_backward_split_body<MUL, VEC>(p);                                                   \
    }
TROP_BACKWARD_SPLIT(plus, false, false)
TROP_BACKWARD_SPLIT(plus_vec, false, true)
TROP_BACKWARD_SPLIT(mul, true, false)
TROP_BACKWARD_SPLIT(mul_vec, true, true)

#define TROP_BACKWARD_STAGED(NAME, MUL, LM)                                                      \
    extern "C" __global__ __launch_bounds__(GBT_THREADS) void trop_gemm_backward_staged_##NAME(   \
        TropBackwardParams p) {                                                                  \
        gemm_backward_staged_body<MUL, LM>(p);                                                   \
    }
// item loads: e = elements, i = 16-byte along items, s = 16-byte across segments
TROP_BACKWARD_STAGED(plus_e, false, GBT_LOAD_ELEM)
TROP_BACKWARD_STAGED(plus_i, false, GBT_LOAD_ITEMS)
TROP_BACKWARD_STAGED(plus_s, false, GBT_LOAD_SEGS)
TROP_BACKWARD_STAGED(mul_e, true, GBT_LOAD_ELEM)
TROP_BACKWARD_STAGED(mul_i, true, GBT_LOAD_ITEMS)
TROP_BACKWARD_STAGED(mul_s, true, GBT_LOAD_SEGS)

// both gradients in one launch; suffix: each job's item loads
#define TROP_BACKWARD_STAGED2(NAME, MUL, LA, LB)                                                 \
    extern "C" __global__ __launch_bounds__(GBT_THREADS) void trop_gemm_backward_staged2_##NAME(  \
        TropBackwardPairParams q) {                                                              \
        gemm_backward_staged_pair_body<MUL, LA, LB>(q);                                          \
    }
#define TROP_BACKWARD_STAGED2_ALL(NAME, MUL)                                           \
    TROP_BACKWARD_STAGED2(NAME##_ee, MUL, GBT_LOAD_ELEM, GBT_LOAD_ELEM)                \
    TROP_BACKWARD_STAGED2(NAME##_ei, MUL, GBT_LOAD_ELEM, GBT_LOAD_ITEMS)               \
    TROP_BACKWARD_STAGED2(NAME##_es, MUL, GBT_LOAD_ELEM, GBT_LOAD_SEGS)                \
    TROP_BACKWARD_STAGED2(NAME##_ie, MUL, GBT_LOAD_ITEMS, GBT_LOAD_ELEM)               \
    TROP_BACKWARD_STAGED2(NAME##_ii, MUL, GBT_LOAD_ITEMS, GBT_LOAD_ITEMS)              \
    TROP_BACKWARD_STAGED2(NAME##_is, MUL, GBT_LOAD_ITEMS, GBT_LOAD_SEGS)               \
    TROP_BACKWARD_STAGED2(NAME##_se, MUL, GBT_LOAD_SEGS, GBT_LOAD_ELEM)                \
    TROP_BACKWARD_STAGED2(NAME##_si, MUL, GBT_LOAD_SEGS, GBT_LOAD_ITEMS)               \
    TROP_BACKWARD_STAGED2(NAME##_ss, MUL, GBT_LOAD_SEGS, GBT_LOAD_SEGS)
TROP_BACKWARD_STAGED2_ALL(plus, false)
TROP_BACKWARD_STAGED2_ALL(mul, true)
