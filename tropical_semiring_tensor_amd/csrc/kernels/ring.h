// Semiring element operations for the device kernels.
//
// The three semirings are the ones the batched kernels of tropical-gemm
// PR #35 ("feat: batched GPU ops with DLPack zero-copy output", Key
// changes) are named after: max-plus, min-plus and max-mul.  The page does
// not spell the operations out; the standard tropical algebra is used:
//   max-plus  (+) max  (x) +   zero -inf (int32 -2^30)
//   min-plus  (+) min  (x) +   zero +inf (int32 +2^30)
//   max-mul   (+) max  (x) *   zero +0   (int32: 0)
// float32 (x) is one IEEE add / multiply (the code is built without fast
// math, FTZ or FMA contraction); int32 (x) is a saturating add, which gfx950
// does in one instruction (v_add_i32 with the clamp bit), or for max-mul the
// exact product clamped to the int32 range (the pages define no int32
// max-mul; this extends the saturating rule to the product).
//
// add2() is the two-input (+).  add3() folds two terms into a running value
// with one v_max3 / v_min3; it
// is written as op(op(r, x), y) so that a chain of add3() calls maps onto
// one 3-input instruction per call rather than a re-balanced tree.
// IEEE mode is on, so a NaN term is ignored by max / min: it can never
// become the running value, the same outcome as the strict "better" scan.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../kernel_params.h"

namespace trop {

template <int SR, typename T>
struct Ring;

template <>
struct Ring<TROP_SR_MAX_PLUS, float> {
    static __device__ __forceinline__ float zero() { return __int_as_float(0xff800000u); }
    static __device__ __forceinline__ float one() { return 0.0f; }
    static __device__ __forceinline__ float mul(float a, float b) { return a + b; }
    static __device__ __forceinline__ bool better(float t, float b) { return t > b; }
    static __device__ __forceinline__ float add2(float x, float y) { return __builtin_fmaxf(x, y); }
    static __device__ __forceinline__ float add3(float r, float x, float y) {
        return __builtin_fmaxf(__builtin_fmaxf(r, x), y);
    }
};

template <>
struct Ring<TROP_SR_MIN_PLUS, float> {
    static __device__ __forceinline__ float zero() { return __int_as_float(0x7f800000u); }
    static __device__ __forceinline__ float one() { return 0.0f; }
    static __device__ __forceinline__ float mul(float a, float b) { return a + b; }
    static __device__ __forceinline__ bool better(float t, float b) { return t < b; }
    static __device__ __forceinline__ float add2(float x, float y) { return __builtin_fminf(x, y); }
    static __device__ __forceinline__ float add3(float r, float x, float y) {
        return __builtin_fminf(__builtin_fminf(r, x), y);
    }
};

template <>
struct Ring<TROP_SR_MAX_MUL, float> {
    static __device__ __forceinline__ float zero() { return 0.0f; }
    static __device__ __forceinline__ float one() { return 1.0f; }
    static __device__ __forceinline__ float mul(float a, float b) { return a * b; }
    static __device__ __forceinline__ bool better(float t, float b) { return t > b; }
    static __device__ __forceinline__ float add2(float x, float y) { return __builtin_fmaxf(x, y); }
    static __device__ __forceinline__ float add3(float r, float x, float y) {
        return __builtin_fmaxf(__builtin_fmaxf(r, x), y);
    }
};

template <>
struct Ring<TROP_SR_MAX_PLUS, int32_t> {
    static __device__ __forceinline__ int32_t zero() { return -(1 << 30); }
    static __device__ __forceinline__ int32_t one() { return 0; }
    static __device__ __forceinline__ int32_t mul(int32_t a, int32_t b) {
        return __builtin_elementwise_add_sat(a, b);
    }
    static __device__ __forceinline__ bool better(int32_t t, int32_t b) { return t > b; }
    static __device__ __forceinline__ int32_t add2(int32_t x, int32_t y) { return max(x, y); }
    static __device__ __forceinline__ int32_t add3(int32_t r, int32_t x, int32_t y) {
        return max(max(r, x), y);
    }
};

template <>
struct Ring<TROP_SR_MIN_PLUS, int32_t> {
    static __device__ __forceinline__ int32_t zero() { return 1 << 30; }
    static __device__ __forceinline__ int32_t one() { return 0; }
    static __device__ __forceinline__ int32_t mul(int32_t a, int32_t b) {
        return __builtin_elementwise_add_sat(a, b);
    }
    static __device__ __forceinline__ bool better(int32_t t, int32_t b) { return t < b; }
    static __device__ __forceinline__ int32_t add2(int32_t x, int32_t y) { return min(x, y); }
    static __device__ __forceinline__ int32_t add3(int32_t r, int32_t x, int32_t y) {
        return min(min(r, x), y);
    }
};

template <>
struct Ring<TROP_SR_MAX_MUL, int32_t> {
    static __device__ __forceinline__ int32_t zero() { return 0; }
    static __device__ __forceinline__ int32_t one() { return 1; }
    static __device__ __forceinline__ int32_t mul(int32_t a, int32_t b) {
        const int64_t t = (int64_t)a * (int64_t)b;
        return t > INT32_MAX ? INT32_MAX : (t < INT32_MIN ? INT32_MIN : (int32_t)t);
    }
    static __device__ __forceinline__ bool better(int32_t t, int32_t b) { return t > b; }
    static __device__ __forceinline__ int32_t add2(int32_t x, int32_t y) { return max(x, y); }
    static __device__ __forceinline__ int32_t add3(int32_t r, int32_t x, int32_t y) {
        return max(max(r, x), y);
    }
};

template <typename T>
using vec4 = T __attribute__((ext_vector_type(4)));

}  // namespace trop
