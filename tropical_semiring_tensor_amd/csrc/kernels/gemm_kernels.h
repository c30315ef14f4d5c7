// Strided-batched tropical GEMM: the simple kernel (one thread per output,
// the sequential scan itself) and the K = 0 fill.  The tiled kernel is in
// gemm_tiled.h.
#pragma once
#include "gemm_tiled.h"

namespace trop {

// One thread per output, k ascending, strict compare: the sequential scan
// itself.  Used for small or oddly strided problems and as a check.
template <int SR, typename T>
__device__ __forceinline__ void gemm_simple_body(const TropGemmParams& p) {
    using R = Ring<SR, T>;
    const int64_t mn = p.m * p.n;
    const int64_t total = mn * p.batch;
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
         o += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = o / mn;
        const int64_t ij = o % mn;
        const int64_t i = ij / p.n;
        const int64_t j = ij % p.n;
        const T* A = static_cast<const T*>(p.A) + b * p.sa_batch + i * p.sa_row;
        const T* B = static_cast<const T*>(p.B) + b * p.sb_batch + j * p.sb_col;
        T best = R::zero();
        int arg = 0;
        for (int64_t k = 0; k < p.k; ++k) {
            const T term = R::mul(A[k * p.sa_col], B[k * p.sb_row]);
            if (R::better(term, best)) {
                best = term;
                arg = (int)k;
            }
        }
        const int64_t off = b * p.sc_batch + i * p.sc_row + j * p.sc_col;
        static_cast<T*>(p.C)[off] = best;
        if (p.argmax) p.argmax[off] = arg;
    }
}

__device__ __forceinline__ void fill_body(const TropFillParams& p) {
    const int64_t mn = p.m * p.n;
    const int64_t total = mn * p.batch;
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
         o += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = o / mn;
        const int64_t ij = o % mn;
        const int64_t off = b * p.sc_batch + (ij / p.n) * p.sc_row + (ij % p.n) * p.sc_col;
        static_cast<uint32_t*>(p.C)[off] = p.zero_bits;
        if (p.argmax) p.argmax[off] = 0;
    }
}

}  // namespace trop
