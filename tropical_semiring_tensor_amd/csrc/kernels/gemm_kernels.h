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

// Split-K merge: the partials of the K splits, in split order, each the
// result of the strict scan over its own range of k.  Keeping the first
// strictly better one reproduces the scan over all of K: its value, the
// bits of its first winning term, and the smallest winning k (a split that
// only ties an earlier one loses).  One thread per output.
template <int SR, typename T>
__device__ __forceinline__ void splitk_merge_body(const TropSplitMergeParams& p) {
    using R = Ring<SR, T>;
    const int64_t mn = p.m * p.n;
    const int64_t total = mn * p.batch;
    const T* pv = static_cast<const T*>(p.pval);
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
         o += (int64_t)gridDim.x * blockDim.x) {
        T best = pv[o];
        int32_t arg = p.pidx ? p.pidx[o] : 0;
        for (int64_t s = 1; s < p.ksplit; ++s) {
            const T v = pv[s * total + o];
            if (R::better(v, best)) {
                best = v;
                if (p.pidx) arg = p.pidx[s * total + o];
            }
        }
        const int64_t b = o / mn, ij = o % mn;
        const int64_t off = b * p.sc_batch + (ij / p.n) * p.sc_row + (ij % p.n) * p.sc_col;
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
