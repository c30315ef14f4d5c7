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

// Split-K merge: the partials of the K ranges, in range order, each the
// result of the strict scan over its own range of k.  Keeping the first
// strictly better one reproduces the scan over all of K: its value, the
// bits of its first winning term, and the smallest winning k (a range that
// only ties an earlier one loses).
//
// MERGE_G consecutive lanes share one output: lane c scans its own run of
// consecutive ranges in order (the first taken as is, then only strictly
// better ones), and the lanes then combine pairwise, the better value
// winning and, on equal values, the earlier range.  That is the same first
// strict winner over all ranges, found with MERGE_G loads in flight.
constexpr int MERGE_G = 8;

template <int SR, typename T>
__device__ __forceinline__ void splitk_merge_body(const TropSplitMergeParams& p) {
    using R = Ring<SR, T>;
    const int64_t mn = p.m * p.n;
    const int64_t total = mn * p.batch;
    const T* pv = static_cast<const T*>(p.pval);
    const int32_t nr = (int32_t)p.ksplit;
    const int32_t per = (nr + MERGE_G - 1) / MERGE_G;  // ranges per lane
    // (total * MERGE_G is a multiple of MERGE_G, so the lanes of one output
    // are active or inactive together)
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total * MERGE_G;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t o = t / MERGE_G;
        const int32_t c = (int32_t)(t % MERGE_G);
        const int32_t r0 = c * per, r1 = r0 + per < nr ? r0 + per : nr;
        T best = R::zero();
        int32_t arg = 0;
        int32_t rb = nr;  // range of `best`; nr = none (an empty run)
        for (int32_t r = r0; r < r1; ++r) {
            const T v = pv[(int64_t)r * total + o];
            if (r == r0 || R::better(v, best)) {
                best = v;
                arg = p.pidx ? p.pidx[(int64_t)r * total + o] : 0;
                rb = r;
            }
        }
#pragma unroll
        for (int m = 1; m < MERGE_G; m <<= 1) {
            const T ov = __shfl_xor(best, m);
            const int32_t oa = __shfl_xor(arg, m);
            const int32_t orb = __shfl_xor(rb, m);
            const bool take = R::better(ov, best) || (!R::better(best, ov) && orb < rb);
            best = take ? ov : best;
            arg = take ? oa : arg;
            rb = take ? orb : rb;
        }
        if (c == 0) {
            const int64_t b = o / mn, ij = o % mn;
            const int64_t off = b * p.sc_batch + (ij / p.n) * p.sc_row + (ij % p.n) * p.sc_col;
            static_cast<T*>(p.C)[off] = best;
            if (p.argmax) p.argmax[off] = arg;
        }
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
