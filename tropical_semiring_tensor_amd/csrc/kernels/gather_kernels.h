// Device-side permute and repeated-label diagonal / trace gather.
//
// omeinsum-rs issue #52 ("GPU tropical path: keep tensors device-resident +
// device-side permute", section "Resolved design for step 3") asks for two
// dtype-generic kernels: (a) an N-d permute / strided gather and (b) a
// diagonal / trace gather with the tropical max / min fused in.  Both are
// the same index machinery: the output is contiguous row-major over its
// axes and each output axis walks the input with one stride (for a
// repeated label that stride is the sum of the repeated axes' strides).
// The page names the naive one-thread-per-element version as a first cut
// and a tiled, padded shared-memory transpose as the faster form; here the
// host picks one of three copy paths per call:
//
//  * copy:  the last output axis has input stride 1, so rows are copied
//           with 16-byte vectors (both sides coalesced);
//  * tiled: another output axis `ax_in` has input stride 1; a 64x64 tile
//           of the (ax_in, last) plane goes through LDS with one word of
//           padding per row, so reads are coalesced along ax_in and writes
//           along the last axis, without LDS bank conflicts;
//  * naive: one thread per output element, digits decoded from the
//           linear index (the fallback).
//
// With ntensors = 2 the second tensor is moved with the identical mapping
// in the same launch (the value and its argmax, issue #52 "Acceptance
// criteria").  All elements are 4 bytes and are moved as raw bits.
//
// A reduction over labels absent from the output (the trace) runs one
// thread per output element with the semiring's (+): zero element first,
// then the strict "better" test in row-major order over the reduced labels,
// so the first of equal values keeps its bits.
#pragma once
#include "ring.h"

namespace trop {

constexpr int GATHER_THREADS = 256;
constexpr int TILE = 64;

// Input offset of output row `row` (all axes but the last), by digits.
__device__ __forceinline__ int64_t gather_row_offset(const TropGatherParams& p, int64_t row) {
    int64_t off = 0;
    for (int d = p.ndim - 2; d >= 0; --d) {
        const int64_t e = p.shape[d];
        off += (row % e) * p.istride[d];
        row /= e;
    }
    return off;
}

__device__ __forceinline__ void gather_copy_body(const TropGatherParams& p) {
    const int64_t inner = p.shape[p.ndim - 1];
    const int64_t rows = p.total / inner;
    if (p.vec) {
        // inner % 4 == 0 and every row start is 16-byte aligned on both sides
        const int64_t vpr = inner / 4;
        const int64_t nv = rows * vpr;
        for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nv;
             v += (int64_t)gridDim.x * blockDim.x) {
            const int64_t row = v / vpr;
            const int64_t col = (v % vpr) * 4;
            const int64_t src = gather_row_offset(p, row) + col;
            const int64_t dst = row * inner + col;
            for (int t = 0; t < p.ntensors; ++t) {
                const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint32_t*>(p.in[t]) + src);
                *reinterpret_cast<uint4*>(static_cast<uint32_t*>(p.out[t]) + dst) = x;
            }
        }
    } else {
        for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < p.total;
             o += (int64_t)gridDim.x * blockDim.x) {
            const int64_t row = o / inner;
            const int64_t src = gather_row_offset(p, row) + (o % inner);
            for (int t = 0; t < p.ntensors; ++t)
                static_cast<uint32_t*>(p.out[t])[o] = static_cast<const uint32_t*>(p.in[t])[src];
        }
    }
}

__device__ __forceinline__ void gather_tiled_body(const TropGatherParams& p) {
    __shared__ uint32_t tile[2][TILE][TILE + 1];
    const int nd = p.ndim;
    const int P = p.ax_in;   // read-contiguous axis
    const int Q = nd - 1;    // write-contiguous axis
    const int64_t EP = p.shape[P], EQ = p.shape[Q];
    const int64_t sQ = p.istride[Q];
    // output stride of axis P
    int64_t oP = 1;
    for (int d = P + 1; d < nd; ++d) oP *= p.shape[d];
    const int lane = threadIdx.x & 63;
    const int grp = threadIdx.x >> 6;  // 0..3
    const int64_t per_batch = p.tiles_p * p.tiles_q;
    const int64_t nblk = per_batch * p.nbatch;

    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int64_t tq = blk % p.tiles_q;
        const int64_t tp = (blk / p.tiles_q) % p.tiles_p;
        int64_t bi = blk / per_batch;
        // decode the remaining axes (all but P and Q) of this batch index
        int64_t ibase = 0, obase = 0, ostride = 1;
        for (int d = nd - 1; d >= 0; --d) {
            const int64_t e = p.shape[d];
            if (d != P && d != Q) {
                const int64_t digit = bi % e;
                bi /= e;
                ibase += digit * p.istride[d];
                obase += digit * ostride;
            }
            ostride *= e;
        }
        const int64_t p0 = tp * TILE, q0 = tq * TILE;
        // read: lanes run along P (unit input stride)
        const int64_t pp = p0 + lane;
        for (int qq = grp; qq < TILE; qq += 4) {
            const int64_t q = q0 + qq;
            if (pp < EP && q < EQ) {
                const int64_t src = ibase + pp + q * sQ;
                for (int t = 0; t < p.ntensors; ++t)
                    tile[t][qq][lane] = static_cast<const uint32_t*>(p.in[t])[src];
            }
        }
        __syncthreads();
        // write: lanes run along Q (unit output stride)
        const int64_t q = q0 + lane;
        for (int pl = grp; pl < TILE; pl += 4) {
            const int64_t pv = p0 + pl;
            if (pv < EP && q < EQ) {
                const int64_t dst = obase + pv * oP + q;
                for (int t = 0; t < p.ntensors; ++t)
                    static_cast<uint32_t*>(p.out[t])[dst] = tile[t][lane][pl];
            }
        }
        __syncthreads();
    }
}

__device__ __forceinline__ void gather_naive_body(const TropGatherParams& p) {
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < p.total;
         o += (int64_t)gridDim.x * blockDim.x) {
        int64_t rem = o, src = 0;
        for (int d = p.ndim - 1; d >= 0; --d) {
            const int64_t e = p.shape[d];
            src += (rem % e) * p.istride[d];
            rem /= e;
        }
        for (int t = 0; t < p.ntensors; ++t)
            static_cast<uint32_t*>(p.out[t])[o] = static_cast<const uint32_t*>(p.in[t])[src];
    }
}

template <int SR, typename T>
__device__ __forceinline__ void gather_reduce_body(const TropGatherParams& p) {
    using R = Ring<SR, T>;
    const T* in = static_cast<const T*>(p.in[0]);
    T* out = static_cast<T*>(p.out[0]);
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < p.total;
         o += (int64_t)gridDim.x * blockDim.x) {
        int64_t rem = o, base = 0;
        for (int d = p.ndim - 1; d >= 0; --d) {
            const int64_t e = p.shape[d];
            base += (rem % e) * p.istride[d];
            rem /= e;
        }
        T best = R::zero();
        for (int64_t r = 0; r < p.rtotal; ++r) {
            int64_t rr = r, off = base;
            for (int d = p.nred - 1; d >= 0; --d) {
                const int64_t e = p.rshape[d];
                off += (rr % e) * p.rstride[d];
                rr /= e;
            }
            const T v = in[off];
            if (R::better(v, best)) best = v;
        }
        out[o] = best;
    }
}

}  // namespace trop
