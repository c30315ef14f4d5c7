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
            const T term = R::mul(A[k_offset(k, p.a_krun, p.sa_khi, p.sa_col)],
                                  B[k_offset(k, p.b_krun, p.sb_khi, p.sb_row)]);
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

// Products with a short K (1..SK_MAXK) and up to 256 columns, a multiple
// of 4 (the host takes it for 128..256 columns and many rows).  Each lane
// holds four columns of B (all K rows) in registers; a row takes the 16,
// 32 or 64 lanes that cover its columns, so a wave computes 4, 2 or 1 rows
// per lane group step.  The workgroup stages blocks of SK_ROWS rows of A in
// LDS, and each lane group walks rows SK_RPW at a time, computing the
// lane's outputs as the sequential scan does (k ascending, the zero
// element to start, strict compare: the same values, bits and smallest
// winning k as the simple kernel) and writing them as one 16-byte store
// each for C and the argmax.  A tiled kernel at this K runs one slice per
// tile, its loads, compute and stores one after another; here B is loaded
// once per batch entry and the output writes stream.  Needs C (and the
// argmax) with unit column stride, rows and batch strides multiples of 4
// and 16-byte aligned (checked on the host).
constexpr int SK_MAXK = 16;
constexpr int SK_ROWS = 32;  // rows per unit of work
constexpr int SK_RPW = 2;    // rows a wave computes together (independent chains)

template <int SR, typename T, bool ARG>
__device__ __forceinline__ void gemm_smallk_run(const TropGemmParams& p, T (&As)[SK_ROWS][SK_MAXK]) {
    using R = Ring<SR, T>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwaves = (int)(blockDim.x >> 6);
    const int K = (int)p.k;
    const int64_t m = p.m;
    // lanes per row: the power of two of 16, 32 or 64 that covers n / 4
    // column groups; the wave's 64 / lpr lane groups take different rows
    const int lsh = p.n > 128 ? 6 : (p.n > 64 ? 5 : 4);
    const int lpr = 1 << lsh, sub = lane >> lsh;
    const int64_t j0 = 4 * (int64_t)(lane & (lpr - 1));
    const bool jl = j0 < p.n;  // (n % 4 == 0)
    const int rstep = SK_RPW << (6 - lsh);  // rows a wave covers per step
    const int64_t rblocks = (m + SK_ROWS - 1) / SK_ROWS;
    const int64_t units = rblocks * p.batch;
    const T* A = static_cast<const T*>(p.A);
    const T* B = static_cast<const T*>(p.B);
    T bv[SK_MAXK][4];
    int64_t cur_b = -1;
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        const int64_t b = u / rblocks, r0 = (u - b * rblocks) * SK_ROWS;
        __syncthreads();  // the previous unit's rows are read
        // A's rows: element e of the SK_ROWS x K block is row e % SK_ROWS,
        // term e / SK_ROWS (consecutive threads take consecutive rows)
        for (int e = tid; e < SK_ROWS * SK_MAXK; e += blockDim.x) {
            const int r = e % SK_ROWS, kk = e / SK_ROWS;
            const int64_t i = r0 + r;
            if (i < m && kk < K)
                As[r][kk] = A[b * p.sa_batch + i * p.sa_row + k_offset(kk, p.a_krun, p.sa_khi, p.sa_col)];
        }
        if (b != cur_b) {
            cur_b = b;
            // a row-major B with 16-byte aligned rows: one 16-byte load per k
            const bool bvec = p.sb_col == 1 && p.b_krun == 0 && (p.sb_row & 3) == 0 && (p.sb_batch & 3) == 0 &&
                              (reinterpret_cast<uintptr_t>(B) & 15u) == 0;
#pragma unroll
            for (int kk = 0; kk < SK_MAXK; ++kk) {
                if (jl && kk < K && bvec) {
                    const vec4<T> v = *reinterpret_cast<const vec4<T>*>(B + b * p.sb_batch + kk * p.sb_row + j0);
                    bv[kk][0] = v.x;
                    bv[kk][1] = v.y;
                    bv[kk][2] = v.z;
                    bv[kk][3] = v.w;
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        bv[kk][c] = (jl && kk < K) ? B[b * p.sb_batch + k_offset(kk, p.b_krun, p.sb_khi, p.sb_row) +
                                                       (j0 + c) * p.sb_col]
                                                   : R::zero();
                }
            }
        }
        __syncthreads();
        // rstep rows at a time per wave (SK_RPW per lane group): 4 * SK_RPW
        // independent chains per lane
        for (int rw = wave * rstep; rw < SK_ROWS; rw += nwaves * rstep) {
            if (r0 + rw >= m) break;  // (uniform over the wave)
            const int rr = rw + sub * SK_RPW;  // this lane group's first row
            T best[SK_RPW][4];
            int32_t arg[SK_RPW][4];
#pragma unroll
            for (int h = 0; h < SK_RPW; ++h)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    best[h][c] = R::zero();
                    arg[h][c] = 0;
                }
#pragma unroll
            for (int kk = 0; kk < SK_MAXK; ++kk) {
                if (kk < K) {
#pragma unroll
                    for (int h = 0; h < SK_RPW; ++h) {
                        const T a = As[rr + h][kk];  // (rows past m: staged garbage, never stored)
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const T t = R::mul(a, bv[kk][c]);
                            const bool up = R::better(t, best[h][c]);
                            best[h][c] = up ? t : best[h][c];
                            if (ARG) arg[h][c] = up ? kk : arg[h][c];
                        }
                    }
                }
            }
            if (jl) {
#pragma unroll
                for (int h = 0; h < SK_RPW; ++h) {
                    const int64_t i = r0 + rr + h;
                    if (i < m) {
                        const int64_t off = b * p.sc_batch + i * p.sc_row + j0;
                        *reinterpret_cast<vec4<T>*>(static_cast<T*>(p.C) + off) =
                            vec4<T>{best[h][0], best[h][1], best[h][2], best[h][3]};
                        if (ARG)
                            *reinterpret_cast<vec4<int32_t>*>(p.argmax + off) =
                                vec4<int32_t>{arg[h][0], arg[h][1], arg[h][2], arg[h][3]};
                    }
                }
            }
        }
    }
}

template <int SR, typename T>
__device__ __forceinline__ void gemm_smallk_body(const TropGemmParams& p) {
    __shared__ T As[SK_ROWS][SK_MAXK];
    if (p.argmax)
        gemm_smallk_run<SR, T, true>(p, As);
    else
        gemm_smallk_run<SR, T, false>(p, As);
}

// Split-K merge: the partials of the K ranges, in range order, each the
// result of the strict scan over its own range of k.  Keeping the first
// strictly better one reproduces the scan over all of K: its value, the
// bits of its first winning term, and the smallest winning k (a range that
// only ties an earlier one loses).
//
// G consecutive lanes share one output (G = p.lanes, a power of two up to
// MERGE_G, about one lane per MERGE_U ranges): lane c scans its own run of
// consecutive ranges in order (the first taken as is, then only strictly
// better ones), and the lanes then combine pairwise, the better value
// winning and, on equal values, the earlier range.  That is the same first
// strict winner over all ranges, found with G x MERGE_U loads in flight per
// output.
constexpr int MERGE_G = TROP_MERGE_LANES;
constexpr int MERGE_U = 8;  // ranges per lane whose loads are in flight together

template <int SR, typename T>
__device__ __forceinline__ void splitk_merge_body(const TropSplitMergeParams& p) {
    using R = Ring<SR, T>;
    const int64_t mn = p.m * p.n;
    const int64_t total = mn * p.batch;
    const T* pv = static_cast<const T*>(p.pval);
    // (value only: the index loads read the values, in bounds, and are not used)
    const int32_t* pi = p.pidx ? p.pidx : reinterpret_cast<const int32_t*>(pv);
    const int32_t nr = (int32_t)p.ksplit;
    const int32_t G = p.lanes, gsh = __builtin_ctz((uint32_t)G);
    const int32_t per = (nr + G - 1) / G;  // ranges per lane
    // (total * G is a multiple of G, so the lanes of one output are active
    // or inactive together)
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total * G;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t o = t >> gsh;
        const int32_t c = (int32_t)(t & (G - 1));
        const int32_t r0 = c * per, r1 = r0 + per < nr ? r0 + per : nr;
        T best = R::zero();
        int32_t arg = 0;
        int32_t rb = nr;  // range of `best`; nr = none (an empty run)
        // MERGE_U ranges at a time: their loads issued together (a range past
        // r1 re-reads range r0, in bounds, and is not considered), then
        // scanned in order
        for (int32_t ra = r0; ra < r1; ra += MERGE_U) {
            T v[MERGE_U];
            int32_t a[MERGE_U];
#pragma unroll
            for (int u = 0; u < MERGE_U; ++u) {
                const int64_t off = (int64_t)(ra + u < r1 ? ra + u : r0) * total + o;
                v[u] = pv[off];
                a[u] = pi[off];
            }
#pragma unroll
            for (int u = 0; u < MERGE_U; ++u) {
                const int32_t r = ra + u;
                const bool take = r < r1 && (r == r0 || R::better(v[u], best));
                best = take ? v[u] : best;
                arg = take ? a[u] : arg;
                rb = take ? r : rb;
            }
        }
        for (int m = 1; m < G; m <<= 1) {  // (uniform)
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

// Domain pre-pass of the float mode of int32 max-plus / min-plus products
// (see zero_of in gemm_tiled.h): is every element of A and B inside the
// semiring's float-exact domain?  min-plus: [0, 2^23) or [2^30, 2^31)
// -- with the top bit of the 31 flipped that is one interval below
// 2^30 + 2^23; max-plus: (-2^23, 2^23), shifted by 2^23 - 1 onto one
// unsigned interval below 2^24 - 1.
template <int SR>
__device__ __forceinline__ uint32_t outside_domain(int32_t x) {
    if constexpr (SR == TROP_SR_MIN_PLUS) {
        return ((uint32_t)x ^ 0x40000000u) >= 0x40800000u;
    } else {
        return (uint32_t)x + 0x7FFFFFu >= 0xFFFFFFu;
    }
}

// Scan one operand: batch entries of r x c elements with strides (sb, sr,
// sc); each workgroup takes rows blockIdx.x, blockIdx.x + gridDim.x, ...,
// its threads run along the unit-stride axis when there is one (16-byte
// loads when aligned).
template <int SR>
__device__ __forceinline__ uint32_t domain_scan(const int32_t* X, int64_t nb, int64_t r, int64_t c, int64_t sb,
                                                int64_t sr, int64_t sc) {
    if (sr == 1 && sc != 1) {
        const int64_t t = r;
        r = c;
        c = t;
        sr = sc;
        sc = 1;
    }
    // one wave per row at a time (rows of different waves in flight
    // together), the row's 16-byte vectors unrolled so that a lane's loads
    // are issued together
    uint32_t bad = 0;
    const int64_t rows = nb * r;
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    const int64_t nw = (int64_t)gridDim.x * (blockDim.x / 64);
    for (int64_t row = wid; row < rows; row += nw) {
        const int64_t b = row / r, i = row - b * r;
        const int32_t* base = X + b * sb + i * sr;
        if (sc == 1 && (reinterpret_cast<uintptr_t>(base) & 15u) == 0) {
            const int64_t nv = c / 4;
#pragma unroll 16
            for (int64_t v = lane; v < nv; v += 64) {
                const vec4<int32_t> x = reinterpret_cast<const vec4<int32_t>*>(base)[v];
                bad |= outside_domain<SR>(x.x) | outside_domain<SR>(x.y) | outside_domain<SR>(x.z) |
                       outside_domain<SR>(x.w);
            }
            for (int64_t e = nv * 4 + lane; e < c; e += 64) bad |= outside_domain<SR>(base[e]);
        } else {
#pragma unroll 8
            for (int64_t e = lane; e < c; e += 64) bad |= outside_domain<SR>(base[e * sc]);
        }
    }
    return bad;
}

template <int SR>
__device__ __forceinline__ void gemm_domain_body(const TropDomainParams& p) {
    uint32_t bad = domain_scan<SR>(p.A, p.batch, p.m, p.k, p.sa_batch, p.sa_row, p.sa_col);
    bad |= domain_scan<SR>(p.B, p.batch, p.k, p.n, p.sb_batch, p.sb_row, p.sb_col);
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) p.flags[blockIdx.x] = bad ? 1 : 0;
}

}  // namespace trop
