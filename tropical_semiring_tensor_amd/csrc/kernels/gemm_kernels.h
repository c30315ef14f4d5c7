// Strided-batched tropical GEMM with argmax for gfx950.
//
// Computes C[b][i][j] = (+)_k A[b][i][k] (x) B[b][k][j] and the smallest k
// whose term is the result -- the batched "with argmax" kernels of
// tropical-gemm PR #35 ("feat: batched GPU ops with DLPack zero-copy
// output", Key changes), re-designed for CDNA4:
//
//  * A max-plus product is not a multiply-accumulate, so it runs on the
//    VALU, not on MFMA.  The value path costs 1.5 VALU instructions per
//    (output, k): one add / multiply per term and one v_max3 / v_min3 per
//    two terms.
//  * An exact per-term argmax would add a compare and two selects per term.
//    Instead the running value is compared once per chunk of BK = 16 terms
//    (one compare + one select: which chunk last improved strictly), and the
//    exact index inside that chunk is resolved afterwards by re-scanning the
//    chunk for the first term equal to the final value.  That re-scan reads
//    the operands from LDS: the kernel keeps a whole K-block of KBLK terms
//    of both operand tiles resident, and resolves at the end of each block
//    every output whose best improved inside it.  The result is the exact
//    first winner: a strictly better chunk is recorded only when it holds a
//    term above everything before it, and inside it the first term equal
//    to the final value is that first winner.
//  * C is written with the bits of the winning term (recomputed at the
//    resolved index), so signed zeros come out as the sequential
//    strict-compare scan produces them; an output that nothing beat keeps
//    the zero element and argmax 0.
//
// Tiling: 256 threads (4 waves), a 64x64 output tile per workgroup, 16
// outputs per thread (rows 2ty, 2ty+1, 2ty+32, 2ty+33 and the same pattern
// of columns, see own()), K staged in BK = 16 slices through LDS.  LDS holds A as [k][i] and B as [k][j] (row
// length 64 + 4 words of padding), whatever the global layout:
// k-contiguous operands are transposed on the way in.  Global loads of the next slice are issued into registers while
// the current slice computes; the next slice is written to LDS at the start
// of the current one, so one barrier per slice suffices.
#pragma once
#include "ring.h"

namespace trop {

constexpr int GEMM_BM = 64;
constexpr int GEMM_BN = 64;
constexpr int GEMM_BK = 16;
constexpr int GEMM_THREADS = 256;
constexpr int GEMM_TM = 4;
constexpr int GEMM_TN = 4;
constexpr int GEMM_LDP = 64 + 4;  // LDS row length (words)
#ifndef TROP_GEMM_KBLK
#define TROP_GEMM_KBLK 128
#endif
// K terms resident in LDS per block.  Larger blocks resolve less often but
// use more LDS (2 x KBLK x 68 words): 128 leaves room for two workgroups
// (eight waves) per CU.
constexpr int GEMM_KBLK = TROP_GEMM_KBLK;
// Words per LDS slice slot.  Slots are skewed by 4 words so that the same
// (k, row) of different slices falls in different LDS banks: the resolve
// reads one slice per lane, chosen by that lane's own data.
constexpr int GEMM_SLOT = GEMM_BK * GEMM_LDP + 4;

// Offset of a thread's r-th row (or column) from 2*ty (2*tx): the thread owns
// the pairs {2t, 2t+1} and {2t+32, 2t+33}, so one ds_read2_b64 fetches its 4
// values at one k, and lanes that read different slices hit different banks.
__device__ __forceinline__ constexpr int own(int r) { return (r & 1) + 32 * (r >> 1); }

// Bijective remap of the linear workgroup id so that each of the 8 XCDs
// (which receive workgroups round-robin) owns one contiguous range of
// logical tiles; neighbouring tiles then share operand panels in one L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t L, int64_t total) {
    constexpr int64_t NX = 8;
    const int64_t per = (total + NX - 1) / NX;
    int64_t tall = total % NX;
    if (tall == 0) tall = NX;
    const int64_t x = L % NX;
    const int64_t local = L / NX;
    if (x < tall) return x * per + local;
    return tall * per + (x - tall) * (per - 1) + local;
}

template <int SR, typename T>
struct GemmTile {
    using R = Ring<SR, T>;
    using V = vec4<T>;

    // Per-thread view of one operand tile: this thread loads 4 elements of
    // every K-slice.  `mn_contig`: the 4 elements run along the row (A) /
    // column (B) axis at one k; otherwise they run along k at one row /
    // column.  `base` points at the thread's first element of slice 0 and
    // `step` advances one slice.
    struct Loader {
        const T* base;
        int64_t step;     // elements per K-slice
        int64_t inner;    // stride between the 4 elements
        int64_t kfirst;   // k of element 0 in slice 0
        int64_t mn0;      // row (A) / column (B) of element 0
        int64_t mn_lim;   // m (A) or n (B)
        int64_t k_lim;    // K
        int64_t mn_str;   // stride of the row / column axis
        int64_t k_str;    // stride of the k axis
        bool mn_contig;
        bool vec;         // 16-byte loads allowed

        // `full`: the whole slice of the whole tile is in range (a uniform
        // condition, so the common case is unguarded and branch-free).
        __device__ __forceinline__ void load(int g, bool full, T pad, T (&r)[4]) const {
            const T* q = base + (int64_t)g * step;
            if (full) {
                if (vec) {
                    const V v = *reinterpret_cast<const V*>(q);
                    r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] = q[e * inner];
                }
            } else {
                const int64_t k = kfirst + (int64_t)g * GEMM_BK;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t kk = mn_contig ? k : k + e;
                    const int64_t mm = mn_contig ? mn0 + e : mn0;
                    r[e] = (kk < k_lim && mm < mn_lim) ? q[e * inner] : pad;
                }
            }
        }
    };

    // mode: TROP_LOAD_*; for A (mn = rows i, str_mn = sa_row, str_k = sa_col),
    // for B (mn = columns j, str_mn = sb_col, str_k = sb_row).
    static __device__ __forceinline__ Loader make(const T* X, int mode, int vec, int64_t mn_start,
                                                  int64_t mn_lim, int64_t k_lim, int64_t str_mn,
                                                  int64_t str_k, int tid) {
        Loader L;
        L.mn_contig = (mode == TROP_LOAD_MN_CONTIG);
        L.mn_lim = mn_lim;
        L.k_lim = k_lim;
        L.mn_str = str_mn;
        L.k_str = str_k;
        L.vec = vec != 0;
        L.step = GEMM_BK * str_k;
        if (L.mn_contig) {
            L.kfirst = tid >> 4;
            L.mn0 = mn_start + (tid & 15) * 4;
            L.inner = str_mn;
        } else {
            L.kfirst = (tid & 3) * 4;
            L.mn0 = mn_start + (tid >> 2);
            L.inner = str_k;
        }
        L.base = X + L.mn0 * str_mn + L.kfirst * str_k;
        return L;
    }

    // Write a slice held in registers into LDS slot `s`: A as [k][i], B as
    // [k][j]; k-contiguous operands are transposed here.
    static __device__ __forceinline__ void store(bool mn_contig, T* S, int s, int tid,
                                                 const T (&r)[4]) {
        T* dst = S + s * GEMM_SLOT;
        if (mn_contig) {
            const V v = {r[0], r[1], r[2], r[3]};
            *reinterpret_cast<V*>(dst + (tid >> 4) * GEMM_LDP + (tid & 15) * 4) = v;
        } else {
            const int mn = tid >> 2, kq = (tid & 3) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(kq + e) * GEMM_LDP + mn] = r[e];
        }
    }
};

// Batch entry and output-tile origin of logical tile L.
struct TileCoord {
    int64_t b, row0, col0;
};

__device__ __forceinline__ TileCoord tile_coord(const TropGemmParams& p, int64_t L, int64_t tiles,
                                                int64_t total) {
    const int64_t lg = p.swizzle ? xcd_remap(L, total) : L;
    const int64_t t = lg % tiles;
    return {lg / tiles, (t / p.tiles_n) * GEMM_BM, (t % p.tiles_n) * GEMM_BN};
}

// The tiled kernel.  A workgroup walks the tiles L = blockIdx.x,
// blockIdx.x + gridDim.x, ... as one stream of (tile, K-slice) steps, so the
// fetch of a tile's first slice overlaps the previous tile's last slice,
// argmax resolve and stores: only the first tile of a workgroup pays the
// latency of starting up.
template <int SR, typename T>
__device__ __forceinline__ void gemm_tiled_body(const TropGemmParams& p) {
    using R = Ring<SR, T>;
    using G = GemmTile<SR, T>;
    using Loader = typename G::Loader;
    constexpr int NST = GEMM_KBLK / GEMM_BK;  // slices per resident K-block
    __shared__ __attribute__((aligned(16))) T As[NST * GEMM_SLOT];
    __shared__ __attribute__((aligned(16))) T Bs[NST * GEMM_SLOT];

    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    const int64_t total = tiles * p.batch;
    const int nslices = (int)((p.k + GEMM_BK - 1) / GEMM_BK);
    const int full_slices = (int)(p.k / GEMM_BK);
    const int64_t stride = gridDim.x;

    int64_t cL = blockIdx.x;  // tile being computed
    if (cL >= total || nslices == 0) return;  // K = 0 is handled by the fill kernel

    // Fetch cursor: the (tile, slice) whose data was last requested into
    // registers, and the loaders of that tile.
    int64_t fL = cL;
    int fg = 0;
    TileCoord ft = tile_coord(p, fL, tiles, total);
    auto make_loaders = [&](const TileCoord& tc, Loader& la, Loader& lb, bool& fa, bool& fb) {
        la = G::make(static_cast<const T*>(p.A) + tc.b * p.sa_batch, p.a_mode, p.a_vec, tc.row0, p.m,
                     p.k, p.sa_row, p.sa_col, tid);
        lb = G::make(static_cast<const T*>(p.B) + tc.b * p.sb_batch, p.b_mode, p.b_vec, tc.col0, p.n,
                     p.k, p.sb_col, p.sb_row, tid);
        fa = tc.row0 + GEMM_BM <= p.m;
        fb = tc.col0 + GEMM_BN <= p.n;
    };
    Loader la, lb;
    bool fa_full, fb_full;
    make_loaders(ft, la, lb, fa_full, fb_full);
    bool fetch_valid = true;
    // advance the fetch cursor by one step and request that slice
    T ra[4], rb[4];
    auto fetch_next = [&]() {
        ++fg;
        if (fg == nslices) {
            fg = 0;
            fL += stride;
            fetch_valid = fL < total;
            if (fetch_valid) {
                ft = tile_coord(p, fL, tiles, total);
                make_loaders(ft, la, lb, fa_full, fb_full);
            }
        }
        if (fetch_valid) {
            la.load(fg, fa_full && fg < full_slices, R::zero(), ra);
            lb.load(fg, fb_full && fg < full_slices, R::one(), rb);
        }
    };

    // prologue: the first slice goes to LDS slot 0, the step after it to
    // registers (both requests in flight together)
    {
        T r0a[4], r0b[4];
        la.load(0, fa_full && 0 < full_slices, R::zero(), r0a);
        lb.load(0, fb_full && 0 < full_slices, R::one(), r0b);
        fetch_next();
        G::store(la.mn_contig, As, 0, tid, r0a);
        G::store(lb.mn_contig, Bs, 0, tid, r0b);
    }
    __syncthreads();

    TileCoord ct = tile_coord(p, cL, tiles, total);
    T best[GEMM_TM][GEMM_TN];
    T cv[GEMM_TM][GEMM_TN];
    int win[GEMM_TM][GEMM_TN];
    int idx[GEMM_TM][GEMM_TN];
    auto reset_outputs = [&]() {
#pragma unroll
        for (int r = 0; r < GEMM_TM; ++r)
#pragma unroll
            for (int c = 0; c < GEMM_TN; ++c) {
                best[r][c] = R::zero();
                cv[r][c] = R::zero();
                win[r][c] = -1;
                idx[r][c] = 0;
            }
    };
    reset_outputs();

    int g = 0;           // slice of the current tile
    int block_k0 = 0;    // first k of the resident block
    for (;;) {
        const int s = g % NST;
        const bool last = (g + 1 == nslices);
        const bool boundary = last || ((g + 1) % NST == 0);
        // The registers hold slice g+1 of this tile: inside a block its LDS
        // slot is free, so park it now and fetch the step after it; both
        // overlap this slice's compute.
        if (!boundary) {
            G::store(la.mn_contig, As, s + 1, tid, ra);
            G::store(lb.mn_contig, Bs, s + 1, tid, rb);
            fetch_next();
        }

        const T* as = As + s * GEMM_SLOT + 2 * ty;
        const T* bs = Bs + s * GEMM_SLOT + 2 * tx;
        T run[GEMM_TM][GEMM_TN];
#pragma unroll
        for (int r = 0; r < GEMM_TM; ++r)
#pragma unroll
            for (int c = 0; c < GEMM_TN; ++c) run[r][c] = best[r][c];
        // fragments of term pairs, double-buffered: pair p+1 is read from
        // LDS while pair p computes
        T fa[2][2][GEMM_TM], fb[2][2][GEMM_TN];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int r = 0; r < GEMM_TM; ++r) fa[0][h][r] = as[h * GEMM_LDP + own(r)];
#pragma unroll
            for (int c = 0; c < GEMM_TN; ++c) fb[0][h][c] = bs[h * GEMM_LDP + own(c)];
        }
#pragma unroll
        for (int pr = 0; pr < GEMM_BK / 2; ++pr) {
            const int cur = pr & 1, nxt = cur ^ 1;
            if (pr + 1 < GEMM_BK / 2) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kk = 2 * pr + 2 + h;
#pragma unroll
                    for (int r = 0; r < GEMM_TM; ++r) fa[nxt][h][r] = as[kk * GEMM_LDP + own(r)];
#pragma unroll
                    for (int c = 0; c < GEMM_TN; ++c) fb[nxt][h][c] = bs[kk * GEMM_LDP + own(c)];
                }
            }
#pragma unroll
            for (int r = 0; r < GEMM_TM; ++r)
#pragma unroll
                for (int c = 0; c < GEMM_TN; ++c)
                    run[r][c] = R::add3(run[r][c], R::mul(fa[cur][0][r], fb[cur][0][c]),
                                        R::mul(fa[cur][1][r], fb[cur][1][c]));
        }
#pragma unroll
        for (int r = 0; r < GEMM_TM; ++r)
#pragma unroll
            for (int c = 0; c < GEMM_TN; ++c) {
                if (R::better(run[r][c], best[r][c])) win[r][c] = s;
                best[r][c] = run[r][c];
            }

        if (boundary) {
            // Resolve the outputs whose best improved inside this block: the
            // first term of the winning slice equal to the best.  The four
            // outputs of a row are scanned together (independent chains, no
            // branch); an output that did not improve scans slot 0 and keeps
            // its earlier result.
#pragma unroll
            for (int r = 0; r < GEMM_TM; ++r) {
                const T* ac[GEMM_TN];
                const T* bc[GEMM_TN];
                int found[GEMM_TN];
#pragma unroll
                for (int c = 0; c < GEMM_TN; ++c) {
                    const int w = win[r][c] < 0 ? 0 : win[r][c];
                    ac[c] = As + w * GEMM_SLOT + 2 * ty + own(r);
                    bc[c] = Bs + w * GEMM_SLOT + 2 * tx + own(c);
                    found[c] = GEMM_BK - 1;
                }
#pragma unroll
                for (int kk = GEMM_BK - 1; kk >= 0; --kk)
#pragma unroll
                    for (int c = 0; c < GEMM_TN; ++c) {
                        const T term = R::mul(ac[c][kk * GEMM_LDP], bc[c][kk * GEMM_LDP]);
                        found[c] = (term == best[r][c]) ? kk : found[c];
                    }
#pragma unroll
                for (int c = 0; c < GEMM_TN; ++c) {
                    const T term = R::mul(ac[c][found[c] * GEMM_LDP], bc[c][found[c] * GEMM_LDP]);
                    const bool hit = win[r][c] >= 0;
                    idx[r][c] = hit ? block_k0 + win[r][c] * GEMM_BK + found[c] : idx[r][c];
                    cv[r][c] = hit ? term : cv[r][c];
                    win[r][c] = -1;
                }
            }
            block_k0 += GEMM_KBLK;

            if (last) {
                // the tile is complete: store C and argmax
                T* __restrict__ C = static_cast<T*>(p.C) + ct.b * p.sc_batch;
                int32_t* __restrict__ I = p.argmax ? p.argmax + ct.b * p.sc_batch : nullptr;
                const bool pairs = p.c_vec2 && ct.col0 + GEMM_BN <= p.n;
#pragma unroll
                for (int r = 0; r < GEMM_TM; ++r) {
                    const int64_t i = ct.row0 + 2 * ty + own(r);
                    if (i >= p.m) continue;
#pragma unroll
                    for (int c = 0; c < GEMM_TN; c += 2) {
                        const int64_t j = ct.col0 + 2 * tx + own(c);
                        const int64_t off = i * p.sc_row + j;
                        if (pairs) {
                            using V2 = T __attribute__((ext_vector_type(2)));
                            using I2 = int32_t __attribute__((ext_vector_type(2)));
                            *reinterpret_cast<V2*>(C + off) = V2{cv[r][c], cv[r][c + 1]};
                            if (I) *reinterpret_cast<I2*>(I + off) = I2{idx[r][c], idx[r][c + 1]};
                        } else {
#pragma unroll
                            for (int e = 0; e < 2; ++e) {
                                const int64_t jj = j + e;
                                if (jj >= p.n) continue;
                                const int64_t o = i * p.sc_row + jj * p.sc_col;
                                C[o] = cv[r][c + e];
                                if (I) I[o] = idx[r][c + e];
                            }
                        }
                    }
                }
            }
            if (!fetch_valid) break;  // no further step for this workgroup
            __syncthreads();          // every wave is done with this block's LDS
            G::store(la.mn_contig, As, 0, tid, ra);
            G::store(lb.mn_contig, Bs, 0, tid, rb);
            fetch_next();
            if (last) {
                cL += stride;
                ct = tile_coord(p, cL, tiles, total);
                reset_outputs();
                g = -1;
                block_k0 = 0;
            }
        }
        __syncthreads();  // the next slice is visible in LDS
        ++g;
    }
}

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
