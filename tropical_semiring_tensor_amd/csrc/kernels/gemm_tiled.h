// Strided-batched tropical GEMM with argmax: the tiled kernel for gfx950.
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
//    Instead the running value is compared once per chunk of CH terms (16;
//    8 in the wide float kernels, whose K-block is short) (one compare + one
//    select: which chunk last improved strictly).  The
//    kernel keeps a whole K-block of KBLK terms of both operand tiles
//    resident in LDS; at the end of each block every output whose best
//    improved inside it re-scans its winning chunk for the first term equal
//    to the block's best.  That is the exact first winner: a chunk is
//    recorded only when it holds a term above everything before it, and
//    inside it the first term equal to the final value is that first winner.
//  * LDS holds both operands k-contiguous ([row][k] for A, [column][k] for
//    B, rows padded by 4 words), so the main loop reads four k at a time
//    per row or column with one 16-byte LDS read, and the re-scan reads its
//    16 terms with four.  k-contiguous global operands are copied in as
//    16-byte vectors; row- or column-contiguous ones are transposed on the
//    way in.
//  * C takes the bits of the first winning term.  Those differ from the
//    running maximum's bits only for a zero result (+0 against -0), so only
//    outputs whose value is zero are recomputed from global memory at the
//    resolved index; an output that nothing beat holds the zero element.
//
// Tiling: 256 threads (4 waves) or 512 (8 waves), a 64x64 output tile per
// workgroup, 16 or 8 outputs per thread at rows ty + RS r and columns
// tx + 16 c (tx = tid % 16, ty = tid / 16, RS = threads / 16).  The forms
// with one 16-column group per thread (NC = 1: products with at most 16
// columns, small products) take 64 x 16 tiles, c = 0 only.  K is staged
// through LDS in slices of SL terms;
// the slice after next is fetched into registers while the current one
// computes and the next one is written to LDS at its start, so one barrier
// per slice suffices (one more at the end of each resident block).
//
// Without an argmax output the same loop runs with no record and no
// re-scan, and LDS holds a ring of two slices instead of a block.
//
// Global resolve (GRES, products with a long K): LDS holds the same ring of
// two slices as the value-only kernel, the record keeps the index of the
// last strictly improving chunk over the tile's whole K, and the first
// winner is found once per output and tile, after the last slice, by
// re-reading that one chunk of both operands from global memory (it was
// streamed through the tile moments before, so it comes from L2 or the
// memory-side cache).  That replaces one LDS re-scan per resident block
// (16 of them at K = 2048) with one 128-byte re-read per output; for short
// K the re-read outweighs the re-scans and the resident-block forms stay.
#pragma once
#include <type_traits>

#include "ring.h"

namespace trop {

#ifndef TROP_GEMM_THREADS
#define TROP_GEMM_THREADS 512
#endif
constexpr int GEMM_THREADS = TROP_GEMM_THREADS;  // 256 or 512
static_assert(GEMM_THREADS == 256 || GEMM_THREADS == 512, "4 or 8 waves");
// Thread tx = tid % 16, ty = tid / 16 owns rows ty + GEMM_RS r (r < GEMM_TR)
// and columns tx + 16 c (c < 4) of the 64x64 tile.
constexpr int GEMM_RS = GEMM_THREADS / 16;
constexpr int GEMM_TR = 64 / GEMM_RS;
constexpr int GEMM_BM = 64;
constexpr int GEMM_BN = 64;
constexpr int GEMM_CH = 16;  // argmax chunk (terms)
// Chunk record: 1 = the running best flows through the chunk's max3 chain
// and is compared with its value before the chunk (one compare, one
// select; with an even number of chunks per slice the two values trade
// registers with no copies); 0 = a separate per-chunk (+) is compared with
// the running best (one compare, two selects).
#ifndef TROP_GEMM_CHAIN_RECORD
#define TROP_GEMM_CHAIN_RECORD 1
#endif
constexpr bool GEMM_CHAIN_RECORD = TROP_GEMM_CHAIN_RECORD != 0;
// LDS staging slice (terms) of the argmax and the value-only kernels
#ifndef TROP_GEMM_SLICE_ARG
#define TROP_GEMM_SLICE_ARG 64
#endif
#ifndef TROP_GEMM_SLICE_VO
#define TROP_GEMM_SLICE_VO 32
#endif
#ifndef TROP_GEMM_KBLK
#define TROP_GEMM_KBLK 256
#endif
// The wide float argmax kernels (many tiles): K-block 128, slices of 32
// terms, and no second LDS fragment or re-scan buffer in flight.  That fits
// them in 128 VGPRs (from 170), so two 512-thread workgroups share a CU (4
// waves per SIMD instead of 2) and the adds of one wave pair with the max3s
// of another: against the setting below, +6% on 64 x 256^3, +9% at
// K = 1024, +5% on max-mul.  With one tile per CU or less the second
// workgroup has nothing to do, the loads are no longer hidden and the
// K = 256 products re-scan twice: there (NARROW) and in the split-K
// kernels, and in the int32 kernels (their adds do not pair; the extra
// waves cost them 12%), the K-block is 256, slices 64, both buffers kept.
#ifndef TROP_GEMM_F32_KBLK
#define TROP_GEMM_F32_KBLK 128
#endif
#ifndef TROP_GEMM_F32_SLICE_ARG
#define TROP_GEMM_F32_SLICE_ARG 32
#endif

// Global-resolve kernels: slice (terms) and whether the next LDS fragment
// is loaded ahead in the main loop.
#ifndef TROP_GEMM_SLICE_GR
#define TROP_GEMM_SLICE_GR 32
#endif
#ifndef TROP_GEMM_GR_PF
#define TROP_GEMM_GR_PF 0
#endif
#ifndef TROP_GEMM_CH_GR
#define TROP_GEMM_CH_GR 16  // argmax chunk of the global-resolve kernels (terms)
#endif
// Argmax chunk of the wide float kernels (K-block 128: each output re-scans
// one chunk per block, so a shorter chunk halves the re-scan for one more
// record per 8 terms)
#ifndef TROP_GEMM_CH_WIDE
#define TROP_GEMM_CH_WIDE 8
#endif

template <bool ARG, typename T, bool NARROW, bool GRES = false>
struct GemmCfg {
    static constexpr bool F32A = ARG && std::is_same<T, float>::value && !NARROW && !GRES;
    // an LDS block resident for the argmax re-scan (else a ring of two slices)
    static constexpr bool BLOCK = ARG && !GRES;
    // K terms resident in LDS: a block (argmax) or a ring of two slices
    static constexpr int SL = GRES ? TROP_GEMM_SLICE_GR
                                   : ARG ? (F32A ? TROP_GEMM_F32_SLICE_ARG : TROP_GEMM_SLICE_ARG)
                                         : TROP_GEMM_SLICE_VO;  // slice (terms)
    static constexpr int KB = BLOCK ? (F32A ? TROP_GEMM_F32_KBLK : TROP_GEMM_KBLK) : 2 * SL;
    // next LDS fragment (main loop) and next chunk (re-scan) loaded ahead
    static constexpr bool PF = GRES ? TROP_GEMM_GR_PF != 0 : !F32A;
    // argmax chunk (terms): one record per chunk and output
    static constexpr int CH = GRES ? TROP_GEMM_CH_GR : F32A ? TROP_GEMM_CH_WIDE : GEMM_CH;
    static constexpr int NSL = KB / SL;  // slices per block
    static_assert(SL % CH == 0 && KB % SL == 0, "whole chunks per slice, whole slices per block");
    // LDS row length in words: 4 words of padding put rows r and r + 1 in
    // different 16-byte bank groups, so 16 lanes reading 16 consecutive rows
    // at one k take distinct banks
    static constexpr int LDR = KB + 4;
};

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

// Batch entry, K split, output-tile origin and K extent of logical tile L.
struct TileCoord {
    int64_t b, s, row0, col0, kt;
};

// floor(n / d) with the host's magic pair (d = 1: n itself)
__device__ __forceinline__ uint32_t mdiv(uint32_t n, uint32_t d, uint32_t m, uint32_t sh) {
    return d == 1 ? n : (__umulhi(n, m) >> sh);
}

// Element offset of k along an operand's k axis: k stride sk, or (krun > 0)
// the two-level k of TropGemmParams (k / krun at stride khi, k % krun on the
// unit-stride axis).
__device__ __forceinline__ int64_t k_offset(int64_t k, int32_t krun, int64_t khi, int64_t sk) {
    if (krun > 0) {
        const int sh = __builtin_ctz((uint32_t)krun);
        return (k >> sh) * khi + (k & (krun - 1));
    }
    return k * sk;
}

// k_offset in an instance built with the two-level k (KR), plain strides
// otherwise (the fixed-layout instances: no registers spent on it).
template <bool KR>
__device__ __forceinline__ int64_t k_off(int64_t k, int32_t krun, int64_t khi, int64_t sk) {
    if constexpr (KR) return k_offset(k, krun, khi, sk);
    return k * sk;
}

// BN: the columns of a tile (64; 16 for the forms whose threads compute one
// 16-column group)
template <bool SPLIT, int BN = GEMM_BN>
__device__ __forceinline__ TileCoord tile_coord(const TropGemmParams& p, int64_t L, int64_t tiles,
                                                int64_t total) {
    if (p.coord32) {
        // the same decode in 32 bits (every index < 2^31)
        const uint32_t nx = 8, tot = (uint32_t)total;
        uint32_t lg = (uint32_t)L;
        if (p.swizzle) {
            const uint32_t per = (tot + nx - 1) / nx;
            uint32_t tall = tot % nx;
            if (tall == 0) tall = nx;
            const uint32_t x = lg % nx, local = lg / nx;
            lg = x < tall ? x * per + local : tall * per + (x - tall) * (per - 1) + local;
        }
        const uint32_t tl = (uint32_t)tiles, tn = (uint32_t)p.tiles_n;
        const uint32_t bs = mdiv(lg, tl, p.tl_m, p.tl_s);
        const uint32_t t = lg - bs * tl;
        uint32_t tr, tc;
        if (p.group_rows > 1) {
            const uint32_t G = (uint32_t)p.group_rows;
            const uint32_t gsz = G * tn;
            const uint32_t gi = mdiv(t, gsz, p.gr_m, p.gr_s);
            const uint32_t r0 = gi * G;
            const uint32_t rows = min(G, (uint32_t)p.tiles_m - r0);
            const uint32_t w = t - gi * gsz;
            tc = w / rows;
            tr = r0 + (w - tc * rows);
        } else {
            tr = mdiv(t, tn, p.tn_m, p.tn_s);
            tc = t - tr * tn;
        }
        TileCoord c{bs, 0, (int64_t)tr * GEMM_BM, (int64_t)tc * BN, p.k};
        if constexpr (SPLIT) {
            const uint32_t ks = (uint32_t)p.ksplit;
            const uint32_t b = mdiv(bs, ks, p.ks_m, p.ks_s);
            c.b = b;
            c.s = bs - b * ks;
            const int64_t rest = p.k - c.s * p.kchunk;
            c.kt = rest < p.kchunk ? rest : p.kchunk;
        }
        return c;
    }
    const int64_t lg = p.swizzle ? xcd_remap(L, total) : L;
    const int64_t t = lg % tiles;
    const int64_t bs = lg / tiles;
    int64_t tr, tc;
    if (p.group_rows > 1) {
        const int64_t G = p.group_rows;
        const int64_t gsz = G * p.tiles_n;
        const int64_t r0 = t / gsz * G;
        const int64_t rows = p.tiles_m - r0 < G ? p.tiles_m - r0 : G;
        const int64_t w = t - r0 * p.tiles_n;
        tc = w / rows;
        tr = r0 + (w - tc * rows);
    } else {
        tr = t / p.tiles_n;
        tc = t % p.tiles_n;
    }
    TileCoord c{bs, 0, tr * GEMM_BM, tc * BN, p.k};
    if constexpr (SPLIT) {
        c.b = bs / p.ksplit;
        c.s = bs % p.ksplit;
        const int64_t rest = p.k - c.s * p.kchunk;
        c.kt = rest < p.kchunk ? rest : p.kchunk;
    }
    return c;
}

// One thread's share of one operand tile per slice: NV vectors of 4
// elements.  K_CONTIG: a vector runs along k at one row (A) / column (B);
// MN_CONTIG: along the rows / columns at one k.  Vector v sits 16 k after
// vector v - 1.
// Vector vi = tid + GEMM_THREADS v of a slice; K_CONTIG: 8 consecutive
// vectors take 8 rows at one k, so their 16-byte LDS writes fall in distinct
// bank groups; MN_CONTIG: 16 consecutive vectors cover 64 rows at one k.
__device__ __forceinline__ int kc_row(int vi) { return (vi & 7) + 8 * ((vi >> 5) & 7); }
__device__ __forceinline__ int kc_k(int vi) { return ((vi >> 3) & 3) * 4 + 16 * (vi >> 8); }
__device__ __forceinline__ int mc_row(int vi) { return (vi & 15) * 4; }
__device__ __forceinline__ int mc_k(int vi) { return vi >> 4; }

// B's LDS rows are swizzled: logical column k of row j sits at k ^ bsw(j),
// bsw(j) = 4 ((j / 16) mod 4).  That only permutes the 16-byte quads inside
// each aligned group of four, so 16-byte reads stay whole, and it makes the
// transposed stores of a row-contiguous B (16 rows 4 apart at 4 k per
// instruction) hit distinct banks.  A thread's columns tx + 16 c all share
// bsw = 4 c, a compile-time constant in the compute loop.
__device__ __forceinline__ int bsw(int row) { return ((row >> 4) & 3) << 2; }

// Exact conversion of a staged element to the compute type (int32 data
// computed in float: see the float mode of the int32 products below).
template <typename T, typename TG>
__device__ __forceinline__ T to_compute(TG x) {
    return static_cast<T>(x);
}

// Operand layout of a kernel instance: read from the launch's arguments
// (LAYOUT_ANY), or fixed at compile time to 16-byte vectors along k
// (LAYOUT_KV) or along the rows / columns (LAYOUT_MV), which removes the
// other paths and their registers.
constexpr int LAYOUT_ANY = 0, LAYOUT_KV = 1, LAYOUT_MV = 2;

template <typename T, int NV, int LDR, bool SWZ, int SL, typename TG = T, int LAYOUT = LAYOUT_ANY>
struct OpLoad {
    using V = vec4<TG>;
    const TG* q0;      // element 0 of vector 0 of slice 0
    int64_t k_step;    // elements per slice along k
    int64_t v_step;    // elements between vectors v and v + 1
    int64_t e_str;     // elements between the 4 elements of a vector
    int64_t mn;        // row / column of element 0
    int64_t k0;        // k of element 0 in slice 0
    int64_t koff0;     // element offset of k0 along the k axis
    int64_t mn_lim, k_lim;
    int lds0;          // LDS word offset of element 0 (slot 0)
    int lds_v;         // LDS words between vectors v and v + 1
    int kv;            // k between vectors v and v + 1
    bool mn_c_, vec_, mn_full;
    __device__ __forceinline__ bool mn_c() const { return LAYOUT == LAYOUT_ANY ? mn_c_ : LAYOUT == LAYOUT_MV; }
    __device__ __forceinline__ bool vec() const { return LAYOUT == LAYOUT_ANY ? vec_ : true; }

    // Position of this thread's elements (independent of the tile).
    __device__ __forceinline__ void init(int mode, int v16, int64_t str_mn, int64_t str_k,
                                         int64_t mnl, int64_t kl, int tid, int32_t krun, int64_t khi) {
        mn_c_ = (mode == TROP_LOAD_MN_CONTIG);
        vec_ = v16 != 0;
        mn_lim = mnl;
        k_lim = kl;
        k_step = (int64_t)SL * str_k;
        // vector v + 1 = vector index + GEMM_THREADS: the same row, k further
        // on by GEMM_THREADS / 16 (MN_CONTIG) or 16 GEMM_THREADS / 256
        // (K_CONTIG)
        kv = mn_c() ? mc_k(GEMM_THREADS) : kc_k(GEMM_THREADS);
        v_step = kv * str_k;
        lds_v = kv;
        // (the swizzle only touches bits 2-3 of k, and the slot offset and
        // vector steps added later are multiples of 16)
        if (mn_c()) {
            e_str = str_mn;
            k0 = mc_k(tid);
            mn = mc_row(tid);
            lds0 = mc_row(tid) * LDR + (mc_k(tid) ^ (SWZ ? bsw(mc_row(tid)) : 0));
        } else {
            e_str = str_k;
            k0 = kc_k(tid);
            mn = kc_row(tid);
            lds0 = kc_row(tid) * LDR + (kc_k(tid) ^ (SWZ ? bsw(kc_row(tid)) : 0));
        }
        koff0 = k0 * str_k;
        if (!mn_c() && krun > 0) {
            // two-level k: a slice, the vector step and a thread's first k
            // are whole runs of krun apart plus a place inside a run (SL and
            // kv are multiples of 16, k0 of 4, krun divides 16)
            const int sh = __builtin_ctz((uint32_t)krun);
            k_step = (int64_t)(SL >> sh) * khi;
            v_step = (int64_t)(kv >> sh) * khi;
            koff0 = (int64_t)(k0 >> sh) * khi + (k0 & (krun - 1));
        }
    }

    // Point at a tile: X is the operand of the batch entry, mn_start the
    // tile's first row / column, str_mn the stride along it.
    __device__ __forceinline__ void at(const TG* X, int64_t mn_start, int64_t str_mn, int64_t str_k,
                                       int tid) {
        const int64_t m_rel = mn_c() ? mc_row(tid) : kc_row(tid);
        mn = mn_start + m_rel;
        q0 = X + mn * str_mn + koff0;
        mn_full = mn_start + 64 <= mn_lim;
    }

    __device__ __forceinline__ void load(int g, T pad, T (&r)[NV][4]) const {
        const TG* q = q0 + (int64_t)g * k_step;
        // K < 2^31 (the host's limit: int32 argmax), so the slice bounds
        // compare in 32 bits (a scalar compare; 64-bit ones go to the VALU)
        const uint32_t kb = (uint32_t)k0 + (uint32_t)g * SL;
        const bool full = mn_full && (uint32_t)(g + 1) * (uint32_t)SL <= (uint32_t)k_lim;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const TG* qv = q + v * v_step;
            if (full) {
                if (vec()) {
                    const V x = *reinterpret_cast<const V*>(qv);
                    r[v][0] = to_compute<T>(x.x);
                    r[v][1] = to_compute<T>(x.y);
                    r[v][2] = to_compute<T>(x.z);
                    r[v][3] = to_compute<T>(x.w);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[v][e] = to_compute<T>(qv[e * e_str]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t kk = kb + (uint32_t)(kv * v + (mn_c() ? 0 : e));
                    const int64_t mm = mn + (mn_c() ? e : 0);
                    r[v][e] = (kk < (uint32_t)k_lim && mm < mn_lim) ? to_compute<T>(qv[e * e_str]) : pad;
                }
            }
        }
    }

    // Write a slice held in registers to LDS at k offset `sk` of the block.
    __device__ __forceinline__ void store(T* S, int sk, const T (&r)[NV][4]) const {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            T* d = S + lds0 + sk + lds_v * v;
            if (mn_c()) {
#pragma unroll
                for (int e = 0; e < 4; ++e) d[e * LDR] = r[v][e];
            } else {
                *reinterpret_cast<vec4<T>*>(d) = vec4<T>{r[v][0], r[v][1], r[v][2], r[v][3]};
            }
        }
    }
};

// C bits of the outputs whose value is zero (max-plus / min-plus float32):
// the bits of the first winning term, recomputed from global memory at the
// resolved index (with argmax) or found by a scan along k (value only).
// Rare and only taken by a wave that holds such an output.
template <int SR, typename T, bool ARG, bool SPLIT, bool KR, int NC>
__device__ __forceinline__ void zero_bits_fixup(const TropGemmParams& p, TileCoord ct, int tx,
                                                          int ty, T (&best)[GEMM_TR][NC],
                                                          const int (&idx)[GEMM_TR][NC]) {
    using R = Ring<SR, T>;
    const T* A = static_cast<const T*>(p.A) + ct.b * p.sa_batch +
                 (SPLIT ? k_off<KR>(ct.s * p.kchunk, p.a_krun, p.sa_khi, p.sa_col) : 0);
    const T* B = static_cast<const T*>(p.B) + ct.b * p.sb_batch +
                 (SPLIT ? k_off<KR>(ct.s * p.kchunk, p.b_krun, p.sb_khi, p.sb_row) : 0);
    for (int r = 0; r < GEMM_TR; ++r)
        for (int c = 0; c < NC; ++c) {
            const int64_t i = ct.row0 + ty + GEMM_RS * r, j = ct.col0 + tx + 16 * c;
            if (i >= p.m || j >= p.n || !(best[r][c] == (T)0)) continue;
            const T* a = A + i * p.sa_row;
            const T* b = B + j * p.sb_col;
            if constexpr (ARG) {
                const int64_t k = idx[r][c];
                best[r][c] = R::mul(a[k_off<KR>(k, p.a_krun, p.sa_khi, p.sa_col)],
                                    b[k_off<KR>(k, p.b_krun, p.sb_khi, p.sb_row)]);
            } else {
                for (int64_t k = 0; k < (SPLIT ? ct.kt : p.k); ++k) {
                    const T t = R::mul(a[k_off<KR>(k, p.a_krun, p.sa_khi, p.sa_col)],
                                       b[k_off<KR>(k, p.b_krun, p.sb_khi, p.sb_row)]);
                    if (t == best[r][c]) {
                        best[r][c] = t;
                        break;
                    }
                }
            }
        }
}

// Global resolve of a finished tile, with the whole workgroup.  Each thread
// has parked its outputs' values and chunk records in LDS (`rv`, `rw`: the
// 64 x 64 tile row by row, rows GEMM_RLD words apart).  A wave then takes
// 512 of the outputs, four lanes to an output: lane q of the four re-reads
// terms 4q .. 4q + 3 of the output's last improving chunk from global
// memory (one 16-byte load per operand when k is the unit-stride axis, so
// a load instruction touches 16 cache lines, not 64) and finds the first
// of them equal to the final value; the four answers combine by shuffles
// into the first in the chunk, written back to `rw` as the relative k (0 for
// an output that nothing beat).  Terms past the tile's K extent are not
// read: they are padding in the main loop and cannot win.  Loads are
// issued for every lane (an output with nothing to resolve reads the tile's
// first element), so the compiler can keep several steps in flight.
constexpr int GEMM_RLD = 65;  // row length of the parked tile (words; odd: rows in different banks)
#ifndef TROP_GEMM_RESOLVE_UNROLL
#define TROP_GEMM_RESOLVE_UNROLL 4  // resolve steps (16 outputs each) per group of loads
#endif
#define TROP_PRAGMA_(x) _Pragma(#x)
#define TROP_PRAGMA(x) TROP_PRAGMA_(x)

#ifndef TROP_GEMM_RESOLVE_CALL
#define TROP_GEMM_RESOLVE_CALL 0
#endif
#if TROP_GEMM_RESOLVE_CALL
// a call, not inlined: its registers are saved once per tile at the call
// instead of constraining the allocation of the main loop
#define TROP_RESOLVE_ATTR __attribute__((noinline))
#else
#define TROP_RESOLVE_ATTR __forceinline__
#endif
template <int SR, typename T, bool SPLIT, int CH, typename TG = T, bool FIXED_KV = false, bool KR = true>
__device__ TROP_RESOLVE_ATTR void resolve_tile(const TropGemmParams& p, TileCoord ct, int tid, const T* rv,
                                             int* rw) {
    using R = Ring<SR, T>;
    using V = vec4<TG>;
    constexpr int QL = CH / 16;  // quads per lane: lane q reads quads q, q + 4, ...
    static_assert(CH % 16 == 0, "four lanes share a chunk of whole quads");
    const int64_t kt = SPLIT ? ct.kt : p.k;
    const TG* const A = static_cast<const TG*>(p.A) + ct.b * p.sa_batch +
                        (SPLIT ? k_off<KR>(ct.s * p.kchunk, p.a_krun, p.sa_khi, p.sa_col) : 0);
    const TG* const B = static_cast<const TG*>(p.B) + ct.b * p.sb_batch +
                        (SPLIT ? k_off<KR>(ct.s * p.kchunk, p.b_krun, p.sb_khi, p.sb_row) : 0);
    // 16-byte loads along k: k is the unit-stride axis with aligned rows
    // (A) / columns (B); a quad starts at a multiple of 4 terms
    const bool a_kv = p.a_mode == TROP_LOAD_K_CONTIG && p.a_vec;
    const bool b_kv = p.b_mode == TROP_LOAD_K_CONTIG && p.b_vec;
    const int lane = tid & 63, wave = tid >> 6, q = lane & 3;
    constexpr int WAVES = GEMM_THREADS / 64;
    constexpr int PER_WAVE = GEMM_BM * GEMM_BN / WAVES;  // outputs per wave
    const int rlim = (int)(p.m - ct.row0 < GEMM_BM ? p.m - ct.row0 : GEMM_BM);
    const int clim = (int)(p.n - ct.col0 < GEMM_BN ? p.n - ct.col0 : GEMM_BN);
    const int kt32 = (int)kt;  // K < 2^31
    // (FIXED_KV: an instance for operands read along k in 16-byte vectors,
    // launched only when K is a multiple of 4)
    if (FIXED_KV || (a_kv && b_kv && (kt32 & 3) == 0)) {
        // both operands k-contiguous and K a multiple of 4: every quad is
        // wholly inside or wholly past K, and each lane makes one 16-byte
        // load per operand and quad (a lane with nothing to read loads the
        // tile's first quad and ignores it).  Steps go in groups of G: all
        // of a group's LDS reads, then its loads, its compares and its LDS
        // writes, so the writes of one step cannot hold back the loads of
        // the next.
        constexpr int G = TROP_GEMM_RESOLVE_UNROLL;
        static_assert((PER_WAVE / 16) % G == 0, "whole groups of steps");
        const TG* const Ar = A + ct.row0 * p.sa_row;
        const TG* const Bc = B + ct.col0 * p.sb_col;
        // FIXED_KV: the host launches this instance only when every element
        // of the tile's row and column panels lies below 2^29 elements from
        // the panel's start, so a quad's place is a 32-bit byte offset from a
        // wave-uniform base (no 64-bit address arithmetic per step)
        const uint32_t sa_b = (uint32_t)p.sa_row * (uint32_t)sizeof(TG);
        const uint32_t sb_b = (uint32_t)p.sb_col * (uint32_t)sizeof(TG);
        // byte offset of a quad's first k (two-level k: whole runs at the
        // run stride, then the place inside the run)
        const int a_sh = p.a_krun > 0 ? __builtin_ctz((uint32_t)p.a_krun) : 0;
        const int b_sh = p.b_krun > 0 ? __builtin_ctz((uint32_t)p.b_krun) : 0;
        const uint32_t a_hi = p.a_krun > 0 ? (uint32_t)p.sa_khi * (uint32_t)sizeof(TG) : 0u;
        const uint32_t b_hi = p.b_krun > 0 ? (uint32_t)p.sb_khi * (uint32_t)sizeof(TG) : 0u;
        const uint32_t a_lo = p.a_krun > 0 ? (uint32_t)p.a_krun - 1 : ~0u;
        const uint32_t b_lo = p.b_krun > 0 ? (uint32_t)p.b_krun - 1 : ~0u;
        // one copy of the loop per k layout (a uniform choice, made once)
        auto steps = [&](auto two_c) {
            constexpr bool TWO = decltype(two_c)::value;
#pragma unroll 1
            for (int st0 = 0; st0 < PER_WAVE / 16; st0 += G) {
                T bst[G];
                int w[G], off[G], row[G], col[G];
                bool live[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int o = wave * PER_WAVE + 16 * (st0 + g) + (lane >> 2);
                    row[g] = o >> 6;
                    col[g] = o & 63;
                    off[g] = row[g] * GEMM_RLD + col[g];
                    bst[g] = rv[off[g]];
                    w[g] = rw[off[g]];
                    live[g] = row[g] < rlim && col[g] < clim;
                }
                V x[G][QL], y[G][QL];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    live[g] = live[g] && w[g] >= 0;
#pragma unroll
                    for (int h = 0; h < QL; ++h) {
                        const int k0 = w[g] * CH + 4 * (q + 4 * h);
                        const bool in = live[g] && k0 < kt32;
                        if constexpr (FIXED_KV) {
                            const uint32_t ku = (uint32_t)k0;
                            uint32_t ka = ku * (uint32_t)sizeof(TG), kb = ka;
                            if constexpr (TWO) {
                                ka = (ku >> a_sh) * a_hi + (ku & a_lo) * (uint32_t)sizeof(TG);
                                kb = (ku >> b_sh) * b_hi + (ku & b_lo) * (uint32_t)sizeof(TG);
                            }
                            const uint32_t oa = in ? (uint32_t)row[g] * sa_b + ka : 0u;
                            const uint32_t ob = in ? (uint32_t)col[g] * sb_b + kb : 0u;
                            x[g][h] = *reinterpret_cast<const V*>(reinterpret_cast<const char*>(Ar) + oa);
                            y[g][h] = *reinterpret_cast<const V*>(reinterpret_cast<const char*>(Bc) + ob);
                        } else {
                            const int64_t ka = TWO ? k_offset(k0, p.a_krun, p.sa_khi, 1) : k0;
                            const int64_t kb = TWO ? k_offset(k0, p.b_krun, p.sb_khi, 1) : k0;
                            x[g][h] = *reinterpret_cast<const V*>(Ar + (in ? row[g] * p.sa_row + ka : 0));
                            y[g][h] = *reinterpret_cast<const V*>(Bc + (in ? col[g] * p.sb_col + kb : 0));
                        }
                    }
                }
                int f[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    f[g] = CH;  // first matching term of this lane's quads, as its place in the chunk
#pragma unroll
                    for (int h = QL - 1; h >= 0; --h) {
                        const int kq = 4 * (q + 4 * h);
                        const bool in = live[g] && w[g] * CH + kq < kt32;
                        const V& xa = x[g][h];
                        const V& yb = y[g][h];
                        f[g] = in && R::mul(to_compute<T>(xa.w), to_compute<T>(yb.w)) == bst[g] ? kq + 3 : f[g];
                        f[g] = in && R::mul(to_compute<T>(xa.z), to_compute<T>(yb.z)) == bst[g] ? kq + 2 : f[g];
                        f[g] = in && R::mul(to_compute<T>(xa.y), to_compute<T>(yb.y)) == bst[g] ? kq + 1 : f[g];
                        f[g] = in && R::mul(to_compute<T>(xa.x), to_compute<T>(yb.x)) == bst[g] ? kq : f[g];
                    }
                    // the first match among the output's four lanes (quad permutes)
                    f[g] = min(f[g], __builtin_amdgcn_mov_dpp(f[g], 0xB1, 0xF, 0xF, true));  // lane ^ 1
                    f[g] = min(f[g], __builtin_amdgcn_mov_dpp(f[g], 0x4E, 0xF, 0xF, true));  // lane ^ 2
                }
#pragma unroll
                for (int g = 0; g < G; ++g)
                    if (q == 0) rw[off[g]] = live[g] ? w[g] * CH + f[g] : 0;
            }
        };
        if (KR && (p.a_krun | p.b_krun) != 0)
            steps(std::integral_constant<bool, KR>{});
        else
            steps(std::false_type{});
        return;
    }
    if constexpr (FIXED_KV) return;
    for (int st = 0; st < PER_WAVE / 16; ++st) {
        const int o = wave * PER_WAVE + 16 * st + (lane >> 2);
        const int row = o >> 6, col = o & 63;
        const T bst = rv[row * GEMM_RLD + col];
        const int w = rw[row * GEMM_RLD + col];
        const bool live = w >= 0 && row < rlim && col < clim;
        int f = CH;
#pragma unroll
        for (int h = QL - 1; h >= 0; --h) {
            const int kq = 4 * (q + 4 * h);  // the quad's first term within the chunk
            const int64_t k0 = live ? (int64_t)w * CH + kq : 0;
            // (a quad lies inside one run of a two-level k: krun is a
            // multiple of 4, so its 4 terms are at unit stride)
            const TG* a = A + (ct.row0 + (live ? row : 0)) * p.sa_row + k_off<KR>(k0, p.a_krun, p.sa_khi, p.sa_col);
            const TG* b = B + (ct.col0 + (live ? col : 0)) * p.sb_col + k_off<KR>(k0, p.b_krun, p.sb_khi, p.sb_row);
            T ta[4], tb[4];
            if (a_kv && k0 + 4 <= kt) {
                const V x = *reinterpret_cast<const V*>(a);
                ta[0] = to_compute<T>(x.x), ta[1] = to_compute<T>(x.y), ta[2] = to_compute<T>(x.z),
                ta[3] = to_compute<T>(x.w);
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) ta[u] = k0 + u < kt ? to_compute<T>(a[u * p.sa_col]) : R::zero();
            }
            if (b_kv && k0 + 4 <= kt) {
                const V x = *reinterpret_cast<const V*>(b);
                tb[0] = to_compute<T>(x.x), tb[1] = to_compute<T>(x.y), tb[2] = to_compute<T>(x.z),
                tb[3] = to_compute<T>(x.w);
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) tb[u] = k0 + u < kt ? to_compute<T>(b[u * p.sb_row]) : R::one();
            }
#pragma unroll
            for (int u = 3; u >= 0; --u) f = (R::mul(ta[u], tb[u]) == bst) ? kq + u : f;
        }
        f = min(f, __shfl_xor(f, 1));
        f = min(f, __shfl_xor(f, 2));
        if (q == 0) rw[row * GEMM_RLD + col] = live ? w * CH + f : 0;
    }
}

// The tiled kernel.  A workgroup walks the tiles L = blockIdx.x,
// blockIdx.x + gridDim.x, ... as one stream of (tile, slice) steps, so the
// fetch of a tile's first slice overlaps the previous tile's last slice,
// re-scan and stores.  SPLIT: the stream also covers the K ranges of a
// split-K product (a separate instantiation, so that the unsplit kernel
// keeps one slice count and one K for every tile).
// Float mode of int32 max-plus / min-plus products (TG = int32_t, T =
// float): the operands are converted on staging and every term is one f32
// add.  A separate pre-pass has checked that all of A and B lie in a domain
// where that is exact for every term that can win -- min-plus: [0, 2^23) or
// [2^30, 2^31) (a sum of two values below 2^23 is an integer below 2^24; a
// sum with a value of 2^30 or more is at least 2^30 in both rings and never
// beats the zero element 2^30); max-plus: (-2^23, 2^23) (every sum exact).
// The running value starts at the int32 zero element, +-2^30, exact in
// float, so the same terms win, and C is that exact integer.
template <int SR, typename T, typename TG>
__device__ __forceinline__ T zero_of() {
    if constexpr (std::is_same<T, TG>::value) {
        return Ring<SR, T>::zero();
    } else {
        static_assert(SR != TROP_SR_MAX_MUL, "no float mode for max-mul");
        return SR == TROP_SR_MIN_PLUS ? (T)(1 << 30) : -(T)(1 << 30);
    }
}

// Launch gate: a product whose int32 data was checked by the domain
// pre-pass is launched twice, once in float mode (mode_run = 1) and once
// with int32 arithmetic (mode_run = 0); each launch reads the pre-pass
// flags (one per pre-pass workgroup, nonzero = a value outside the domain)
// and only the one that matches proceeds.  Uniform over the workgroup.
__device__ __forceinline__ bool mode_gate_open(const TropGemmParams& p) {
    if (!p.mode_flags) return true;
    int bad = 0;
    for (int i = threadIdx.x; i < p.mode_slots; i += blockDim.x) bad |= p.mode_flags[i];
    const bool in_domain = __syncthreads_or(bad) == 0;
    return in_domain == (p.mode_run != 0);
}

template <int SR, typename T, bool ARG, bool SPLIT, bool NARROW = SPLIT, bool GRES = false, typename TG = T,
          int LAYOUT_A = LAYOUT_ANY, int LAYOUT_B = LAYOUT_ANY, bool KR = true, int NC = 4>
__device__ __forceinline__ void gemm_tiled_body(const TropGemmParams& p) {
    using R = Ring<SR, T>;
    using V = vec4<T>;
    using Cfg = GemmCfg<ARG, T, NARROW, GRES>;
    static_assert(!GRES || ARG, "the global resolve is an argmax form");
    // NC: 16-column groups a thread computes (4: the 64 x 64 tile; 1: only
    // the tile's first 16 columns, for products with at most 16 columns --
    // the rest of the tile would be padding)
    static_assert(NC == 4 || (NC == 1 && !GRES), "one column group: resident-block and value-only forms");
    constexpr bool FM = !std::is_same<T, TG>::value;  // int32 data computed in float
    constexpr bool BLK = Cfg::BLOCK;  // resident block + LDS re-scan
    constexpr int NSL = Cfg::NSL, LDR = Cfg::LDR, GEMM_SL = Cfg::SL;
    constexpr int NV = 16 * GEMM_SL / GEMM_THREADS;  // vectors per thread, operand and slice
    static_assert(NV >= 1 && NV * GEMM_THREADS == 16 * GEMM_SL, "whole vectors per thread");
    constexpr int NQ = GEMM_SL / 4;         // k-quads per slice
    constexpr int CH = Cfg::CH;              // argmax chunk (terms)
    constexpr int QPC = CH / 4;              // k-quads per chunk
    constexpr int CPS = GEMM_SL / CH;        // chunks per slice
    using LA = OpLoad<T, NV, LDR, false, GEMM_SL, TG, LAYOUT_A>;
    using LB = OpLoad<T, NV, LDR, true, GEMM_SL, TG, LAYOUT_B>;
    static_assert(GEMM_SL % 16 == 0 && LDR % 4 == 0, "slots and rows keep the swizzle inside 16-word groups");
    // A's rows, then B's columns (one array: the global resolve parks a
    // finished tile over both)
    __shared__ __attribute__((aligned(16))) T Ss[(GEMM_BM + GEMM_BN) * LDR];
    T* const As = Ss;
    T* const Bs = Ss + GEMM_BM * LDR;
    static_assert(!GRES || (GEMM_BM + GEMM_BN) * LDR >= 2 * GEMM_BM * GEMM_RLD,
                  "the parked tile fits in the operand rings");

    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    const int64_t total = tiles * p.batch * (SPLIT ? p.ksplit : 1);
    const int64_t gstride = gridDim.x;
    // slices of a tile (its K extent: the split's, or the whole K)
    const int nslices_k = (int)((p.k + GEMM_SL - 1) / GEMM_SL);
    auto slices_of = [&](const TileCoord& tc) {
        return SPLIT ? (int)((tc.kt + GEMM_SL - 1) / GEMM_SL) : nslices_k;
    };

    int64_t cL = blockIdx.x;  // tile being computed
    if (cL >= total || p.k == 0) return;  // K = 0 is handled by the fill kernel
    if (blockDim.x != GEMM_THREADS) return;   // launched with a block it was not built for
    if (!mode_gate_open(p)) return;          // the other launch of a checked int32 product runs

    LA la;
    LB lb;
    // (KR: the instance reads a two-level k when the launch asks for one)
    la.init(p.a_mode, p.a_vec, p.sa_row, p.sa_col, p.m, p.k, tid, KR ? p.a_krun : 0, KR ? p.sa_khi : 0);
    lb.init(p.b_mode, p.b_vec, p.sb_col, p.sb_row, p.n, p.k, tid, KR ? p.b_krun : 0, KR ? p.sb_khi : 0);
    const TG* const Ag = static_cast<const TG*>(p.A);
    const TG* const Bg = static_cast<const TG*>(p.B);
    int f_nsl = 0;  // slices of the tile being fetched
    auto point = [&](const TileCoord& tc) {
        la.at(Ag + tc.b * p.sa_batch + (SPLIT ? k_off<KR>(tc.s * p.kchunk, p.a_krun, p.sa_khi, p.sa_col) : 0),
              tc.row0, p.sa_row, p.sa_col, tid);
        lb.at(Bg + tc.b * p.sb_batch + (SPLIT ? k_off<KR>(tc.s * p.kchunk, p.b_krun, p.sb_khi, p.sb_row) : 0),
              tc.col0, p.sb_col, p.sb_row, tid);
        if constexpr (SPLIT) {
            la.k_lim = tc.kt;
            lb.k_lim = tc.kt;
        }
        f_nsl = slices_of(tc);
    };

    // Fetch cursor: the (tile, slice) whose data was last requested.
    int64_t fL = cL;
    int fg = 0;
    point(tile_coord<SPLIT, 16 * NC>(p, fL, tiles, total));
    bool fetch_valid = true;
    T ra[NV][4], rb[NV][4];
    auto fetch_next = [&]() {
        ++fg;
        if (fg == (SPLIT ? f_nsl : nslices_k)) {
            fg = 0;
            fL += gstride;
            fetch_valid = fL < total;
            if (fetch_valid) point(tile_coord<SPLIT, 16 * NC>(p, fL, tiles, total));
        }
        if (fetch_valid) {
            la.load(fg, R::zero(), ra);
            lb.load(fg, R::one(), rb);
        }
    };

    // prologue: slice 0 goes to LDS slot 0, slice 1 to registers
    {
        T r0a[NV][4], r0b[NV][4];
        la.load(0, R::zero(), r0a);
        lb.load(0, R::one(), r0b);
        fetch_next();
        la.store(As, 0, r0a);
        lb.store(Bs, 0, r0b);
    }
    __syncthreads();

    TileCoord ct = tile_coord<SPLIT, 16 * NC>(p, cL, tiles, total);
    int c_nsl = slices_of(ct);  // slices of the tile being computed
    T best[GEMM_TR][NC];
    int win[GEMM_TR][NC];
    int idx[GEMM_TR][NC];
    auto reset_outputs = [&]() {
#pragma unroll
        for (int r = 0; r < GEMM_TR; ++r)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                best[r][c] = zero_of<SR, T, TG>();
                win[r][c] = -1;
                idx[r][c] = 0;
            }
    };
    reset_outputs();

    const T* const a_row = As + ty * LDR;  // row ty + GEMM_RS r at + GEMM_RS r LDR
    const T* const b_col = Bs + tx * LDR;

    int g = 0;           // slice of the current tile
    int64_t blk_k0 = 0;  // first k of the resident block
    int ring = 0;        // value only: ring slot of the current slice
    for (;;) {
        const int s = BLK ? g % NSL : ring;
        const bool last = (g + 1 == (SPLIT ? c_nsl : nslices_k));
        const bool bend = BLK ? (last || s == NSL - 1) : last;
        // The registers hold slice g + 1 of this tile: its LDS slot is free
        // (argmax: inside the block; value only: the ring slot read two
        // slices ago), so park it now and fetch the step after it.
        if (!bend) {
            const int sn = (BLK ? s + 1 : s ^ 1) * GEMM_SL;
            la.store(As, sn, ra);
            lb.store(Bs, sn, rb);
            fetch_next();
        }

        // ---- compute the slice: 4 k per 16-byte fragment ----
        {
            const int sk = s * GEMM_SL;
            // Chunks of the last slice that lie wholly past K hold only
            // padding (terms that cannot win): they are skipped, which makes
            // a small K cost its own chunks and not a whole slice.  Not in
            // the global-resolve kernels (K > 256, at most one partial
            // slice): there the exit would make the running values' register
            // depend on where the slice ended, which costs a copy of every
            // one of them per slice.
            const int64_t k_left = (SPLIT ? ct.kt : p.k) - (int64_t)g * GEMM_SL;
            const int q_end = k_left >= GEMM_SL ? NQ : (int)((k_left + CH - 1) / CH) * QPC;
            V fa[2][GEMM_TR], fb[2][NC];
#pragma unroll
            for (int r = 0; r < GEMM_TR; ++r) fa[0][r] = *reinterpret_cast<const V*>(a_row + r * GEMM_RS * LDR + sk);
#pragma unroll
            for (int c = 0; c < NC; ++c) fb[0][c] = *reinterpret_cast<const V*>(b_col + c * 16 * LDR + sk + 4 * c);
            T cm[GEMM_TR][NC];    // argmax: (+) of the current chunk's terms
            T prev[GEMM_TR][NC];  // argmax: the best before the current chunk
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                if (!GRES && q % QPC == 0 && q > 0 && q >= q_end) break;  // uniform over the workgroup
                const int cur = Cfg::PF ? q & 1 : 0, nxt = cur ^ 1;
                if constexpr (Cfg::PF) {
                    if (q + 1 < NQ) {
#pragma unroll
                        for (int r = 0; r < GEMM_TR; ++r)
                            fa[nxt][r] = *reinterpret_cast<const V*>(a_row + r * GEMM_RS * LDR + sk + 4 * (q + 1));
#pragma unroll
                        for (int c = 0; c < NC; ++c)
                            fb[nxt][c] = *reinterpret_cast<const V*>(b_col + c * 16 * LDR + sk +
                                                                     4 * (((q + 1) & ~3) | (((q + 1) & 3) ^ c)));
                    }
                } else if (q > 0) {
#pragma unroll
                    for (int r = 0; r < GEMM_TR; ++r)
                        fa[0][r] = *reinterpret_cast<const V*>(a_row + r * GEMM_RS * LDR + sk + 4 * q);
#pragma unroll
                    for (int c = 0; c < NC; ++c)
                        fb[0][c] = *reinterpret_cast<const V*>(b_col + c * 16 * LDR + sk + 4 * ((q & ~3) | ((q & 3) ^ c)));
                }
#pragma unroll
                for (int r = 0; r < GEMM_TR; ++r)
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        const V a = fa[cur][r], b = fb[cur][c];
                        if constexpr (ARG && !GEMM_CHAIN_RECORD) {
                            T v = (q % QPC == 0) ? R::add2(R::mul(a.x, b.x), R::mul(a.y, b.y))
                                                 : R::add3(cm[r][c], R::mul(a.x, b.x), R::mul(a.y, b.y));
                            cm[r][c] = R::add3(v, R::mul(a.z, b.z), R::mul(a.w, b.w));
                        } else {
                            if (ARG && q % QPC == 0) prev[r][c] = best[r][c];
                            T v = R::add3(best[r][c], R::mul(a.x, b.x), R::mul(a.y, b.y));
                            best[r][c] = R::add3(v, R::mul(a.z, b.z), R::mul(a.w, b.w));
                        }
                    }
                if constexpr (ARG) {
                    if (q % QPC == QPC - 1) {
                        // record the chunk if it beats everything before it
                        // chunk within the block, or (GRES) within the tile's K
                        const int cid = (GRES ? g : s) * CPS + q / QPC;
                        if constexpr (GEMM_CHAIN_RECORD && GRES) {
                            // all compares, then all selects: the compares
                            // write separate lane masks instead of each
                            // select waiting on the one before it (the
                            // headline product 5.94 -> 5.86 ms; the wide
                            // kernels measured slower this way)
                            bool upd[GEMM_TR][NC];
#pragma unroll
                            for (int r = 0; r < GEMM_TR; ++r)
#pragma unroll
                                for (int c = 0; c < NC; ++c) upd[r][c] = R::better(best[r][c], prev[r][c]);
                            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                            for (int r = 0; r < GEMM_TR; ++r)
#pragma unroll
                                for (int c = 0; c < NC; ++c) win[r][c] = upd[r][c] ? cid : win[r][c];
                        } else
#pragma unroll
                        for (int r = 0; r < GEMM_TR; ++r)
#pragma unroll
                            for (int c = 0; c < NC; ++c) {
                                // one compare feeds both selects (a select,
                                // unlike max, needs no NaN canonicalisation)
                                if constexpr (GEMM_CHAIN_RECORD) {
                                    win[r][c] = R::better(best[r][c], prev[r][c]) ? cid : win[r][c];
                                } else {
                                    const bool up = R::better(cm[r][c], best[r][c]);
                                    win[r][c] = up ? cid : win[r][c];
                                    best[r][c] = up ? cm[r][c] : best[r][c];
                                }
                            }
                    }
                }
            }
        }

        if (bend) {
            if constexpr (BLK) {
                // Re-scan the winning chunk of every output that improved in
                // this block: the first term equal to the best.  Slots run in
                // sequence with the 16-byte reads of the next slot issued
                // before the current slot's scan.  A slot that did not improve
                // scans chunk 0 and keeps its index.
                constexpr int NS = GEMM_TR * NC;
                V av[2][QPC], bv[2][QPC];
                auto rs_load = [&](int n, int buf) {
                    const int r = n / NC, c = n % NC;
                    const int w = win[r][c] < 0 ? 0 : win[r][c];
                    const T* ap = a_row + r * GEMM_RS * LDR + w * CH;
                    const T* bp = b_col + c * 16 * LDR;
#pragma unroll
                    for (int u = 0; u < QPC; ++u) {
                        av[buf][u] = *reinterpret_cast<const V*>(ap + 4 * u);
                        // (B's quads are swizzled: quad q of column c-group at q ^ c)
                        bv[buf][u] = *reinterpret_cast<const V*>(bp + 4 * ((w * QPC + u) ^ c));
                    }
                };
                if constexpr (Cfg::PF) rs_load(0, 0);
#pragma unroll
                for (int n = 0; n < NS; ++n) {
                    const int r = n / NC, c = n % NC, cur = Cfg::PF ? n & 1 : 0;
                    if constexpr (Cfg::PF) {
                        if (n + 1 < NS) rs_load(n + 1, cur ^ 1);
                    } else {
                        rs_load(n, 0);
                    }
                    const T bst = best[r][c];
                    int f = CH - 1;
#pragma unroll
                    for (int u = QPC - 1; u >= 0; --u) {
                        const V a = av[cur][u], b = bv[cur][u];
                        f = (R::mul(a.w, b.w) == bst) ? 4 * u + 3 : f;
                        f = (R::mul(a.z, b.z) == bst) ? 4 * u + 2 : f;
                        f = (R::mul(a.y, b.y) == bst) ? 4 * u + 1 : f;
                        f = (R::mul(a.x, b.x) == bst) ? 4 * u : f;
                    }
                    idx[r][c] = win[r][c] >= 0 ? (int)blk_k0 + win[r][c] * CH + f : idx[r][c];
                    win[r][c] = -1;
                }
                blk_k0 += Cfg::KB;
            }

            if (last) {
                if constexpr (GRES) {
                    // park values and chunk records, resolve, read back
                    T* const rv = Ss;
                    int* const rw = reinterpret_cast<int*>(Ss + GEMM_BM * GEMM_RLD);
                    __syncthreads();  // every wave is done with the operand rings
#pragma unroll
                    for (int r = 0; r < GEMM_TR; ++r)
#pragma unroll
                        for (int c = 0; c < NC; ++c) {
                            const int o = (ty + GEMM_RS * r) * GEMM_RLD + tx + 16 * c;
                            rv[o] = best[r][c];
                            rw[o] = win[r][c];
                        }
                    __syncthreads();
                    resolve_tile<SR, T, SPLIT, CH, TG, LAYOUT_A == LAYOUT_KV && LAYOUT_B == LAYOUT_KV, KR>(p, ct, tid, rv,
                                                                                            rw);
                    __syncthreads();
#pragma unroll
                    for (int r = 0; r < GEMM_TR; ++r)
#pragma unroll
                        for (int c = 0; c < NC; ++c) {
                            const int o = (ty + GEMM_RS * r) * GEMM_RLD + tx + 16 * c;
                            idx[r][c] = rw[o];
                            best[r][c] = rv[o];  // (reloaded: nothing stays live across the resolve)
                        }
                    __syncthreads();  // the rings are refilled below
                }
                // The tile is complete.  C takes the bits of the first
                // winning term; they can differ from the running maximum's
                // only for a zero value (+0 against -0).
                if constexpr (std::is_same<TG, float>::value) {
                    if constexpr (SR == TROP_SR_MAX_MUL) {
                        // the zero element is +0 and a term must exceed it to
                        // win: a zero value means nothing won
#pragma unroll
                        for (int r = 0; r < GEMM_TR; ++r)
#pragma unroll
                            for (int c = 0; c < NC; ++c)
                                best[r][c] = best[r][c] == (T)0 ? R::zero() : best[r][c];
                    } else {
                        bool any0 = false;
#pragma unroll
                        for (int r = 0; r < GEMM_TR; ++r)
#pragma unroll
                            for (int c = 0; c < NC; ++c) any0 |= best[r][c] == (T)0;
                        if (__any(any0))
                            zero_bits_fixup<SR, T, ARG, SPLIT, KR, NC>(p, ct, tx, ty, best, idx);
                    }
                }
                const int64_t c_off = ct.b * p.sc_batch + (SPLIT ? ct.s * p.c_split : 0);
                TG* __restrict__ C = static_cast<TG*>(p.C) + c_off;
                int32_t* __restrict__ I = ARG ? p.argmax + c_off : nullptr;
                const int k_off = SPLIT ? (int)(ct.s * p.kchunk) : 0;  // a split's argmax is global
#pragma unroll
                for (int r = 0; r < GEMM_TR; ++r) {
                    const int64_t i = ct.row0 + ty + GEMM_RS * r;
                    if (i >= p.m) continue;
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        const int64_t j = ct.col0 + tx + 16 * c;
                        if (j >= p.n) continue;
                        const int64_t o = i * p.sc_row + j * p.sc_col;
                        C[o] = static_cast<TG>(best[r][c]);  // (float mode: an exact integer)
                        if constexpr (ARG) I[o] = idx[r][c] + k_off;
                    }
                }
            }
            if (!fetch_valid) break;  // no further step for this workgroup
            if constexpr (BLK) __syncthreads();  // every wave is done with this block
            const int sn = BLK ? 0 : (s ^ 1) * GEMM_SL;
            la.store(As, sn, ra);
            lb.store(Bs, sn, rb);
            fetch_next();
            if (last) {
                cL += gstride;
                ct = tile_coord<SPLIT, 16 * NC>(p, cL, tiles, total);
                c_nsl = slices_of(ct);
                reset_outputs();
                g = -1;
                blk_k0 = 0;
            }
        }
        __syncthreads();  // the next slice is visible in LDS
        ++g;
        ring ^= 1;
    }
}

}  // namespace trop
