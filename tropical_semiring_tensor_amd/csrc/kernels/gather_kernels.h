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
// host picks one of these paths per call:
//
//  * copy:  the last output axis has input stride 1, so rows are copied
//           with 16-byte vectors (both sides coalesced);
//  * tiled: another output axis `ax_in` has input stride 1; a 64x64 tile
//           of the (ax_in, last) plane goes through LDS with one word of
//           padding per row, so reads are coalesced along ax_in and writes
//           along the last axis, without LDS bank conflicts;
//  * runs:  the last output axis is a short run (2 to 16 words) with input
//           stride 1 and another output axis steps from run to run in the
//           input; tiles of runs go through LDS so that reads and writes
//           are long contiguous segments (a transpose of wide elements);
//  * flat:  short read- or write-contiguous axes (small bonds, many small
//           axes): each side of the tile is a group of axes, walked in
//           input order to read and in output order to write;
//  * naive: one thread per output element, digits decoded from the
//           linear index (the fallback).
//
// The copy path uses 32-bit indices with magic-number division when the
// output has fewer than 2^31 elements; the tiled path has a vectorised form
// (16-byte loads along ax_in, 16-byte stores along the last axis).
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

// Streaming accesses.  Every element of a permute or gather is read once and
// written once, so loads and stores carry the non-temporal hint: on gfx950
// that keeps the streams from filling L2 and the memory-side cache with
// lines that are never reused, which is worth 1.4x on a 256 MiB copy.
#ifndef TROP_GATHER_NT
#define TROP_GATHER_NT 1
#endif
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 ld16(const uint32_t* p) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    if (TROP_GATHER_NT) return __builtin_nontemporal_load(q);
    return *q;
}
__device__ __forceinline__ void st16(uint32_t* p, u32x4 v) {
    u32x4* q = reinterpret_cast<u32x4*>(p);
    if (TROP_GATHER_NT)
        __builtin_nontemporal_store(v, q);
    else
        *q = v;
}
__device__ __forceinline__ uint32_t ld4(const uint32_t* p) {
    if (TROP_GATHER_NT) return __builtin_nontemporal_load(p);
    return *p;
}
__device__ __forceinline__ void st4(uint32_t* p, uint32_t v) {
    if (TROP_GATHER_NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// floor(n / d) for n < 2^31 with the host-computed magic pair of d >= 2.
__device__ __forceinline__ uint32_t fdiv(uint32_t n, uint32_t m, uint32_t sh) {
    return __umulhi(n, m) >> sh;
}

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

#ifndef GC_UNROLL
#define GC_UNROLL 4  // independent 16-byte vectors per thread and iteration
#endif

__device__ __forceinline__ void gather_copy_body(const TropGatherParams& p) {
    const int64_t inner = p.shape[p.ndim - 1];
    if (p.vec && p.idx32) {
        // 16-byte vectors, 32-bit indices, magic-number division; each thread
        // keeps GC_UNROLL independent vectors in flight per iteration
        const uint32_t nv = (uint32_t)(p.total / 4);
        const uint32_t vpr = p.vpr;
        const uint32_t step = gridDim.x * blockDim.x;
        auto offsets = [&](uint32_t v, int64_t& src, int64_t& dst) {
            const uint32_t row = vpr == 1 ? v : fdiv(v, p.vpr_m, p.vpr_s);
            const uint32_t col = (v - row * vpr) * 4;
            src = col;
            uint32_t r = row;
            for (int d = p.ndim - 2; d >= 0; --d) {
                const uint32_t q = fdiv(r, p.mag_m[d], p.mag_s[d]);
                src += (int64_t)(r - q * (uint32_t)p.shape[d]) * p.istride[d];
                r = q;
            }
            dst = (int64_t)row * inner + col;
        };
        for (uint32_t v0 = blockIdx.x * blockDim.x + threadIdx.x; v0 < nv; v0 += GC_UNROLL * step) {
            int64_t src[GC_UNROLL], dst[GC_UNROLL];
            bool ok[GC_UNROLL];
#pragma unroll
            for (int u = 0; u < GC_UNROLL; ++u) {
                const uint32_t v = v0 + u * step;
                ok[u] = v < nv && v >= v0;  // (v >= v0 guards wrap-around)
                if (ok[u]) offsets(v, src[u], dst[u]);
            }
            for (int t = 0; t < p.ntensors; ++t) {
                const uint32_t* in = static_cast<const uint32_t*>(p.in[t]);
                uint32_t* out = static_cast<uint32_t*>(p.out[t]);
                u32x4 x[GC_UNROLL];
#pragma unroll
                for (int u = 0; u < GC_UNROLL; ++u)
                    if (ok[u]) x[u] = ld16(in + src[u]);
#pragma unroll
                for (int u = 0; u < GC_UNROLL; ++u)
                    if (ok[u]) st16(out + dst[u], x[u]);
            }
        }
        return;
    }
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
            for (int t = 0; t < p.ntensors; ++t)
                st16(static_cast<uint32_t*>(p.out[t]) + dst, ld16(static_cast<const uint32_t*>(p.in[t]) + src));
        }
    } else {
        for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < p.total;
             o += (int64_t)gridDim.x * blockDim.x) {
            const int64_t row = o / inner;
            const int64_t src = gather_row_offset(p, row) + (o % inner);
            for (int t = 0; t < p.ntensors; ++t)
                st4(static_cast<uint32_t*>(p.out[t]) + o, ld4(static_cast<const uint32_t*>(p.in[t]) + src));
        }
    }
}

// Transpose through LDS with 16-byte accesses everywhere.  A tile covers TP
// elements along ax_in (P, input stride 1) and TQ = 4096 / TP along the last
// output axis (Q, output stride 1).  LDS holds the tile row by row along P
// (row q: TP words), and quad c of row q sits at quad c ^ s(q),
// s(q) = (q / 4) mod (TP / 4).
//   read:  each thread loads four 16-byte vectors along P (four q, RPP
//          apart) and writes each as one 16-byte LDS store: the lanes of a
//          row fill it (a permutation of its quads), so no two lanes of a
//          16-lane group share a bank;
//   write: each thread takes one 4 x 4 block (q-quad bq, p-quad bp): four
//          16-byte LDS reads of rows 4 bq .. 4 bq + 3, a transpose in
//          registers, and four 16-byte stores along Q, one per p.  Lanes run
//          along bq, so their reads fall on the quads bp ^ bq of rows TP words
//          apart: distinct quads for up to TP / 4 neighbouring lanes (and,
//          with the row exchange below for narrow tiles, distinct banks for
//          16).
// Every LDS access is 16 bytes wide (four times fewer LDS instructions than
// word accesses).  Needs EP, EQ, the input stride of Q and of every other
// axis to be multiples of 4 and both pointers 16-byte aligned (checked on the
// host).  Workgroup b0 of a set of bstep workgroups walks tiles b0,
// b0 + bstep, ...
template <int TP, int NT>
__device__ __forceinline__ void gather_tiled_vec_body(const TropGatherParams& p, int64_t b0, int64_t bstep) {
    constexpr int TQ = 4096 / TP;
    constexpr int NQP = TP / 4;                 // quads per LDS row
    constexpr int LPR = TP / 4;                 // read phase: lanes per q-row
    constexpr int RPP = GATHER_THREADS / LPR;   // q-rows per pass
    constexpr int BQ = TQ / 4;                  // write phase: q-quads per tile
    static_assert(RPP * 4 == TQ && BQ * NQP == GATHER_THREADS, "four read passes, one block per thread");
    __shared__ __attribute__((aligned(16))) uint32_t tile[NT][TQ * TP];
    const int nd = p.ndim;
    const int P = p.ax_in, Q = nd - 1;
    const int64_t EP = p.shape[P], EQ = p.shape[Q];
    const int64_t sQ = p.istride[Q];
    int64_t oP = 1;
    for (int d = P + 1; d < nd; ++d) oP *= p.shape[d];
    const int tid = threadIdx.x;
    const int64_t per_batch = p.tiles_p * p.tiles_q;
    const int64_t nblk = per_batch * p.nbatch;
    const int rc = tid % LPR, rq = tid / LPR;   // read phase: p-quad, q-row within a pass
    const int bq = tid % BQ, bp = tid / BQ;     // write phase: the thread's 4 x 4 block
    auto swz = [](int q) { return (q >> 2) & (NQP - 1); };
    // Rows narrower than the 64 banks (TP = 16, 32) also trade places inside
    // groups of RG = 64 / TP rows, so that the lanes of a 16-lane group whose
    // quads coincide read rows in different bank ranges.
    constexpr int RG = TP >= 64 ? 1 : 64 / TP;
    constexpr int RSH = TP == 16 ? 4 : 5;  // log2(TP / 4) + 2
    auto prow = [](int q) { return RG == 1 ? q : q ^ ((q >> RSH) & (RG - 1)); };

    for (int64_t blk = b0; blk < nblk; blk += bstep) {
        const int64_t tq = blk % p.tiles_q;
        const int64_t tp = (blk / p.tiles_q) % p.tiles_p;
        int64_t bi = blk / per_batch;
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
        const int64_t p0 = tp * TP, q0 = tq * TQ;
        const int64_t pp = p0 + 4 * rc;
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
            const int ql = pass * RPP + rq;
            const int64_t q = q0 + ql;
            if (pp < EP && q < EQ) {
                const int64_t src = ibase + pp + q * sQ;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const u32x4 x = ld16(static_cast<const uint32_t*>(p.in[t]) + src);
                    *reinterpret_cast<u32x4*>(&tile[t][prow(ql) * TP + 4 * (rc ^ swz(ql))]) = x;
                }
            }
        }
        __syncthreads();
        const int64_t qv = q0 + 4 * bq;
        const int64_t pv0 = p0 + 4 * bp;
        if (qv < EQ && pv0 < EP) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                u32x4 r[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    r[j] = *reinterpret_cast<const u32x4*>(&tile[t][prow(4 * bq + j) * TP + 4 * (bp ^ swz(4 * bq))]);
                uint32_t* out = static_cast<uint32_t*>(p.out[t]) + obase + pv0 * oP + qv;
                st16(out, u32x4{r[0].x, r[1].x, r[2].x, r[3].x});
                st16(out + oP, u32x4{r[0].y, r[1].y, r[2].y, r[3].y});
                st16(out + 2 * oP, u32x4{r[0].z, r[1].z, r[2].z, r[3].z});
                st16(out + 3 * oP, u32x4{r[0].w, r[1].w, r[2].w, r[3].w});
            }
        }
        __syncthreads();
    }
}

// Runs path.  Axes: Z = the last output axis (extent R = 2^run_shift words,
// input stride 1), Q = the one before it, P = ax_in with input stride R, so
// for fixed q the runs p, p + 1, ... are adjacent in the input, and for
// fixed p the runs q, q + 1, ... are adjacent in the output.  A tile holds
// RUN_TQ q-rows of RUN_TPR words (RUN_TPR / R runs along P):
//   read:  each q-row is one contiguous input segment of RUN_TPR words;
//   write: each p-row is one contiguous output segment of RUN_TQ R words.
// VEC: 16-byte accesses (every segment start is a multiple of 4 words and
// both pointers are 16-byte aligned; checked on the host); otherwise words.
constexpr int RUN_TPR = 128;
constexpr int RUN_TQ = 32;

template <bool VEC, int NT>
__device__ __forceinline__ void gather_runs_body(const TropGatherParams& p) {
    constexpr int LDT = RUN_TPR + 4;  // LDS q-row (keeps 16-byte alignment)
    __shared__ __attribute__((aligned(16))) uint32_t tile[NT][RUN_TQ * LDT];
    const int nd = p.ndim;
    const int P = p.ax_in, Q = nd - 2, Z = nd - 1;
    const int lr = p.run_shift;
    const int R = 1 << lr;
    const int TP = RUN_TPR >> lr;  // runs per tile along P
    const int64_t EP = p.shape[P], EQ = p.shape[Q];
    const int64_t sQ = p.istride[Q];
    int64_t oP = 1;  // output stride of P
    for (int d = P + 1; d < nd; ++d) oP *= p.shape[d];
    const int tid = threadIdx.x;
    const int64_t per_batch = p.tiles_p * p.tiles_q;
    const int64_t nblk = per_batch * p.nbatch;
    constexpr int RVEC = RUN_TQ * RUN_TPR / 4;  // 16-byte slots of a tile
    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int64_t tq = blk % p.tiles_q;
        const int64_t tp = (blk / p.tiles_q) % p.tiles_p;
        int64_t bi = blk / per_batch;
        int64_t ibase = 0, obase = 0, ostride = 1;
        for (int d = nd - 1; d >= 0; --d) {
            const int64_t e = p.shape[d];
            if (d != P && d != Q && d != Z) {
                const int64_t digit = bi % e;
                bi /= e;
                ibase += digit * p.istride[d];
                obase += digit * ostride;
            }
            ostride *= e;
        }
        const int64_t p0 = tp * TP, q0 = tq * RUN_TQ;
        const int np = (int)(EP - p0 < TP ? EP - p0 : TP);
        const int nq = (int)(EQ - q0 < RUN_TQ ? EQ - q0 : RUN_TQ);
        const int rw = np << lr;  // words per q-row
        // read phase: q-row ql, words w .. w + 3
        for (int v = tid; v < RVEC; v += GATHER_THREADS) {
            const int ql = v / (RUN_TPR / 4), w = (v % (RUN_TPR / 4)) * 4;
            if (ql >= nq || w >= rw) continue;
            const int64_t src = ibase + (p0 << lr) + (q0 + ql) * sQ + w;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint32_t* in = static_cast<const uint32_t*>(p.in[t]);
                uint32_t* row = &tile[t][ql * LDT + w];
                if (VEC && w + 4 <= rw) {
                    const u32x4 x = ld16(in + src);
                    *reinterpret_cast<u32x4*>(row) = x;
                } else {
                    for (int e = 0; e < 4 && w + e < rw; ++e) row[e] = ld4(in + src + e);
                }
            }
        }
        __syncthreads();
        // write phase: p-row pl, words w .. w + 3 of its nq R words
        const int vpr = (RUN_TQ * R) / 4;  // 16-byte slots per p-row
        const int ow = nq << lr;           // words per p-row
        for (int v = tid; v < TP * vpr; v += GATHER_THREADS) {
            const int pl = v / vpr, w = (v % vpr) * 4;
            if (pl >= np || w >= ow) continue;
            const int64_t dst = obase + (p0 + pl) * oP + (q0 << lr) + w;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                uint32_t x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int wi = w + e;
                    x[e] = tile[t][(wi >> lr) * LDT + (pl << lr) + (wi & (R - 1))];
                }
                uint32_t* out = static_cast<uint32_t*>(p.out[t]);
                if (VEC && w + 4 <= ow) {
                    st16(out + dst, u32x4{x[0], x[1], x[2], x[3]});
                } else {
                    for (int e = 0; e < 4 && w + e < ow; ++e) st4(out + dst + e, x[e]);
                }
            }
        }
        __syncthreads();
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
                    tile[t][qq][lane] = ld4(static_cast<const uint32_t*>(p.in[t]) + src);
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
                    st4(static_cast<uint32_t*>(p.out[t]) + dst, tile[t][lane][pl]);
            }
        }
        __syncthreads();
    }
}

// Flat-tile path for transposes whose read- and write-contiguous axes are
// short (a bond of 2..32, the words of a wide element against a short
// axis, many small axes).  The fixed tiles above span one axis each way and
// waste most of the tile there: a 64-wide tile of a 2-wide axis moves 2
// useful columns, and an 8^8 tensor's 8 x 8 planes fill 1/64 of a tile.
// Here each side of the tile is a group of axes:
//   P group: output axes that form one contiguous block of the input
//            (input strides R, R e0, R e0 e1, ...);
//   Q group: the last output axes (before the element's words, if any),
//            one contiguous block of the output;
// each with its inner axes whole and a chunk of its outermost axis, so a
// P position p is input word p R and a Q position q output word q R.  The
// other side's offsets (output offsets of the P positions, input offsets
// of the Q positions) are the same for every tile and sit in an LDS table
// built once per workgroup.  When the whole P x Q block is small (a batched
// transpose of 16 x 16 matrices) and another axis steps from block to
// block in the input or in the output, a tile holds several consecutive
// blocks along it.  The read phase walks the tile in input order
// (q, then p, then the word) and the write phase in output order (p, then
// q, then the word), so each side moves in contiguous segments.  The LDS
// row of a fixed q is flat_ld words (odd: the write phase's column walk is
// conflict-free).  4-byte accesses, up to 16 loads in flight per thread.
// GROUPS = false: both groups are single axes, whose offsets are a
// multiply (no table; the larger LDS tile keeps one more workgroup per CU).
constexpr int FLAT_WORDS = 4096;
constexpr int FLAT_LDS_AXES = 6144;    // >= flat_tq * flat_ld (checked on the host)
constexpr int FLAT_LDS_GROUPS = 5120;  // the same with the table beside it
constexpr int FLAT_TAB = 2050;         // >= flat_tp + flat_tq (checked on the host)
constexpr int FLAT_PER_THREAD = FLAT_WORDS / GATHER_THREADS;

// BLOCKS = false: one P x Q block per tile (flat_nx = 1); the block index
// math is compiled out (the kernel is close to VALU-bound: ~20 VALU per
// word moved at ~2 words per clock per CU each way).
template <int NT, bool GROUPS, bool BLOCKS>
__device__ __forceinline__ void gather_flat_body(const TropGatherParams& p) {
    __shared__ uint32_t tile[NT][GROUPS ? FLAT_LDS_GROUPS : FLAT_LDS_AXES];
    __shared__ uint32_t tab[GROUPS ? FLAT_TAB : 1];  // [0, tp): output offsets of P positions; then input offsets of Q positions
    const int nd = p.ndim;
    const int lr = p.run_shift;  // log2 words per element
    const uint32_t tpn = (uint32_t)p.flat_tp, tqn = (uint32_t)p.flat_tq;
    const int tid = threadIdx.x;
    // offsets inside a tile fit in 31 bits (checked on the host)
    const uint32_t pstr32 = (uint32_t)p.fc_postr[0], qstr32 = (uint32_t)p.fc_qistr[0];
    for (uint32_t i = tid; GROUPS && i < tpn + tqn; i += GATHER_THREADS) {
        const bool isp = i < tpn;
        const int n = isp ? p.fc_np : p.fc_nq;
        uint32_t r = isp ? i : i - tpn;
        int64_t off = 0;
        for (int a = 0; a < n; ++a) {
            const int ax = isp ? p.fc_pax[a] : p.fc_qax[a];
            const int64_t st = isp ? p.fc_postr[a] : p.fc_qistr[a];
            const uint32_t e = (uint32_t)p.shape[ax];
            const uint32_t digit = a + 1 < n ? r % e : r;  // the outermost axis: the rest of the index
            off += (int64_t)digit * st;
            r = a + 1 < n ? r / e : 0;
        }
        tab[i] = (uint32_t)off;
    }
    uint32_t grp = p.flat_z ? 1u << (nd - 1) : 0u;  // axes outside the batch
    for (int a = 0; a < p.fc_np; ++a) grp |= 1u << p.fc_pax[a];
    for (int a = 0; a < p.fc_nq; ++a) grp |= 1u << p.fc_qax[a];
    if (p.fc_xax >= 0) grp |= 1u << p.fc_xax;
    const int64_t pstep = p.fc_postr[p.fc_np - 1], qstep = p.fc_qistr[p.fc_nq - 1];
    // a tile's chunk of the outermost axis of each group (tile sides are
    // multiples of the inner axes' products)
    const int64_t pchunk = (uint32_t)tpn / (uint32_t)p.fc_pin, qchunk = (uint32_t)tqn / (uint32_t)p.fc_qin;
    const uint32_t rw = tpn << lr;  // words of a tile row (fixed q)
    const uint32_t cw = tqn << lr;  // words of a tile column (fixed p)
    const uint32_t nwb = rw * tqn;  // words of one P x Q block
    const uint32_t nx = BLOCKS ? (uint32_t)p.flat_nx : 1u;
    const uint32_t nw = nwb * nx;   // words of a full tile, <= FLAT_WORDS
    const uint32_t ld = (uint32_t)p.flat_ld;
    const uint32_t lb = tqn * ld;   // LDS words of one block
    const uint32_t wmask = (1u << lr) - 1;
    const int64_t bstr = p.fc_xstr, bostr = p.fc_xostr;
    const int64_t EX = p.fc_xax >= 0 ? p.shape[p.fc_xax] : 1;
    const int64_t per_batch = p.tiles_p * p.tiles_q * p.tiles_x;
    const int64_t nblk = per_batch * p.nbatch;
    __syncthreads();

    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        int64_t tq, tp, tx;
        int64_t ibase = 0, obase = 0, ostride = 1;
        if (p.idx32) {
            // every tile index is below 2^31: 32-bit magic divisions (the
            // 64-bit ones are long software sequences, per tile)
            auto div = [](uint32_t n, int64_t d, uint32_t m, uint32_t sh) { return d == 1 ? n : fdiv(n, m, sh); };
            const uint32_t b = (uint32_t)blk;
            const uint32_t b1 = div(b, p.tiles_q, p.tl_m[0], p.tl_s[0]);
            const uint32_t b2 = div(b1, p.tiles_p, p.tl_m[1], p.tl_s[1]);
            uint32_t bi = div(b2, p.tiles_x, p.tl_m[2], p.tl_s[2]);
            tq = b - b1 * (uint32_t)p.tiles_q;
            tp = b1 - b2 * (uint32_t)p.tiles_p;
            tx = b2 - bi * (uint32_t)p.tiles_x;
            for (int d = nd - 1; d >= 0; --d) {
                const int64_t e = p.shape[d];
                if (!((grp >> d) & 1u)) {
                    const uint32_t q = fdiv(bi, p.mag_m[d], p.mag_s[d]);  // batch axes have extents >= 2
                    const uint32_t digit = bi - q * (uint32_t)e;
                    bi = q;
                    ibase += (int64_t)digit * p.istride[d];
                    obase += (int64_t)digit * ostride;
                }
                ostride *= e;
            }
        } else {
            tq = blk % p.tiles_q;
            tp = (blk / p.tiles_q) % p.tiles_p;
            tx = (blk / (p.tiles_q * p.tiles_p)) % p.tiles_x;
            int64_t bi = blk / per_batch;
            for (int d = nd - 1; d >= 0; --d) {
                const int64_t e = p.shape[d];
                if (!((grp >> d) & 1u)) {
                    const int64_t digit = bi % e;
                    bi /= e;
                    ibase += digit * p.istride[d];
                    obase += digit * ostride;
                }
                ostride *= e;
            }
        }
        const int64_t p0 = tp * tpn, q0 = tq * tqn;
        const uint32_t np = (uint32_t)(p.fc_ptot - p0 < tpn ? p.fc_ptot - p0 : tpn);
        const uint32_t nq = (uint32_t)(p.fc_qtot - q0 < tqn ? p.fc_qtot - q0 : tqn);
        const int64_t x0 = tx * nx;
        const uint32_t nxv = (uint32_t)(EX - x0 < nx ? EX - x0 : nx);  // blocks in range
        ibase += (p0 << lr) + tq * qchunk * qstep + x0 * bstr;   // the tile's first word in the input
        obase += tp * pchunk * pstep + (q0 << lr) + x0 * bostr;  // and in the output
        // The per-element index math below is the same for every tile; an
        // opaque copy of the thread id keeps the compiler from hoisting all
        // 16 elements' worth of it out of the loop (150+ live registers).
        uint32_t tid_t = (uint32_t)tid;
        asm volatile("" : "+v"(tid_t));
        // read, in input order; all loads issued before the LDS stores
        uint32_t v[NT][FLAT_PER_THREAD];
        uint32_t slot[FLAT_PER_THREAD];
#pragma unroll
        for (int i = 0; i < FLAT_PER_THREAD; ++i) {
            const uint32_t f = tid_t + (uint32_t)i * GATHER_THREADS;
            const uint32_t xb = BLOCKS ? fdiv(f, p.fl_m3, p.fl_s3) : 0u;  // block: f / nwb
            const uint32_t fb = f - xb * nwb;
            const uint32_t ql = fdiv(fb, p.fl_m1, p.fl_s1);  // fb / rw
            const uint32_t rem = fb - ql * rw;                // pl * R + w
            const bool ok = f < nw && (!BLOCKS || xb < nxv) && (rem >> lr) < np && ql < nq;
            slot[i] = ok ? xb * lb + ql * ld + rem : 0xffffffffu;
            // (an element outside the tile loads the tile's first word, which exists)
            const uint32_t qo = GROUPS ? tab[tpn + (ok ? ql : 0u)] : ql * qstr32;
            const uint32_t off = ok ? (uint32_t)(xb * bstr) + rem + qo : 0u;
#pragma unroll
            for (int t = 0; t < NT; ++t) v[t][i] = ld4(static_cast<const uint32_t*>(p.in[t]) + ibase + off);
        }
#pragma unroll
        for (int i = 0; i < FLAT_PER_THREAD; ++i)
            if (slot[i] != 0xffffffffu)
#pragma unroll
                for (int t = 0; t < NT; ++t) tile[t][slot[i]] = v[t][i];
        __syncthreads();
        // write, in output order
#pragma unroll
        for (int i = 0; i < FLAT_PER_THREAD; ++i) {
            const uint32_t f = tid_t + (uint32_t)i * GATHER_THREADS;
            const uint32_t xb = BLOCKS ? fdiv(f, p.fl_m3, p.fl_s3) : 0u;  // block: f / nwb
            const uint32_t fb = f - xb * nwb;
            const uint32_t pl = fdiv(fb, p.fl_m2, p.fl_s2);  // fb / cw
            const uint32_t rem = fb - pl * cw;                // ql * R + w
            const uint32_t ql = rem >> lr;
            if (f < nw && (!BLOCKS || xb < nxv) && pl < np && ql < nq) {
                const uint32_t a = xb * lb + ql * ld + (pl << lr) + (rem & wmask);
                const uint32_t off = (uint32_t)(xb * bostr) + rem + (GROUPS ? tab[pl] : pl * pstr32);
#pragma unroll
                for (int t = 0; t < NT; ++t) st4(static_cast<uint32_t*>(p.out[t]) + obase + off, tile[t][a]);
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
            st4(static_cast<uint32_t*>(p.out[t]) + o, ld4(static_cast<const uint32_t*>(p.in[t]) + src));
    }
}

// Reduction over labels absent from the output (trace, pre-pass (+)).
// The semiring's (+) is a max or a min: a selection, exact in any grouping.
// The sequential definition -- start from the zero element, take a value
// only when strictly better -- yields the first position (row-major over
// the reduced axes) whose value equals the extreme, or the zero element
// with position 0 when nothing beats it (NaN never does).  Here each output
// is reduced by 256 / red_o threads, each over an interleaved slice of the
// positions in ascending order, and the slices' (value, position) pairs
// are merged with "strictly better, or equal with an earlier position":
// the same first position, the same bits (+0 against -0 included), in any
// grouping.  Slices merge by wave shuffles, then (across waves) in LDS.
template <int SR, typename T>
__device__ __forceinline__ void reduce_merge(T& b, int64_t& w, T v, int64_t r) {
    using R = Ring<SR, T>;
    // w < 0: nothing beat the zero element yet; a real partial (r >= 0) is
    // strictly better than the zero element, and never NaN
    if (r < 0) return;
    if (w < 0 || R::better(v, b) || (!R::better(b, v) && r < w)) {
        b = v;
        w = r;
    }
}

template <int SR, typename T>
__device__ __forceinline__ T shfl_xor_t(T v, int m) {
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, __shfl_xor(__builtin_bit_cast(int, v), m));
    }
}

// Reduction with many outputs whose last axis is contiguous in the input
// (one thread per output would read 4 bytes at a time, a long-strided walk
// per thread): each thread takes four adjacent outputs and reads the four
// values at each reduction position with one 16-byte load, eight positions
// in flight, then scans them in ascending position with the strict test --
// the same first winner and bits as the sequential definition, per output.
// The host checks: the last output axis has input stride 1 and extent a
// multiple of 4, every other output and reduction stride is a multiple of
// 4, the reduction has fewer than 2^31 positions, and the input and outputs
// are 16-byte aligned.
template <int SR, typename T>
__device__ __forceinline__ void gather_reduce_vec_body(const TropGatherParams& p) {
    using R = Ring<SR, T>;
    using V = vec4<T>;
    constexpr int U = 8;  // reduction positions in flight
    const T* in = static_cast<const T*>(p.in[0]);
    T* out = static_cast<T*>(p.out[0]);
    int32_t* win_out = p.ntensors == 2 ? static_cast<int32_t*>(p.out[1]) : nullptr;
    const int64_t inner = p.shape[p.ndim - 1];
    const int64_t nvec = p.total / 4;
    const int rt = (int)p.rtotal;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec;
         v += (int64_t)gridDim.x * blockDim.x) {
        const int64_t o = 4 * v;
        const int64_t base = gather_row_offset(p, o / inner) + o % inner;
        T best[4] = {R::zero(), R::zero(), R::zero(), R::zero()};
        int win[4] = {0, 0, 0, 0};
        auto offset = [&](int r) -> int64_t {
            if (p.nred == 1) return (int64_t)r * p.rstride[0];
            int64_t off = 0;
            uint32_t rr = (uint32_t)r;
            for (int d = p.nred - 1; d >= 0; --d) {
                const uint32_t q = fdiv(rr, p.rmag_m[d], p.rmag_s[d]);
                off += (int64_t)(rr - q * (uint32_t)p.rshape[d]) * p.rstride[d];
                rr = q;
            }
            return off;
        };
        auto take = [&](const V& x, int r) {
            const T e[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool up = R::better(e[c], best[c]);
                best[c] = up ? e[c] : best[c];
                win[c] = up ? r : win[c];
            }
        };
        int r = 0;
        for (; r + U <= rt; r += U) {
            V x[U];
#pragma unroll
            for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(reinterpret_cast<const V*>(in + base + offset(r + u)));
#pragma unroll
            for (int u = 0; u < U; ++u) take(x[u], r + u);
        }
        for (; r < rt; ++r) take(__builtin_nontemporal_load(reinterpret_cast<const V*>(in + base + offset(r))), r);
        __builtin_nontemporal_store(V{best[0], best[1], best[2], best[3]}, reinterpret_cast<V*>(out + o));
        if (win_out)
            __builtin_nontemporal_store(vec4<int32_t>{win[0], win[1], win[2], win[3]},
                                        reinterpret_cast<vec4<int32_t>*>(win_out + o));
    }
}

template <int SR, typename T>
__device__ __forceinline__ void gather_reduce_body(const TropGatherParams& p) {
    using R = Ring<SR, T>;
    __shared__ T part_v[GATHER_THREADS];
    __shared__ int64_t part_r[GATHER_THREADS];
    const T* in = static_cast<const T*>(p.in[0]);
    T* out = static_cast<T*>(p.out[0]);
    // with ntensors = 2, out[1] receives each output's winner position
    int32_t* win_out = p.ntensors == 2 ? static_cast<int32_t*>(p.out[1]) : nullptr;
    const int O = p.red_o, S = GATHER_THREADS / O;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool sfast = p.red_sfast != 0;
    const int ol = sfast ? tid / S : tid % O;  // output of this thread within the block
    const int s = sfast ? tid % S : tid / O;   // its slice
    for (int64_t ob = (int64_t)blockIdx.x * O; ob < p.total; ob += (int64_t)gridDim.x * O) {
        const int64_t o = ob + ol;
        T best = R::zero();
        int64_t win = -1;
        if (o < p.total) {
            int64_t rem = o, base = 0;
            for (int d = p.ndim - 1; d >= 0; --d) {
                const int64_t e = p.shape[d];
                base += (rem % e) * p.istride[d];
                rem /= e;
            }
            auto offset = [&](int64_t r) -> int64_t {
                if (p.nred == 1) return r * p.rstride[0];
                int64_t off = 0;
                if (p.red_idx32) {
                    uint32_t rr = (uint32_t)r;
                    for (int d = p.nred - 1; d >= 0; --d) {
                        const uint32_t q = fdiv(rr, p.rmag_m[d], p.rmag_s[d]);
                        off += (int64_t)(rr - q * (uint32_t)p.rshape[d]) * p.rstride[d];
                        rr = q;
                    }
                } else {
                    int64_t rr = r;
                    for (int d = p.nred - 1; d >= 0; --d) {
                        off += (rr % p.rshape[d]) * p.rstride[d];
                        rr /= p.rshape[d];
                    }
                }
                return off;
            };
            // four positions' loads in flight, then taken in ascending order
            int64_t r = s;
            for (; r + 3 * (int64_t)S < p.rtotal; r += 4 * (int64_t)S) {
                T v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = in[base + offset(r + u * (int64_t)S)];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (R::better(v[u], best)) {
                        best = v[u];
                        win = r + u * (int64_t)S;
                    }
            }
            for (; r < p.rtotal; r += S) {
                const T v = in[base + offset(r)];
                if (R::better(v, best)) {
                    best = v;
                    win = r;
                }
            }
        }
        // merge the slices of each output: inside the wave by shuffles
        // (sfast: the S lanes of an output are neighbours; else, with
        // O < 64, lanes O apart share an output), then across the waves in
        // LDS (the butterfly leaves every lane with its wave's merge)
        const int lo = sfast ? 1 : O, hi = sfast ? S : 64;
        for (int m = lo; m < hi; m <<= 1) {
            const T v = shfl_xor_t<SR, T>(best, m);
            const int64_t rr = __shfl_xor(win, m);
            reduce_merge<SR, T>(best, win, v, rr);
        }
        if (sfast || S == 1) {
            // the output's slices were all in this wave (sfast: S <= 64)
            if (o < p.total && s == 0) {
                out[o] = best;
                if (win_out) win_out[o] = (int32_t)(win < 0 ? 0 : win);
            }
        } else {
            part_v[tid] = best;
            part_r[tid] = win;
            __syncthreads();
            if (tid < O && ob + tid < p.total) {
                // O < 64: lane tid of each wave holds that wave's merge;
                // else the S slices sit O threads apart
                const int n = O < 64 ? GATHER_THREADS / 64 : S;
                const int step = O < 64 ? 64 : O;
                T b = part_v[tid];
                int64_t w = part_r[tid];
                for (int q = 1; q < n; ++q) reduce_merge<SR, T>(b, w, part_v[tid + q * step], part_r[tid + q * step]);
                out[ob + tid] = b;
                if (win_out) win_out[ob + tid] = (int32_t)(w < 0 ? 0 : w);
            }
            __syncthreads();
        }
    }
}

// Argmax through pre-pass reductions: one thread per output of the GEMM's
// canonical result, in place (TropComposeParams).
__device__ __forceinline__ void argmax_compose_body(const TropComposeParams& p) {
    const int64_t rc = p.rows * p.cols;
    const int64_t total = rc * p.batch;
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
         o += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = o / rc, t = o % rc, r = t / p.cols, c = t % p.cols;
        const int64_t k = p.idx[o];
        int64_t v = k * p.ra_n * p.rb_n;
        if (p.wa) v += (int64_t)p.wa[b * p.wa_b + r * p.wa_r + c * p.wa_c + k * p.wa_k] * p.rb_n;
        if (p.wb) v += p.wb[b * p.wb_b + r * p.wb_r + c * p.wb_c + k * p.wb_k];
        p.idx[o] = (int32_t)v;
    }
}

}  // namespace trop
