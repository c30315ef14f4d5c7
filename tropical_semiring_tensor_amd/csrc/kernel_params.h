// Kernel argument blocks, passed by value to every launch.  Plain structs
// shared by the host runtime and the device code so that both agree on the
// layout; no pointer in them is kept after a call returns.
#pragma once
#include <stdint.h>

#define TROP_MAX_DIMS 8

// Semiring ids (match trop_semiring in include/tropical.h).
#define TROP_SR_MAX_PLUS 0
#define TROP_SR_MIN_PLUS 1
#define TROP_SR_MAX_MUL 2

// How a GEMM operand tile is read from global memory.
#define TROP_LOAD_K_CONTIG 0   // k is the unit-stride axis (or neither is)
#define TROP_LOAD_MN_CONTIG 1  // the row (A) / column (B) axis is unit-stride

// tile-rows per group of the GEMM's grouped raster (see group_rows)
#define TROP_GEMM_GROUP_ROWS 4

struct TropGemmParams {
    const void* A;
    const void* B;
    void* C;
    int32_t* argmax;  // may be null
    int64_t sa_row, sa_col, sa_batch;
    int64_t sb_row, sb_col, sb_batch;
    int64_t sc_row, sc_col, sc_batch;
    int64_t m, n, k, batch;
    int32_t tiles_m, tiles_n;  // tiled kernel: tile counts along m and n
    int32_t a_mode, b_mode;    // TROP_LOAD_*
    int32_t a_vec, b_vec;      // 16-byte vector loads are aligned and legal
    int32_t swizzle;           // remap workgroups so each XCD owns a tile range
    int32_t pad_;
    // split K: the tile stream covers (batch entry, split, tile); split s
    // takes k in [s kchunk, min((s + 1) kchunk, k)) and writes its partial
    // value and (global) argmax at C / argmax + s c_split.  ksplit = 1: no
    // split (kchunk = k, c_split = 0).
    int64_t ksplit, kchunk, c_split;
    // coord32 = 1: every logical tile index is below 2^31, and the tile
    // decode divides with 32-bit magic numbers: floor(n / d) =
    // umulhi(n, *_m) >> *_s for d = tiles_m * tiles_n (tl_*), tiles_n (tn_*)
    // and ksplit (ks_*); a divisor of 1 is not divided by
    int32_t coord32;
    uint32_t tl_m, tl_s, tn_m, tn_s, ks_m, ks_s;
    // grouped raster: inside a batch entry the tiles run in groups of
    // group_rows tile-rows (the last group may be shorter), column by column
    // and down the rows inside a group, so the workgroups that run at the
    // same time share a few operand panels.  group_rows = 1: row by row.
    // gr_m / gr_s: magic pair of group_rows * tiles_n (coord32).
    int32_t group_rows;
    uint32_t gr_m, gr_s;
    // launch gate of a checked int32 product (float mode): mode_slots flags
    // from the domain pre-pass, nonzero = some value outside the domain; the
    // launch proceeds only if (all flags zero) == mode_run.  NULL: no gate.
    const int32_t* mode_flags;
    int32_t mode_slots, mode_run;
    // two-level k of an operand read along k: a_krun > 0 splits A's k as
    // k = hi a_krun + lo, lo on the unit-stride axis (sa_col = 1, a_krun a
    // power of two from 4 to 16) and hi at stride sa_khi, so element (i, k)
    // sits at i sa_row + (k / a_krun) sa_khi + k % a_krun -- an operand whose
    // contracted axes lie on both sides of its free axes, read in place.
    // 0: k at stride sa_col.  b_krun / sb_khi: the same for B (sb_row = 1).
    int32_t a_krun, b_krun;
    int64_t sa_khi, sb_khi;
};

// Domain pre-pass of an int32 max-plus / min-plus product (float mode):
// workgroup w writes flags[w] = 1 if some element of A (batch, m, k) or B
// (batch, k, n) that it scanned lies outside the semiring's float-exact
// domain, else 0.  Every flag is written.
struct TropDomainParams {
    const int32_t* A;
    const int32_t* B;
    int32_t* flags;
    int64_t sa_row, sa_col, sa_batch;
    int64_t sb_row, sb_col, sb_batch;
    int64_t m, n, k, batch;
};

// Merge of split-K partials: out = the first strictly better of the
// ksplit partials (split 0 first), stored [split][batch][m][n] contiguous.
// Most lanes of the split-K merge per output (a power of two up to 64).
#define TROP_MERGE_LANES 16

struct TropSplitMergeParams {
    const void* pval;
    const int32_t* pidx;  // may be null (value only)
    void* C;
    int32_t* argmax;      // may be null
    int64_t sc_row, sc_col, sc_batch;
    int64_t m, n, batch, ksplit;
    // lanes per output: a power of two from 1 to TROP_MERGE_LANES (the grid
    // has one thread per lane and output)
    int32_t lanes, pad_;
};

struct TropFillParams {
    void* C;
    int32_t* argmax;  // may be null
    int64_t sc_row, sc_col, sc_batch;
    int64_t m, n, batch;
    uint32_t zero_bits;  // bit pattern of the semiring's zero element
    int32_t pad_;
};

// Gather: out (contiguous, row-major over `shape`) from an input walked with
// one stride per output axis; optional (+)-reduction over extra axes.
struct TropGatherParams {
    const void* in[2];
    void* out[2];
    int32_t ntensors;  // 1 or 2 (same mapping for both)
    int32_t ndim;      // output rank, 1..TROP_MAX_DIMS
    int64_t shape[TROP_MAX_DIMS];
    int64_t istride[TROP_MAX_DIMS];
    int64_t total;     // number of output elements
    // tiled transpose: the output axis `ax_in` has input stride 1 and the
    // last output axis has output stride 1
    int32_t ax_in;
    int32_t vec;       // copy path: 16-byte vectors along the last axis
    int64_t tiles_p, tiles_q;  // tiles along ax_in (p) and the last axis (q)
    int64_t nbatch;            // product of the remaining axes
    // 32-bit index math: every output linear index is below 2^31, and
    // floor(n / shape[d]) = umulhi(n, mag_m[d]) >> mag_s[d] (shape[d] >= 2)
    int32_t idx32;
    uint32_t mag_m[TROP_MAX_DIMS];
    uint32_t mag_s[TROP_MAX_DIMS];
    uint32_t vpr, vpr_m, vpr_s;  // copy path: 16-byte vectors per output row
    int32_t tile_p;              // vectorised tiled path: tile extent along ax_in
    int32_t run_shift;           // runs / flat path: log2 of the run length R (words)
    // flat path.  The P group: output axes fc_pax[0..fc_np) that are one
    // contiguous block of the input (fc_pax[0] innermost); the Q group:
    // the last output axes fc_qax[0..fc_nq) (fc_qax[0] = the last one
    // before the element's words), one contiguous block of the output.  A
    // tile is flat_tp elements of the P group by flat_tq of the Q group,
    // whole inner axes (products fc_pin, fc_qin) and a chunk of the
    // outermost one; group totals fc_ptot, fc_qtot.  fc_postr: output
    // stride of each P axis, fc_qistr: input stride of each Q axis (words).
    // LDS row of flat_ld words; flat_z = 1 when the last axis is the
    // element's words; floor(f / (flat_tp R)) and floor(f / (flat_tq R))
    // by the magic pairs (fl_m1, fl_s1) and (fl_m2, fl_s2)
    int32_t flat_tp, flat_tq, flat_ld, flat_z;
    uint32_t fl_m1, fl_s1, fl_m2, fl_s2;
    int32_t fc_np, fc_nq;
    int32_t fc_pax[4], fc_qax[4];
    int64_t fc_postr[4], fc_qistr[4];
    int64_t fc_ptot, fc_qtot, fc_pin, fc_qin;
    // blocks: when the whole P x Q block is small, a tile holds flat_nx
    // consecutive blocks along the axis fc_xax, which steps by fc_xstr
    // words in the input and fc_xostr in the output (one of them the
    // block itself: blocks adjacent on that side); fc_xax = -1,
    // flat_nx = 1: none; floor(f / block words) by (fl_m3, fl_s3)
    int32_t fc_xax, flat_nx;
    int64_t fc_xstr, fc_xostr, tiles_x;
    uint32_t fl_m3, fl_s3;
    // floor(n / tiles_q), floor(n / tiles_p), floor(n / tiles_x) by magic
    // pairs (for idx32 plans; a divisor of 1 is taken as is)
    uint32_t tl_m[3], tl_s[3];
    // reduction (trace)
    int32_t nred;
    int64_t rshape[TROP_MAX_DIMS];
    int64_t rstride[TROP_MAX_DIMS];
    int64_t rtotal;
    // reduce path: red_o outputs per 256-thread workgroup, 256 / red_o
    // slices of the reduction each; red_sfast: a slice's lanes are
    // neighbours (the reduction's last axis has input stride 1), else the
    // outputs' lanes are; floor(r / rshape[d]) by (rmag_m, rmag_s) when
    // red_idx32 (every reduction index below 2^31)
    int32_t red_o, red_sfast, red_idx32;
    // red_vec: the four-outputs-per-thread form applies (strides and
    // extents allow it; the pointers' alignment is checked at launch)
    int32_t red_vec;
    uint32_t rmag_m[TROP_MAX_DIMS];
    uint32_t rmag_s[TROP_MAX_DIMS];
};

// Two gathers of the vectorised tiled path in one launch: workgroups
// [0, split) run p[0] and the rest run p[1], each over its own tiles.
struct TropGatherPairParams {
    TropGatherParams p[2];
    int32_t split;
};

// Argmax through pre-pass reductions: I[o] (the product's k, in the GEMM's
// canonical (batch, row, col) layout) becomes
//     k * ra_n * rb_n + wa[k] * rb_n + wb[k]
// where wa / wb are the pre-pass winners of A and B (null: no reduction on
// that side), addressed at (batch, row, col, k) through the strides below
// (a stride of 0 for the GEMM axis the operand does not carry).
struct TropComposeParams {
    int32_t* idx;
    const int32_t* wa;
    const int32_t* wb;
    int64_t wa_b, wa_r, wa_c, wa_k;
    int64_t wb_b, wb_r, wb_c, wb_k;
    int64_t ra_n, rb_n;
    int64_t rows, cols, batch;
};

// Backward (winner routing): one segmented histogram, either the rows of
// grad_a (segments i, items j, bins k) or the columns of grad_b (segments
// j, items i, bins k).  The max-mul weight of item t with key k sits at
// w + b * w_batch + k * w_key + t * w_item.
struct TropBackwardParams {
    const int32_t* idx;  // argmax
    const float* grad;   // upstream gradient, strides of argmax
    const float* w;      // max-mul weight operand (B for grad_a, A for grad_b)
    float* out;          // grad_a or grad_b
    int64_t c_batch, c_seg, c_item;  // argmax / gradient strides
    int64_t w_batch, w_key, w_item;  // weight operand strides
    int64_t o_batch, o_seg, o_bin;   // output strides
    int64_t segs, batch, items, bins;
    int32_t mul;  // max-mul: multiply by the weight
    int32_t pad_;
};

// Two gradients in one launch (the staged backward): workgroups below
// `split` take p[0], the rest p[1].
struct TropBackwardPairParams {
    TropBackwardParams p[2];
    int64_t split;
};
