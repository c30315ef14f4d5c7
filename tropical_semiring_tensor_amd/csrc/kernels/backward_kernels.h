// Backward of the tropical product: the gradient routed along the argmax.
//
// With k* = argmax[b][i][j] the product is C = A[b][i][k*] (x) B[b][k*][j],
// so the gradients of L = sum G * C are
//     dA[b][i][k] = sum over j with k* = k of G[b][i][j] * dC/dA
//     dB[b][k][j] = sum over i with k* = k of G[b][i][j] * dC/dB
// (dC/dA = dC/dB = 1 for max-plus and min-plus, B[b][k*][j] and A[b][i][k*]
// for max-mul).  This is the winner routing of omeinsum-rs issue #52
// ("Acceptance criteria": backward consistent with the CPU path through the
// argmax buffer) and the scatter-add of tropical-gemm PR #35's autograd
// functions, done the way the rustytorch commit "rtx-backend-cuda: native
// index_select / index_add" does scatter-add: deterministically, by walking
// the adjoint of the selection in a fixed order (the LDS adds below never
// let two lanes race on one bin).
//
// Both gradients are one pattern, a segmented histogram: a segment (a row
// of dA, or a column of dB) has `items` entries, each with a key (its k*)
// and a value, and each of its `bins` outputs is the sum of the values with
// that key, added in ascending item order starting from +0.0 -- the order
// of a sequential loop, so results are bit-identical to one.
//
// One wave owns one segment at a time; its bins live in LDS (chunks of at
// most NB).  Items are taken 64 at a time, one per lane.  Lanes whose
// keys collide must add in lane order, so each round every pending lane
// claims its key's slot with an LDS atomic min of its lane id, the lowest
// lane of each slot adds its value and releases the slot, and the rest try
// again next round.  A wave's LDS operations complete in program order, so
// no barrier is needed; rounds per 64 items = the largest number of pending
// lanes that share a slot.
#pragma once
#include "ring.h"

namespace trop {

constexpr int GBW_THREADS = 256;
constexpr int GBW_WAVES = GBW_THREADS / 64;
constexpr int GBW_SLOTS = 256;  // claim slots per wave (bin mod 256)
constexpr int GBW_UNROLL = 4;   // 64-item chunks whose loads are issued together

// Compiler-only fence: the claim protocol relies on the wave's LDS
// operations staying in program order; the hardware keeps a wave's LDS
// operations in order, this keeps the compiler from moving or caching them.
__device__ __forceinline__ void lds_order() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// Adds v into an LDS float with the LDS unit's own add (ds_add_f32, no value
// returned): an IEEE single-precision add rounded to nearest even, with
// denormals kept.  Where a bin is only ever added to by one lane, the wave's
// in-order LDS pipeline applies its adds in program order, so the bin is
// the same sequential sum a plain load-add-store loop gives, without the
// wave waiting on the load.
__device__ __forceinline__ void lds_add(float* a, float v) {
    __hip_atomic_fetch_add(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

// NB: bins per LDS chunk and wave (the host picks the smallest of 256, 1024,
// 4096 that holds all bins, or 4096 and several passes).
template <int NB>
__device__ __forceinline__ void gemm_backward_body(const TropBackwardParams& p) {
    __shared__ float bins_all[GBW_WAVES][NB];
    __shared__ uint32_t claim_all[GBW_WAVES][GBW_SLOTS];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    float(&bins)[NB] = bins_all[wave];
    uint32_t(&claim)[GBW_SLOTS] = claim_all[wave];
    for (int e = lane; e < GBW_SLOTS; e += 64) claim[e] = 64u;  // free
    lds_order();

    const int64_t nseg = p.segs * p.batch;
    const int64_t kc_max = p.bins < NB ? p.bins : NB;
    for (int64_t seg = (int64_t)blockIdx.x * GBW_WAVES + wave; seg < nseg;
         seg += (int64_t)gridDim.x * GBW_WAVES) {
        const int64_t b = seg / p.segs, s = seg % p.segs;
        const int32_t* idx = p.idx + b * p.c_batch + s * p.c_seg;
        const float* grad = p.grad + b * p.c_batch + s * p.c_seg;
        const float* w = p.mul ? p.w + b * p.w_batch : nullptr;
        float* out = p.out + b * p.o_batch + s * p.o_seg;
        for (int64_t kc0 = 0; kc0 < p.bins; kc0 += kc_max) {
            const int64_t kcn = (p.bins - kc0) < kc_max ? (p.bins - kc0) : kc_max;
            for (int64_t e = lane; e < kcn; e += 64) bins[e] = 0.0f;
            lds_order();
            for (int64_t t0 = 0; t0 < p.items; t0 += 64 * GBW_UNROLL) {
                // the keys and values of GBW_UNROLL chunks, requested together
                int64_t key[GBW_UNROLL];
                float val[GBW_UNROLL];
#pragma unroll
                for (int u = 0; u < GBW_UNROLL; ++u) {
                    const int64_t t = t0 + 64 * u + lane;
                    key[u] = t < p.items ? (int64_t)idx[t * p.c_item] : -1;
                    val[u] = t < p.items ? grad[t * p.c_item] : 0.0f;
                }
                bool pend[GBW_UNROLL];
#pragma unroll
                for (int u = 0; u < GBW_UNROLL; ++u) {
                    pend[u] = key[u] >= kc0 && key[u] < kc0 + kcn;  // also drops keys outside [0, bins)
                    if (p.mul && pend[u]) val[u] = val[u] * w[key[u] * p.w_key + (t0 + 64 * u + lane) * p.w_item];
                }
                // the chunks in item order; inside a chunk, colliding lanes
                // commit in lane order
#pragma unroll
                for (int u = 0; u < GBW_UNROLL; ++u) {
                    const int bin = pend[u] ? (int)(key[u] - kc0) : 0;
                    const int slot = bin & (GBW_SLOTS - 1);
                    bool pd = pend[u];
                    while (__any(pd)) {
                        if (pd) atomicMin(&claim[slot], (uint32_t)lane);
                        lds_order();
                        const bool win = pd && claim[slot] == (uint32_t)lane;
                        lds_order();
                        if (win) {
                            bins[bin] = bins[bin] + val[u];
                            claim[slot] = 64u;
                        }
                        lds_order();
                        pd = pd && !win;
                    }
                }
            }
            lds_order();
            for (int64_t e = lane; e < kcn; e += 64) out[(kc0 + e) * p.o_bin] = bins[e];
            lds_order();
        }
    }
}

// Lane-per-segment form for up to GBL_BINS bins: each of the 64 lanes of a
// one-wave workgroup walks its own segment item by item, in order, adding
// each item into its own LDS row of bins with lds_add (no lane touches
// another's row until the walk is over, so every bin is summed in item
// order).  Keys and values are fetched GBL_PF items ahead.  After the walk the wave's bins are written out with
// unit-stride accesses, along bins or along segments, whichever the output
// allows.
constexpr int GBL_BINS = 256;
constexpr int GBL_LDR = GBL_BINS + 1;  // padded row: lane l, bin k at bank (l + k) mod 64
constexpr int GBR_BINS = 64;           // bins per workgroup in the range form
constexpr int GBL_PF = 16;             // items fetched per step (4 groups of 4)

// MUL: multiply by the weight operand.  VEC: items are contiguous
// (c_item == 1), their count is a multiple of 4 and every segment start is
// 16-byte aligned, so each lane reads four items with one 16-byte load.
//
// NB < GBL_BINS (range form): a workgroup holds the bins [lo, lo + NB) of its
// 64 segments, so a group of segments is ceil(bins / NB) units of work, each
// walking all items and adding those whose key is in its range.  The units
// of one group go to workgroups b, b + 8, b + 16, ... (one XCD under the
// round-robin dispatch), whose repeated item reads then hit the same L2.
template <bool MUL, bool VEC, int NB = GBL_BINS>
__device__ __forceinline__ void gemm_backward_lane_body(const TropBackwardParams& p) {
    constexpr int LDR = NB + 1;  // padded row: lane l, bin k at bank (l + k) mod 64
    constexpr bool RANGE = NB < GBL_BINS;
    __shared__ float bins[64 * LDR];
    const int lane = threadIdx.x & 63;
    const int64_t nseg = p.segs * p.batch;
    const int32_t K = (int32_t)p.bins;  // <= GBL_BINS (checked on the host)
    const int64_t items = p.items;
    float* row = bins + lane * LDR;
    const int64_t ngroups = (nseg + 63) / 64;
    const int32_t nr = RANGE ? (K + NB - 1) / NB : 1;  // bin ranges per group
    const int64_t units = RANGE ? (ngroups + 7) / 8 * 8 * nr : ngroups;
    for (int64_t w = blockIdx.x; w < units; w += gridDim.x) {
        int64_t g = w;
        int32_t lo = 0;
        if (RANGE) {
            const int64_t per = 8 * (int64_t)nr, blk = w / per;
            const int32_t r = (int32_t)(w - blk * per);
            g = blk * 8 + (r & 7);
            lo = (r >> 3) * NB;
            if (g >= ngroups) continue;  // (uniform over the workgroup)
        }
        const int32_t kn = RANGE ? min(NB, K - lo) : K;  // bins of this unit
        const int64_t seg0 = g * 64;
        const int64_t seg = seg0 + lane;
        const bool live = seg < nseg;
        const int64_t b = live ? seg / p.segs : 0, s = live ? seg % p.segs : 0;
        const int32_t* ip = p.idx + b * p.c_batch + s * p.c_seg;
        const float* gp = p.grad + b * p.c_batch + s * p.c_seg;
        const float* wp = MUL ? p.w + b * p.w_batch : nullptr;
        for (int32_t k = 0; k < kn; ++k) row[k] = 0.0f;
        lds_order();

        // items GBL_PF at a time, the next group fetched while this one adds
        int32_t kb[2][GBL_PF];
        float vb[2][GBL_PF];
        auto fetch = [&](int64_t t0, int buf) {
#pragma unroll
            for (int q = 0; q < GBL_PF / 4; ++q) {
                const int64_t t = t0 + 4 * q;
                if (VEC) {
                    // whole groups of 4 are in range or out (items % 4 == 0)
                    const bool ok = live && t < items;
                    const int64_t tc = ok ? t : 0;
                    const int4 k4 = *reinterpret_cast<const int4*>(ip + tc);
                    const float4 v4 = *reinterpret_cast<const float4*>(gp + tc);
                    kb[buf][4 * q + 0] = ok ? k4.x : -1;
                    kb[buf][4 * q + 1] = ok ? k4.y : -1;
                    kb[buf][4 * q + 2] = ok ? k4.z : -1;
                    kb[buf][4 * q + 3] = ok ? k4.w : -1;
                    vb[buf][4 * q + 0] = v4.x;
                    vb[buf][4 * q + 1] = v4.y;
                    vb[buf][4 * q + 2] = v4.z;
                    vb[buf][4 * q + 3] = v4.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool ok = live && t + e < items;
                        const int64_t off = (ok ? t + e : 0) * p.c_item;
                        kb[buf][4 * q + e] = ok ? ip[off] : -1;
                        vb[buf][4 * q + e] = gp[off];
                    }
                }
            }
        };
        // (no load at all when a segment has no items: the host does not
        // validate the argmax / gradient pointers then, and an empty view's
        // pointer may be NULL)
        if (items > 0) fetch(0, 0);
        for (int64_t t0 = 0; t0 < items; t0 += 2 * GBL_PF) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t tb = t0 + h * GBL_PF;
                if (tb >= items) break;
                if (tb + GBL_PF < items) fetch(tb + GBL_PF, h ^ 1);
#pragma unroll
                for (int u = 0; u < GBL_PF; ++u) {
                    const int32_t key = kb[h][u];
                    // an item, with a key in [lo, lo + kn) (a subset of [0, bins))
                    const bool valid = (uint32_t)key - (uint32_t)lo < (uint32_t)kn;  // unsigned: no overflow for any key
                    float v = vb[h][u];
                    // (an invalid item reads the weight at (0, 0), which is in range)
                    if (MUL) v = v * wp[(int64_t)(valid ? key : 0) * p.w_key + (valid ? tb + u : 0) * p.w_item];
                    if (valid) lds_add(&row[key - lo], v);
                }
            }
        }
        lds_order();
        // write the 64 segments' bins
        if (p.o_bin == 1) {
            for (int r = 0; r < 64; ++r) {
                const int64_t sg = seg0 + r;
                if (sg >= nseg) break;
                float* out = p.out + (sg / p.segs) * p.o_batch + (sg % p.segs) * p.o_seg + lo;
                for (int32_t k = lane; k < kn; k += 64) out[k] = bins[r * LDR + k];
            }
        } else if (live) {
            float* out = p.out + b * p.o_batch + s * p.o_seg + (int64_t)lo * p.o_bin;
            for (int32_t k = 0; k < kn; ++k) out[k * p.o_bin] = row[k];
        }
        lds_order();
    }
}

// Split form for up to GBS_LPS * GBS_BPL = 256 bins when the segments alone
// are too few to fill the device: GBS_LPS neighbouring lanes share one
// segment, each owning a contiguous range of at most GBS_BPL bins.  Every
// lane walks all of its segment's items in order (the lanes of a segment
// load the same addresses at the same time, so the loads are shared) and
// adds only the items whose key falls in its range, with lds_add as in the
// lane-per-segment form.  Each bin is still one lane's sequential sum in
// ascending item order.  The bins are
// then written with the lanes of a segment side by side along the bins.
constexpr int GBS_LPS = 16;
constexpr int GBS_BPL = 16;
constexpr int GBS_LDR = GBS_BPL + 1;
constexpr int GBS_THREADS = 256;

template <bool MUL, bool VEC>
__device__ __forceinline__ void gemm_backward_split_body(const TropBackwardParams& p) {
    __shared__ float bins_all[GBS_THREADS * GBS_LDR];
    const int tid = threadIdx.x;
    const int sub = tid % GBS_LPS;
    const int64_t nseg = p.segs * p.batch;
    const int32_t K = (int32_t)p.bins;  // <= GBS_LPS * GBS_BPL (checked on the host)
    const int32_t bpl = (K + GBS_LPS - 1) / GBS_LPS;
    const int32_t lo = sub * bpl;
    const int32_t hi = lo + bpl < K ? lo + bpl : K;
    const int64_t items = p.items;
    float* row = bins_all + tid * GBS_LDR;
    constexpr int SPB = GBS_THREADS / GBS_LPS;  // segments per workgroup
    for (int64_t seg0 = (int64_t)blockIdx.x * SPB; seg0 < nseg; seg0 += (int64_t)gridDim.x * SPB) {
        const int64_t seg = seg0 + tid / GBS_LPS;
        const bool live = seg < nseg;
        const int64_t b = live ? seg / p.segs : 0, s = live ? seg % p.segs : 0;
        const int32_t* ip = p.idx + b * p.c_batch + s * p.c_seg;
        const float* gp = p.grad + b * p.c_batch + s * p.c_seg;
        const float* wp = MUL ? p.w + b * p.w_batch : nullptr;
        for (int32_t q = 0; q < bpl; ++q) row[q] = 0.0f;
        lds_order();

        int32_t kb[2][GBL_PF];
        float vb[2][GBL_PF];
        auto fetch = [&](int64_t t0, int buf) {
#pragma unroll
            for (int q = 0; q < GBL_PF / 4; ++q) {
                const int64_t t = t0 + 4 * q;
                if (VEC) {
                    const bool ok = live && t < items;
                    const int64_t tc = ok ? t : 0;
                    const int4 k4 = *reinterpret_cast<const int4*>(ip + tc);
                    const float4 v4 = *reinterpret_cast<const float4*>(gp + tc);
                    kb[buf][4 * q + 0] = ok ? k4.x : -1;
                    kb[buf][4 * q + 1] = ok ? k4.y : -1;
                    kb[buf][4 * q + 2] = ok ? k4.z : -1;
                    kb[buf][4 * q + 3] = ok ? k4.w : -1;
                    vb[buf][4 * q + 0] = v4.x;
                    vb[buf][4 * q + 1] = v4.y;
                    vb[buf][4 * q + 2] = v4.z;
                    vb[buf][4 * q + 3] = v4.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool ok = live && t + e < items;
                        const int64_t off = (ok ? t + e : 0) * p.c_item;
                        kb[buf][4 * q + e] = ok ? ip[off] : -1;
                        vb[buf][4 * q + e] = gp[off];
                    }
                }
            }
        };
        // (no load at all when a segment has no items: the host does not
        // validate the argmax / gradient pointers then)
        if (items > 0) fetch(0, 0);
        for (int64_t t0 = 0; t0 < items; t0 += 2 * GBL_PF) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t tb = t0 + h * GBL_PF;
                if (tb >= items) break;
                if (tb + GBL_PF < items) fetch(tb + GBL_PF, h ^ 1);
#pragma unroll
                for (int u = 0; u < GBL_PF; ++u) {
                    const int32_t key = kb[h][u];
                    const bool valid = key >= lo && key < hi;  // an item with a key in this lane's range
                    float v = vb[h][u];
                    if (MUL && valid) v = v * wp[(int64_t)key * p.w_key + (tb + u) * p.w_item];
                    if (valid) lds_add(&row[key - lo], v);
                }
            }
        }
        lds_order();
        // write: lane `sub` of a segment takes bins sub, sub + 16, ... (the
        // bin's owner lane is bin / bpl, its slot bin % bpl; all in one wave)
        if (live) {
            float* out = p.out + b * p.o_batch + s * p.o_seg;
            const float* seg_rows = bins_all + (tid - sub) * GBS_LDR;
            for (int32_t k = sub; k < K; k += GBS_LPS)
                out[(int64_t)k * p.o_bin] = seg_rows[(k / bpl) * GBS_LDR + k % bpl];
        }
        lds_order();
    }
}

// Staged form for up to GBT_WAVES * GBT_RW = 256 bins: a workgroup owns 64
// segments at a time and GBT_WAVES waves, wave w holding bins
// [w W, w W + W) (W = ceil(bins / GBT_WAVES)) of all 64 segments, lane l
// those of segment l, in LDS.  The segments' items come in pieces of GBT_T:
// the whole workgroup loads a piece into registers (each thread a few items;
// 16-byte loads along the items or across four segments where the layout
// allows; the piece after next already in flight while a piece is walked),
// multiplies in the max-mul weights and writes keys (16-bit) and values to
// an LDS stage laid out [item][segment].  Then every wave walks the piece in
// item order, lane l reading item t of its own segment and adding it to its
// bin with a plain LDS read, add and write, two items per round trip (see
// the walk).  A bin is one lane's sum in ascending item order, so the result
// is the sequential one.  The walk reads LDS only: the memory latency of the
// items is paid once per piece for the whole workgroup instead of once per
// few items per lane, and no LDS atomic is used (the LDS float add costs
// about four cycles per active lane).  A workgroup takes 77 KB of LDS, so
// two share a CU; the paired entry runs both gradients in one launch, one
// workgroup of each per CU, and their phases overlap.
constexpr int GBT_WAVES = 4;
constexpr int GBT_THREADS = 64 * GBT_WAVES;
constexpr int GBT_RW = 64;              // most bins per wave
constexpr int GBT_LDR = GBT_RW + 1;     // padded row: lane l, bin k at bank (l + k) mod 64
constexpr int GBT_T = 16;               // items per staged piece
constexpr int GBT_G = 2;                // items per group of the walk (bins read together)
constexpr int GBT_IPT = GBT_T * 64 / GBT_THREADS;  // items loaded per thread and piece
static_assert(GBT_IPT % 4 == 0 && GBT_T % (4 * GBT_WAVES) == 0, "whole quads per thread");

// VEC: items contiguous (c_item == 1), their count a multiple of 4 and every
// segment start 16-byte aligned: a thread loads quads of items with one
// 16-byte load per tensor; otherwise item t of the 64 segments is loaded
// with one element load per lane (coalesced when segments are contiguous).
// The workgroup's LDS: the bins of its four ranges and the two stage
// buffers (keys as 16-bit words: bins <= 256, GBT_NOKEY for no item or a key
// outside [0, bins)).  77 KB, so that two workgroups share a CU.
constexpr uint16_t GBT_NOKEY = 0xFFFF;
struct GbtLds {
    alignas(16) float bins[GBT_WAVES * 64 * GBT_LDR];
    uint16_t stage_k[2][GBT_T][64];
    float stage_v[2][GBT_T][64];
};

// Item loads of the staged form: elements (one per lane and item), 16-byte
// vectors along the items (items contiguous), or 16-byte vectors across four
// neighbouring segments (segments contiguous, their count a multiple of 4).
constexpr int GBT_LOAD_ELEM = 0, GBT_LOAD_ITEMS = 1, GBT_LOAD_SEGS = 2;

// Walks groups g0, g0 + gstep, ... of 64 segments.
template <bool MUL, int LM>
__device__ __forceinline__ void gemm_backward_staged_run(const TropBackwardParams& p, int64_t g0, int64_t gstep,
                                                         GbtLds& L) {
    float* const bins = L.bins;
    uint16_t(&stage_k)[2][GBT_T][64] = L.stage_k;
    float(&stage_v)[2][GBT_T][64] = L.stage_v;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int32_t K = (int32_t)p.bins;  // <= GBT_WAVES * GBT_RW (checked on the host)
    const int32_t W = (K + GBT_WAVES - 1) / GBT_WAVES;
    const int32_t lo = wave * W;
    const int32_t kn = K - lo < W ? (K - lo > 0 ? K - lo : 0) : W;  // bins of this wave (uniform)
    float* const row = bins + (wave * 64 + lane) * GBT_LDR;
    const int64_t nseg = p.segs * p.batch;
    const int64_t items = p.items;
    const int64_t ngroups = (nseg + 63) / 64;
    const int64_t npieces = (items + GBT_T - 1) / GBT_T;
    constexpr bool VEC = LM == GBT_LOAD_ITEMS, SVEC = LM == GBT_LOAD_SEGS;
    // The j-th value this thread loads: its item within the piece and its
    // segment within the group (the stage column).  Items along: quads
    // wave + GBT_WAVES h of segment `lane`; elements: items wave + GBT_WAVES j
    // of segment `lane`; across segments: item (tid / 16) + 16 (j / 4) of
    // segments 4 (tid % 16) .. 4 (tid % 16) + 3.
    constexpr int SQ = GBT_THREADS / 16;  // across segments: items per pass
    auto item_of = [&](int j) -> int {
        return VEC ? 4 * (wave + GBT_WAVES * (j / 4)) + (j & 3)
                   : (SVEC ? tid / 16 + SQ * (j / 4) : wave + GBT_WAVES * j);
    };
    auto col_of = [&](int j) -> int { return SVEC ? 4 * (tid & 15) + (j & 3) : lane; };
    static_assert(!SVEC || (GBT_IPT / 4) * SQ == GBT_T, "across segments: whole passes per piece");

    for (int64_t g = g0; g < ngroups; g += gstep) {
        const int64_t seg0 = g * 64;
        const int64_t seg = seg0 + lane;  // this thread's segment, for loads and the walk
        const bool live = seg < nseg;
        const int64_t b = live ? seg / p.segs : 0, s = live ? seg % p.segs : 0;
        const int32_t* ip = p.idx + b * p.c_batch + s * p.c_seg;
        const float* gp = p.grad + b * p.c_batch + s * p.c_seg;
        const float* wp = MUL ? p.w + b * p.w_batch : nullptr;
        // across segments: this thread loads segments seg0 + 4 (tid % 16) ..
        // + 3, which share a batch entry (segs % 4 == 0)
        const int64_t lseg = SVEC ? seg0 + 4 * (tid & 15) : seg;
        const bool llive = lseg < nseg;
        const int64_t lb = SVEC ? (llive ? lseg / p.segs : 0) : b, ls = SVEC ? (llive ? lseg % p.segs : 0) : s;
        const int32_t* lip = SVEC ? p.idx + lb * p.c_batch + ls : ip;
        const float* lgp = SVEC ? p.grad + lb * p.c_batch + ls : gp;
        const float* lwp = MUL ? p.w + lb * p.w_batch : nullptr;
        {
            // the wave's 64 rows are one contiguous block: cleared with
            // 16-byte stores (padding and unread words included)
            float4* const wrows = reinterpret_cast<float4*>(bins + wave * 64 * GBT_LDR);
            for (int v = lane; v < 64 * GBT_LDR / 4; v += 64) wrows[v] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        lds_order();

        int32_t ka[GBT_IPT], kb[GBT_IPT];
        float va[GBT_IPT], vb[GBT_IPT], wa[GBT_IPT];
        // Piece pc's loads keep the raw values: whether an item exists (its
        // segment is live and it lies before `items`) is applied when it is
        // staged, so that no instruction right after a load waits on it, and
        // every step issues the same loads (past the last piece they re-read
        // the segment's last items, which is harmless), so the waits before
        // staging count only the loads issued since.  A lane past the last
        // segment reads the first segment's items.
        // (a missing item's load is clamped to the segment's last item, an
        // arithmetic clamp rather than a select, so that the compiler keeps
        // the loads free of branches)
        auto exists = [&](int64_t pc, int j) { return llive && pc * GBT_T + item_of(j) < items; };
        auto load = [&](int64_t pc, int32_t(&kr)[GBT_IPT], float(&vr)[GBT_IPT]) {
            if (SVEC) {
#pragma unroll
                for (int h = 0; h < GBT_IPT / 4; ++h) {
                    const int64_t off = min(pc * GBT_T + item_of(4 * h), items - 1) * p.c_item;
                    const int4 k4 = *reinterpret_cast<const int4*>(lip + off);
                    const float4 v4 = *reinterpret_cast<const float4*>(lgp + off);
                    kr[4 * h + 0] = k4.x;
                    kr[4 * h + 1] = k4.y;
                    kr[4 * h + 2] = k4.z;
                    kr[4 * h + 3] = k4.w;
                    vr[4 * h + 0] = v4.x;
                    vr[4 * h + 1] = v4.y;
                    vr[4 * h + 2] = v4.z;
                    vr[4 * h + 3] = v4.w;
                }
            } else if (VEC) {
#pragma unroll
                for (int h = 0; h < GBT_IPT / 4; ++h) {
                    const int64_t tc = min(pc * GBT_T + item_of(4 * h), items - 4);  // whole quads
                    const int4 k4 = *reinterpret_cast<const int4*>(ip + tc);
                    const float4 v4 = *reinterpret_cast<const float4*>(gp + tc);
                    kr[4 * h + 0] = k4.x;
                    kr[4 * h + 1] = k4.y;
                    kr[4 * h + 2] = k4.z;
                    kr[4 * h + 3] = k4.w;
                    vr[4 * h + 0] = v4.x;
                    vr[4 * h + 1] = v4.y;
                    vr[4 * h + 2] = v4.z;
                    vr[4 * h + 3] = v4.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < GBT_IPT; ++j) {
                    const int64_t off = min(pc * GBT_T + item_of(j), items - 1) * p.c_item;
                    kr[j] = ip[off];
                    vr[j] = gp[off];
                }
            }
        };
        // max-mul: the weight of each item with a key in [0, bins) (others
        // read the weight at (0, 0), which is in range, and are not added;
        // the address is masked, not selected, for the same reason)
        auto weights = [&](int64_t pc, const int32_t(&kr)[GBT_IPT]) {
#pragma unroll
            for (int j = 0; j < GBT_IPT; ++j) {
                const bool valid = exists(pc, j) && (uint32_t)kr[j] < (uint32_t)K;
                const int64_t t = pc * GBT_T + item_of(j);
                wa[j] = lwp[((int64_t)kr[j] * p.w_key + t * p.w_item) & -(int64_t)valid];
            }
        };
        auto stage = [&](int buf, int64_t pc, const int32_t(&kr)[GBT_IPT], const float(&vr)[GBT_IPT]) {
#pragma unroll
            for (int j = 0; j < GBT_IPT; ++j) {
                stage_k[buf][item_of(j)][col_of(j)] =
                    exists(pc, j) && (uint32_t)kr[j] < (uint32_t)K ? (uint16_t)kr[j] : GBT_NOKEY;
                stage_v[buf][item_of(j)][col_of(j)] = MUL ? vr[j] * wa[j] : vr[j];
            }
        };

        // (no load at all when a segment has no items: the host does not
        // validate the argmax / gradient pointers then)
        if (npieces > 0) {
            load(0, ka, va);
            if (MUL) weights(0, ka);
            stage(0, 0, ka, va);
            load(1, ka, va);
        }
        __syncthreads();
        // Piece pc: its keys and values are in stage buffer pc % 2, piece
        // pc + 1 in registers `cur` (loaded one step ago), and piece pc + 2
        // is loaded into `nxt` before the walk.  Two steps per iteration
        // with the register sets swapped, so that no copy waits on a load.
        auto step = [&](int64_t pc, int32_t(&ck)[GBT_IPT], float(&cv)[GBT_IPT], int32_t(&nk)[GBT_IPT],
                        float(&nv)[GBT_IPT]) {
            const int buf = (int)(pc & 1);
            if (MUL) weights(pc + 1, ck);
            load(pc + 2, nk, nv);
            if (kn > 0) {
                // the piece's keys and values first (the reads in flight
                // together), then the adds in item order
                uint32_t kk[GBT_T];
                float vv[GBT_T];
#pragma unroll
                for (int t = 0; t < GBT_T; ++t) {
                    kk[t] = stage_k[buf][t][lane];
                    vv[t] = stage_v[buf][t][lane];
                }
                // Groups of GBT_G items: the group's bins are read together,
                // each new sum starts from the latest earlier item of the
                // group with the same bin (else from the read), and the sums
                // are written in item order, so a bin sees its items in
                // order with one LDS round trip per group.  Keys outside
                // [lo, lo + kn) (-1 included) use bins kn .. GBT_RW of the
                // row, which are never read out.
#pragma unroll
                for (int t0 = 0; t0 < GBT_T; t0 += GBT_G) {
                    uint32_t ix[GBT_G];
                    float rd[GBT_G], nw[GBT_G];
#pragma unroll
                    for (int u = 0; u < GBT_G; ++u) {
                        ix[u] = min(kk[t0 + u] - (uint32_t)lo, (uint32_t)GBT_RW);  // unsigned: GBT_NOKEY and keys below lo land past GBT_RW
                        rd[u] = row[ix[u]];
                    }
#pragma unroll
                    for (int u = 0; u < GBT_G; ++u) {
                        float a = rd[u];
#pragma unroll
                        for (int e = 0; e < u; ++e) a = ix[u] == ix[e] ? nw[e] : a;  // later e wins
                        nw[u] = a + vv[t0 + u];
                    }
#pragma unroll
                    for (int u = 0; u < GBT_G; ++u) row[ix[u]] = nw[u];
                }
            }
            if (pc + 1 < npieces) stage(buf ^ 1, pc + 1, ck, cv);
            __syncthreads();  // piece pc + 1 staged; piece pc's buffer is free
        };
        for (int64_t pc = 0; pc < npieces; pc += 2) {
            step(pc, ka, va, kb, vb);
            if (pc + 1 < npieces) step(pc + 1, kb, vb, ka, va);
        }
        lds_order();
        // write the 64 segments' bins of this wave's range
        if (kn > 0) {
            constexpr int WB = 8;  // LDS reads in flight per batch of stores
            const bool vec_out = p.o_bin == 1 && kn % 4 == 0 && lo % 4 == 0 && p.o_seg % 4 == 0 &&
                                 p.o_batch % 4 == 0 && (reinterpret_cast<uintptr_t>(p.out) & 15u) == 0;
            if (vec_out) {
                // 16 lanes per segment, four bins each: one 16-byte store per
                // lane, four segments per instruction
                const int rr = lane >> 4, q = lane & 15;
                int64_t sg = seg0 + rr;
                int64_t ob = sg / p.segs, os = sg - ob * p.segs;  // segment seg0 + r0 + rr, stepped by 4
                for (int r0 = 0; r0 < 64; r0 += 16) {
                    float4 v[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float* src = bins + (wave * 64 + r0 + 4 * u + rr) * GBT_LDR + 4 * q;
                        v[u] = make_float4(src[0], src[1], src[2], src[3]);
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        if (sg < nseg && 4 * q < kn)
                            *reinterpret_cast<float4*>(p.out + ob * p.o_batch + os * p.o_seg + lo + 4 * q) = v[u];
                        sg += 4;
                        os += 4;
                        while (os >= p.segs) {
                            os -= p.segs;
                            ++ob;
                        }
                    }
                }
            } else if (p.o_bin == 1) {
                // lane = bin: each segment's bins are one contiguous store
                int64_t ob = seg0 / p.segs, os = seg0 - ob * p.segs;  // segment seg0 + r, stepped
                for (int r0 = 0; r0 < 64; r0 += WB) {
                    float v[WB];
#pragma unroll
                    for (int u = 0; u < WB; ++u) v[u] = bins[(wave * 64 + r0 + u) * GBT_LDR + lane];
#pragma unroll
                    for (int u = 0; u < WB; ++u) {
                        if (seg0 + r0 + u < nseg && lane < kn) p.out[ob * p.o_batch + os * p.o_seg + lo + lane] = v[u];
                        if (++os == p.segs) {
                            os = 0;
                            ++ob;
                        }
                    }
                }
            } else if (p.o_seg == 1 && kn % 4 == 0 && p.segs % 4 == 0 && p.o_bin % 4 == 0 && p.o_batch % 4 == 0 &&
                       (reinterpret_cast<uintptr_t>(p.out) & 15u) == 0) {
                // segments side by side in the output: lane (sq, kb) writes
                // bin k0 + kb of segments 4 sq .. 4 sq + 3 (one batch entry,
                // since segs % 4 == 0) with one 16-byte store
                const int sq = lane & 15, kb = lane >> 4;
                const int64_t sg = seg0 + 4 * sq;
                const int64_t qb = sg / p.segs, qs = sg - qb * p.segs;
                float* out = p.out + qb * p.o_batch + qs + (int64_t)lo * p.o_bin;
                const float* src = bins + (wave * 64 + 4 * sq) * GBT_LDR;
                for (int32_t k0 = 0; k0 < kn; k0 += 16) {
                    float4 v[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int k = min(k0 + 4 * u + kb, GBT_RW);
                        v[u] = make_float4(src[k], src[GBT_LDR + k], src[2 * GBT_LDR + k], src[3 * GBT_LDR + k]);
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int k = k0 + 4 * u + kb;
                        if (sg < nseg && k < kn) *reinterpret_cast<float4*>(out + (int64_t)k * p.o_bin) = v[u];
                    }
                }
            } else if (live) {
                // lane = segment: bin k of the 64 segments side by side
                float* out = p.out + b * p.o_batch + s * p.o_seg + (int64_t)lo * p.o_bin;
                for (int32_t k0 = 0; k0 < kn; k0 += WB) {
                    float v[WB];
#pragma unroll
                    for (int u = 0; u < WB; ++u) v[u] = row[k0 + u < GBT_RW ? k0 + u : GBT_RW];
#pragma unroll
                    for (int u = 0; u < WB; ++u)
                        if (k0 + u < kn) out[(int64_t)(k0 + u) * p.o_bin] = v[u];
                }
            }
        }
        lds_order();
    }
}

template <bool MUL, int LM>
__device__ __forceinline__ void gemm_backward_staged_body(const TropBackwardParams& p) {
    __shared__ GbtLds L;
    gemm_backward_staged_run<MUL, LM>(p, blockIdx.x, gridDim.x, L);
}

// Both gradients in one launch: workgroups [0, split) take the first job's
// groups, the rest the second's.  With two workgroups per CU, a CU then holds
// one of each, and the phases of one (item loads, staging, the output
// write) overlap the other's walk.
template <bool MUL, int LA, int LB>
__device__ __forceinline__ void gemm_backward_staged_pair_body(const TropBackwardPairParams& q) {
    __shared__ GbtLds L;
    if ((int64_t)blockIdx.x < q.split)
        gemm_backward_staged_run<MUL, LA>(q.p[0], blockIdx.x, q.split, L);
    else
        gemm_backward_staged_run<MUL, LB>(q.p[1], blockIdx.x - q.split, gridDim.x - q.split, L);
}

}  // namespace trop
