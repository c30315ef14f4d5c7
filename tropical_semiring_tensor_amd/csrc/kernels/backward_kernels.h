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

}  // namespace trop
