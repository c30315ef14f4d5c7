// tropical_permute and tropical_diag_gather: planning and launch.
//
// Kernels (a) and (b) of omeinsum-rs issue #52 ("GPU tropical path: keep
// tensors device-resident + device-side permute", "Resolved design for
// step 3") share one description here: the output is contiguous row-major,
// each output axis walks the input with one stride (the sum of strides for
// a repeated label), and optional extra axes are (+)-reduced.  Planning
// drops size-1 axes and merges output neighbours that are also contiguous
// in the input, then picks the copy / tiled / naive / reduce kernel.
#include <cstdlib>
#include <cstring>
#include <string>

#include "internal.h"

namespace trop {

namespace {

constexpr uint32_t kMaxGrid = 1u << 30;

uint32_t grid_for(int64_t work, int64_t per_block) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g > kMaxGrid) g = kMaxGrid;
    return (uint32_t)g;
}

bool env_flag(const char* name) {
    const char* v = std::getenv(name);
    return v && *v && std::strcmp(v, "0") != 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

long env_long(const char* name, long dflt) {
    const char* v = std::getenv(name);
    if (!v || !*v) return dflt;
    const long x = std::strtol(v, nullptr, 10);
    return x > 0 ? x : dflt;
}

// Grid of a grid-stride streaming kernel with `work` thread-items: a few
// workgroups per CU, each looping, keeps enough 16-byte requests in flight
// without paying for hundreds of thousands of workgroup launches.
uint32_t stream_grid(int dev, int64_t work) {
    const int64_t per_cu = env_long("TROPICAL_GATHER_BLOCKS_PER_CU", 2);  // tuning knob
    const int64_t cap = (int64_t)device_cu_count(dev) * per_cu;
    const int64_t g = (work + 255) / 256;
    return (uint32_t)(g < cap ? (g < 1 ? 1 : g) : cap);
}

// Grid of the tiled transpose: one workgroup per tile up to a cap of
// resident workgroups, each looping over tiles.  Measured on 256 MiB
// transposes (cold cache): 4 per CU is best for the 4-byte tiled kernel;
// the runs kernel (wide elements, short runs) gains 1-16% at 5.
uint32_t tile_grid(int dev, int64_t tiles, const char* knob = "TROPICAL_TILED_BLOCKS_PER_CU",
                   long per_cu_default = 4) {
    const int64_t per_cu = env_long(knob, per_cu_default);  // tuning knob
    const int64_t cap = (int64_t)device_cu_count(dev) * per_cu;
    return (uint32_t)(tiles < cap ? tiles : cap);
}

void magic(uint64_t d, uint32_t* m, uint32_t* sh) { magic_u31(d, m, sh); }

}  // namespace

const char* gather_path_name(GatherPath p) {
    switch (p) {
        case GP_NONE: return "none";
        case GP_COPY: return "copy";
        case GP_TILED: return "tiled";
        case GP_NAIVE: return "naive";
        case GP_REDUCE: return "reduce";
        case GP_RUNS: return "runs";
        case GP_FLAT: return "flat";
    }
    return "?";
}

namespace {

// Fraction of a tile sweep along an axis of extent e that is in range.
double tile_use(int64_t e, int64_t t) { return (double)e / (double)(((e + t - 1) / t) * t); }

// The tiled or runs plan `p` (ax_in set; lr = log2 words per element, z =
// whether the last axis is the element's words) switches to the flat path
// where that measured faster (256 MiB transposes, cold cache):
//  - always in place of the scalar 64 x 64 tile (shapes or pointers that
//    rule out 16-byte accesses): 0.3-1.9 TB/s there against 2.6-5.2 flat;
//  - in place of the 16-byte tiled or the runs kernel when at most half of
//    its fixed tile is in range (a 2-wide axis fills 2/64 of a tile, the
//    8 x 8 planes of an 8^8 tensor 1/64).
// The flat tile's sides are groups of axes: the P group grows from ax_in
// through the axes that continue it in the input, the Q group from the
// last axis (before the element's words) towards the front of the output,
// each until it holds 64 elements, then either while the tile is short of
// 4096 words (at most 4 axes each); a small whole block is repeated along
// an axis that steps from block to block on at least one side.
// `fixed_vec`: whether the tiled kernel would use 16-byte accesses (at
// planning time, as far as shapes and strides tell).  TROPICAL_FLAT_PATH=0
// keeps the fixed tiles; =force takes the flat path whenever its tile is
// valid (tests).
bool consider_flat(TropGatherParams& p, int lr, int z, bool fixed_vec) {
    const char* mode = std::getenv("TROPICAL_FLAT_PATH");
    if (mode && std::strcmp(mode, "0") == 0) return false;
    const bool force = mode && std::strcmp(mode, "force") == 0;
    const int nd = p.ndim, P = p.ax_in, Q = nd - 1 - z;
    const int64_t R = int64_t(1) << lr;
    if (P == Q || P < 0 || Q < 0) return false;
    const int64_t EP = p.shape[P], EQ = p.shape[Q];
    // share of the fixed tile in range
    double fixed;
    if (z) {
        fixed = tile_use(EP, 128 / R) * tile_use(EQ, 32);
    } else {
        const int64_t tp = fixed_vec ? (EP >= 64 ? 64 : (EP >= 32 ? 32 : 16)) : 64;
        fixed = tile_use(EP, tp) * tile_use(EQ, fixed_vec ? 4096 / tp : 64);
    }
    // the groups
    int pax[4] = {P, 0, 0, 0}, qax[4] = {Q, 0, 0, 0};
    int np = 1, nq = 1;
    int64_t pprod = EP, qprod = EQ;
    auto taken = [&](int d) {
        for (int a = 0; a < np; ++a)
            if (pax[a] == d) return true;
        for (int a = 0; a < nq; ++a)
            if (qax[a] == d) return true;
        return d == nd - 1 && z;
    };
    // both groups to 64 elements first; then, while the tile is short of
    // 4096 words, whichever can still grow (one group may be blocked by
    // the other: its next axis is already the other's)
    for (int phase = 0; phase < 2; ++phase)
    for (bool grew = true; grew;) {
        grew = false;
        if (phase == 1 && pprod * qprod * R >= 4096) break;
        if ((phase == 1 || pprod < 64) && np < 4) {
            for (int d = 0; d < nd; ++d) {
                if (!taken(d) && p.istride[d] == pprod * R) {
                    pax[np++] = d;
                    pprod *= p.shape[d];
                    grew = true;
                    break;
                }
            }
        }
        if (phase == 1 && grew) continue;  // one axis at a time, P first
        if ((phase == 1 || qprod < 64) && nq < 4) {
            const int d = qax[nq - 1] - 1;
            if (d >= 0 && !taken(d)) {
                qax[nq++] = d;
                qprod *= p.shape[d];
                grew = true;
            }
        }
    }
    const int64_t pin = pprod / p.shape[pax[np - 1]], qin = qprod / p.shape[qax[nq - 1]];
    // tile: the side with fewer elements whole up to 64 (or 64 when both
    // are longer), the other side filled up to 4096 words; each side a
    // multiple of its inner axes' product, a multiple of 32 elements where
    // it has no inner axes and is that long (128-byte segments)
    auto fit = [](int64_t total, int64_t inner, int64_t cap) {
        int64_t t = total < cap ? total : cap;
        if (inner == 1 && t >= 64) t -= t % 32;
        return t - t % inner;
    };
    const int64_t budget = 4096 / R;
    int64_t tp, tq;
    if (pprod <= qprod) {
        tp = fit(pprod, pin, pprod <= 64 ? pprod : 64);
        tq = tp > 0 ? fit(qprod, qin, budget / tp) : 0;
    } else {
        tq = fit(qprod, qin, qprod <= 64 ? qprod : 64);
        tp = tq > 0 ? fit(pprod, pin, budget / tq) : 0;
    }
    if (tp < pin || tq < qin || tp < 1 || tq < 1) return false;
    const int64_t rw = tp * R;
    const int64_t ld = rw % 2 == 0 ? rw + 1 : rw;
    const bool groups = np > 1 || nq > 1;
    const int64_t lds = groups ? 5120 : 6144;  // the kernel's LDS tile (words)
    if (tq * ld > lds) tq = fit(qprod, qin, lds / ld);
    const int64_t cw = tq * R;
    if (tq < qin || rw < 2 || cw < 2 || rw * tq > 4096 || tq * ld > lds || (groups && tp + tq > 2050)) return false;
    // output strides (words)
    int64_t ostr[TROP_MAX_DIMS];
    int64_t acc = 1;
    for (int d = nd - 1; d >= 0; --d) {
        ostr[d] = acc;
        acc *= p.shape[d];
    }
    // blocks: with the whole P x Q block in a tile and short of 4096 words,
    // a tile holds several blocks along an axis that steps by one block on
    // at least one side: first one contiguous on both sides (the output
    // axis just outside the block, every later output axis in a group,
    // stepping by the dense block in the input too), then one contiguous
    // in the input, then the output axis just outside the block
    int xax = -1;
    int64_t nx = 1, bsz = 0, bosz = 0;
    const int last = nd - 1 - z;
    if (tp == pprod && tq == qprod && 2 * rw * tq <= 4096) {
        int m = nd;
        int64_t mx = R - 1;  // the block's last word in the input, relative to its first
        for (int a = 0; a < np; ++a) {
            m = pax[a] < m ? pax[a] : m;
            mx += (p.shape[pax[a]] - 1) * p.istride[pax[a]];
        }
        for (int a = 0; a < nq; ++a) {
            m = qax[a] < m ? qax[a] : m;
            mx += (p.shape[qax[a]] - 1) * p.istride[qax[a]];
        }
        const int64_t blk = rw * tq;
        const bool in_dense = mx + 1 == blk;
        const bool out_adj = m >= 1 && np + nq == last - m + 1;  // axis m - 1 steps by the block in the output
        if (out_adj && in_dense && p.istride[m - 1] == blk) {
            xax = m - 1;
        } else {
            for (int d = 0; d < nd && in_dense && xax < 0; ++d)
                if (!taken(d) && p.istride[d] == blk) xax = d;
            if (xax < 0 && out_adj) xax = m - 1;
        }
        if (xax >= 0) {
            bsz = p.istride[xax];
            bosz = ostr[xax];
            nx = 4096 / blk;
            if (nx * tq * ld > lds) nx = lds / (tq * ld);
            if (nx > p.shape[xax]) nx = p.shape[xax];
            if (nx < 2) xax = -1, nx = 1, bsz = bosz = 0;
        }
    }
    if (rw * tq * nx < 512) return false;  // too little per tile: per-tile costs dominate
    // offsets inside a tile in 31 bits
    const int64_t lim = int64_t(1) << 31;
    int64_t pmax = (tp / pin - 1) * ostr[pax[np - 1]], qmax = (tq / qin - 1) * p.istride[qax[nq - 1]];
    for (int a = 0; a + 1 < np; ++a) pmax += (p.shape[pax[a]] - 1) * ostr[pax[a]];
    for (int a = 0; a + 1 < nq; ++a) qmax += (p.shape[qax[a]] - 1) * p.istride[qax[a]];
    if (pmax + cw >= lim || qmax + rw >= lim || nx * bsz >= lim || nx * bosz >= lim) return false;
    const int64_t pct = env_long("TROPICAL_FLAT_MAX_FIXED_USE_PCT", 50);  // tuning knob
    const bool scalar_fixed = !z && !fixed_vec;
    if (!force && !scalar_fixed && !(fixed * 100.0 <= (double)pct)) return false;
    p.run_shift = lr;
    p.flat_z = z;
    p.flat_tp = (int32_t)tp;
    p.flat_tq = (int32_t)tq;
    p.flat_ld = (int32_t)ld;
    magic((uint64_t)rw, &p.fl_m1, &p.fl_s1);
    magic((uint64_t)cw, &p.fl_m2, &p.fl_s2);
    p.fc_np = np;
    p.fc_nq = nq;
    for (int a = 0; a < 4; ++a) {
        p.fc_pax[a] = a < np ? pax[a] : 0;
        p.fc_qax[a] = a < nq ? qax[a] : 0;
        p.fc_postr[a] = a < np ? ostr[pax[a]] : 0;
        p.fc_qistr[a] = a < nq ? p.istride[qax[a]] : 0;
    }
    p.fc_ptot = pprod;
    p.fc_qtot = qprod;
    p.fc_pin = pin;
    p.fc_qin = qin;
    p.tiles_p = (pprod + tp - 1) / tp;
    p.tiles_q = (qprod + tq - 1) / tq;
    p.fc_xax = xax;
    p.flat_nx = (int32_t)nx;
    p.fc_xstr = bsz;
    p.fc_xostr = bosz;
    magic((uint64_t)(rw * tq), &p.fl_m3, &p.fl_s3);
    const int64_t ex = xax >= 0 ? p.shape[xax] : 1;
    p.tiles_x = (ex + nx - 1) / nx;
    p.nbatch = p.total / (pprod * qprod * R * ex);
    const int64_t tl[3] = {p.tiles_q, p.tiles_p, p.tiles_x};
    for (int i = 0; i < 3; ++i)
        if (tl[i] >= 2 && p.idx32) magic((uint64_t)tl[i], &p.tl_m[i], &p.tl_s[i]);
    return true;
}

// Whether the tiled kernel can use 16-byte accesses on these shapes and
// strides (pointers aside).
bool tiled_vec_shape(const TropGatherParams& p) {
    const int nd = p.ndim, P = p.ax_in, Q = nd - 1;
    bool vec = p.shape[P] % 4 == 0 && p.shape[Q] % 4 == 0 && p.shape[P] >= 4;
    for (int d = 0; d < nd && vec; ++d)
        if (d != P) vec = p.istride[d] % 4 == 0;
    return vec;
}

}  // namespace

trop_status plan_gather(int ndim, const int64_t* oshape, const int64_t* ostride, int nred,
                        const int64_t* rshape, const int64_t* rstride, GatherPlan* plan) {
    std::memset(plan, 0, sizeof(*plan));
    TropGatherParams& p = plan->params;
    if (ndim < 0 || ndim > TROP_MAX_DIMS || nred < 0 || nred > TROP_MAX_DIMS)
        return fail(TROP_ERR_INVALID_ARGUMENT, "rank above 8");
    int64_t total = 1;
    for (int d = 0; d < ndim; ++d) {
        if (oshape[d] < 0 || ostride[d] < 0) return fail(TROP_ERR_INVALID_ARGUMENT, "negative extent or stride");
        if (__builtin_mul_overflow(total, oshape[d], &total))
            return fail(TROP_ERR_INVALID_ARGUMENT, "output too large");
    }
    int64_t rtotal = 1;
    for (int d = 0; d < nred; ++d) {
        if (rshape[d] < 0 || rstride[d] < 0) return fail(TROP_ERR_INVALID_ARGUMENT, "negative extent or stride");
        if (__builtin_mul_overflow(rtotal, rshape[d], &rtotal))
            return fail(TROP_ERR_INVALID_ARGUMENT, "reduction too large");
    }
    if (total == 0) {
        plan->path = GP_NONE;
        return TROP_OK;
    }
    // An empty reduction yields the zero element everywhere: keep it on the
    // reduce path, whose loop then runs zero times.

    // input span (for the allocation check)
    int64_t span = 0;
    if (!max_offset(ndim, oshape, ostride, &span)) return fail(TROP_ERR_INVALID_ARGUMENT, "input extent overflows");
    if (rtotal > 0) {
        int64_t rs = 0;
        if (!max_offset(nred, rshape, rstride, &rs) || __builtin_add_overflow(span, rs, &span))
            return fail(TROP_ERR_INVALID_ARGUMENT, "input extent overflows");
        plan->in_span = span + 1;
    } else {
        plan->in_span = 0;
    }

    // normalise output axes: drop extent 1, merge contiguous neighbours
    int nd = 0;
    for (int d = 0; d < ndim; ++d) {
        if (oshape[d] == 1) continue;
        if (nd > 0 && p.istride[nd - 1] == ostride[d] * oshape[d]) {
            p.shape[nd - 1] *= oshape[d];
            p.istride[nd - 1] = ostride[d];
        } else {
            p.shape[nd] = oshape[d];
            p.istride[nd] = ostride[d];
            ++nd;
        }
    }
    if (nd == 0) {  // a single element
        p.shape[0] = 1;
        p.istride[0] = 0;
        nd = 1;
    }
    p.ndim = nd;
    p.total = total;
    p.idx32 = total < (int64_t(1) << 31) ? 1 : 0;
    for (int d = 0; d < nd && p.idx32; ++d)
        if (p.shape[d] >= 2) magic((uint64_t)p.shape[d], &p.mag_m[d], &p.mag_s[d]);

    int nr = 0;
    for (int d = 0; d < nred; ++d) {
        if (rshape[d] == 1) continue;
        p.rshape[nr] = rshape[d];
        p.rstride[nr] = rstride[d];
        ++nr;
    }
    p.nred = nr;
    p.rtotal = rtotal;
    if (nr > 0 || rtotal == 0) {
        plan->path = GP_REDUCE;
        // Slices per output: doubled while the grid is short of 256k threads
        // and the reduction has two positions per slice, at most 64 when a
        // slice's lanes are neighbours (the reduction's last axis has input
        // stride 1: coalesced along it), else 256.  One thread per output
        // reading a long reduction alone ran at 0.2 TB/s (a 2048-long max
        // over an outer axis) and took 4.6 ms for the trace of an 8192^2
        // matrix.
        const bool sfast = nr > 0 && p.rstride[nr - 1] == 1 && rtotal >= 8;
        const int64_t smax = sfast ? 64 : 256;
        int64_t S = 1;
        while (S < smax && total * S < 256 * 1024 && 2 * S <= rtotal) S *= 2;
        const long forced = env_long("TROPICAL_REDUCE_SLICES", 0);  // tests: 1 .. smax, a power of two
        if (forced > 0 && forced <= smax && (forced & (forced - 1)) == 0) S = forced;
        p.red_o = (int32_t)(256 / S);
        p.red_sfast = sfast && S > 1 ? 1 : 0;
        p.red_idx32 = rtotal < (int64_t(1) << 31) ? 1 : 0;
        for (int d = 0; d < nr && p.red_idx32; ++d)
            if (p.rshape[d] >= 2) magic((uint64_t)p.rshape[d], &p.rmag_m[d], &p.rmag_s[d]);
        // One slice per output and the last output axis contiguous in the
        // input with every stride a multiple of 4 elements: four adjacent
        // outputs per thread with 16-byte loads (TROPICAL_REDUCE_VEC=0: never)
        bool vec = S == 1 && p.red_idx32 && p.istride[nd - 1] == 1 && p.shape[nd - 1] % 4 == 0 &&
                   !(env_long("TROPICAL_REDUCE_VEC", 1) == 0);
        for (int d = 0; d < nd - 1 && vec; ++d) vec = p.istride[d] % 4 == 0;
        for (int d = 0; d < nr && vec; ++d) vec = p.rstride[d] % 4 == 0;
        p.red_vec = vec ? 1 : 0;
        return TROP_OK;
    }
    if (env_flag("TROPICAL_FORCE_NAIVE_PERMUTE")) {
        plan->path = GP_NAIVE;
        return TROP_OK;
    }
    if (p.istride[nd - 1] == 1) {
        // A short last axis (a run of 2 to 16 words, e.g. the words of an
        // 8- or 16-byte element) that another axis steps over in the input:
        // transpose whole runs through LDS instead of copying short rows.
        const int64_t R = p.shape[nd - 1];
        if (nd >= 3 && (R == 2 || R == 4 || R == 8 || R == 16) && !env_flag("TROPICAL_NO_RUNS_PATH")) {
            for (int d = nd - 3; d >= 0; --d) {
                if (p.istride[d] != R) continue;
                plan->path = GP_RUNS;
                p.ax_in = d;
                p.run_shift = R == 2 ? 1 : (R == 4 ? 2 : (R == 8 ? 3 : 4));
                const int64_t tp = 128 / R;
                p.tiles_p = (p.shape[d] + tp - 1) / tp;
                p.tiles_q = (p.shape[nd - 2] + 31) / 32;
                p.nbatch = total / (p.shape[d] * p.shape[nd - 2] * R);
                if (consider_flat(p, p.run_shift, 1, false)) plan->path = GP_FLAT;
                return TROP_OK;
            }
        }
        plan->path = GP_COPY;
        return TROP_OK;
    }
    for (int d = nd - 2; d >= 0; --d) {
        if (p.istride[d] == 1) {
            plan->path = GP_TILED;
            p.ax_in = d;
            p.tiles_p = (p.shape[d] + 63) / 64;
            p.tiles_q = (p.shape[nd - 1] + 63) / 64;
            p.nbatch = total / (p.shape[d] * p.shape[nd - 1]);
            if (consider_flat(p, 0, 0, tiled_vec_shape(p))) plan->path = GP_FLAT;
            return TROP_OK;
        }
    }
    plan->path = GP_NAIVE;
    return TROP_OK;
}

trop_status plan_diag(int in_ndim, const int64_t* in_shape, const int64_t* in_strides,
                      const int32_t* in_labels, int out_ndim, const int32_t* out_labels,
                      GatherPlan* plan) {
    if (in_ndim < 0 || in_ndim > TROP_MAX_DIMS || out_ndim < 0 || out_ndim > TROP_MAX_DIMS)
        return fail(TROP_ERR_INVALID_ARGUMENT, "rank above 8");
    if ((in_ndim > 0 && (!in_shape || !in_strides || !in_labels)) || (out_ndim > 0 && !out_labels))
        return fail(TROP_ERR_INVALID_ARGUMENT, "NULL shape / stride / label array");
    int32_t lab[TROP_MAX_DIMS];
    int64_t ext[TROP_MAX_DIMS], str[TROP_MAX_DIMS];
    int nlab = 0;
    for (int a = 0; a < in_ndim; ++a) {
        if (in_shape[a] < 0 || in_strides[a] < 0)
            return fail(TROP_ERR_INVALID_ARGUMENT, "negative extent or stride");
        int f = -1;
        for (int l = 0; l < nlab; ++l)
            if (lab[l] == in_labels[a]) f = l;
        if (f < 0) {
            lab[nlab] = in_labels[a];
            ext[nlab] = in_shape[a];
            str[nlab] = in_strides[a];
            ++nlab;
        } else {
            if (ext[f] != in_shape[a])
                return fail(TROP_ERR_INVALID_ARGUMENT, "axes with the same label differ in extent");
            str[f] += in_strides[a];
        }
    }
    bool used[TROP_MAX_DIMS] = {false};
    int64_t oshape[TROP_MAX_DIMS], ostride[TROP_MAX_DIMS];
    for (int d = 0; d < out_ndim; ++d) {
        int f = -1;
        for (int l = 0; l < nlab; ++l)
            if (lab[l] == out_labels[d]) f = l;
        if (f < 0) return fail(TROP_ERR_INVALID_ARGUMENT, "output label not present in the input");
        if (used[f]) return fail(TROP_ERR_INVALID_ARGUMENT, "output label repeated");
        used[f] = true;
        oshape[d] = ext[f];
        ostride[d] = str[f];
    }
    int64_t rshape[TROP_MAX_DIMS], rstride[TROP_MAX_DIMS];
    int nred = 0;
    for (int l = 0; l < nlab; ++l) {
        if (used[l]) continue;
        rshape[nred] = ext[l];
        rstride[nred] = str[l];
        ++nred;
    }
    return plan_gather(out_ndim, oshape, ostride, nred, rshape, rstride, plan);
}

namespace {

void set_pointers(TropGatherParams& p, int ntensors, const void* const* in, void* const* out) {
    p.ntensors = ntensors;
    for (int t = 0; t < 2; ++t) {
        p.in[t] = t < ntensors ? in[t] : nullptr;
        p.out[t] = t < ntensors ? out[t] : nullptr;
    }
}

// Tiled path: the kernel for these pointers (16-byte accesses on both sides
// when every stride, extent and pointer allows) and its number of tiles.
KernelId prepare_tiled(TropGatherParams& p, int ntensors, int64_t* nblk) {
    const int nd = p.ndim, P = p.ax_in, Q = nd - 1;
    const int64_t EP = p.shape[P], EQ = p.shape[Q];
    bool vec = EP % 4 == 0 && EQ % 4 == 0 && EP >= 4;
    for (int d = 0; d < nd && vec; ++d)
        if (d != P) vec = p.istride[d] % 4 == 0;
    for (int t = 0; t < ntensors && vec; ++t) vec = aligned16(p.in[t]) && aligned16(p.out[t]);
    KernelId kid = K_GATHER_TILED;
    if (vec) {
        const int tp = EP >= 64 ? 64 : (EP >= 32 ? 32 : 16);
        p.tile_p = tp;
        p.tiles_p = (EP + tp - 1) / tp;
        p.tiles_q = (EQ + 4096 / tp - 1) / (4096 / tp);
        const int base = ntensors == 2 ? K_GATHER_TILED_V16_N2 : K_GATHER_TILED_V16_N1;
        kid = (KernelId)(base + (tp == 64 ? 2 : (tp == 32 ? 1 : 0)));
    }
    *nblk = p.tiles_p * p.tiles_q * p.nbatch;
    return kid;
}

}  // namespace

namespace {

// Flat path launch: more workgroups than fit at once (6 per CU by LDS and
// registers) balanced the tiles best: 8 per CU measured 5.2 TB/s on 2-wide
// transposes against 4.4-4.9 at 4.
trop_status launch_flat(int dev, TropGatherParams& p, int ntensors, hipStream_t stream) {
    const int64_t nblk = p.tiles_p * p.tiles_q * p.tiles_x * p.nbatch;
    const bool groups = p.fc_np > 1 || p.fc_nq > 1, blocks = p.flat_nx > 1;
    const int n2 = ntensors == 2 ? 1 : 0;
    const KernelId kid = (KernelId)((blocks ? (groups ? K_GATHER_FLATGB_N1 : K_GATHER_FLATB_N1)
                                            : (groups ? K_GATHER_FLATG_N1 : K_GATHER_FLAT_N1)) + n2);
    return launch(dev, kid, TROP_K_GATHER_TILED, tile_grid(dev, nblk, "TROPICAL_FLAT_BLOCKS_PER_CU", 8), 256, &p,
                  stream);
}

}  // namespace

trop_status run_gather_pair(int dev, GatherPlan& g0, int nt0, const void* const* in0, void* const* out0,
                            GatherPlan& g1, int nt1, const void* const* in1, void* const* out1,
                            trop_semiring sr, trop_dtype dt, hipStream_t stream) {
    if (g0.path == GP_TILED && g1.path == GP_TILED && !env_long("TROPICAL_NO_PAIRED_GATHER", 0)) {
        TropGatherPairParams q{};
        q.p[0] = g0.params;
        q.p[1] = g1.params;
        set_pointers(q.p[0], nt0, in0, out0);
        set_pointers(q.p[1], nt1, in1, out1);
        int64_t n0 = 0, n1 = 0;
        const KernelId k0 = prepare_tiled(q.p[0], nt0, &n0);
        const KernelId k1 = prepare_tiled(q.p[1], nt1, &n1);
        if (k0 == k1 && k0 >= K_GATHER_TILED_V16_N1 && k0 <= K_GATHER_TILED_V64_N2 && n0 > 0 && n1 > 0) {
            // workgroups in proportion to the two gathers' tiles (all of them
            // when both fit under the resident cap), at least one each
            const int64_t grid = tile_grid(dev, n0 + n1);
            int64_t s0 = grid == n0 + n1 ? n0 : (grid * n0 + (n0 + n1) / 2) / (n0 + n1);
            if (s0 < 1) s0 = 1;
            if (s0 > grid - 1) s0 = grid - 1;
            q.split = (int32_t)s0;
            const KernelId kp = (KernelId)(K_GATHER_TILED2_V16_N1 + (k0 - K_GATHER_TILED_V16_N1));
            return launch(dev, kp, TROP_K_GATHER_TILED, (uint32_t)grid, 256, &q, stream);
        }
    }
    trop_status st = run_gather(dev, g0, nt0, in0, out0, sr, dt, stream);
    if (st != TROP_OK) return st;
    return run_gather(dev, g1, nt1, in1, out1, sr, dt, stream);
}

trop_status run_gather(int dev, GatherPlan& plan, int ntensors, const void* const* in, void* const* out,
                       trop_semiring sr, trop_dtype dt, hipStream_t stream) {
    TropGatherParams& p = plan.params;
    set_pointers(p, ntensors, in, out);
    switch (plan.path) {
        case GP_NONE:
            return TROP_OK;
        case GP_COPY: {
            const int64_t inner = p.shape[p.ndim - 1];
            bool vec = inner % 4 == 0;
            for (int d = 0; d < p.ndim - 1 && vec; ++d) vec = p.istride[d] % 4 == 0;
            for (int t = 0; t < ntensors && vec; ++t) vec = aligned16(p.in[t]) && aligned16(p.out[t]);
            p.vec = vec ? 1 : 0;
            if (vec) {
                p.vpr = (uint32_t)(inner / 4);
                if (p.vpr >= 2 && p.idx32) magic(p.vpr, &p.vpr_m, &p.vpr_s);
            }
            // the 32-bit vector path moves four vectors per thread and pass
            const int64_t work = vec ? (p.idx32 ? (p.total / 4 + 3) / 4 : p.total / 4) : p.total;
            return launch(dev, K_GATHER_COPY, TROP_K_GATHER_COPY, stream_grid(dev, work), 256, &p, stream);
        }
        case GP_TILED: {
            int64_t nblk = 0;
            const KernelId kid = prepare_tiled(p, ntensors, &nblk);
            if (kid == K_GATHER_TILED) {
                // pointers that rule out 16-byte accesses: the flat tile
                // beats the scalar 64 x 64 one
                TropGatherParams f = p;
                if (consider_flat(f, 0, 0, false)) return launch_flat(dev, f, ntensors, stream);
            }
            return launch(dev, kid, TROP_K_GATHER_TILED, tile_grid(dev, nblk), 256, &p, stream);
        }
        case GP_RUNS: {
            const int nd = p.ndim, P = p.ax_in, Q = nd - 2;
            // 16-byte accesses when every segment starts on a 4-word boundary
            bool vec = p.istride[Q] % 4 == 0;
            int64_t ostr = 1;
            for (int d = nd - 1; d >= 0 && vec; --d) {
                if (d < Q && d != P) vec = p.istride[d] % 4 == 0 && ostr % 4 == 0;
                if (d == P) vec = ostr % 4 == 0;
                ostr *= p.shape[d];
            }
            for (int t = 0; t < ntensors && vec; ++t) vec = aligned16(p.in[t]) && aligned16(p.out[t]);
            const KernelId kid = vec ? (ntensors == 2 ? K_GATHER_RUNS_V_N2 : K_GATHER_RUNS_V_N1)
                                     : (ntensors == 2 ? K_GATHER_RUNS_S_N2 : K_GATHER_RUNS_S_N1);
            const int64_t nblk = p.tiles_p * p.tiles_q * p.nbatch;
            return launch(dev, kid, TROP_K_GATHER_TILED, tile_grid(dev, nblk, "TROPICAL_RUNS_BLOCKS_PER_CU", 5),
                          256, &p, stream);
        }
        case GP_FLAT:
            return launch_flat(dev, p, ntensors, stream);
        case GP_NAIVE:
            return launch(dev, K_GATHER_NAIVE, TROP_K_GATHER_NAIVE, grid_for(p.total, 256), 256, &p, stream);
        case GP_REDUCE: {
            const int ri = ring_index(sr, dt);
            if (ri < 0) return fail(TROP_ERR_UNSUPPORTED, "no such semiring / dtype pair");
            const bool vec = p.red_vec && aligned16(p.in[0]) && aligned16(p.out[0]) &&
                             (ntensors < 2 || aligned16(p.out[1])) && p.rtotal > 0;
            if (vec)
                return launch(dev, (KernelId)(K_GATHER_REDUCE_VEC_MAXPLUS_F32 + ri), TROP_K_GATHER_REDUCE,
                              grid_for(p.total / 4, 256), 256, &p, stream);
            return launch(dev, (KernelId)(K_GATHER_REDUCE_MAXPLUS_F32 + ri), TROP_K_GATHER_REDUCE,
                          grid_for(p.total, p.red_o), 256, &p, stream);
        }
    }
    return fail(TROP_ERR_INVALID_ARGUMENT, "bad gather plan");
}

}  // namespace trop

using namespace trop;

extern "C" trop_status tropical_permute(size_t elem_bytes, int ndim, const int64_t* shape,
                                        const int64_t* in_strides, const int32_t* perm, int ntensors,
                                        const void* const* in, void* const* out, void* stream) {
    if (ndim < 0 || ndim > TROP_MAX_DIMS) return fail(TROP_ERR_INVALID_ARGUMENT, "ndim must be 0..8");
    if (ntensors != 1 && ntensors != 2) return fail(TROP_ERR_INVALID_ARGUMENT, "ntensors must be 1 or 2");
    if (ndim > 0 && (!shape || !in_strides || !perm))
        return fail(TROP_ERR_INVALID_ARGUMENT, "NULL shape / stride / perm array");
    if (!in || !out) return fail(TROP_ERR_INVALID_ARGUMENT, "NULL tensor array");
    bool seen[TROP_MAX_DIMS] = {false};
    if (elem_bytes != 4 && elem_bytes != 8 && elem_bytes != 16)
        return fail(TROP_ERR_UNSUPPORTED, "elements of 4, 8 or 16 bytes only");
    // An element of W = elem_bytes / 4 words is moved as W words: every
    // stride is scaled by W and a last axis of W words with unit stride is
    // appended (omeinsum-rs issue #52, "Resolved design for step 3", kernel
    // (a) serves f32 / f64 / c32 / c64 tensors and the u32 argmax alike).
    const int64_t W = (int64_t)(elem_bytes / 4);
    int64_t oshape[TROP_MAX_DIMS + 1], ostride[TROP_MAX_DIMS + 1];
    for (int d = 0; d < ndim; ++d) {
        const int q = perm[d];
        if (q < 0 || q >= ndim || seen[q]) return fail(TROP_ERR_INVALID_ARGUMENT, "perm is not a permutation");
        seen[q] = true;
        if (shape[q] < 0 || in_strides[q] < 0) return fail(TROP_ERR_INVALID_ARGUMENT, "negative extent or stride");
        if (__builtin_mul_overflow(in_strides[q], W, &ostride[d]))
            return fail(TROP_ERR_INVALID_ARGUMENT, "stride overflows");
        oshape[d] = shape[q];
    }
    int nd = ndim;
    if (W > 1) {
        oshape[nd] = W;
        ostride[nd] = 1;
        ++nd;
        // drop extent-1 axes and merge neighbours contiguous in the input
        // (the word axis merges into a last axis of unit element stride),
        // so that a rank-8 tensor usually still fits the 8 kernel axes
        int k = 0;
        for (int d = 0; d < nd; ++d) {
            if (oshape[d] == 1) continue;
            if (k > 0 && ostride[k - 1] == ostride[d] * oshape[d]) {
                oshape[k - 1] *= oshape[d];
                ostride[k - 1] = ostride[d];
            } else {
                oshape[k] = oshape[d];
                ostride[k] = ostride[d];
                ++k;
            }
        }
        nd = k;
        if (nd > TROP_MAX_DIMS)
            return fail(TROP_ERR_UNSUPPORTED, "8 output axes that stay apart, with 8- or 16-byte elements");
    }
    GatherPlan plan;
    trop_status st = plan_gather(nd, oshape, ostride, 0, nullptr, nullptr, &plan);
    if (st != TROP_OK) return st;
    if (plan.path == GP_NONE) return ok();
    int dev = -1;
    st = current_device(&dev);
    if (st != TROP_OK) return st;
    for (int t = 0; t < ntensors; ++t) {
        st = check_device_span(in[t], dev, plan.in_span, 4, t ? "in[1]" : "in[0]");
        if (st != TROP_OK) return st;
        st = check_device_span(out[t], dev, plan.params.total, 4, t ? "out[1]" : "out[0]");
        if (st != TROP_OK) return st;
    }
    st = run_gather(dev, plan, ntensors, in, out, TROP_MAX_PLUS, TROP_F32, static_cast<hipStream_t>(stream));
    return st == TROP_OK ? ok() : st;
}

extern "C" trop_status tropical_diag_gather(trop_semiring semiring, trop_dtype dtype, int in_ndim,
                                            const int64_t* in_shape, const int64_t* in_strides,
                                            const int32_t* in_labels, int out_ndim,
                                            const int32_t* out_labels, const void* in, void* out,
                                            void* stream) {
    if (dtype != TROP_F32 && dtype != TROP_I32) return fail(TROP_ERR_INVALID_ARGUMENT, "unknown dtype");
    if (semiring < TROP_MAX_PLUS || semiring > TROP_MAX_MUL)
        return fail(TROP_ERR_INVALID_ARGUMENT, "unknown semiring");
    GatherPlan plan;
    trop_status st = plan_diag(in_ndim, in_shape, in_strides, in_labels, out_ndim, out_labels, &plan);
    if (st != TROP_OK) return st;
    if (plan.path == GP_REDUCE && ring_index(semiring, dtype) < 0)
        return fail(TROP_ERR_UNSUPPORTED, "no such semiring / dtype pair");
    if (plan.path == GP_NONE) return ok();
    int dev = -1;
    st = current_device(&dev);
    if (st != TROP_OK) return st;
    if (plan.in_span > 0) {
        st = check_device_span(in, dev, plan.in_span, 4, "in");
        if (st != TROP_OK) return st;
    }
    st = check_device_span(out, dev, plan.params.total, 4, "out");
    if (st != TROP_OK) return st;
    const void* ins[1] = {in};
    void* outs[1] = {out};
    st = run_gather(dev, plan, 1, ins, outs, semiring, dtype, static_cast<hipStream_t>(stream));
    return st == TROP_OK ? ok() : st;
}
