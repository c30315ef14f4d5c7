// tropical_gemm_backward: argument checks and the two launches (one per
// requested gradient) of the winner-routing kernel.
//
// The gradient of a tropical product flows only through the term that won:
// omeinsum-rs issue #52 ("Acceptance criteria": forward, backward and argmax
// consistent with the CPU path, the argmax buffer being the winner routing)
// and tropical-gemm PR #35 (batched autograd functions that route gradients
// through the argmax).  Both gradients are segmented histograms -- rows of
// grad_a, columns of grad_b -- that the kernel accumulates deterministically
// in LDS (see backward_kernels.h), in the spirit of the rustytorch commit
// "rtx-backend-cuda: native index_select / index_add" (scatter-add with no
// atomics, bit-identical to the host).
#include <cstdlib>
#include <string>

#include "internal.h"

namespace trop {
namespace {

bool env_flag_set(const char* name) {  // tuning / test knob
    const char* v = std::getenv(name);
    return v && *v && v[0] != '0';
}

trop_status check_span3(const void* p, int dev, int64_t batch, int64_t rows, int64_t cols,
                        trop_strides s, const char* what) {
    if (s.row < 0 || s.col < 0 || s.batch < 0)
        return fail(TROP_ERR_INVALID_ARGUMENT, std::string("negative stride for ") + what);
    const int64_t e[3] = {batch, rows, cols}, st[3] = {s.batch, s.row, s.col};
    int64_t span = 0;
    if (!max_offset(3, e, st, &span)) return fail(TROP_ERR_INVALID_ARGUMENT, std::string(what) + " extent overflows");
    return check_device_span(p, dev, span + 1, 4, what);
}

// One gradient's launch parameters.  seg_*: strides that step between
// segments, item_* within a segment; the weight of item t with key k is at
// w + b * w.batch + k * w_key + t * w_item.
struct GradJob {
    TropBackwardParams p;
    bool vec;     // 16-byte loads along the items
    int mode;     // the staged form's item loads: 0 elements, 1 along items, 2 across segments
    bool staged;  // the staged form (up to 256 bins, no knob forcing another form)
};

GradJob make_job(const int32_t* argmax, const float* grad_c, trop_strides sC, int64_t c_seg, int64_t c_item,
                 const float* w, int64_t w_batch, int64_t w_key, int64_t w_item, bool mul, float* out,
                 int64_t o_batch, int64_t o_seg, int64_t o_bin, int64_t segs, int64_t items, int64_t bins,
                 int64_t batch) {
    GradJob j{};
    TropBackwardParams& p = j.p;
    p.idx = argmax;
    p.grad = grad_c;
    p.w = mul ? w : nullptr;
    p.out = out;
    p.c_batch = sC.batch;
    p.c_seg = c_seg;
    p.c_item = c_item;
    p.w_batch = w_batch;
    p.w_key = w_key;
    p.w_item = w_item;
    p.o_batch = o_batch;
    p.o_seg = o_seg;
    p.o_bin = o_bin;
    p.segs = segs;
    p.batch = batch;
    p.items = items;
    p.bins = bins;
    p.mul = mul ? 1 : 0;
    // 16-byte item loads when items are contiguous, a multiple of 4, and
    // every segment start is 16-byte aligned
    const bool aligned =
        (reinterpret_cast<uintptr_t>(argmax) & 15u) == 0 && (reinterpret_cast<uintptr_t>(grad_c) & 15u) == 0;
    j.vec = c_item == 1 && items % 4 == 0 && sC.batch % 4 == 0 && c_seg % 4 == 0 && aligned;
    // 16-byte loads across four segments when the segments are contiguous,
    // their count a multiple of 4 and every item row 16-byte aligned
    const bool svec = c_seg == 1 && segs % 4 == 0 && sC.batch % 4 == 0 && c_item % 4 == 0 && aligned;
    j.mode = j.vec ? 1 : (svec ? 2 : 0);
    // The staged form: 64 segments and four bin ranges per workgroup, items
    // loaded a piece at a time by the whole workgroup and walked from LDS.
    // The other forms stay for the knobs that force them
    // (TROPICAL_BACKWARD_LANE / _SPLIT / _RANGE / _WAVE;
    // TROPICAL_BACKWARD_STAGED=0 keeps the choice among them).
    const char* sv = std::getenv("TROPICAL_BACKWARD_STAGED");
    j.staged = bins <= 256 && !env_flag_set("TROPICAL_BACKWARD_WAVE") && !env_flag_set("TROPICAL_BACKWARD_LANE") &&
               !env_flag_set("TROPICAL_BACKWARD_SPLIT") && !std::getenv("TROPICAL_BACKWARD_RANGE") &&
               !(sv && *sv && sv[0] == '0');
    return j;
}

// Both gradients in one launch of the staged form: two workgroups per CU,
// one of each gradient, whose phases overlap.  Each gradient gets at most
// half of the resident workgroups.
trop_status launch_staged_pair(int dev, const GradJob& a, const GradJob& b, hipStream_t stream) {
    const bool mul = a.p.mul != 0;
    const KernelId kid =
        (KernelId)((mul ? K_GEMM_BACKWARD_STAGED2_MUL : K_GEMM_BACKWARD_STAGED2_PLUS) + 3 * a.mode + b.mode);
    int occ = kernel_occupancy(dev, kid);
    if (occ < 1) occ = 1;
    const int64_t cap = (int64_t)device_cu_count(dev) * occ;
    const int64_t half = cap / 2 > 0 ? cap / 2 : 1;
    const int64_t ga = (a.p.segs * a.p.batch + 63) / 64, gb = (b.p.segs * b.p.batch + 63) / 64;
    const int64_t na = ga < half ? ga : half;
    const int64_t nb = gb < cap - na ? gb : cap - na;
    TropBackwardPairParams q{};
    q.p[0] = a.p;
    q.p[1] = b.p;
    q.split = na < 1 ? 1 : na;
    const int64_t grid = q.split + (nb < 1 ? 1 : nb);
    return launch(dev, kid, TROP_K_GEMM_BACKWARD, (uint32_t)grid, 256, &q, stream);
}

// Enqueue one gradient.
trop_status launch_grad(int dev, const GradJob& job, hipStream_t stream) {
    TropBackwardParams p = job.p;
    const bool mul = p.mul != 0, vec = job.vec;
    const int64_t c_item = p.c_item, segs = p.segs, batch = p.batch, bins = p.bins;
    // Up to 256 bins: one lane per segment and bin range, each walking its
    // items in order (cheap whatever the key distribution).  More bins: one
    // wave per segment with the bins in LDS, the smallest chunk that holds
    // them all (else 4096 and several passes).
    if (bins <= 256 && !env_flag_set("TROPICAL_BACKWARD_WAVE")) {
        if (job.staged) {
            const KernelId tk = (KernelId)((mul ? K_GEMM_BACKWARD_STAGED_MUL : K_GEMM_BACKWARD_STAGED_PLUS) + job.mode);
            const int64_t groups = (segs * batch + 63) / 64;  // 64 segments per workgroup
            int occ = kernel_occupancy(dev, tk);
            if (occ < 1) occ = 1;
            const int64_t cap = (int64_t)device_cu_count(dev) * occ;
            const int64_t grid = groups < cap ? groups : cap;
            return launch(dev, tk, TROP_K_GEMM_BACKWARD, (uint32_t)(grid < 1 ? 1 : grid), 256, &p, stream);
        }
        // Items contiguous in a segment (rows of grad_a) but too few
        // segments for one lane each to fill the device (fewer than 4 waves
        // per CU): 16 lanes per segment, each owning a range of bins.  (With
        // strided items -- columns of grad_b -- the 16 lanes of a segment
        // load 16 bytes per item and wave, and the lane form measures faster.)
        const int64_t lane_waves = (segs * batch + 63) / 64;
        const bool split_any = env_flag_set("TROPICAL_BACKWARD_SPLIT");  // tests: the split form for strided items too
        if ((c_item == 1 || split_any) && lane_waves < 4 * (int64_t)device_cu_count(dev) &&
            !env_flag_set("TROPICAL_BACKWARD_LANE")) {
            const KernelId sk =
                (KernelId)((mul ? K_GEMM_BACKWARD_SPLIT_MUL : K_GEMM_BACKWARD_SPLIT_PLUS) + (vec ? 1 : 0));
            const int64_t groups = (segs * batch + 15) / 16;  // 16 segments per workgroup
            int occ = kernel_occupancy(dev, sk);
            if (occ < 1) occ = 1;
            const int64_t cap = (int64_t)device_cu_count(dev) * occ;
            const int64_t grid = groups < cap ? groups : cap;
            return launch(dev, sk, TROP_K_GEMM_BACKWARD, (uint32_t)(grid < 1 ? 1 : grid), 256, &p, stream);
        }
        const int64_t groups = (segs * batch + 63) / 64;
        // Strided items (columns of grad_b) with too few segments for one
        // lane each to fill the device: the range form, 64 bins per
        // workgroup, ceil(bins / 64) workgroups per 64 segments.
        // TROPICAL_BACKWARD_LANE (the plain lane form) wins over everything;
        // otherwise TROPICAL_BACKWARD_RANGE=1 forces the range form for any
        // segments (tests) and =0 keeps the lane form.
        const char* rv = std::getenv("TROPICAL_BACKWARD_RANGE");
        const bool range = !env_flag_set("TROPICAL_BACKWARD_LANE") &&
                           (rv && *rv ? rv[0] != '0'
                                      : c_item != 1 && bins > 64 && lane_waves < 4 * (int64_t)device_cu_count(dev));
        if (range) {
            const KernelId rk = mul ? K_GEMM_BACKWARD_RANGE_MUL : K_GEMM_BACKWARD_RANGE_PLUS;
            const int64_t units = (groups + 7) / 8 * 8 * ((bins + 63) / 64);
            int occ = kernel_occupancy(dev, rk);
            if (occ < 1) occ = 1;
            const int64_t cap = (int64_t)device_cu_count(dev) * occ;
            const int64_t grid = units < cap ? units : cap;
            return launch(dev, rk, TROP_K_GEMM_BACKWARD, (uint32_t)(grid < 1 ? 1 : grid), 64, &p, stream);
        }
        const KernelId lk = (KernelId)((mul ? K_GEMM_BACKWARD_LANE_MUL : K_GEMM_BACKWARD_LANE_PLUS) + (vec ? 1 : 0));
        int occ = kernel_occupancy(dev, lk);
        if (occ < 1) occ = 1;
        const int64_t cap = (int64_t)device_cu_count(dev) * occ;
        const int64_t grid = groups < cap ? groups : cap;
        return launch(dev, lk, TROP_K_GEMM_BACKWARD, (uint32_t)(grid < 1 ? 1 : grid), 64, &p, stream);
    }
    const KernelId kid = bins <= 256 ? K_GEMM_BACKWARD_B256
                                     : (bins <= 1024 ? K_GEMM_BACKWARD_B1024 : K_GEMM_BACKWARD_B4096);
    // one wave per segment, four waves per workgroup, as many workgroups as
    // are resident at once, each looping
    const int64_t waves = segs * batch;
    int64_t grid = (waves + 3) / 4;
    int occ = kernel_occupancy(dev, kid);
    if (occ < 1) occ = 1;
    const int64_t cap = (int64_t)device_cu_count(dev) * occ;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    return launch(dev, kid, TROP_K_GEMM_BACKWARD, (uint32_t)grid, 256, &p, stream);
}

}  // namespace
}  // namespace trop

extern "C" trop_status tropical_gemm_backward(trop_semiring semiring, trop_dtype dtype, const void* A,
                                              trop_strides sA, const void* B, trop_strides sB,
                                              const int32_t* argmax, const float* grad_c, trop_strides sC,
                                              float* grad_a, trop_strides sGA, float* grad_b,
                                              trop_strides sGB, int64_t m, int64_t n, int64_t k,
                                              int64_t batch, void* stream) {
    using namespace trop;
    if (semiring < TROP_MAX_PLUS || semiring > TROP_MAX_MUL)
        return fail(TROP_ERR_INVALID_ARGUMENT, "unknown semiring " + std::to_string((int)semiring));
    if (dtype != TROP_F32 && dtype != TROP_I32)
        return fail(TROP_ERR_INVALID_ARGUMENT, "unknown dtype " + std::to_string((int)dtype));
    // the max-mul weight is the other operand as float32; an int32 max-mul
    // product (saturating) has no gradient defined here
    if (semiring == TROP_MAX_MUL && dtype == TROP_I32)
        return fail(TROP_ERR_UNSUPPORTED, "the backward of int32 max-mul is not defined");
    if (m < 0 || n < 0 || k < 0 || batch < 0) return fail(TROP_ERR_INVALID_ARGUMENT, "negative size");
    const bool mul = semiring == TROP_MAX_MUL;
    const bool want_a = grad_a && batch > 0 && m > 0 && k > 0;
    const bool want_b = grad_b && batch > 0 && n > 0 && k > 0;
    if (!want_a && !want_b) return ok();
    if (mul && ((want_a && !B) || (want_b && !A)))
        return fail(TROP_ERR_INVALID_ARGUMENT, "max-mul gradients need the operands A and B");
    int dev = -1;
    trop_status st = current_device(&dev);
    if (st != TROP_OK) return st;
    if (m > 0 && n > 0) {
        st = check_span3(argmax, dev, batch, m, n, sC, "argmax");
        if (st != TROP_OK) return st;
        st = check_span3(grad_c, dev, batch, m, n, sC, "grad_c");
        if (st != TROP_OK) return st;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (want_a) {
        st = check_span3(grad_a, dev, batch, m, k, sGA, "grad_a");
        if (st == TROP_OK && mul && n > 0) st = check_span3(B, dev, batch, k, n, sB, "B");
        if (st != TROP_OK) return st;
    }
    if (want_b) {
        st = check_span3(grad_b, dev, batch, k, n, sGB, "grad_b");
        if (st == TROP_OK && mul && m > 0) st = check_span3(A, dev, batch, m, k, sA, "A");
        if (st != TROP_OK) return st;
    }
    // rows of grad_a: segments i, items j, bins k; weight B[b][k][j]
    const GradJob ja = make_job(argmax, grad_c, sC, sC.row, sC.col, static_cast<const float*>(B), sB.batch, sB.row,
                                sB.col, mul, grad_a, sGA.batch, sGA.row, sGA.col, m, n, k, batch);
    // columns of grad_b: segments j, items i, bins k; weight A[b][i][k]
    const GradJob jb = make_job(argmax, grad_c, sC, sC.col, sC.row, static_cast<const float*>(A), sA.batch, sA.col,
                                sA.row, mul, grad_b, sGB.batch, sGB.col, sGB.row, n, m, k, batch);
    if (want_a && want_b && ja.staged && jb.staged && !env_flag_set("TROPICAL_BACKWARD_NO_PAIR"))
        return launch_staged_pair(dev, ja, jb, s);
    if (want_a) {
        st = launch_grad(dev, ja, s);
        if (st != TROP_OK) return st;
    }
    if (want_b) {
        st = launch_grad(dev, jb, s);
        if (st != TROP_OK) return st;
    }
    return ok();
}
