// The plan of one pairwise tropical contraction, shared by
// tropical_contract_pair (contract.cpp) and the contraction-tree executor
// (tree.cpp).  A plan is built once on the host from subscripts, shapes and
// strides; running it only sets pointers and enqueues kernels.
#pragma once
#include <string>

#include "internal.h"

namespace trop {

constexpr size_t kWsAlign = 256;
inline size_t ws_align(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

struct PairOperand {
    std::string sub;  // subscript
    int64_t shape[TROP_MAX_DIMS];
    int64_t stride[TROP_MAX_DIMS];
};

struct PairPlan {
    std::string la, lb, lo;
    // label roles: batch / left / right in output order, contracted and the
    // pre-pass reductions in operand-subscript order
    std::string batch, left, right, contracted, a_red, b_red;
    int64_t ext[128];
    int64_t nb = 1, M = 1, N = 1, K = 1;
    int64_t out_total = 1;
    int64_t span_a = 0, span_b = 0;  // elements of A / B reached (0: empty operand)
    bool a_fold = false, b_fold = false, c_direct = false;
    bool b_kcol = false;  // the GEMM's right operand gathered in (batch, cols, contracted) order
    // swap: the GEMM's left operand is B and its right operand is A, so that
    // the product comes out as (batch, right, left), the output order
    bool swap = false;
    int64_t gm = 1, gn = 1;  // GEMM rows and columns
    trop_strides sA{}, sB{};
    GatherPlan ga{}, gb{}, gc{};
    // workspace layout of the step (bytes, relative to its scratch base);
    // split_bytes > 0: the GEMM's own workspace at off_split (split-K
    // partials when gemm_split, else the float-mode domain flags)
    size_t off_a = 0, off_b = 0, off_c = 0, off_i = 0, off_split = 0, split_bytes = 0, ws = 0;
    bool gemm_split = false;
    // argmax through pre-pass reductions: the winners of the GEMM's left /
    // right operand's reduction (when it has one), in its canonical layout,
    // and the extents of A's and B's reduced labels
    size_t off_wl = 0, off_wr = 0;
    bool red_l = false, red_r = false;
    int64_t ra_n = 1, rb_n = 1;
    bool route_fits = true;  // K * ra_n * rb_n < 2^31
    // an operand folded with a two-level k (its contracted labels on both
    // sides of its free ones): a_run / a_hi for the GEMM's left operand,
    // b_run / b_hi for its right one (0: plain fold or gathered)
    GemmKRuns kr{};
};

// "lhs,rhs->out" into its three subscripts (spaces ignored).
trop_status pair_parse(const char* spec, std::string* la, std::string* lb, std::string* lo);

// Plan `la,lb->lo` for operands of these shapes and element strides
// (strides NULL: contiguous row-major).  value_only: a call without an
// argmax output (a long K then keeps a right operand read in place: only
// the argmax form gains from reading it along k); its workspace is at most
// that of the argmax plan.
trop_status pair_plan(const std::string& la, const std::string& lb, const std::string& lo,
                      const int64_t* shapeA, const int64_t* stridesA, const int64_t* shapeB,
                      const int64_t* stridesB, PairPlan& P, bool value_only = false);

std::string pair_describe(const PairPlan& P);

// tropical_contract_pair with its argument and pointer checks: `workspace`
// holds `workspace_bytes`; fixed_scratch: it is the library's own
// allocation-free scratch (not checked as a caller pointer, and a plan that
// needs more is rejected with that limit in the message).
trop_status contract_pair_call(const char* spec, trop_semiring semiring, trop_dtype dtype, const void* A,
                               const int64_t* shapeA, const int64_t* stridesA, const void* B,
                               const int64_t* shapeB, const int64_t* stridesB, void* C, int32_t* argmax,
                               void* workspace, size_t workspace_bytes, bool fixed_scratch, void* stream);

// Enqueue a planned contraction on `stream`: no pointer checks here (the
// callers check spans).  `scratch` holds P.ws bytes.  Requesting `argmax`
// with a pre-pass reduction is the caller's error to reject.
trop_status pair_run(int dev, const PairPlan& P, trop_semiring sr, trop_dtype dt, const void* A,
                     const void* B, void* C, int32_t* argmax, void* scratch, hipStream_t stream);

}  // namespace trop
