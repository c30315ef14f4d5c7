// tropical_contract_pair: one pairwise tropical einsum, device-resident.
//
// omeinsum-rs issue #52 ("GPU tropical path: keep tensors device-resident +
// device-side permute") describes the data flow this reproduces on one
// stream: repeated labels are handled by a unary pre-pass so that the GEMM
// core only sees clean operands ("Structural lessons from OMEinsum"), the
// operands are permuted into canonical order, one strided-batched tropical
// GEMM runs, and its value and argmax are permuted into the output order
// with one shared mapping ("Acceptance criteria") -- or, when the output
// order is (batch, B-side labels, A-side labels), the product is taken as
// B (x) A and lands in the output order with no permute.  Nothing leaves the
// device and the host never waits: all intermediates live in the caller's
// workspace and every step is enqueued on the caller's stream.  The same
// section's advice to let GEMM strides absorb a permute "where the layout
// allows" is followed for operands: an operand whose batch, row and column
// label groups each collapse to one stride, with a unit row or column
// stride, is read in place instead of being gathered.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "contract_plan.h"

namespace trop {

namespace {

using Plan = PairPlan;
using Operand = PairOperand;
size_t align_up(size_t x) { return ws_align(x); }

bool is_label(char c) { return (c >= 'a' && c <= 'z') || (c >= 'A' && c <= 'Z'); }

bool has(const std::string& s, char c) { return s.find(c) != std::string::npos; }

std::string unique(const std::string& s) {
    std::string u;
    for (char c : s)
        if (!has(u, c)) u.push_back(c);
    return u;
}

trop_status assign_roles(Plan& P) {
    for (const std::string* part : {&P.la, &P.lb, &P.lo}) {
        if (part->size() > TROP_MAX_DIMS) return fail(TROP_ERR_INVALID_ARGUMENT, "subscript longer than 8");
        for (char c : *part)
            if (!is_label(c)) return fail(TROP_ERR_INVALID_ARGUMENT, std::string("bad label '") + c + "'");
    }
    if (unique(P.lo).size() != P.lo.size()) return fail(TROP_ERR_INVALID_ARGUMENT, "repeated output label");
    for (char c : P.lo)
        if (!has(P.la, c) && !has(P.lb, c))
            return fail(TROP_ERR_INVALID_ARGUMENT, std::string("output label '") + c + "' is in no operand");
    // label roles, in output order for batch / left / right and in
    // A-subscript order for contracted labels
    for (char c : P.lo) {
        const bool a = has(P.la, c), b = has(P.lb, c);
        if (a && b) P.batch.push_back(c);
        else if (a) P.left.push_back(c);
        else P.right.push_back(c);
    }
    for (char c : unique(P.la)) {
        if (has(P.lo, c)) continue;
        if (has(P.lb, c)) P.contracted.push_back(c);
        else P.a_red.push_back(c);
    }
    for (char c : unique(P.lb))
        if (!has(P.lo, c) && !has(P.la, c)) P.b_red.push_back(c);
    return TROP_OK;
}

trop_status bind_shapes(Plan& P, const int64_t* shapeA, const int64_t* shapeB) {
    for (int i = 0; i < 128; ++i) P.ext[i] = -1;
    const std::string* subs[2] = {&P.la, &P.lb};
    const int64_t* shapes[2] = {shapeA, shapeB};
    for (int o = 0; o < 2; ++o) {
        if (!subs[o]->empty() && !shapes[o]) return fail(TROP_ERR_INVALID_ARGUMENT, "NULL shape");
        for (size_t d = 0; d < subs[o]->size(); ++d) {
            const char c = (*subs[o])[d];
            const int64_t e = shapes[o][d];
            if (e < 0) return fail(TROP_ERR_INVALID_ARGUMENT, "negative extent");
            if (P.ext[(int)c] >= 0 && P.ext[(int)c] != e)
                return fail(TROP_ERR_INVALID_ARGUMENT, std::string("extent mismatch for label '") + c + "'");
            P.ext[(int)c] = e;
        }
    }
    auto prod = [&](const std::string& labels, int64_t* out) {
        int64_t p = 1;
        for (char c : labels)
            if (__builtin_mul_overflow(p, P.ext[(int)c], &p)) return false;
        *out = p;
        return true;
    };
    if (!prod(P.batch, &P.nb) || !prod(P.left, &P.M) || !prod(P.right, &P.N) || !prod(P.contracted, &P.K) ||
        !prod(P.lo, &P.out_total))
        return fail(TROP_ERR_INVALID_ARGUMENT, "sizes overflow");
    if (P.K > INT32_MAX) return fail(TROP_ERR_INVALID_ARGUMENT, "contracted size must be < 2^31 (int32 argmax)");
    int64_t t;
    if (__builtin_mul_overflow(P.nb, P.M, &t) || __builtin_mul_overflow(t, P.K, &t) ||
        __builtin_mul_overflow(P.nb, P.K, &t) || __builtin_mul_overflow(t, P.N, &t) ||
        __builtin_mul_overflow(P.nb * P.M, P.N, &t))
        return fail(TROP_ERR_INVALID_ARGUMENT, "sizes overflow");
    return TROP_OK;
}

// Stride of a label group when it collapses to one axis of `op` (labels in
// group order, outermost first).  Returns false if the group is not
// collapsible or a label of it is repeated in the operand.
}  // namespace

trop_status pair_parse(const char* spec, std::string* la, std::string* lb, std::string* lo) {
    if (!spec) return fail(TROP_ERR_INVALID_ARGUMENT, "spec is NULL");
    std::string s;
    for (const char* q = spec; *q; ++q)
        if (*q != ' ') s.push_back(*q);
    const size_t arrow = s.find("->");
    if (arrow == std::string::npos || s.find("->", arrow + 2) != std::string::npos)
        return fail(TROP_ERR_INVALID_ARGUMENT, "spec needs exactly one '->' (explicit output)");
    const std::string lhs = s.substr(0, arrow);
    *lo = s.substr(arrow + 2);
    const size_t comma = lhs.find(',');
    if (comma == std::string::npos || lhs.find(',', comma + 1) != std::string::npos)
        return fail(TROP_ERR_INVALID_ARGUMENT, "spec needs exactly two operands");
    *la = lhs.substr(0, comma);
    *lb = lhs.substr(comma + 1);
    return TROP_OK;
}

namespace {

bool group_stride(const Plan& P, const Operand& op, const std::string& group, int64_t* out) {
    int64_t want = -1;  // stride the next (outer) label must have
    int64_t s_inner = 0;
    bool any = false;
    for (int g = (int)group.size() - 1; g >= 0; --g) {
        const char c = group[g];
        int pos = -1, count = 0;
        for (size_t d = 0; d < op.sub.size(); ++d)
            if (op.sub[d] == c) {
                pos = (int)d;
                ++count;
            }
        if (count != 1) return false;
        const int64_t e = P.ext[(int)c];
        if (e == 1) continue;
        const int64_t s = op.stride[pos];
        if (!any) {
            s_inner = s;
            any = true;
        } else if (s != want) {
            return false;
        }
        want = s * e;
    }
    *out = any ? s_inner : 0;
    return true;
}

// Can `op` be read in place as a batched matrix (batch, rows, cols)?
bool try_fold(const Plan& P, const Operand& op, const std::string& reduce, const std::string& gb,
              const std::string& gr, const std::string& gc, trop_strides* s) {
    if (!reduce.empty()) return false;
    if (unique(op.sub).size() != op.sub.size()) return false;  // repeated label: needs the diagonal pass
    int64_t sb, sr, sc;
    if (!group_stride(P, op, gb, &sb) || !group_stride(P, op, gr, &sr) || !group_stride(P, op, gc, &sc))
        return false;
    const int64_t rows = [&] { int64_t p = 1; for (char c : gr) p *= P.ext[(int)c]; return p; }();
    const int64_t cols = [&] { int64_t p = 1; for (char c : gc) p *= P.ext[(int)c]; return p; }();
    // a unit stride on the row or column axis keeps the GEMM loads coalesced
    const bool unit = (sc == 1 || cols == 1) || (sr == 1 || rows == 1);
    if (!unit) return false;
    s->batch = sb;
    s->row = sr;
    s->col = sc;
    return true;
}

// Can `op` be read in place with a two-level k?  The batch group and the
// free group (rows of the GEMM's left operand, columns of its right one)
// each collapse to one stride; the contracted group `gk` splits into outer
// labels that collapse to one stride (hi) and inner labels that collapse to
// unit stride with 4, 8 or 16 elements in all (the run), so that k =
// outer index * run + inner index is the row-major index over gk.  The
// GEMM then reads 16-byte vectors inside the runs instead of a gathered
// copy.  k_is_col: gk is the operand's column group (the left operand).
bool try_fold_two(const Plan& P, const Operand& op, const std::string& reduce, const std::string& gb,
                  const std::string& gfree, const std::string& gk, bool k_is_col, trop_strides* s,
                  int32_t* run, int64_t* hi) {
    if (!reduce.empty()) return false;
    if (const char* v = std::getenv("TROPICAL_NO_KRUN_FOLD"))  // tests: gather instead
        if (*v && *v != '0') return false;
    if (unique(op.sub).size() != op.sub.size()) return false;
    int64_t sb, sf;
    if (!group_stride(P, op, gb, &sb) || !group_stride(P, op, gfree, &sf)) return false;
    for (size_t j = 1; j < gk.size(); ++j) {
        const std::string outer = gk.substr(0, gk.size() - j), inner = gk.substr(gk.size() - j);
        int64_t r = 1;
        for (char c : inner) r = r > 16 ? r : r * P.ext[(int)c];
        if (!krun_ok((int32_t)std::min<int64_t>(r, 17))) continue;
        int64_t si = 0, so = 0;
        if (!group_stride(P, op, inner, &si) || si != 1) continue;
        if (!group_stride(P, op, outer, &so)) continue;
        *run = (int32_t)r;
        *hi = so;
        s->batch = sb;
        s->row = k_is_col ? sf : 1;
        s->col = k_is_col ? 1 : sf;
        return true;
    }
    return false;
}

trop_status plan_operand(const Plan& P, const Operand& op, const std::string& canonical, GatherPlan* g) {
    int32_t in_lab[TROP_MAX_DIMS], out_lab[TROP_MAX_DIMS];
    for (size_t d = 0; d < op.sub.size(); ++d) in_lab[d] = op.sub[d];
    for (size_t d = 0; d < canonical.size(); ++d) out_lab[d] = canonical[d];
    return plan_diag((int)op.sub.size(), op.shape, op.stride, in_lab, (int)canonical.size(), out_lab, g);
}

void default_strides(Operand& op) {
    int64_t s = 1;
    for (int d = (int)op.sub.size() - 1; d >= 0; --d) {
        op.stride[d] = s;
        s *= op.shape[d] > 0 ? op.shape[d] : 1;
    }
}

// Elements of `op` reached from its base (0 when it has no element).
bool operand_span(const Operand& op, int64_t* span) {
    *span = 0;
    for (size_t d = 0; d < op.sub.size(); ++d)
        if (op.shape[d] == 0) return true;
    int64_t off = 0;
    if (!max_offset((int)op.sub.size(), op.shape, op.stride, &off)) return false;
    *span = off + 1;
    return true;
}

}  // namespace

trop_status pair_plan(const std::string& la, const std::string& lb, const std::string& lo,
                      const int64_t* shapeA, const int64_t* stridesA, const int64_t* shapeB,
                      const int64_t* stridesB, Plan& P, bool value_only) {
    P = Plan();
    P.la = la;
    P.lb = lb;
    P.lo = lo;
    trop_status st = assign_roles(P);
    if (st != TROP_OK) return st;
    st = bind_shapes(P, shapeA, shapeB);
    if (st != TROP_OK) return st;
    Operand A, B;
    A.sub = P.la;
    B.sub = P.lb;
    for (size_t d = 0; d < A.sub.size(); ++d) A.shape[d] = shapeA[d];
    for (size_t d = 0; d < B.sub.size(); ++d) B.shape[d] = shapeB[d];
    if (stridesA) {
        for (size_t d = 0; d < A.sub.size(); ++d) A.stride[d] = stridesA[d];
    } else {
        default_strides(A);
    }
    if (stridesB) {
        for (size_t d = 0; d < B.sub.size(); ++d) B.stride[d] = stridesB[d];
    } else {
        default_strides(B);
    }
    for (size_t d = 0; d < A.sub.size(); ++d)
        if (A.stride[d] < 0) return fail(TROP_ERR_INVALID_ARGUMENT, "negative stride in A");
    for (size_t d = 0; d < B.sub.size(); ++d)
        if (B.stride[d] < 0) return fail(TROP_ERR_INVALID_ARGUMENT, "negative stride in B");
    if (!operand_span(A, &P.span_a) || !operand_span(B, &P.span_b))
        return fail(TROP_ERR_INVALID_ARGUMENT, "operand extent overflows");

    // Every (x) here is commutative bit for bit (IEEE add and multiply,
    // saturating int32 add), so the product may be taken as B (x) A when
    // that writes the output order directly: C[b][r][l] = (+)_k B[b][r][k]
    // (x) A[b][k][l].  The contracted labels keep A-subscript order on both
    // sides, so the argmax index means the same either way.
    P.swap = (P.batch + P.left + P.right != P.lo) && (P.batch + P.right + P.left == P.lo);
    const std::string rows = P.swap ? P.right : P.left;   // GEMM row labels
    const std::string cols = P.swap ? P.left : P.right;   // GEMM column labels
    P.gm = P.swap ? P.N : P.M;
    P.gn = P.swap ? P.M : P.N;
    const std::string canL = P.batch + rows + P.contracted;  // GEMM left operand
    const std::string canR = P.batch + P.contracted + cols;  // GEMM right operand
    const std::string canC = P.batch + rows + cols;
    // ga / sA / a_fold describe the GEMM's left operand (A, or B when
    // swapped), gb / sB / b_fold its right operand
    const Operand& L = P.swap ? B : A;
    const Operand& Rt = P.swap ? A : B;
    const std::string& l_red = P.swap ? P.b_red : P.a_red;
    const std::string& r_red = P.swap ? P.a_red : P.b_red;

    P.a_fold = try_fold(P, L, l_red, P.batch, rows, P.contracted, &P.sA) ||
               try_fold_two(P, L, l_red, P.batch, rows, P.contracted, true, &P.sA, &P.kr.a_run, &P.kr.a_hi);
    // A long K (the size rule of kcol_b_pays): the GEMM reads both operands
    // along k in its global-resolve form, so a left operand that would be
    // read with its free index at unit stride is gathered in (batch, rows,
    // contracted) order, and the right one likewise below
    const bool long_k = kcol_b_pays(P.gm, P.gn, P.K, P.nb);
    if (P.a_fold && long_k && P.kr.a_run == 0 && !(P.sA.col == 1 && P.sA.row % 4 == 0 && P.sA.batch % 4 == 0))
        P.a_fold = false;
    if (!P.a_fold) {
        st = plan_operand(P, L, canL, &P.ga);
        if (st != TROP_OK) return st;
        P.sA = {P.K, 1, P.gm * P.K};
    }
    P.b_fold = try_fold(P, Rt, r_red, P.batch, P.contracted, cols, &P.sB) ||
               try_fold_two(P, Rt, r_red, P.batch, cols, P.contracted, false, &P.sB, &P.kr.b_run, &P.kr.b_hi);
    // the right operand: read along k from a copy in (batch, cols,
    // contracted) order where it would otherwise be read with its free
    // index at unit stride (the left one is read along k by now); not
    // without an argmax output, whose kernel reads either layout as fast
    // (the copy would only add its traffic)
    const bool b_kcol = long_k && !value_only;
    if (P.b_fold && b_kcol && P.kr.b_run == 0 && P.sB.row != 1) P.b_fold = false;
    P.b_kcol = !P.b_fold && b_kcol;
    if (!P.b_fold) {
        st = plan_operand(P, Rt, b_kcol ? P.batch + cols + P.contracted : canR, &P.gb);
        if (st != TROP_OK) return st;
        P.sB = b_kcol ? trop_strides{1, P.K, P.K * P.gn} : trop_strides{P.gn, 1, P.K * P.gn};
    }
    P.c_direct = (canC == P.lo);
    if (!P.c_direct) {
        // C'' is contiguous over canC; the output walks it in P.lo order
        int64_t cstr[TROP_MAX_DIMS];
        int64_t s = 1;
        for (int d = (int)canC.size() - 1; d >= 0; --d) {
            cstr[d] = s;
            s *= P.ext[(int)canC[d]];
        }
        int64_t oshape[TROP_MAX_DIMS], ostride[TROP_MAX_DIMS];
        for (size_t d = 0; d < P.lo.size(); ++d) {
            const size_t pos = canC.find(P.lo[d]);
            oshape[d] = P.ext[(int)P.lo[d]];
            ostride[d] = cstr[pos];
        }
        st = plan_gather((int)P.lo.size(), oshape, ostride, 0, nullptr, nullptr, &P.gc);
        if (st != TROP_OK) return st;
    }
    // workspace layout
    size_t off = 0;
    if (!P.a_fold) {
        P.off_a = off;
        off += align_up((size_t)(P.nb * P.gm * P.K) * 4);
    }
    if (!P.b_fold) {
        P.off_b = off;
        off += align_up((size_t)(P.nb * P.K * P.gn) * 4);
    }
    if (!P.c_direct) {
        P.off_c = off;
        off += align_up((size_t)(P.nb * P.M * P.N) * 4);
        P.off_i = off;
        off += align_up((size_t)(P.nb * P.M * P.N) * 4);
    }
    // winners of the pre-pass reductions (for an argmax routed through them)
    P.red_l = !l_red.empty();
    P.red_r = !r_red.empty();
    for (char c : P.a_red) P.ra_n *= P.ext[(int)c];
    for (char c : P.b_red) P.rb_n *= P.ext[(int)c];
    {
        int64_t t = 0;
        P.route_fits = !__builtin_mul_overflow(P.K, P.ra_n, &t) && !__builtin_mul_overflow(t, P.rb_n, &t) &&
                       t <= (int64_t)INT32_MAX + 1;
    }
    if (P.red_l) {
        P.off_wl = off;
        off += align_up((size_t)(P.nb * P.gm * P.K) * 4);
    }
    if (P.red_r) {
        P.off_wr = off;
        off += align_up((size_t)(P.nb * P.K * P.gn) * 4);
    }
    // the GEMM's own workspace: split-K partials, or the domain flags of
    // the float mode of int32 products
    P.gemm_split = plan_splitk(P.gm, P.gn, P.K, P.nb).ksplit > 1;
    const size_t gws = gemm_workspace_bytes(P.gm, P.gn, P.K, P.nb);
    if (gws > 0) {
        P.off_split = off;
        P.split_bytes = gws;
        off += ws_align(gws);
    }
    P.ws = off;
    return TROP_OK;
}

std::string pair_describe(const Plan& P) {
    // how the GEMM reads A and B: "fold" (in place), "fold:krunR" (in place
    // with a two-level k of run R) or "gather:<path>"
    auto how = [&](bool fold, int32_t run, const GatherPlan& g) {
        if (!fold) return std::string("gather:") + gather_path_name(g.path);
        return run > 0 ? "fold:krun" + std::to_string(run) : std::string("fold");
    };
    // (":kcol": the GEMM's right operand gathered with k at unit stride)
    const std::string hr = how(P.b_fold, P.kr.b_run, P.gb) + (P.b_kcol ? ":kcol" : "");
    const std::string ha = P.swap ? hr : how(P.a_fold, P.kr.a_run, P.ga);
    const std::string hb = P.swap ? how(P.a_fold, P.kr.a_run, P.ga) : hr;
    char buf[640];
    std::snprintf(buf, sizeof(buf),
                  "batch=%s left=%s right=%s contracted=%s reduceA=%s reduceB=%s; gemm %s batch=%lld m=%lld "
                  "n=%lld k=%lld%s; A=%s B=%s out=%s%s; workspace=%zu",
                  P.batch.c_str(), P.left.c_str(), P.right.c_str(), P.contracted.c_str(), P.a_red.c_str(),
                  P.b_red.c_str(), P.swap ? "B(x)A" : "A(x)B", (long long)P.nb, (long long)P.gm,
                  (long long)P.gn, (long long)P.K, P.gemm_split ? " splitK" : "", ha.c_str(), hb.c_str(),
                  P.c_direct ? "direct" : "permute:", P.c_direct ? "" : gather_path_name(P.gc.path), P.ws);
    return buf;
}

trop_status pair_run(int dev, const Plan& P, trop_semiring semiring, trop_dtype dtype, const void* Aptr,
                     const void* Bptr, void* C, int32_t* argmax, void* scratch, hipStream_t s) {
    if (P.out_total == 0) return TROP_OK;
    char* ws = static_cast<char*>(scratch);
    trop_status st;
    // 1. unary pre-pass + permute into canonical operand order (a_* is the
    // GEMM's left operand: A, or B when the product is taken as B (x) A).
    // The gather plans are copied: running sets their pointers, and a plan
    // may be run from several threads at once.
    const void* l_ptr = P.swap ? Bptr : Aptr;
    const void* r_ptr = P.swap ? Aptr : Bptr;
    const void* a_use = l_ptr;
    const void* b_use = r_ptr;
    // an argmax routed through a pre-pass reduction keeps its winners
    const bool route = argmax && (P.red_l || P.red_r) && P.K > 0;
    if (!P.a_fold && !P.b_fold) {
        // both operands: one launch when both take the same tiled kernel
        GatherPlan g0 = P.ga, g1 = P.gb;
        const void* in0[2] = {l_ptr, nullptr};
        void* out0[2] = {ws + P.off_a, ws + P.off_wl};
        const void* in1[2] = {r_ptr, nullptr};
        void* out1[2] = {ws + P.off_b, ws + P.off_wr};
        st = run_gather_pair(dev, g0, route && P.red_l ? 2 : 1, in0, out0, g1, route && P.red_r ? 2 : 1, in1,
                             out1, semiring, dtype, s);
        if (st != TROP_OK) return st;
        a_use = ws + P.off_a;
        b_use = ws + P.off_b;
    } else if (!P.a_fold) {
        GatherPlan g = P.ga;
        void* dst = ws + P.off_a;
        const void* in[2] = {l_ptr, nullptr};
        void* out[2] = {dst, ws + P.off_wl};
        st = run_gather(dev, g, route && P.red_l ? 2 : 1, in, out, semiring, dtype, s);
        if (st != TROP_OK) return st;
        a_use = dst;
    } else if (!P.b_fold) {
        GatherPlan g = P.gb;
        void* dst = ws + P.off_b;
        const void* in[2] = {r_ptr, nullptr};
        void* out[2] = {dst, ws + P.off_wr};
        st = run_gather(dev, g, route && P.red_r ? 2 : 1, in, out, semiring, dtype, s);
        if (st != TROP_OK) return st;
        b_use = dst;
    }
    // 2. batched GEMM into the canonical (batch, rows, cols) result
    void* c_gemm = P.c_direct ? C : static_cast<void*>(ws + P.off_c);
    int32_t* i_gemm = P.c_direct ? argmax : (argmax ? reinterpret_cast<int32_t*>(ws + P.off_i) : nullptr);
    const trop_strides sC = {P.gn, 1, P.gm * P.gn};
    st = run_gemm(dev, semiring, dtype, a_use, P.sA, b_use, P.sB, c_gemm, sC, i_gemm, P.gm, P.gn, P.K, P.nb, s,
                  P.split_bytes ? ws + P.off_split : nullptr, P.split_bytes, &P.kr);
    if (st != TROP_OK) return st;
    if (route) {
        // the product's k, then the reduction winners at that k, as one
        // row-major index over (contracted, A's reduced, B's reduced)
        TropComposeParams cp{};
        cp.idx = i_gemm;
        const int32_t* wl = P.red_l ? reinterpret_cast<const int32_t*>(ws + P.off_wl) : nullptr;
        const int32_t* wr = P.red_r ? reinterpret_cast<const int32_t*>(ws + P.off_wr) : nullptr;
        // left operand [nb][gm][K], right operand [nb][K][gn] (or
        // [nb][gn][K] when gathered along k)
        const int64_t l_str[4] = {P.gm * P.K, P.K, 0, 1};
        const int64_t r_str[4] = {P.K * P.gn, 0, P.b_kcol ? P.K : 1, P.b_kcol ? 1 : P.gn};
        const int32_t* wa = P.swap ? wr : wl;
        const int32_t* wb = P.swap ? wl : wr;
        const int64_t* sa = P.swap ? r_str : l_str;
        const int64_t* sb = P.swap ? l_str : r_str;
        cp.wa = wa;
        cp.wb = wb;
        cp.wa_b = sa[0], cp.wa_r = sa[1], cp.wa_c = sa[2], cp.wa_k = sa[3];
        cp.wb_b = sb[0], cp.wb_r = sb[1], cp.wb_c = sb[2], cp.wb_k = sb[3];
        cp.ra_n = P.ra_n;
        cp.rb_n = P.rb_n;
        cp.rows = P.gm;
        cp.cols = P.gn;
        cp.batch = P.nb;
        const int64_t tot = P.nb * P.gm * P.gn;
        const uint32_t grid = (uint32_t)std::min<int64_t>((tot + 255) / 256, int64_t(1) << 30);
        st = launch(dev, K_ARGMAX_COMPOSE, TROP_K_ARGMAX_COMPOSE, grid, 256, &cp, s);
        if (st != TROP_OK) return st;
    }
    // 3. one paired permute of value and argmax into the output order
    if (!P.c_direct) {
        GatherPlan g = P.gc;
        const void* in[2] = {c_gemm, i_gemm};
        void* out[2] = {C, argmax};
        st = run_gather(dev, g, argmax ? 2 : 1, in, out, semiring, dtype, s);
        if (st != TROP_OK) return st;
    }
    return TROP_OK;
}

namespace {

trop_status build_plan(const char* spec, const int64_t* shapeA, const int64_t* stridesA, const int64_t* shapeB,
                       const int64_t* stridesB, Plan& P, bool value_only = false) {
    std::string la, lb, lo;
    trop_status st = pair_parse(spec, &la, &lb, &lo);
    if (st != TROP_OK) return st;
    return pair_plan(la, lb, lo, shapeA, stridesA, shapeB, stridesB, P, value_only);
}

}  // namespace

}  // namespace trop

using namespace trop;

extern "C" trop_status tropical_contract_pair_workspace_size(const char* spec, const int64_t* shapeA,
                                                             const int64_t* shapeB, size_t* bytes) {
    if (!bytes) return fail(TROP_ERR_INVALID_ARGUMENT, "bytes is NULL");
    Plan P;
    // default (contiguous) strides: the bound below does not depend on them
    trop_status st = build_plan(spec, shapeA, nullptr, shapeB, nullptr, P);
    if (st != TROP_OK) return st;
    // upper bound: room for both operand pre-passes and the output permute
    size_t ws = align_up((size_t)(P.nb * P.M * P.K) * 4) + align_up((size_t)(P.nb * P.K * P.N) * 4);
    if (!P.c_direct) ws += 2 * align_up((size_t)(P.nb * P.M * P.N) * 4);
    ws += ws_align(gemm_workspace_bytes(P.M, P.N, P.K, P.nb));  // split K, or int32 float-mode flags
    // winners of the pre-pass reductions, for an argmax routed through them
    if (!P.a_red.empty()) ws += align_up((size_t)(P.nb * P.M * P.K) * 4);
    if (!P.b_red.empty()) ws += align_up((size_t)(P.nb * P.K * P.N) * 4);
    *bytes = ws;
    return ok();
}

extern "C" trop_status tropical_contract_pair_describe(const char* spec, const int64_t* shapeA,
                                                       const int64_t* stridesA, const int64_t* shapeB,
                                                       const int64_t* stridesB, char* buf, size_t buflen) {
    Plan P;
    trop_status st = build_plan(spec, shapeA, stridesA, shapeB, stridesB, P);
    if (st != TROP_OK) return st;
    const std::string d = pair_describe(P);
    if (buf && buflen > 0) {
        std::strncpy(buf, d.c_str(), buflen - 1);
        buf[buflen - 1] = '\0';
    }
    return ok();
}

namespace trop {

trop_status contract_pair_call(const char* spec, trop_semiring semiring, trop_dtype dtype, const void* Aptr,
                               const int64_t* shapeA, const int64_t* stridesA, const void* Bptr,
                               const int64_t* shapeB, const int64_t* stridesB, void* C, int32_t* argmax,
                               void* workspace, size_t workspace_bytes, bool fixed_scratch, void* stream) {
    if (semiring < TROP_MAX_PLUS || semiring > TROP_MAX_MUL) return fail(TROP_ERR_INVALID_ARGUMENT, "unknown semiring");
    if (dtype != TROP_F32 && dtype != TROP_I32) return fail(TROP_ERR_INVALID_ARGUMENT, "unknown dtype");
    if (ring_index(semiring, dtype) < 0) return fail(TROP_ERR_UNSUPPORTED, "no such semiring / dtype pair");
    Plan P;
    trop_status st = build_plan(spec, shapeA, stridesA, shapeB, stridesB, P, argmax == nullptr);
    if (st != TROP_OK) return st;
    if (argmax && !P.route_fits)
        return fail(TROP_ERR_INVALID_ARGUMENT, "the argmax index over the contracted and reduced labels exceeds int32");
    if (P.out_total == 0) return ok();
    if (P.ws > 0 && workspace_bytes < P.ws) {
        if (fixed_scratch)
            return fail(TROP_ERR_WORKSPACE_TOO_SMALL,
                        "this contraction needs " + std::to_string(P.ws) +
                            " bytes of scratch; the allocation-free call holds at most " +
                            std::to_string(workspace_bytes) + " (use tropical_contract_pair with a workspace)");
        return fail(TROP_ERR_WORKSPACE_TOO_SMALL,
                    "workspace needs " + std::to_string(P.ws) + " bytes, got " + std::to_string(workspace_bytes));
    }

    int dev = -1;
    st = current_device(&dev);
    if (st != TROP_OK) return st;
    if (P.span_a > 0) {
        st = check_device_span(Aptr, dev, P.span_a, 4, "A");
        if (st != TROP_OK) return st;
    }
    if (P.span_b > 0) {
        st = check_device_span(Bptr, dev, P.span_b, 4, "B");
        if (st != TROP_OK) return st;
    }
    st = check_device_span(C, dev, P.out_total, 4, "C");
    if (st != TROP_OK) return st;
    if (argmax) {
        st = check_device_span(argmax, dev, P.out_total, 4, "argmax");
        if (st != TROP_OK) return st;
    }
    if (P.ws > 0 && !fixed_scratch) {
        st = check_device_span(workspace, dev, (int64_t)(P.ws / 4), 4, "workspace");
        if (st != TROP_OK) return st;
    }
    st = pair_run(dev, P, semiring, dtype, Aptr, Bptr, C, argmax, workspace, static_cast<hipStream_t>(stream));
    if (st != TROP_OK) return st;
    return ok();
}

}  // namespace trop

extern "C" trop_status tropical_contract_pair(const char* spec, trop_semiring semiring, trop_dtype dtype,
                                              const void* Aptr, const int64_t* shapeA, const int64_t* stridesA,
                                              const void* Bptr, const int64_t* shapeB, const int64_t* stridesB,
                                              void* C, int32_t* argmax, void* workspace,
                                              size_t workspace_bytes, void* stream) {
    return contract_pair_call(spec, semiring, dtype, Aptr, shapeA, stridesA, Bptr, shapeB, stridesB, C, argmax,
                              workspace, workspace_bytes, false, stream);
}
