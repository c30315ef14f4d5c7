/*
 * tropical_oracle.c -- plain, slow CPU oracle for the tropical contraction
 * hot path.
 *
 * THIS IS TEST INFRASTRUCTURE.  Only the test suite, the package smoke check
 * and the benchmark's CPU-baseline leg may load or call it.  The HIP library
 * never links, includes or calls anything here, and this file includes
 * nothing from the HIP library: the two implementations share no code.
 *
 * What it computes (sources are the web pages the method is taken from):
 *
 *  - orc_gemm / orc_gemm_points: the strided-batched tropical matrix product
 *    with a per-element argmax, over the three semirings named in
 *    tropical-gemm PR #35 "feat: batched GPU ops with DLPack zero-copy
 *    output" (Summary, Key changes: max-plus, min-plus and max-mul batched
 *    kernels "with argmax", batch as the third grid axis, strided access).
 *    The pages never write out the semiring operations, so the standard
 *    tropical algebra is used:
 *        max-plus:  a (+) b = max(a, b),  a (x) b = a + b,  zero = -inf
 *        min-plus:  a (+) b = min(a, b),  a (x) b = a + b,  zero = +inf
 *        max-mul :  a (+) b = max(a, b),  a (x) b = a * b,  zero = +0
 *    For int32 the zero elements are -2^30 / +2^30 and (x) is a saturating
 *    32-bit add.  int32 max-mul, which the pages do not cover, takes the
 *    same rule for its product: the exact product clamped to the int32
 *    range; its zero is 0 (a term must exceed 0 to win, as for float32).
 *    The argmax is the index k of the first term that achieves the result:
 *    the scan starts from the zero element, goes over k in ascending order
 *    and replaces the running best only on a strictly better term.  A term
 *    that never beats the zero element (a NaN, or a term equal to zero)
 *    leaves the argmax at 0.
 *
 *  - orc_gemm_backward: gradients of the product routed along its argmax
 *    (winner routing), see the function's comment.
 *
 *  - orc_permute: the generic N-d permute of omeinsum-rs issue #52 "GPU
 *    tropical path: keep tensors device-resident + device-side permute",
 *    section "Resolved design for step 3", kernel (a): for each output
 *    element, decode its linear index against the output shape and
 *    recombine the digits with the permuted input strides.
 *
 *  - orc_diag_gather: kernel (b) of the same section: the repeated-label
 *    diagonal / trace unary pre-pass.  An input axis pair that carries the
 *    same label is walked with one shared index (its strides add up); a
 *    label that is absent from the output is reduced with the semiring's
 *    (+) (the tropical max / min fused into the gather).
 *
 *  - orc_einsum_brute: the pairwise contraction evaluated by enumerating
 *    every assignment of the summed labels.  It is an independent second
 *    route to the result of the pipeline described in the same issue
 *    ("Structural lessons from OMEinsum": unary pre-pass, permute,
 *    batched GEMM, output permute).
 *
 * Floating point: one IEEE add or multiply per term, round-to-nearest-even,
 * build with -ffp-contract=off and without fast-math, so that denormals are
 * kept and no FMA contraction can occur.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_MAX_PLUS = 0, ORC_MIN_PLUS = 1, ORC_MAX_MUL = 2 };
enum { ORC_F32 = 0, ORC_I32 = 1 };
enum { ORC_OK = 0, ORC_BAD_ARG = 1, ORC_UNSUPPORTED = 2 };

#define ORC_I32_INF (1 << 30) /* int32 stand-in for infinity */
#define ORC_MAX_RANK 16

/* ------------------------------------------------------------------ */
/* semiring elements                                                    */
/* ------------------------------------------------------------------ */

static float zero_f32(int sr)
{
    if (sr == ORC_MAX_PLUS) return -INFINITY;
    if (sr == ORC_MIN_PLUS) return INFINITY;
    return 0.0f; /* max-mul on [0, inf) */
}

static int32_t zero_i32(int sr)
{
    if (sr == ORC_MAX_MUL) return 0;
    return sr == ORC_MIN_PLUS ? ORC_I32_INF : -ORC_I32_INF;
}

static float otimes_f32(int sr, float a, float b)
{
    if (sr == ORC_MAX_MUL) return a * b;
    return a + b;
}

static int32_t otimes_i32(int sr, int32_t a, int32_t b)
{
    int64_t s = (sr == ORC_MAX_MUL) ? (int64_t)a * (int64_t)b : (int64_t)a + (int64_t)b;
    if (s > INT32_MAX) return INT32_MAX;
    if (s < INT32_MIN) return INT32_MIN;
    return (int32_t)s;
}

/* "t is strictly better than best" under the semiring's (+). */
static int better_f32(int sr, float t, float best)
{
    if (sr == ORC_MIN_PLUS) return t < best;
    return t > best;
}

static int better_i32(int sr, int32_t t, int32_t best)
{
    if (sr == ORC_MIN_PLUS) return t < best;
    return t > best;
}

static int valid_pair(int sr, int dt)
{
    if (sr < ORC_MAX_PLUS || sr > ORC_MAX_MUL) return ORC_BAD_ARG;
    if (dt != ORC_F32 && dt != ORC_I32) return ORC_BAD_ARG;
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* tropical GEMM                                                        */
/* ------------------------------------------------------------------ */

/*
 * One output element C[b][i][j] = (+)_k A[b][i][k] (x) B[b][k][j] and its
 * argmax.  Strides are in elements: s[0] = row, s[1] = column, s[2] = batch.
 */
static void gemm_one(int sr, int dt,
                     const void* A, const int64_t* sA,
                     const void* B, const int64_t* sB,
                     int64_t k, int64_t b, int64_t i, int64_t j,
                     void* cval, int32_t* arg_out)
{
    int32_t arg = 0;
    if (dt == ORC_F32) {
        const float* a = (const float*)A;
        const float* bm = (const float*)B;
        float best = zero_f32(sr);
        for (int64_t kk = 0; kk < k; ++kk) {
            float x = a[b * sA[2] + i * sA[0] + kk * sA[1]];
            float y = bm[b * sB[2] + kk * sB[0] + j * sB[1]];
            float t = otimes_f32(sr, x, y);
            if (better_f32(sr, t, best)) {
                best = t;
                arg = (int32_t)kk;
            }
        }
        *(float*)cval = best;
    } else {
        const int32_t* a = (const int32_t*)A;
        const int32_t* bm = (const int32_t*)B;
        int32_t best = zero_i32(sr);
        for (int64_t kk = 0; kk < k; ++kk) {
            int32_t x = a[b * sA[2] + i * sA[0] + kk * sA[1]];
            int32_t y = bm[b * sB[2] + kk * sB[0] + j * sB[1]];
            int32_t t = otimes_i32(sr, x, y);
            if (better_i32(sr, t, best)) {
                best = t;
                arg = (int32_t)kk;
            }
        }
        *(int32_t*)cval = best;
    }
    *arg_out = arg;
}

/*
 * Full strided-batched product.  C and argmax share the strides sC;
 * argmax may be NULL.
 */
int orc_gemm(int sr, int dt,
             const void* A, const int64_t* sA,
             const void* B, const int64_t* sB,
             void* C, const int64_t* sC, int32_t* argmax,
             int64_t m, int64_t n, int64_t k, int64_t batch)
{
    int st = valid_pair(sr, dt);
    if (st != ORC_OK) return st;
    if (m < 0 || n < 0 || k < 0 || batch < 0) return ORC_BAD_ARG;
    if (k > INT32_MAX) return ORC_BAD_ARG;

    int64_t rows = batch * m;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / m;
        int64_t i = r % m;
        for (int64_t j = 0; j < n; ++j) {
            int64_t off = b * sC[2] + i * sC[0] + j * sC[1];
            int32_t arg;
            if (dt == ORC_F32) {
                float v;
                gemm_one(sr, dt, A, sA, B, sB, k, b, i, j, &v, &arg);
                ((float*)C)[off] = v;
            } else {
                int32_t v;
                gemm_one(sr, dt, A, sA, B, sB, k, b, i, j, &v, &arg);
                ((int32_t*)C)[off] = v;
            }
            if (argmax) argmax[off] = arg;
        }
    }
    return ORC_OK;
}

/*
 * The same product at a list of output points only: pts holds npts
 * (b, i, j) triples; values and argmaxes are written densely.
 */
int orc_gemm_points(int sr, int dt,
                    const void* A, const int64_t* sA,
                    const void* B, const int64_t* sB,
                    int64_t k, const int64_t* pts, int64_t npts,
                    void* cvals, int32_t* args)
{
    int st = valid_pair(sr, dt);
    if (st != ORC_OK) return st;
    if (k < 0 || npts < 0 || k > INT32_MAX) return ORC_BAD_ARG;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npts; ++p) {
        void* dst = (char*)cvals + 4 * p;
        gemm_one(sr, dt, A, sA, B, sB, k, pts[3 * p], pts[3 * p + 1], pts[3 * p + 2],
                 dst, &args[p]);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* backward: winner routing                                             */
/* ------------------------------------------------------------------ */

/*
 * Gradients of L = sum_{b,i,j} G[b][i][j] * C[b][i][j] through the tropical
 * product, routed along its argmax.  The pages ask for the backward to stay
 * consistent with the CPU path and to use the argmax the forward produces:
 * omeinsum-rs issue #52 ("Acceptance criteria": forward, backward and argmax
 * bit-for-bit; the u32 argmax buffer is the "tropical winner-routing"),
 * tropical-gemm PR #35 (the batched autograd functions route the gradient
 * through the argmax with scatter_add_ / gather, review comments), and the
 * rustytorch commit "rtx-backend-cuda: native index_select / index_add"
 * (scatter-add as a deterministic walk of the adjoint of the selection).
 *
 * With k* = argmax[b][i][j], C[b][i][j] = A[b][i][k*] (x) B[b][k*][j], so
 *     dA[b][i][k] = sum over j with k* = k of G[b][i][j] * dC/dA
 *     dB[b][k][j] = sum over i with k* = k of G[b][i][j] * dC/dB
 * where dC/dA = dC/dB = 1 for max-plus and min-plus (x = +), and
 * dC/dA = B[b][k*][j], dC/dB = A[b][i][k*] for max-mul (x = *).  Every
 * output that has an argmax routes its gradient, also one that nothing beat
 * (its argmax is 0).  Each sum starts at +0.0 and adds its terms in
 * ascending j (dA) or ascending i (dB), one IEEE multiply (max-mul) and one
 * IEEE add per term.  Argmax entries outside [0, k) route nothing.  The
 * float operands A and B are read for max-mul only and may be NULL
 * otherwise; either gradient may be NULL (not computed).  Strides: s[0] row,
 * s[1] column, s[2] batch; G shares the argmax's strides sC.
 */
int orc_gemm_backward(int sr, const float* A, const int64_t* sA,
                      const float* B, const int64_t* sB,
                      const int32_t* argmax, const float* G, const int64_t* sC,
                      float* dA, const int64_t* sdA, float* dB, const int64_t* sdB,
                      int64_t m, int64_t n, int64_t k, int64_t batch)
{
    if (sr < ORC_MAX_PLUS || sr > ORC_MAX_MUL) return ORC_BAD_ARG;
    if (m < 0 || n < 0 || k < 0 || batch < 0) return ORC_BAD_ARG;
    if (sr == ORC_MAX_MUL && ((dA && !B) || (dB && !A))) return ORC_BAD_ARG;
    const int mul = sr == ORC_MAX_MUL;
    if (dA) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t r = 0; r < batch * m; ++r) {
            int64_t b = r / m, i = r % m;
            for (int64_t kk = 0; kk < k; ++kk) dA[b * sdA[2] + i * sdA[0] + kk * sdA[1]] = 0.0f;
            for (int64_t j = 0; j < n; ++j) {
                int64_t c = b * sC[2] + i * sC[0] + j * sC[1];
                int32_t ks = argmax[c];
                if (ks < 0 || ks >= k) continue;
                float v = G[c];
                if (mul) v = v * B[b * sB[2] + ks * sB[0] + j * sB[1]];
                float* d = &dA[b * sdA[2] + i * sdA[0] + ks * sdA[1]];
                *d = *d + v;
            }
        }
    }
    if (dB) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t r = 0; r < batch * n; ++r) {
            int64_t b = r / n, j = r % n;
            for (int64_t kk = 0; kk < k; ++kk) dB[b * sdB[2] + kk * sdB[0] + j * sdB[1]] = 0.0f;
            for (int64_t i = 0; i < m; ++i) {
                int64_t c = b * sC[2] + i * sC[0] + j * sC[1];
                int32_t ks = argmax[c];
                if (ks < 0 || ks >= k) continue;
                float v = G[c];
                if (mul) v = v * A[b * sA[2] + i * sA[0] + ks * sA[1]];
                float* d = &dB[b * sdB[2] + ks * sdB[0] + j * sdB[1]];
                *d = *d + v;
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* permute                                                              */
/* ------------------------------------------------------------------ */

/*
 * out is contiguous row-major with shape[perm[0]], ..., shape[perm[ndim-1]]:
 * out[o_0, ..., o_{n-1}] = in[sum_d o_d * in_strides[perm[d]]].
 */
int orc_permute(int elem_bytes, int ndim, const int64_t* shape,
                const int64_t* in_strides, const int32_t* perm,
                const void* in, void* out)
{
    if (ndim < 0 || ndim > ORC_MAX_RANK) return ORC_BAD_ARG;
    if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8 && elem_bytes != 16)
        return ORC_BAD_ARG;
    int seen[ORC_MAX_RANK] = {0};
    int64_t out_shape[ORC_MAX_RANK];
    int64_t total = 1;
    for (int d = 0; d < ndim; ++d) {
        if (perm[d] < 0 || perm[d] >= ndim || seen[perm[d]]) return ORC_BAD_ARG;
        seen[perm[d]] = 1;
        if (shape[perm[d]] < 0) return ORC_BAD_ARG;
        out_shape[d] = shape[perm[d]];
        total *= out_shape[d];
    }
    for (int64_t o = 0; o < total; ++o) {
        int64_t rem = o;
        int64_t off = 0;
        for (int d = ndim - 1; d >= 0; --d) {
            int64_t digit = rem % out_shape[d];
            rem /= out_shape[d];
            off += digit * in_strides[perm[d]];
        }
        memcpy((char*)out + o * elem_bytes, (const char*)in + off * elem_bytes,
               (size_t)elem_bytes);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* repeated-label diagonal / trace gather                               */
/* ------------------------------------------------------------------ */

/*
 * in has in_ndim axes, each carrying a label id.  Axes that share a label
 * are walked together (a diagonal): their extents must agree and their
 * strides add.  The output is contiguous row-major over out_labels.  Input
 * labels missing from out_labels are reduced with the semiring's (+),
 * starting from its zero element with the strict "better" test, in
 * row-major order over those labels (first one slowest).
 */
int orc_diag_gather(int sr, int dt, int in_ndim, const int64_t* in_shape,
                    const int64_t* in_strides, const int32_t* in_labels,
                    int out_ndim, const int32_t* out_labels,
                    const void* in, void* out, int32_t* arg_out)
{
    if (in_ndim < 0 || in_ndim > ORC_MAX_RANK) return ORC_BAD_ARG;
    if (out_ndim < 0 || out_ndim > ORC_MAX_RANK) return ORC_BAD_ARG;

    /* distinct input labels, in order of first appearance */
    int32_t lab[ORC_MAX_RANK];
    int64_t ext[ORC_MAX_RANK];
    int64_t str[ORC_MAX_RANK];
    int nlab = 0;
    for (int a = 0; a < in_ndim; ++a) {
        if (in_shape[a] < 0) return ORC_BAD_ARG;
        int found = -1;
        for (int l = 0; l < nlab; ++l)
            if (lab[l] == in_labels[a]) found = l;
        if (found < 0) {
            lab[nlab] = in_labels[a];
            ext[nlab] = in_shape[a];
            str[nlab] = in_strides[a];
            ++nlab;
        } else {
            if (ext[found] != in_shape[a]) return ORC_BAD_ARG;
            str[found] += in_strides[a];
        }
    }

    /* output labels: distinct and present in the input */
    int out_pos[ORC_MAX_RANK];
    int is_out[ORC_MAX_RANK] = {0};
    for (int d = 0; d < out_ndim; ++d) {
        int found = -1;
        for (int l = 0; l < nlab; ++l)
            if (lab[l] == out_labels[d]) found = l;
        if (found < 0 || is_out[found]) return ORC_BAD_ARG;
        is_out[found] = 1;
        out_pos[d] = found;
    }
    int red_pos[ORC_MAX_RANK];
    int nred = 0;
    for (int l = 0; l < nlab; ++l)
        if (!is_out[l]) red_pos[nred++] = l;

    if (nred > 0) {
        int st = valid_pair(sr, dt);
        if (st != ORC_OK) return st;
    } else if (dt != ORC_F32 && dt != ORC_I32) {
        return ORC_BAD_ARG;
    }

    int64_t total = 1;
    for (int d = 0; d < out_ndim; ++d) total *= ext[out_pos[d]];
    int64_t rtotal = 1;
    for (int r = 0; r < nred; ++r) rtotal *= ext[red_pos[r]];

    for (int64_t o = 0; o < total; ++o) {
        int64_t rem = o;
        int64_t base = 0;
        for (int d = out_ndim - 1; d >= 0; --d) {
            int64_t e = ext[out_pos[d]];
            base += (rem % e) * str[out_pos[d]];
            rem /= e;
        }
        if (nred == 0) {
            memcpy((char*)out + 4 * o, (const char*)in + 4 * base, 4);
            if (arg_out) arg_out[o] = 0;
            continue;
        }
        /* the winner: the position q (row-major over the reduced labels in
           order of first appearance) of the first strictly better value;
           0 when nothing beats the zero element */
        int32_t win = 0;
        if (dt == ORC_F32) {
            float best = zero_f32(sr);
            for (int64_t q = 0; q < rtotal; ++q) {
                int64_t rr = q, off = base;
                for (int r = nred - 1; r >= 0; --r) {
                    int64_t e = ext[red_pos[r]];
                    off += (rr % e) * str[red_pos[r]];
                    rr /= e;
                }
                float t = ((const float*)in)[off];
                if (better_f32(sr, t, best)) {
                    best = t;
                    win = (int32_t)q;
                }
            }
            ((float*)out)[o] = best;
        } else {
            int32_t best = zero_i32(sr);
            for (int64_t q = 0; q < rtotal; ++q) {
                int64_t rr = q, off = base;
                for (int r = nred - 1; r >= 0; --r) {
                    int64_t e = ext[red_pos[r]];
                    off += (rr % e) * str[red_pos[r]];
                    rr /= e;
                }
                int32_t t = ((const int32_t*)in)[off];
                if (better_i32(sr, t, best)) {
                    best = t;
                    win = (int32_t)q;
                }
            }
            ((int32_t*)out)[o] = best;
        }
        if (arg_out) arg_out[o] = win;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* brute-force pairwise einsum                                          */
/* ------------------------------------------------------------------ */

/*
 * Labels are ids 0 .. nlab-1 with extents extent[].  For every output
 * index (row-major over o_lab) the result is the (+) over every assignment
 * of the summed labels s_lab (row-major, first label slowest) of
 * A[..] (x) B[..]; idx receives the row-major position of the first
 * strictly better assignment (NULL: not written).  Every label of A and B
 * must be either an output or a summed label.
 */
int orc_einsum_brute(int sr, int dt, int nlab, const int64_t* extent,
                     int a_ndim, const int32_t* a_lab, const int64_t* a_str, const void* A,
                     int b_ndim, const int32_t* b_lab, const int64_t* b_str, const void* B,
                     int o_ndim, const int32_t* o_lab, void* C, int32_t* idx,
                     int s_ndim, const int32_t* s_lab)
{
    int st = valid_pair(sr, dt);
    if (st != ORC_OK) return st;
    if (nlab < 0 || nlab > 2 * ORC_MAX_RANK) return ORC_BAD_ARG;
    if (a_ndim < 0 || a_ndim > ORC_MAX_RANK || b_ndim < 0 || b_ndim > ORC_MAX_RANK ||
        o_ndim < 0 || o_ndim > ORC_MAX_RANK || s_ndim < 0 || s_ndim > 2 * ORC_MAX_RANK)
        return ORC_BAD_ARG;
    int role[2 * ORC_MAX_RANK];
    for (int l = 0; l < nlab; ++l) role[l] = 0;
    for (int d = 0; d < o_ndim; ++d) {
        if (o_lab[d] < 0 || o_lab[d] >= nlab || role[o_lab[d]]) return ORC_BAD_ARG;
        role[o_lab[d]] = 1;
    }
    for (int d = 0; d < s_ndim; ++d) {
        if (s_lab[d] < 0 || s_lab[d] >= nlab || role[s_lab[d]]) return ORC_BAD_ARG;
        role[s_lab[d]] = 2;
    }
    for (int d = 0; d < a_ndim; ++d)
        if (a_lab[d] < 0 || a_lab[d] >= nlab || !role[a_lab[d]]) return ORC_BAD_ARG;
    for (int d = 0; d < b_ndim; ++d)
        if (b_lab[d] < 0 || b_lab[d] >= nlab || !role[b_lab[d]]) return ORC_BAD_ARG;

    int64_t total = 1, stotal = 1;
    for (int d = 0; d < o_ndim; ++d) total *= extent[o_lab[d]];
    for (int d = 0; d < s_ndim; ++d) stotal *= extent[s_lab[d]];

    for (int64_t o = 0; o < total; ++o) {
        int64_t val[2 * ORC_MAX_RANK];
        int64_t rem = o;
        for (int d = o_ndim - 1; d >= 0; --d) {
            val[o_lab[d]] = rem % extent[o_lab[d]];
            rem /= extent[o_lab[d]];
        }
        float bestf = zero_f32(sr);
        int32_t besti = zero_i32(sr);
        int32_t arg = 0;
        for (int64_t p = 0; p < stotal; ++p) {
            int64_t pr = p;
            for (int d = s_ndim - 1; d >= 0; --d) {
                val[s_lab[d]] = pr % extent[s_lab[d]];
                pr /= extent[s_lab[d]];
            }
            int64_t ao = 0, bo = 0;
            for (int d = 0; d < a_ndim; ++d) ao += val[a_lab[d]] * a_str[d];
            for (int d = 0; d < b_ndim; ++d) bo += val[b_lab[d]] * b_str[d];
            if (dt == ORC_F32) {
                float t = otimes_f32(sr, ((const float*)A)[ao], ((const float*)B)[bo]);
                if (better_f32(sr, t, bestf)) {
                    bestf = t;
                    arg = (int32_t)p;
                }
            } else {
                int32_t t = otimes_i32(sr, ((const int32_t*)A)[ao], ((const int32_t*)B)[bo]);
                if (better_i32(sr, t, besti)) {
                    besti = t;
                    arg = (int32_t)p;
                }
            }
        }
        if (dt == ORC_F32)
            ((float*)C)[o] = bestf;
        else
            ((int32_t*)C)[o] = besti;
        if (idx) idx[o] = arg;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* threads                                                              */
/* ------------------------------------------------------------------ */

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
