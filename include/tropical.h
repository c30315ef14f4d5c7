/*
 * tropical.h -- C ABI of libtropical.so, the MI355X (gfx950) tropical
 * contraction hot path.
 *
 * Six operations, all device-resident and enqueued on a caller stream:
 *   tropical_gemm_strided_batched  batched tropical matrix product + argmax
 *   tropical_gemm_backward         gradients routed along that argmax
 *   tropical_permute               N-d permute of one or two 4-byte tensors
 *   tropical_diag_gather           repeated-label diagonal / trace pre-pass
 *   tropical_contract_pair         one pairwise einsum built from the three
 *   tropical_tree_run              a contraction tree of pairwise einsums
 *                                  with every intermediate kept on device
 *
 * Sources (web pages the method is taken from):
 *   [PR35]  tropical-gemm PR #35 "feat: batched GPU ops with DLPack zero-copy
 *           output" -- Summary / Key changes (batched max-plus, min-plus,
 *           max-mul f32 kernels with argmax, batch on the third grid axis,
 *           per-device context cache; reject host memory, guard zero-sized
 *           dims, validate same-device tensors).
 *   [I52]   omeinsum-rs issue #52 "GPU tropical path: keep tensors
 *           device-resident + device-side permute" -- "Resolved design for
 *           step 3" kernels (a) permute and (b) diagonal/trace gather;
 *           "Structural lessons from OMEinsum" (unary pre-pass, then permute,
 *           batched GEMM, output permute); "Acceptance criteria"
 *           (intermediates stay in device memory, context and module created
 *           once, value and argmax permuted with one identical mapping;
 *           forward, backward and argmax consistent with the CPU path, the
 *           argmax buffer being the "tropical winner-routing").
 *   [RT]    rustytorch commit "rtx-backend-cuda: native index_select /
 *           index_add" -- scatter-add as a deterministic walk of the
 *           adjoint of the selection, no atomics, bit-identical to the host.
 *   [WR]    tenferro-rs design note "cuTENSOR workspace retirement without a
 *           stream barrier" -- "Problem" (a per-node plan cache smaller than
 *           the number of distinct contractions evicts continuously, and each
 *           eviction releases a workspace behind a stream barrier) and
 *           "Proposal" (stream order as the completion witness for reuse).
 *
 * Conventions for every entry point
 *   - Element strides and sizes are counted in ELEMENTS, not bytes.
 *   - Every data pointer must be device memory of the current HIP device
 *     (hipMalloc / PyTorch's allocator).  Host or pinned-host pointers are
 *     rejected with TROP_ERR_NOT_DEVICE_MEMORY, pointers of another device
 *     with TROP_ERR_INVALID_ARGUMENT.
 *   - Ownership: the caller owns every buffer, including the workspace.
 *     The library allocates no device memory, keeps no pointer after the
 *     call returns and copies shape / stride arrays into kernel arguments.
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the
 *     legacy default stream) and the call returns without synchronising
 *     the host.  Argument errors are returned synchronously and then
 *     nothing is enqueued.  A fault inside a kernel surfaces at the
 *     caller's next synchronisation, as for any HIP launch.
 *   - Errors: a trop_status code; tropical_last_error() returns a
 *     thread-local text for the last failing call of the calling thread.
 *   - Thread safety: per-device module loading is guarded; calls are
 *     otherwise stateless and may be issued from several threads.
 *   - An output with zero elements makes any call a no-op returning
 *     TROP_OK before any pointer is inspected.
 */
#ifndef TROPICAL_H
#define TROPICAL_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define TROP_API __attribute__((visibility("default")))
#else
#define TROP_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TROP_OK = 0,
    TROP_ERR_INVALID_ARGUMENT = 1,
    TROP_ERR_UNSUPPORTED = 2,
    TROP_ERR_NOT_DEVICE_MEMORY = 3,
    TROP_ERR_WORKSPACE_TOO_SMALL = 4,
    TROP_ERR_HIP = 5
} trop_status;

/*
 * The three semirings of [PR35].  The pages name them without writing the
 * operations out; the standard tropical algebra is used:
 *   TROP_MAX_PLUS  (+) = max, (x) = +, zero = -inf (int32: -2^30)
 *   TROP_MIN_PLUS  (+) = min, (x) = +, zero = +inf (int32: +2^30)
 *   TROP_MAX_MUL   (+) = max, (x) = *, zero = +0   (int32: 0)
 * float32 (x) is one IEEE-754 add / multiply, round to nearest even,
 * denormals kept.  int32 (x) is a saturating 32-bit add; for int32 max-mul
 * it is the exact product clamped to [INT32_MIN, INT32_MAX] (the pages
 * define no int32 max-mul; this extends the saturating rule).  As for
 * float32, a max-mul term must exceed the zero element 0 to win.
 */
typedef enum { TROP_MAX_PLUS = 0, TROP_MIN_PLUS = 1, TROP_MAX_MUL = 2 } trop_semiring;
typedef enum { TROP_F32 = 0, TROP_I32 = 1 } trop_dtype;

/* Strides of a batched matrix X[b][r][c] = base[b*batch + r*row + c*col]. */
typedef struct {
    int64_t row, col, batch;
} trop_strides;

/* Kernel families counted by trop_stats.launches[]. */
typedef enum {
    TROP_K_GEMM_TILED = 0,   /* LDS-tiled GEMM with chunked argmax      */
    TROP_K_GEMM_SIMPLE = 1,  /* one-thread-per-output exact GEMM         */
    TROP_K_FILL = 2,         /* K = 0: C = zero, argmax = 0              */
    TROP_K_GATHER_COPY = 3,  /* permute/gather keeping the inner axis    */
    TROP_K_GATHER_TILED = 4, /* permute/gather through an LDS tile       */
    TROP_K_GATHER_NAIVE = 5, /* permute/gather, one thread per element   */
    TROP_K_GATHER_REDUCE = 6,/* gather with a (+)-reduction (trace)      */
    TROP_K_GEMM_BACKWARD = 7,/* gradient routed along the argmax         */
    TROP_K_GEMM_SPLITK_MERGE = 8, /* merge of split-K partials           */
    TROP_K_ARGMAX_COMPOSE = 9,    /* argmax through pre-pass reductions  */
    TROP_K_GEMM_DOMAIN = 10,      /* int32 float-mode domain pre-pass    */
    TROP_K_FAMILIES = 11
} trop_kernel_family;

typedef struct {
    uint64_t module_loads;             /* hipModuleLoadData calls, all devices  */
    uint64_t launches_total;           /* kernels enqueued                      */
    uint64_t launches[TROP_K_FAMILIES];/* per trop_kernel_family                */
} trop_stats;

/*
 * Load the kernel code object on `device` (once per process and device,
 * [I52] "Compilation & caching"; [PR35] per-device context cache).  Optional:
 * every other call loads lazily on the current device.  Idempotent.
 * Errors: TROP_ERR_INVALID_ARGUMENT (no such device), TROP_ERR_HIP (load
 * failed; nothing is cached, a later call retries).
 */
TROP_API trop_status tropical_init(int device);

/*
 * Strided-batched tropical GEMM with argmax ([PR35] batched kernels; [I52]
 * "Proposed plan" step 2):
 *   C[b][i][j] = (+)_{k<K} A[b][i][k] (x) B[b][k][j]
 *   argmax[b][i][j] = the smallest k whose term is the result
 * for b < batch, i < m, j < n.  The scan starts from the zero element and
 * only a strictly better term replaces the running best, so ties go to the
 * smaller k, a NaN term never wins, and a result that nothing beat is the
 * zero element with argmax 0 (C then holds the zero element's bits;
 * otherwise C holds the bits of the winning term, so signed zeros are kept).
 *
 * A, B, C: device pointers of `dtype` elements (float32 or int32).
 * sA, sB, sC: element strides; any non-negative values (A[b][i][k] at
 *   b*sA.batch + i*sA.row + k*sA.col, B[b][k][j] likewise with row = k,
 *   col = j).  Row-major and column-major A and B take the fast path.
 * argmax: device int32 pointer with the strides sC, or NULL (not written).
 * m, n, k, batch >= 0; k < 2^31.  k == 0 writes C = zero, argmax = 0.
 * Errors: TROP_ERR_INVALID_ARGUMENT (bad enum, negative size or stride),
 *   TROP_ERR_NOT_DEVICE_MEMORY, TROP_ERR_HIP (launch failure).
 */
TROP_API trop_status tropical_gemm_strided_batched(trop_semiring semiring, trop_dtype dtype,
                                          const void* A, trop_strides sA,
                                          const void* B, trop_strides sB,
                                          void* C, trop_strides sC, int32_t* argmax,
                                          int64_t m, int64_t n, int64_t k, int64_t batch,
                                          void* stream);

/*
 * Workspace (bytes) with which tropical_gemm_strided_batched_ws splits a
 * product of this shape along K (or, unsplit and large, gives an int32
 * max-plus / min-plus product its float mode); 0 when neither.  Host-only.
 * Errors: TROP_ERR_INVALID_ARGUMENT (negative size, NULL bytes).
 */
TROP_API trop_status tropical_gemm_workspace_size(int64_t m, int64_t n, int64_t k, int64_t batch,
                                         size_t* bytes);

/*
 * Workspace (bytes) for tropical_gemm_strided_batched_ws with these operand
 * strides: tropical_gemm_workspace_size's bytes, or more when the call
 * would copy operands transposed.  The copies are made for a product with
 * K >= 512 and a multiple of 4, at least 256 rows and 2^30 terms, and no
 * split along K: a column-major A (sA.row == 1, sA.col != 1) is copied as
 * [batch][m][k], and, with an argmax output (with_argmax != 0), a
 * row-major B (sB.col == 1) as [batch][n][k] when A is read along k
 * (sA.col == 1, sA.row and sA.batch multiples of 4, A 16-byte aligned, or
 * A copied).  They sit in the workspace 1 KiB in (after the int32
 * float-mode flags), B's first, each batch*rows*k*4 bytes rounded up to
 * 256.  The product then reads both operands along k as it does for a
 * row-major A and a column-major B (one argmax resolve per output tile;
 * the copies hold the same values, so the results are unchanged).  A
 * workspace of tropical_gemm_workspace_size's bytes gets no copy.
 * Host-only.
 * Errors: TROP_ERR_INVALID_ARGUMENT (negative size or stride, NULL bytes).
 */
TROP_API trop_status tropical_gemm_workspace_size_strided(trop_strides sA, trop_strides sB, int with_argmax,
                                                 int64_t m, int64_t n, int64_t k, int64_t batch,
                                                 size_t* bytes);

/*
 * tropical_gemm_strided_batched with a workspace, which lets a product with
 * few output tiles and a long K run on the whole device: K is cut into
 * `ksplit` ranges (of whole 256-term blocks; of 64 terms for a product of
 * at most 64 (tile, 256-term block) pairs), each (tile, range) pair is one
 * unit of the tiled kernel writing a partial value and global argmax into
 * the workspace, and a merge kernel keeps, per output, the first partial
 * (in range order) that is strictly better than those before it.  Every
 * range is scanned with the same strict rule, so the results -- values,
 * their bits and the smallest winning k -- are those of the unsplit call
 * (the tie rule of [PR35]'s argmax survives the split).  The split is used
 * when the product has fewer 64 x 64 output tiles (times batch) than the
 * device has CUs and K >= 512 (K >= 128 for those small products), and the
 * int32 float mode takes 1 KiB of it for a large unsplit product;
 * tropical_gemm_workspace_size reports the bytes (0: neither, and the call
 * equals tropical_gemm_strided_batched).
 * workspace: NULL with workspace_bytes 0 (never split), or device memory of
 *   at least that size, used only by work on `stream`.
 * Errors: as tropical_gemm_strided_batched, plus
 *   TROP_ERR_WORKSPACE_TOO_SMALL (a non-NULL workspace below the size).
 */
TROP_API trop_status tropical_gemm_strided_batched_ws(trop_semiring semiring, trop_dtype dtype,
                                             const void* A, trop_strides sA,
                                             const void* B, trop_strides sB,
                                             void* C, trop_strides sC, int32_t* argmax,
                                             int64_t m, int64_t n, int64_t k, int64_t batch,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream);

/*
 * Backward of tropical_gemm_strided_batched: the gradients of
 * L = sum_{b,i,j} grad_c[b][i][j] * C[b][i][j] routed along the argmax the
 * forward produced (winner routing, [I52] "Acceptance criteria"; the
 * scatter-add of [PR35]'s batched autograd functions, done as in [RT]):
 *   grad_a[b][i][k] = sum over j with argmax[b][i][j] = k of
 *                     grad_c[b][i][j] * w,  w = 1 (max-plus, min-plus)
 *                                           or B[b][k][j] (max-mul)
 *   grad_b[b][k][j] = sum over i with argmax[b][i][j] = k of
 *                     grad_c[b][i][j] * w,  w = 1 or A[b][i][k]
 * Each sum starts at +0.0 and adds its terms in ascending j (grad_a) or
 * ascending i (grad_b), one IEEE multiply and one IEEE add per term, with no
 * atomics: results are deterministic and bit-identical to that sequential
 * loop.  Every output routes its gradient, also one that nothing beat
 * (argmax 0); argmax entries outside [0, k) route nothing.  Every element of
 * the requested gradients is written (zeros where nothing routes).
 *
 * dtype: of A and B.  A and B are read for max-mul only (float32, required
 *   there, may be NULL otherwise); max-plus and min-plus work for float32
 *   and int32 products alike since only the argmax is read.
 * argmax (int32) and grad_c (float32) share the strides sC.
 * grad_a (batch, m, k) with strides sGA, grad_b (batch, k, n) with strides
 *   sGB: float32 device pointers, either may be NULL (not computed); they
 *   must not overlap each other or the inputs.
 * m, n, k, batch >= 0.
 * Errors: TROP_ERR_INVALID_ARGUMENT (bad enum, negative size or stride,
 *   max-mul without A / B), TROP_ERR_UNSUPPORTED (int32 max-mul: its
 *   clamped product has no gradient defined here), TROP_ERR_NOT_DEVICE_MEMORY,
 *   TROP_ERR_HIP.
 */
TROP_API trop_status tropical_gemm_backward(trop_semiring semiring, trop_dtype dtype,
                                   const void* A, trop_strides sA,
                                   const void* B, trop_strides sB,
                                   const int32_t* argmax, const float* grad_c, trop_strides sC,
                                   float* grad_a, trop_strides sGA,
                                   float* grad_b, trop_strides sGB,
                                   int64_t m, int64_t n, int64_t k, int64_t batch,
                                   void* stream);

/*
 * N-d permute ([I52] "Resolved design for step 3", kernel (a)):
 *   out[o_0..o_{d-1}] = in[sum_d o_d * in_strides[perm[d]]]
 * with out contiguous row-major of shape shape[perm[0]], ..., shape[perm[d-1]].
 * ntensors = 1 or 2: with 2, in[1] -> out[1] is moved with the identical
 * mapping in the same launch (value and argmax, [I52] "Acceptance criteria").
 * elem_bytes: 4 (float32, int32, uint32), 8 (float64, int64, complex64) or
 * 16 (complex128) -- [I52] (a) serves f32 / f64 / c32 / c64 tensors and the
 * u32 argmax; elements are moved as opaque bytes (their 4-byte words in
 * order), so any type of that size works.  Pointers need 4-byte alignment
 * (wider alignment enables wider accesses).  ndim <= 8; perm a permutation
 * of 0..ndim-1; shape >= 0; in_strides >= 0, in elements.  in and out must
 * not overlap.
 * Errors: TROP_ERR_INVALID_ARGUMENT, TROP_ERR_UNSUPPORTED (another
 *   elem_bytes; 8- or 16-byte elements with 8 output axes of which no two
 *   neighbours, nor the last axis and the element's own words, are
 *   contiguous in the input), TROP_ERR_NOT_DEVICE_MEMORY, TROP_ERR_HIP.
 */
TROP_API trop_status tropical_permute(size_t elem_bytes, int ndim, const int64_t* shape,
                             const int64_t* in_strides, const int32_t* perm,
                             int ntensors, const void* const* in, void* const* out,
                             void* stream);

/*
 * Repeated-label diagonal / trace gather ([I52] "Resolved design for step
 * 3", kernel (b): the unary pre-pass with the tropical max / min fused in).
 * Input axis a carries label in_labels[a] (any int32 ids).  Axes that share
 * a label are walked with one index (their extents must agree; their strides
 * add).  out is contiguous row-major over out_labels (distinct, each present
 * in the input).  Input labels absent from out_labels are reduced with the
 * semiring's (+), from its zero element with the strict "better" test, in
 * row-major order over those labels; without such labels the semiring is
 * ignored and the call is a pure 4-byte gather.
 * in_ndim, out_ndim <= 8.
 * Errors: TROP_ERR_INVALID_ARGUMENT (extent mismatch, unknown or repeated
 *   output label), TROP_ERR_NOT_DEVICE_MEMORY, TROP_ERR_HIP.
 */
TROP_API trop_status tropical_diag_gather(trop_semiring semiring, trop_dtype dtype,
                                 int in_ndim, const int64_t* in_shape,
                                 const int64_t* in_strides, const int32_t* in_labels,
                                 int out_ndim, const int32_t* out_labels,
                                 const void* in, void* out, void* stream);

/* Scratch held by tropical_contract_pair_noalloc on every device it runs
 * on (a file-scope device array, until the process ends). */
#define TROP_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * Workspace (bytes) that tropical_contract_pair needs for `spec` with these
 * operand shapes.  Host-only, touches no device.  Errors as for
 * tropical_contract_pair's argument checks.
 */
TROP_API trop_status tropical_contract_pair_workspace_size(const char* spec, const int64_t* shapeA,
                                                  const int64_t* shapeB, size_t* bytes);

/*
 * One pairwise tropical einsum, all on `stream` with no host round trip
 * ([I52] "Structural lessons from OMEinsum" and "Acceptance criteria"):
 *   1. diagonal / trace pre-pass and permute of A into (batch, left,
 *      contracted) and of B into (batch, contracted, right);
 *   2. one strided-batched tropical GEMM with argmax;
 *   3. one paired permute of value and argmax into the output order.
 * When the output order is (batch, right, left) the product is taken as
 * B (x) A instead -- B into (batch, right, contracted), A into (batch,
 * contracted, left) -- and lands in the output order with no step 3 (every
 * (x) here is commutative bit for bit, so values and argmax are the same).
 * An operand already collapsible to a batched matrix with a unit row or
 * column stride is used in place.  For a long K (K >= 512, a multiple of
 * 4, at least 256 rows and 2^30 terms, not split) an operand that would be
 * read with its free index at unit stride is gathered with k at unit
 * stride instead ((batch, rows, contracted) for the product's left
 * operand, (batch, cols, contracted) for its right one, the latter only
 * with an argmax output), so that the product reads both operands along k
 * (TROPICAL_GEMM_B_TRANSPOSE as for tropical_gemm_workspace_size_strided).  When both operands need the
 * tiled transpose kernel in step 1, the two run as one launch.
 * spec: "lhs,rhs->out" with single-letter labels a-z A-Z, explicit output,
 *   no ellipsis; every output label appears in an operand, output labels
 *   are distinct.  batch labels are in A, B and out; left in A and out;
 *   right in B and out; contracted in A and B only.  A label found in one
 *   operand only and absent from the output is (+)-reduced in the pre-pass.
 * A, B: device pointers, shapes and element strides (rank = subscript
 *   length, <= 8).  C: contiguous row-major over the output labels.
 * argmax: NULL or a contiguous int32 tensor shaped like C; it holds the
 *   row-major linear index over the contracted labels taken in A-subscript
 *   order.  When a pre-pass reduces labels of A or B, the index continues
 *   over A's reduced labels (A order), then B's (B order): the product's
 *   winning k, then the winners (first strictly better position) of the
 *   reductions that produced the two values it compared.  The whole index
 *   must fit int32 (else TROP_ERR_INVALID_ARGUMENT when requested).
 * workspace: device memory of at least tropical_contract_pair_workspace_size
 *   bytes (may be NULL when that size is 0), used only by work on `stream`.
 * Errors: TROP_ERR_INVALID_ARGUMENT, TROP_ERR_UNSUPPORTED,
 *   TROP_ERR_WORKSPACE_TOO_SMALL, TROP_ERR_NOT_DEVICE_MEMORY, TROP_ERR_HIP.
 */
TROP_API trop_status tropical_contract_pair(const char* spec, trop_semiring semiring, trop_dtype dtype,
                                   const void* A, const int64_t* shapeA, const int64_t* stridesA,
                                   const void* B, const int64_t* shapeB, const int64_t* stridesB,
                                   void* C, int32_t* argmax,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * tropical_contract_pair for callers that cannot allocate device memory or
 * pass a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results and errors,
 * minus the workspace: the intermediates live in the library's own
 * TROP_NOALLOC_SCRATCH_BYTES of device memory per device (a file-scope
 * array whose address is looked up once per device, at tropical_init or on
 * the first call there).  A contraction whose
 * tropical_contract_pair_workspace_size exceeds that limit is rejected with
 * TROP_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.  This call
 * allocates nothing and calls no allocating routine.  Every call on one
 * device shares that device's scratch: calls that overlap on one device
 * (other streams, other host threads) race and must be ordered by the
 * caller; calls on one stream are ordered by it.
 */
TROP_API trop_status tropical_contract_pair_noalloc(const char* spec, trop_semiring semiring, trop_dtype dtype,
                                                    const void* A, const int64_t* shapeA, const int64_t* stridesA,
                                                    const void* B, const int64_t* shapeB, const int64_t* stridesB,
                                                    void* C, int32_t* argmax, void* stream);

/*
 * Host-only: write a one-line text description of the plan that
 * tropical_contract_pair would enqueue (label roles, GEMM sizes, which
 * pre-passes and which kernel paths) into buf (NUL-terminated, truncated to
 * buflen).  Touches no device.
 */
TROP_API trop_status tropical_contract_pair_describe(const char* spec,
                                            const int64_t* shapeA, const int64_t* stridesA,
                                            const int64_t* shapeB, const int64_t* stridesB,
                                            char* buf, size_t buflen);

/*
 * ---- Contraction trees ([I52] "Acceptance criteria": intermediates stay in
 * device memory across the contraction tree; the module is loaded once) ----
 *
 * A tree is planned once and run any number of times.  Tensor slots are
 * numbered inputs first (0 .. n_inputs-1), then the result of step s as
 * slot n_inputs + s.  Step s contracts two earlier slots with
 * tropical_contract_pair's rules ("lhs_sub,rhs_sub->out"); the last step's
 * result is the tree's output.  Every step result except the last must be
 * read by a later step; inputs and results may be read by several steps.
 *
 * The plan holds one pairwise plan per step (so nothing is re-planned, and
 * no plan is ever evicted, whatever the number of distinct contractions --
 * [WR] "Problem") and a fixed layout of ONE workspace: each step's result
 * lives from its step to its last reader, each step's scratch during its
 * step only, and buffers whose lifetimes do not meet share memory.  All
 * steps are enqueued in order on the caller's stream, which is what makes
 * the sharing safe ([WR] "Proposal": stream order is the completion
 * witness); a run allocates, frees and waits for nothing.
 */
typedef struct trop_tree_plan_s* trop_tree_plan;

typedef struct {
    int32_t lhs, rhs;  /* operand slots (earlier inputs or step results)   */
    const char* out;   /* output subscript of the step (copied at planning) */
} trop_tree_step;

/*
 * Plan a tree.  input_subs[i]: subscript of input i (single letters a-z A-Z,
 * rank <= 8, repeated labels allowed); input_shapes[i]: its extents (may be
 * NULL for rank 0); input_strides: NULL (all contiguous row-major) or one
 * entry per input, NULL for a contiguous input, else its element strides.
 * Every step's subscripts follow tropical_contract_pair's rules, with the
 * operands' subscripts taken from their slots.  Host-only: touches no
 * device.  On success *plan owns host memory until
 * tropical_tree_plan_destroy.  A plan is immutable: several threads may run
 * it at once, each with its own workspace.
 * Errors: TROP_ERR_INVALID_ARGUMENT (bad enum, slot, subscript or extent;
 *   a step result that no later step reads).  The message names the
 *   failing step.
 */
TROP_API trop_status tropical_tree_plan_create(trop_semiring semiring, trop_dtype dtype, int n_inputs,
                                      const char* const* input_subs,
                                      const int64_t* const* input_shapes,
                                      const int64_t* const* input_strides,
                                      int n_steps, const trop_tree_step* steps,
                                      trop_tree_plan* plan);

/* Free a plan (NULL is ignored).  Runs already enqueued are unaffected. */
TROP_API void tropical_tree_plan_destroy(trop_tree_plan plan);

/* Device workspace (bytes) a run of this plan needs. */
TROP_API trop_status tropical_tree_workspace_size(trop_tree_plan plan, size_t* bytes);

/*
 * Output of step `step`: its subscript (NUL-terminated, buffer of at least
 * 9 bytes, or NULL), extents (at least rank entries, or NULL) and element
 * count (or NULL).  The argmax of a step, when requested, is a contiguous
 * int32 tensor of that shape.
 */
TROP_API trop_status tropical_tree_step_info(trop_tree_plan plan, int step, char* subscript,
                                    int64_t* shape, int64_t* elements);

/*
 * Run the tree on `stream`:
 *   inputs[i]: device pointer of input i (strides as planned);
 *   out: contiguous device tensor over the last step's subscript;
 *   step_argmax: NULL, or n_steps entries each NULL or a contiguous device
 *     int32 tensor shaped like that step's output, filled with the step's
 *     argmax exactly as tropical_contract_pair defines it (the winner
 *     routing of the tree: following it from the output down selects one
 *     entry of every input);
 *   workspace: at least tropical_tree_workspace_size bytes of device
 *     memory, not touched by other work until this run has finished on
 *     `stream` (a later run of any plan on the same stream may reuse it).
 * All argument checks precede the first launch; on error nothing is
 * enqueued.  Errors: as tropical_contract_pair.
 */
TROP_API trop_status tropical_tree_run(trop_tree_plan plan, const void* const* inputs, void* out,
                              int32_t* const* step_argmax, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Host-only: one line per step (slots, subscripts, workspace offsets and
 * tropical_contract_pair_describe's text), then the workspace size and
 * the sum of the intermediate results' sizes, into buf (truncated).
 */
TROP_API trop_status tropical_tree_describe(trop_tree_plan plan, char* buf, size_t buflen);

/* Text of the calling thread's last error ("" if none). */
TROP_API const char* tropical_last_error(void);

/* Copy the process-wide counters. */
TROP_API trop_status tropical_get_stats(trop_stats* out);

/* Zero the launch counters (module_loads is kept). */
TROP_API void tropical_reset_stats(void);

#ifdef __cplusplus
}
#endif

#endif /* TROPICAL_H */
