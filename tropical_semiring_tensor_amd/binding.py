"""Thin ctypes binding of libtropical.so (see include/tropical.h).

Each function has the name of the C entry point it calls and only marshals
arguments: torch tensors become data pointers, element strides and sizes,
the stream defaults to torch's current stream.  All computation happens in
the library's gfx950 kernels.  There is no fallback: if the library was not
built, the first call raises ``TropicalLibraryMissing``.

Output tensors are allocated with torch when the caller passes none; torch
is used only for device memory and streams.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libtropical.so")

OK, INVALID_ARGUMENT, UNSUPPORTED, NOT_DEVICE_MEMORY, WORKSPACE_TOO_SMALL, HIP_ERROR = range(6)
STATUS_NAMES = {0: "TROP_OK", 1: "TROP_ERR_INVALID_ARGUMENT", 2: "TROP_ERR_UNSUPPORTED",
                3: "TROP_ERR_NOT_DEVICE_MEMORY", 4: "TROP_ERR_WORKSPACE_TOO_SMALL",
                5: "TROP_ERR_HIP"}
SEMIRINGS = {"max_plus": 0, "min_plus": 1, "max_mul": 2}
F32, I32 = 0, 1
KERNEL_FAMILIES = ["gemm_tiled", "gemm_simple", "fill", "gather_copy", "gather_tiled",
                   "gather_naive", "gather_reduce", "gemm_backward", "gemm_splitk_merge",
                   "argmax_compose", "gemm_domain"]
MAX_DIMS = 8


class TropicalLibraryMissing(RuntimeError):
    pass


class TropicalError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


class trop_strides(ctypes.Structure):
    _fields_ = [("row", ctypes.c_int64), ("col", ctypes.c_int64), ("batch", ctypes.c_int64)]


class trop_tree_step(ctypes.Structure):
    _fields_ = [("lhs", ctypes.c_int32), ("rhs", ctypes.c_int32), ("out", ctypes.c_char_p)]


class trop_stats(ctypes.Structure):
    _fields_ = [("module_loads", ctypes.c_uint64), ("launches_total", ctypes.c_uint64),
                ("launches", ctypes.c_uint64 * 11)]


_lib = None


def lib():
    """The loaded library (loaded on first use; raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise TropicalLibraryMissing(
            f"{LIB_PATH} is not built; run __graft_entry__.build() "
            "(python tropical_semiring_tensor_amd/csrc/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    I64P = ctypes.POINTER(ctypes.c_int64)
    I32P = ctypes.POINTER(ctypes.c_int32)
    L.tropical_init.argtypes = [i32]
    L.tropical_gemm_strided_batched.argtypes = [i32, i32, vp, trop_strides, vp, trop_strides, vp,
                                                trop_strides, vp, i64, i64, i64, i64, vp]
    L.tropical_gemm_strided_batched_ws.argtypes = [i32, i32, vp, trop_strides, vp, trop_strides, vp,
                                                   trop_strides, vp, i64, i64, i64, i64, vp, sz, vp]
    L.tropical_gemm_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.POINTER(sz)]
    L.tropical_gemm_workspace_size_strided.argtypes = [trop_strides, trop_strides, i32, i64, i64, i64, i64,
                                                       ctypes.POINTER(sz)]
    L.tropical_gemm_backward.argtypes = [i32, i32, vp, trop_strides, vp, trop_strides, vp, vp,
                                         trop_strides, vp, trop_strides, vp, trop_strides,
                                         i64, i64, i64, i64, vp]
    L.tropical_permute.argtypes = [sz, i32, I64P, I64P, I32P, i32, ctypes.POINTER(vp),
                                   ctypes.POINTER(vp), vp]
    L.tropical_diag_gather.argtypes = [i32, i32, i32, I64P, I64P, I32P, i32, I32P, vp, vp, vp]
    L.tropical_contract_pair_workspace_size.argtypes = [ctypes.c_char_p, I64P, I64P,
                                                        ctypes.POINTER(sz)]
    L.tropical_contract_pair.argtypes = [ctypes.c_char_p, i32, i32, vp, I64P, I64P, vp, I64P, I64P,
                                         vp, vp, vp, sz, vp]
    L.tropical_contract_pair_describe.argtypes = [ctypes.c_char_p, I64P, I64P, I64P, I64P,
                                                  ctypes.c_char_p, sz]
    L.tropical_contract_pair_noalloc.argtypes = [ctypes.c_char_p, i32, i32, vp, I64P, I64P, vp, I64P, I64P,
                                                 vp, vp, vp]
    PP = ctypes.POINTER
    L.tropical_tree_plan_create.argtypes = [i32, i32, i32, PP(ctypes.c_char_p), PP(I64P), PP(I64P), i32,
                                            PP(trop_tree_step), PP(vp)]
    L.tropical_tree_plan_destroy.argtypes = [vp]
    L.tropical_tree_plan_destroy.restype = None
    L.tropical_tree_workspace_size.argtypes = [vp, PP(sz)]
    L.tropical_tree_step_info.argtypes = [vp, i32, ctypes.c_char_p, I64P, I64P]
    L.tropical_tree_run.argtypes = [vp, PP(vp), vp, PP(vp), vp, sz, vp]
    L.tropical_tree_describe.argtypes = [vp, ctypes.c_char_p, sz]
    L.tropical_last_error.restype = ctypes.c_char_p
    L.tropical_get_stats.argtypes = [ctypes.POINTER(trop_stats)]
    L.tropical_reset_stats.restype = None
    for fn in ("tropical_init", "tropical_gemm_strided_batched", "tropical_gemm_backward", "tropical_permute",
               "tropical_gemm_strided_batched_ws", "tropical_gemm_workspace_size",
               "tropical_gemm_workspace_size_strided",
               "tropical_diag_gather", "tropical_contract_pair_workspace_size",
               "tropical_contract_pair", "tropical_contract_pair_describe", "tropical_get_stats",
               "tropical_contract_pair_noalloc",
               "tropical_tree_plan_create", "tropical_tree_workspace_size", "tropical_tree_step_info",
               "tropical_tree_run", "tropical_tree_describe"):
        getattr(L, fn).restype = ctypes.c_int
    # declared argument types: ctypes then converts plain ints (data
    # pointers, sizes) without inspecting each argument's type per call
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.tropical_gemm_strided_batched.argtypes = [ctypes.c_int, ctypes.c_int, vp, trop_strides, vp, trop_strides,
                                                vp, trop_strides, vp, i64, i64, i64, i64, vp]
    _lib = L
    return L


def _check(status, what):
    if status != OK:
        msg = lib().tropical_last_error().decode(errors="replace")
        raise TropicalError(status, f"{what}: {msg}")


def _sr(semiring):
    return SEMIRINGS[semiring] if isinstance(semiring, str) else int(semiring)


def _dt(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.int32:
        return I32
    raise TypeError(f"float32 or int32 tensors only, got {t.dtype}")


# torch's current stream as a raw pointer, without building a Stream object
# per call (the public call below is the fallback)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_ptr(stream, t):
    """Raw stream pointer (int) for a call on tensor t's device."""
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(t.device.index if t.device.index is not None else torch.cuda.current_device())
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _stream(stream):
    if stream is None:
        if _raw_stream is not None:
            return ctypes.c_void_p(_raw_stream(torch.cuda.current_device()))
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _i64(vals):
    return (ctypes.c_int64 * max(1, len(vals)))(*[int(v) for v in vals])


def _i32(vals):
    return (ctypes.c_int32 * max(1, len(vals)))(*[int(v) for v in vals])


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _as3(t):
    return t.unsqueeze(0) if t.dim() == 2 else t


# ---------------------------------------------------------------------------

def tropical_init(device=0):
    _check(lib().tropical_init(int(device)), "tropical_init")


def tropical_gemm_strided_batched(semiring, A, B, C, argmax=None, stream=None):
    """C[b,i,j] = (+)_k A[b,i,k] (x) B[b,k,j] and argmax[b,i,j] = first winning k.

    A: (batch, m, k), B: (batch, k, n), C and argmax: (batch, m, n) views
    (2-d tensors are batch 1).  Any non-negative strides; argmax must share
    C's strides.  Enqueued on `stream` (default: torch's current stream).
    """
    A3, B3, C3 = _as3(A), _as3(B), _as3(C)
    batch, m, k = A3.shape
    n = B3.shape[2]
    a, b, c = A3.stride(), B3.stride(), C3.stride()
    if argmax is not None and _as3(argmax).stride() != c:
        raise ValueError("argmax must have the strides of C")
    st = lib().tropical_gemm_strided_batched(_sr(semiring), _dt(A3), A3.data_ptr(), trop_strides(a[1], a[2], a[0]),
                                             B3.data_ptr(), trop_strides(b[1], b[2], b[0]), C3.data_ptr(),
                                             trop_strides(c[1], c[2], c[0]),
                                             argmax.data_ptr() if argmax is not None else None,
                                             m, n, k, batch, _stream_ptr(stream, A3))
    _check(st, "tropical_gemm_strided_batched")
    return C, argmax


def tropical_gemm_workspace_size(m, n, k, batch=1):
    nb = ctypes.c_size_t(0)
    _check(lib().tropical_gemm_workspace_size(int(m), int(n), int(k), int(batch), ctypes.byref(nb)),
           "tropical_gemm_workspace_size")
    return nb.value


def tropical_gemm_workspace_size_strided(A, B, with_argmax=True):
    """Workspace bytes for tropical_gemm_strided_batched_ws with the shapes
    and strides of the (batch, m, k) and (batch, k, n) tensors A and B."""
    A3, B3 = _as3(A), _as3(B)
    batch, m, k = A3.shape
    n = B3.shape[2]
    sA = trop_strides(A3.stride(1), A3.stride(2), A3.stride(0))
    sB = trop_strides(B3.stride(1), B3.stride(2), B3.stride(0))
    nb = ctypes.c_size_t(0)
    _check(lib().tropical_gemm_workspace_size_strided(sA, sB, 1 if with_argmax else 0, m, n, k, batch,
                                                      ctypes.byref(nb)), "tropical_gemm_workspace_size_strided")
    return nb.value


def tropical_gemm_strided_batched_ws(semiring, A, B, C, argmax=None, workspace=None, stream=None):
    """tropical_gemm_strided_batched with a workspace (split along K when
    the product has few output tiles and a long K; a transposed copy of a
    row-major B for a long-K argmax product).  workspace: None to allocate
    tropical_gemm_workspace_size_strided bytes with torch, or a uint8
    device tensor."""
    A3, B3, C3 = _as3(A), _as3(B), _as3(C)
    batch, m, k = A3.shape
    n = B3.shape[2]
    if argmax is not None and _as3(argmax).stride() != C3.stride():
        raise ValueError("argmax must have the strides of C")
    if workspace is None:
        nb = tropical_gemm_workspace_size_strided(A3, B3, argmax is not None)
        workspace = torch.empty(nb, dtype=torch.uint8, device=A3.device) if nb else None
    sA = trop_strides(A3.stride(1), A3.stride(2), A3.stride(0))
    sB = trop_strides(B3.stride(1), B3.stride(2), B3.stride(0))
    sC = trop_strides(C3.stride(1), C3.stride(2), C3.stride(0))
    st = lib().tropical_gemm_strided_batched_ws(_sr(semiring), _dt(A3), _ptr(A3), sA, _ptr(B3), sB,
                                                _ptr(C3), sC, _ptr(argmax), m, n, k, batch, _ptr(workspace),
                                                workspace.numel() if workspace is not None else 0,
                                                _stream(stream))
    _check(st, "tropical_gemm_strided_batched_ws")
    return C, argmax


def tropical_gemm_backward(semiring, argmax, grad_c, A=None, B=None, k=None, grad_a=True,
                           grad_b=True, stream=None):
    """Gradients of sum(grad_c * C) routed along the forward's argmax.

    argmax (int32) and grad_c (float32): (batch, m, n) with equal strides.
    A (batch, m, k) and B (batch, k, n) are read for max-mul only.  k is the
    contracted size (from A or B when omitted).  grad_a / grad_b: True to
    allocate (float32, contiguous), a tensor to fill, or None to skip.
    Returns (grad_a, grad_b).
    """
    I3, G3 = _as3(argmax), _as3(grad_c)
    if I3.stride() != G3.stride() or I3.shape != G3.shape:
        raise ValueError("argmax and grad_c must share shape and strides")
    batch, m, n = I3.shape
    A3 = _as3(A) if A is not None else None
    B3 = _as3(B) if B is not None else None
    if k is None:
        k = A3.shape[2] if A3 is not None else B3.shape[1]
    dev = I3.device
    if grad_a is True:
        grad_a = torch.empty(batch, m, k, dtype=torch.float32, device=dev)
    if grad_b is True:
        grad_b = torch.empty(batch, k, n, dtype=torch.float32, device=dev)
    ga3 = _as3(grad_a) if grad_a is not None else None
    gb3 = _as3(grad_b) if grad_b is not None else None

    def strides(t):
        return trop_strides(t.stride(1), t.stride(2), t.stride(0)) if t is not None else trop_strides(0, 0, 0)

    dt = _dt(A3) if A3 is not None else (_dt(B3) if B3 is not None else F32)
    st = lib().tropical_gemm_backward(_sr(semiring), dt, _ptr(A3), strides(A3), _ptr(B3), strides(B3),
                                      _ptr(I3), _ptr(G3), strides(I3), _ptr(ga3), strides(ga3),
                                      _ptr(gb3), strides(gb3), m, n, int(k), batch, _stream(stream))
    _check(st, "tropical_gemm_backward")
    return grad_a, grad_b


def tropical_permute(x, perm, out=None, x2=None, out2=None, stream=None):
    """out = x.permute(perm) made contiguous; x2 -> out2 with the same mapping."""
    perm = [int(p) for p in perm]
    shape = [x.shape[p] for p in perm]
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    n = 1
    ins = [x.data_ptr()]
    outs = [out.data_ptr()]
    if x2 is not None:
        if x2.shape != x.shape or x2.stride() != x.stride():
            raise ValueError("x2 must have the shape and strides of x")
        if out2 is None:
            out2 = torch.empty(shape, dtype=x2.dtype, device=x2.device)
        ins.append(x2.data_ptr())
        outs.append(out2.data_ptr())
        n = 2
    in_arr = (ctypes.c_void_p * 2)(*ins, *([0] * (2 - n)))
    out_arr = (ctypes.c_void_p * 2)(*outs, *([0] * (2 - n)))
    st = lib().tropical_permute(x.element_size(), x.dim(), _i64(x.shape), _i64(x.stride()),
                                _i32(perm), n, in_arr, out_arr, _stream(stream))
    _check(st, "tropical_permute")
    return (out, out2) if x2 is not None else out


def _label_ids(labels):
    return [ord(c) if isinstance(c, str) else int(c) for c in labels]


def tropical_diag_gather(semiring, x, in_labels, out_labels, out=None, stream=None):
    """Repeated-label diagonal (and (+)-reduction of labels absent from out)."""
    il, ol = _label_ids(in_labels), _label_ids(out_labels)
    if len(il) != x.dim():
        raise ValueError("one label per input axis")
    ext = {}
    for lab, e in zip(il, x.shape):
        ext.setdefault(lab, e)
    if out is None:
        out = torch.empty([ext.get(lab, 0) for lab in ol], dtype=x.dtype, device=x.device)
    st = lib().tropical_diag_gather(_sr(semiring), _dt(x), x.dim(), _i64(x.shape), _i64(x.stride()),
                                    _i32(il), len(ol), _i32(ol), _ptr(x), _ptr(out),
                                    _stream(stream))
    _check(st, "tropical_diag_gather")
    return out


def tropical_contract_pair_workspace_size(spec, shapeA, shapeB):
    n = ctypes.c_size_t(0)
    st = lib().tropical_contract_pair_workspace_size(spec.encode(), _i64(shapeA), _i64(shapeB),
                                                     ctypes.byref(n))
    _check(st, "tropical_contract_pair_workspace_size")
    return n.value


def tropical_contract_pair_describe(spec, shapeA, shapeB, stridesA=None, stridesB=None):
    buf = ctypes.create_string_buffer(1024)
    st = lib().tropical_contract_pair_describe(
        spec.encode(), _i64(shapeA), _i64(stridesA) if stridesA is not None else None,
        _i64(shapeB), _i64(stridesB) if stridesB is not None else None, buf, len(buf))
    _check(st, "tropical_contract_pair_describe")
    return buf.value.decode()


def _out_shape(spec, A, B):
    lhs, out = spec.replace(" ", "").split("->")
    la, lb = lhs.split(",")
    ext = {}
    for sub, t in ((la, A), (lb, B)):
        for c, e in zip(sub, t.shape):
            ext.setdefault(c, e)
    return [ext.get(c, 0) for c in out]


def tropical_contract_pair(spec, semiring, A, B, C=None, argmax=True, workspace=None, stream=None):
    """Pairwise tropical einsum; returns (C, argmax) (argmax None if not asked).

    argmax=True allocates the int32 argmax; pass a tensor to reuse one, or
    None / False to skip it.  The workspace is allocated with torch when
    not given.
    """
    shape = _out_shape(spec, A, B)
    if C is None:
        C = torch.empty(shape, dtype=A.dtype, device=A.device)
    if argmax is True:
        argmax = torch.empty(shape, dtype=torch.int32, device=A.device)
    elif argmax is False:
        argmax = None
    if workspace is None:
        nbytes = tropical_contract_pair_workspace_size(spec, A.shape, B.shape)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=A.device)
    st = lib().tropical_contract_pair(spec.encode(), _sr(semiring), _dt(A), _ptr(A), _i64(A.shape),
                                      _i64(A.stride()), _ptr(B), _i64(B.shape), _i64(B.stride()),
                                      _ptr(C), _ptr(argmax), _ptr(workspace), workspace.numel(),
                                      _stream(stream))
    _check(st, "tropical_contract_pair")
    return C, argmax


NOALLOC_SCRATCH_BYTES = 32 << 20  # TROP_NOALLOC_SCRATCH_BYTES in include/tropical.h


def tropical_contract_pair_noalloc(spec, semiring, A, B, C, argmax=None, stream=None):
    """Pairwise tropical einsum into the caller's C (and argmax, or None)
    with the library's own scratch: the call allocates nothing, so C (and
    argmax) must be given."""
    st = lib().tropical_contract_pair_noalloc(spec.encode(), _sr(semiring), _dt(A), _ptr(A), _i64(A.shape),
                                              _i64(A.stride()), _ptr(B), _i64(B.shape), _i64(B.stride()),
                                              _ptr(C), _ptr(argmax), _stream(stream))
    _check(st, "tropical_contract_pair_noalloc")
    return C, argmax


class TreePlan:
    """Handle of a planned contraction tree (owns the library's plan)."""

    def __init__(self, handle, n_inputs, n_steps, dtype):
        self.handle = handle
        self.n_inputs = n_inputs
        self.n_steps = n_steps
        self.dtype = dtype

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.tropical_tree_plan_destroy(self.handle)
            self.handle = None


def tropical_tree_plan_create(semiring, dtype, subs, shapes, steps, strides=None):
    """Plan a tree.  subs / shapes: per input; strides: None, or per input
    None (contiguous) or its element strides; steps: (lhs_slot, rhs_slot,
    out_subscript) with slots 0..n-1 the inputs and n + s step s's result.
    dtype: torch.float32 or torch.int32."""
    n, m = len(subs), len(steps)
    dt = F32 if dtype == torch.float32 else (I32 if dtype == torch.int32 else None)
    if dt is None:
        raise TypeError(f"float32 or int32 only, got {dtype}")
    sub_arr = (ctypes.c_char_p * n)(*[x.encode() for x in subs])
    shape_keep = [_i64(sh) for sh in shapes]
    I64P = ctypes.POINTER(ctypes.c_int64)
    shape_arr = (I64P * n)(*[ctypes.cast(a, I64P) for a in shape_keep])
    stride_arr = None
    if strides is not None:
        stride_keep = [_i64(st) if st is not None else None for st in strides]
        stride_arr = (I64P * n)(*[ctypes.cast(a, I64P) if a is not None else I64P() for a in stride_keep])
    out_keep = [o.encode() for _, _, o in steps]
    step_arr = (trop_tree_step * m)(*[trop_tree_step(int(a), int(b), o) for (a, b, _), o in zip(steps, out_keep)])
    h = ctypes.c_void_p(0)
    st = lib().tropical_tree_plan_create(_sr(semiring), dt, n, sub_arr, shape_arr, stride_arr, m, step_arr,
                                         ctypes.byref(h))
    _check(st, "tropical_tree_plan_create")
    return TreePlan(h.value, n, m, dtype)


def tropical_tree_plan_destroy(plan):
    if plan.handle:
        lib().tropical_tree_plan_destroy(plan.handle)
        plan.handle = None


def tropical_tree_workspace_size(plan):
    n = ctypes.c_size_t(0)
    _check(lib().tropical_tree_workspace_size(plan.handle, ctypes.byref(n)), "tropical_tree_workspace_size")
    return n.value


def tropical_tree_step_info(plan, step):
    """(subscript, shape) of step `step`'s output."""
    sub = ctypes.create_string_buffer(16)
    shape = (ctypes.c_int64 * 8)()
    _check(lib().tropical_tree_step_info(plan.handle, int(step), sub, shape, None), "tropical_tree_step_info")
    s = sub.value.decode()
    return s, [shape[d] for d in range(len(s))]


def tropical_tree_describe(plan):
    buf = ctypes.create_string_buffer(64 * 1024)
    _check(lib().tropical_tree_describe(plan.handle, buf, len(buf)), "tropical_tree_describe")
    return buf.value.decode()


def tropical_tree_run(plan, inputs, out=None, argmax=False, workspace=None, stream=None):
    """Run a planned tree; returns (out, [argmax of each step or None]).

    argmax: False (none), True (every step) or one flag / tensor / None per
    step; requested ones are allocated as contiguous int32 tensors.  The
    workspace is allocated with torch when not given.
    """
    if len(inputs) != plan.n_inputs:
        raise ValueError(f"the plan has {plan.n_inputs} inputs")
    dev = inputs[0].device
    if out is None:
        _, shape = tropical_tree_step_info(plan, plan.n_steps - 1)
        out = torch.empty(shape, dtype=plan.dtype, device=dev)
    flags = [argmax] * plan.n_steps if isinstance(argmax, bool) else list(argmax)
    if len(flags) != plan.n_steps:
        raise ValueError("one argmax entry per step")
    ams = []
    for s, f in enumerate(flags):
        if f is True:
            ams.append(torch.empty(tropical_tree_step_info(plan, s)[1], dtype=torch.int32, device=dev))
        elif f is False or f is None:
            ams.append(None)
        else:
            ams.append(f)
    if workspace is None:
        workspace = torch.empty(max(tropical_tree_workspace_size(plan), 1), dtype=torch.uint8, device=dev)
    in_arr = (ctypes.c_void_p * len(inputs))(*[t.data_ptr() for t in inputs])
    am_arr = (ctypes.c_void_p * plan.n_steps)(*[a.data_ptr() if a is not None else 0 for a in ams])
    st = lib().tropical_tree_run(plan.handle, in_arr, _ptr(out), am_arr, _ptr(workspace), workspace.numel(),
                                 _stream(stream))
    _check(st, "tropical_tree_run")
    return out, ams


def tropical_get_stats():
    s = trop_stats()
    _check(lib().tropical_get_stats(ctypes.byref(s)), "tropical_get_stats")
    return {"module_loads": s.module_loads, "launches_total": s.launches_total,
            "launches": {name: s.launches[i] for i, name in enumerate(KERNEL_FAMILIES)}}


def tropical_reset_stats():
    lib().tropical_reset_stats()


def tropical_last_error():
    return lib().tropical_last_error().decode(errors="replace")
