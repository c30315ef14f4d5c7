"""CPU oracle for the tropical contraction hot path.

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only ``tests/``, the package's
``smoke()`` check and the benchmark's ``cpu_baseline`` leg may import it.
The HIP library and its Python binding never import, load or call anything
here, and nothing here imports them.

The arithmetic lives in ``tropical_oracle.c`` (plain loops, see its header
for the semiring definitions and the sources they follow).  This module
only marshals numpy arrays into that library and, in ``contract.py``,
plans a pairwise einsum the way omeinsum-rs issue #52 ("GPU tropical path:
keep tensors device-resident + device-side permute", section "Resolved
design for step 3") describes it: a diagonal/trace unary pre-pass, a
permute into canonical operand order, one batched tropical GEMM, and a
permute of the value and the argmax into the output order; a contraction
tree is a sequence of such pairwise steps whose results feed later steps.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(hand-worked examples, library routines, algebraic identities, a textbook
shortest-path algorithm, brute force over every label assignment of small
networks, and the routing of each tree's argmax back to its inputs); none
is "parity unpinned".
"""
import ctypes
import os

import numpy as np

from . import build as _build

MAX_PLUS, MIN_PLUS, MAX_MUL = 0, 1, 2
F32, I32 = 0, 1
I32_INF = 1 << 30

SEMIRINGS = {"max_plus": MAX_PLUS, "min_plus": MIN_PLUS, "max_mul": MAX_MUL}
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported"}

_I64P = ctypes.POINTER(ctypes.c_int64)
_I32P = ctypes.POINTER(ctypes.c_int32)


class OracleError(RuntimeError):
    pass


def _dt_code(arr):
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.int32:
        return I32
    raise TypeError(f"oracle handles float32 and int32 only, got {arr.dtype}")


def _sr_code(sr):
    if isinstance(sr, str):
        return SEMIRINGS[sr]
    return int(sr)


def _elem_strides(arr):
    if any(s < 0 for s in arr.strides):
        raise ValueError("negative strides are not supported")
    return [s // arr.itemsize for s in arr.strides]


def _i64(vals):
    return (ctypes.c_int64 * max(1, len(vals)))(*vals)


def _i32(vals):
    return (ctypes.c_int32 * max(1, len(vals)))(*vals)


def _ptr(arr):
    return ctypes.c_void_p(arr.ctypes.data)


class Oracle:
    """ctypes handle on one build of ``tropical_oracle.c``."""

    def __init__(self, lib_path=None):
        if lib_path is None:
            lib_path = _build.LIB
            # (re)build when missing or older than its source
            if not os.path.exists(lib_path) or os.path.getmtime(_build.SRC) > os.path.getmtime(lib_path):
                _build.build()
        self.path = lib_path
        self.lib = ctypes.CDLL(lib_path)
        L = self.lib
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_gemm.argtypes = [i32, i32, vp, _I64P, vp, _I64P, vp, _I64P, _I32P,
                               i64, i64, i64, i64]
        L.orc_gemm_points.argtypes = [i32, i32, vp, _I64P, vp, _I64P, i64, _I64P, i64,
                                      vp, _I32P]
        L.orc_permute.argtypes = [i32, i32, _I64P, _I64P, _I32P, vp, vp]
        L.orc_diag_gather.argtypes = [i32, i32, i32, _I64P, _I64P, _I32P, i32, _I32P,
                                      vp, vp, _I32P]
        L.orc_einsum_brute.argtypes = [i32, i32, i32, _I64P,
                                       i32, _I32P, _I64P, vp,
                                       i32, _I32P, _I64P, vp,
                                       i32, _I32P, vp, _I32P,
                                       i32, _I32P]
        L.orc_gemm_backward.argtypes = [i32, vp, _I64P, vp, _I64P, _I32P, vp, _I64P,
                                        vp, _I64P, vp, _I64P, i64, i64, i64, i64]
        L.orc_max_threads.restype = ctypes.c_int
        L.orc_set_threads.argtypes = [ctypes.c_int]
        for fn in ("orc_gemm", "orc_gemm_points", "orc_permute", "orc_diag_gather",
                   "orc_einsum_brute", "orc_gemm_backward"):
            getattr(L, fn).restype = ctypes.c_int

    @staticmethod
    def _check(st, what):
        if st != 0:
            raise OracleError(f"{what}: {_STATUS.get(st, st)}")

    # -- threads --------------------------------------------------------
    def max_threads(self):
        return self.lib.orc_max_threads()

    def set_threads(self, n):
        self.lib.orc_set_threads(int(n))

    # -- GEMM -------------------------------------------------------------
    def gemm(self, sr, A, B, argmax=True):
        """Batched tropical product of A (batch, m, k) and B (batch, k, n).

        A and B may be any non-negatively strided views (2-d inputs are
        taken as batch 1).  Returns (C, argmax) as contiguous arrays of
        shape (batch, m, n); argmax is int32 (None if not requested).
        """
        A = np.asarray(A)
        B = np.asarray(B)
        if A.ndim == 2:
            A = A[None]
        if B.ndim == 2:
            B = B[None]
        if A.dtype != B.dtype:
            raise TypeError("A and B must have the same dtype")
        batch, m, k = A.shape
        if B.shape[0] != batch or B.shape[1] != k:
            raise ValueError(f"shape mismatch {A.shape} x {B.shape}")
        n = B.shape[2]
        C = np.empty((batch, m, n), dtype=A.dtype)
        idx = np.empty((batch, m, n), dtype=np.int32) if argmax else None
        sa, sb = _elem_strides(A), _elem_strides(B)
        sA = _i64([sa[1], sa[2], sa[0]])
        sB = _i64([sb[1], sb[2], sb[0]])
        sC = _i64([n, 1, m * n])
        st = self.lib.orc_gemm(_sr_code(sr), _dt_code(A), _ptr(A), sA, _ptr(B), sB,
                               _ptr(C), sC,
                               idx.ctypes.data_as(_I32P) if idx is not None else None,
                               m, n, k, batch)
        self._check(st, "orc_gemm")
        return C, idx

    def gemm_points(self, sr, A, B, points):
        """Values and argmax of the product at the (b, i, j) rows of `points`."""
        A = np.asarray(A)
        B = np.asarray(B)
        if A.ndim == 2:
            A = A[None]
        if B.ndim == 2:
            B = B[None]
        pts = np.ascontiguousarray(points, dtype=np.int64).reshape(-1, 3)
        k = A.shape[2]
        sa, sb = _elem_strides(A), _elem_strides(B)
        vals = np.empty(len(pts), dtype=A.dtype)
        args = np.empty(len(pts), dtype=np.int32)
        st = self.lib.orc_gemm_points(_sr_code(sr), _dt_code(A), _ptr(A),
                                      _i64([sa[1], sa[2], sa[0]]), _ptr(B),
                                      _i64([sb[1], sb[2], sb[0]]), k,
                                      pts.ctypes.data_as(_I64P), len(pts),
                                      _ptr(vals), args.ctypes.data_as(_I32P))
        self._check(st, "orc_gemm_points")
        return vals, args

    def gemm_backward(self, sr, argmax, G, A=None, B=None, k=None, grad_a=True, grad_b=True):
        """Gradients routed along the argmax (winner routing).

        argmax and G are (batch, m, n) (int32 / float32, same strides); A
        (batch, m, k) and B (batch, k, n) are float32 and needed for max-mul
        only.  k is the contracted size (taken from A or B when omitted).
        Returns (dA (batch, m, k), dB (batch, k, n)) as float32, each None
        if not requested.
        """
        argmax = np.asarray(argmax)
        G = np.asarray(G)
        if argmax.ndim == 2:
            argmax, G = argmax[None], G[None]
        if argmax.dtype != np.int32 or G.dtype != np.float32 or argmax.shape != G.shape:
            raise TypeError("argmax must be int32 and G float32 of one shape")
        if _elem_strides(argmax) != _elem_strides(G):
            G = np.ascontiguousarray(G)
            argmax = np.ascontiguousarray(argmax)
        batch, m, n = argmax.shape
        A = None if A is None else np.asarray(A, dtype=np.float32)
        B = None if B is None else np.asarray(B, dtype=np.float32)
        if A is not None and A.ndim == 2:
            A = A[None]
        if B is not None and B.ndim == 2:
            B = B[None]
        if k is None:
            k = A.shape[2] if A is not None else B.shape[1]
        sc = _elem_strides(argmax)
        sa = _elem_strides(A) if A is not None else [0, 0, 0]
        sb = _elem_strides(B) if B is not None else [0, 0, 0]
        dA = np.empty((batch, m, k), dtype=np.float32) if grad_a else None
        dB = np.empty((batch, k, n), dtype=np.float32) if grad_b else None
        sda = _elem_strides(dA) if grad_a else [0, 0, 0]
        sdb = _elem_strides(dB) if grad_b else [0, 0, 0]
        nul = ctypes.c_void_p(0)
        st = self.lib.orc_gemm_backward(
            _sr_code(sr), _ptr(A) if A is not None else nul, _i64([sa[1], sa[2], sa[0]]),
            _ptr(B) if B is not None else nul, _i64([sb[1], sb[2], sb[0]]),
            argmax.ctypes.data_as(_I32P), _ptr(G), _i64([sc[1], sc[2], sc[0]]),
            _ptr(dA) if grad_a else nul, _i64([sda[1], sda[2], sda[0]]),
            _ptr(dB) if grad_b else nul, _i64([sdb[1], sdb[2], sdb[0]]), m, n, k, batch)
        self._check(st, "orc_gemm_backward")
        return dA, dB

    # -- permute ----------------------------------------------------------
    def permute(self, x, perm):
        """Contiguous copy of x with its axes reordered: out axis d = x axis perm[d]."""
        x = np.asarray(x)
        perm = [int(p) for p in perm]
        out = np.empty([x.shape[p] for p in perm], dtype=x.dtype)
        st = self.lib.orc_permute(x.itemsize, x.ndim, _i64(list(x.shape)),
                                  _i64(_elem_strides(x)), _i32(perm), _ptr(x), _ptr(out))
        self._check(st, "orc_permute")
        return out

    # -- diagonal / trace ----------------------------------------------------
    def diag_gather(self, sr, x, in_labels, out_labels, argmax=False):
        """Repeated-label diagonal with (+)-reduction of labels absent from out.

        Labels are strings of single characters (or int sequences).  With
        argmax, also returns the reduction's winner per output: the
        row-major position over the reduced labels (in order of first
        appearance) of the first strictly better value, 0 if none.
        """
        x = np.asarray(x)
        ids = {}
        def lid(c):
            return ids.setdefault(c, len(ids))
        il = [lid(c) for c in in_labels]
        if len(il) != x.ndim:
            raise ValueError("one label per input axis")
        ext = {}
        for c, e in zip(in_labels, x.shape):
            ext.setdefault(c, e)
        ol = []
        for c in out_labels:
            if c not in ids:
                raise OracleError("orc_diag_gather: invalid argument")
            ol.append(ids[c])
        out = np.empty([ext[c] for c in out_labels], dtype=x.dtype)
        arg = np.empty(out.shape, dtype=np.int32) if argmax else None
        st = self.lib.orc_diag_gather(_sr_code(sr), _dt_code(x), x.ndim, _i64(list(x.shape)),
                                      _i64(_elem_strides(x)), _i32(il), len(ol), _i32(ol),
                                      _ptr(x), _ptr(out),
                                      arg.ctypes.data_as(_I32P) if argmax else None)
        self._check(st, "orc_diag_gather")
        return (out, arg) if argmax else out

    # -- brute-force einsum -------------------------------------------------
    def einsum_brute(self, sr, spec, A, B, sum_order=None, argmax=True):
        """Evaluate `spec` by enumerating every assignment of the summed labels.

        Summed labels default to: labels of A absent from the output, in A
        order, then labels of B absent from both, in B order.  The argmax
        is the row-major position in that enumeration.
        """
        A = np.asarray(A)
        B = np.asarray(B)
        lhs, out = spec.replace(" ", "").split("->")
        la, lb = lhs.split(",")
        labels = []
        for c in la + lb + out:
            if c not in labels:
                labels.append(c)
        ids = {c: n for n, c in enumerate(labels)}
        ext = [0] * len(labels)
        seen = [False] * len(labels)
        for sub, arr in ((la, A), (lb, B)):
            if len(sub) != arr.ndim:
                raise ValueError("subscript rank mismatch")
            for c, e in zip(sub, arr.shape):
                if seen[ids[c]] and ext[ids[c]] != e:
                    raise ValueError(f"extent mismatch for label {c}")
                ext[ids[c]] = e
                seen[ids[c]] = True
        if sum_order is None:
            sum_order = []
            for c in la + lb:
                if c not in out and c not in sum_order:
                    sum_order.append(c)
        C = np.empty([ext[ids[c]] for c in out], dtype=A.dtype)
        idx = np.empty(C.shape, dtype=np.int32) if argmax else None
        st = self.lib.orc_einsum_brute(
            _sr_code(sr), _dt_code(A), len(labels), _i64(ext),
            A.ndim, _i32([ids[c] for c in la]), _i64(_elem_strides(A)), _ptr(A),
            B.ndim, _i32([ids[c] for c in lb]), _i64(_elem_strides(B)), _ptr(B),
            len(out), _i32([ids[c] for c in out]), _ptr(C),
            idx.ctypes.data_as(_I32P) if idx is not None else None,
            len(sum_order), _i32([ids[c] for c in sum_order]))
        self._check(st, "orc_einsum_brute")
        return C, idx

    # -- decomposed pairwise contraction --------------------------------------
    def contract_pair(self, spec, sr, A, B, argmax=True):
        from .contract import contract_pair
        return contract_pair(self, spec, sr, A, B, argmax=argmax)

    def contract_tree(self, sr, inputs, subs, steps, argmax=True):
        from .contract import contract_tree
        return contract_tree(self, sr, inputs, subs, steps, argmax=argmax)


_default = None


def default():
    """The oracle built from this directory's source (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
