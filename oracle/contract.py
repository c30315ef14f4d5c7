"""Decomposed pairwise tropical einsum, the oracle's version.

TEST INFRASTRUCTURE (see the package docstring).

Follows the pipeline of omeinsum-rs issue #52 ("GPU tropical path: keep
tensors device-resident + device-side permute"), section "Resolved design
for step 3" and its "Structural lessons from OMEinsum": repeated labels are
removed by a separate unary pre-pass (diagonal, or a (+)-reduction for a
label that appears in one operand only), the operands are permuted into
canonical order, one batched tropical GEMM runs, and its value and argmax
are permuted into the output order with one and the same index mapping.

Canonical orders (row-major):
    A'' = (batch..., left..., contracted...)
    B'' = (batch..., contracted..., right...)
    C'' = (batch..., left..., right...)
batch / left / right labels are taken in output order, contracted labels in
the order they first appear in A's subscript.  The argmax is therefore the
row-major linear index over the contracted labels in A-subscript order.

When a pre-pass reduces labels found in one operand only, its winners are
kept and the argmax covers them too: the row-major linear index over the
contracted labels (A order), then A's reduced labels (A order), then B's
(B order) -- the product's winning k, then the pre-pass winner of A at
that k, then B's.  The contracted labels lead because the product's k is
chosen first; the pre-pass winners are the ones that produced the values
the product compared.
"""
import numpy as np

from . import OracleError


def parse(spec):
    spec = spec.replace(" ", "")
    if spec.count("->") != 1:
        raise OracleError("spec needs exactly one '->'")
    lhs, out = spec.split("->")
    if lhs.count(",") != 1:
        raise OracleError("spec needs exactly two operands")
    la, lb = lhs.split(",")
    for c in la + lb + out:
        if not c.isalpha() or not c.isascii():
            raise OracleError(f"bad label {c!r}")
    if len(set(out)) != len(out):
        raise OracleError("repeated output label")
    for c in out:
        if c not in la and c not in lb:
            raise OracleError(f"output label {c!r} appears in no operand")
    return la, lb, out


def _unique(s):
    seen = []
    for c in s:
        if c not in seen:
            seen.append(c)
    return seen


def roles(la, lb, out):
    batch = [c for c in out if c in la and c in lb]
    left = [c for c in out if c in la and c not in lb]
    right = [c for c in out if c in lb and c not in la]
    contracted = [c for c in _unique(la) if c in lb and c not in out]
    a_reduce = [c for c in _unique(la) if c not in lb and c not in out]
    b_reduce = [c for c in _unique(lb) if c not in la and c not in out]
    return batch, left, right, contracted, a_reduce, b_reduce


def _prepare(orc, sr, x, sub, reduce_labels, canonical, winners=False):
    """Unary pre-pass (diagonal / trace), then permute to `canonical`; with
    `winners`, also the pre-pass reduction's winner index, permuted alike."""
    kept = [c for c in _unique(sub) if c not in reduce_labels]
    perm = [kept.index(c) for c in canonical]
    if winners:
        y, w = orc.diag_gather(sr, x, sub, "".join(kept), argmax=True)
        return orc.permute(y, perm), orc.permute(w, perm)
    y = orc.diag_gather(sr, x, sub, "".join(kept))
    return orc.permute(y, perm)


def prod_of(labels, ext):
    p = 1
    for c in labels:
        p *= ext[c]
    return p


def contract_pair(orc, spec, sr, A, B, argmax=True):
    A = np.asarray(A)
    B = np.asarray(B)
    la, lb, out = parse(spec)
    if len(la) != A.ndim or len(lb) != B.ndim:
        raise OracleError("subscript rank mismatch")
    ext = {}
    for sub, arr in ((la, A), (lb, B)):
        for c, e in zip(sub, arr.shape):
            if c in ext and ext[c] != e:
                raise OracleError(f"extent mismatch for label {c!r}")
            ext[c] = e
    batch, left, right, contracted, a_red, b_red = roles(la, lb, out)
    # (with K = 0 nothing wins anywhere: every index, routed or not, is 0)
    route = argmax and bool(a_red or b_red) and prod_of(contracted, ext) > 0

    def prod(labels):
        p = 1
        for c in labels:
            p *= ext[c]
        return p

    nb, m, n, k = prod(batch), prod(left), prod(right), prod(contracted)
    if route:
        A2, WA = _prepare(orc, sr, A, la, a_red, batch + left + contracted, winners=True)
        B2, WB = _prepare(orc, sr, B, lb, b_red, batch + contracted + right, winners=True)
    else:
        A2 = _prepare(orc, sr, A, la, a_red, batch + left + contracted)
        B2 = _prepare(orc, sr, B, lb, b_red, batch + contracted + right)
    C2, I2 = orc.gemm(sr, A2.reshape(nb, m, k), B2.reshape(nb, k, n), argmax=argmax)
    if route:
        # the product's k, then the pre-pass winners at that k
        ra, rb = prod(a_red), prod(b_red)
        bi, ii, jj = np.meshgrid(np.arange(nb), np.arange(m), np.arange(n), indexing="ij")
        wa = WA.reshape(nb, m, k)[bi, ii, I2].astype(np.int64)
        wb = WB.reshape(nb, k, n)[bi, I2, jj].astype(np.int64)
        full = I2.astype(np.int64) * (ra * rb) + wa * rb + wb
        if full.size and full.max() >= 2 ** 31:
            raise OracleError("argmax index does not fit int32")
        I2 = full.astype(np.int32)

    canon = batch + left + right
    shape = [ext[c] for c in canon]
    perm = [canon.index(c) for c in out]
    C = orc.permute(C2.reshape(shape), perm)
    I = orc.permute(I2.reshape(shape), perm) if argmax else None
    return C, I


def contract_tree(orc, sr, inputs, subs, steps, argmax=True):
    """A contraction tree evaluated one pairwise step at a time.

    omeinsum-rs issue #52 asks for the pairwise path to run "across the
    contraction tree" with every intermediate kept where it was made
    ("Acceptance criteria"); this is that tree, on the CPU.  Tensor slots
    are numbered inputs first (0 .. n-1), then the result of step s as slot
    n + s.  Step s is ``(lhs, rhs, out)``: the pairwise contraction
    ``subs[lhs],subs[rhs]->out`` of two earlier slots, done by
    ``contract_pair`` above.  The last step's result is the tree's result.

    ``argmax``: True / False for every step, or one flag per step.
    Returns (result, [argmax of each step or None]).
    """
    if len(inputs) != len(subs):
        raise OracleError("one subscript per input")
    if not steps:
        raise OracleError("a tree needs at least one step")
    flags = [bool(argmax)] * len(steps) if isinstance(argmax, bool) else [bool(f) for f in argmax]
    if len(flags) != len(steps):
        raise OracleError("one argmax flag per step")
    slots = [(sub, np.asarray(x)) for sub, x in zip(subs, inputs)]
    winners = []
    for s, (lhs, rhs, out) in enumerate(steps):
        if not (0 <= lhs < len(slots) and 0 <= rhs < len(slots)):
            raise OracleError(f"step {s} names a slot that does not exist yet")
        la, A = slots[lhs]
        lb, B = slots[rhs]
        C, I = contract_pair(orc, f"{la},{lb}->{out}", sr, A, B, argmax=flags[s])
        slots.append((out, C))
        winners.append(I)
    return slots[-1][1], winners
