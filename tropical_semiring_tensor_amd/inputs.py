"""Seeded synthetic inputs for the five tropical workloads.

This module holds no tropical arithmetic: it only draws random tensors on
the CPU (so both the HIP path and the CPU oracle see identical bits) with
the shapes, layouts and value distributions of the workloads below.  Every
draw uses ``torch.Generator('cpu').manual_seed(20261202 + workload)``.

Workloads (sizes as used by the benchmark and the parity tests):
  1  max-plus f32, batch 1, 64x64x64, integer values in [-8, 8] (tie-heavy)
  2  max-plus f32, batch 64, 256x256x256, N(0, 1), contiguous batches
  3  min-plus i32, 4096x4096x4096, U{1..1000} with 20% of entries 2^30
  4  max-mul f32, batch 16, 2048^3, U(0, 1], B column-major
  5  max-plus f32 einsum 'iijb,kjb->bki', A (128,128,256,32) N(0,1),
     B (256,256,32) U[-1, 1]
  6  a square-lattice tropical network (one tensor per site, one label per
     bond) contracted site by site down to a scalar; see grid_network
"""
import string

import torch

SEED_BASE = 20261202
I32_INF = 1 << 30

WORKLOADS = {
    1: dict(name="maxplus_f32_b1_64", semiring="max_plus", dtype="f32",
            batch=1, m=64, n=64, k=64),
    2: dict(name="maxplus_f32_b64_256", semiring="max_plus", dtype="f32",
            batch=64, m=256, n=256, k=256),
    3: dict(name="minplus_i32_b1_4096", semiring="min_plus", dtype="i32",
            batch=1, m=4096, n=4096, k=4096),
    4: dict(name="maxmul_f32_b16_2048_colB", semiring="max_mul", dtype="f32",
            batch=16, m=2048, n=2048, k=2048),
    5: dict(name="einsum_iijb_kjb_bki_f32", semiring="max_plus", dtype="f32",
            spec="iijb,kjb->bki", shape_a=(128, 128, 256, 32), shape_b=(256, 256, 32)),
}


def generator(workload, salt=0):
    g = torch.Generator(device="cpu")
    g.manual_seed(SEED_BASE + workload + 1000 * salt)
    return g


def int_uniform_f32(shape, lo, hi, g):
    """Integer values in [lo, hi] stored as float32."""
    return torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int32).to(torch.float32)


def normal_f32(shape, g):
    return torch.randn(shape, generator=g, dtype=torch.float32)


def unit_open_closed_f32(shape, g):
    """U(0, 1]: one minus torch's U[0, 1) draw (a multiple of 2^-24, so exact)."""
    return 1.0 - torch.rand(shape, generator=g, dtype=torch.float32)


def symmetric_unit_f32(shape, g):
    """U[-1, 1): 2 * U[0, 1) - 1."""
    return 2.0 * torch.rand(shape, generator=g, dtype=torch.float32) - 1.0


def sparse_inf_i32(shape, g, lo=1, hi=1000, p_inf=0.2, inf=I32_INF):
    """Integers uniform on [lo, hi]; each entry independently replaced by
    `inf` with probability p_inf."""
    x = torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int32)
    mask = torch.rand(shape, generator=g) < p_inf
    x[mask] = inf
    return x


def gemm_operands(workload, batch=None, m=None, n=None, k=None, salt=0):
    """(A, B) on the CPU for GEMM workloads 1-4, optionally at other sizes.

    A is (batch, m, k) row-major.  B is (batch, k, n); for workload 4 it is
    a column-major view (the storage is (batch, n, k) contiguous).
    """
    w = WORKLOADS[workload]
    batch = w["batch"] if batch is None else batch
    m = w["m"] if m is None else m
    n = w["n"] if n is None else n
    k = w["k"] if k is None else k
    g = generator(workload, salt)
    if workload == 1:
        A = int_uniform_f32((batch, m, k), -8, 8, g)
        B = int_uniform_f32((batch, k, n), -8, 8, g)
    elif workload == 2:
        A = normal_f32((batch, m, k), g)
        B = normal_f32((batch, k, n), g)
    elif workload == 3:
        A = sparse_inf_i32((batch, m, k), g)
        B = sparse_inf_i32((batch, k, n), g)
    elif workload == 4:
        A = unit_open_closed_f32((batch, m, k), g)
        B = unit_open_closed_f32((batch, n, k), g).transpose(1, 2)
    else:
        raise ValueError(f"workload {workload} is not a plain GEMM")
    return A, B


def einsum_operands(shape_a=None, shape_b=None, salt=0):
    """(A, B) on the CPU for workload 5, optionally at other sizes."""
    w = WORKLOADS[5]
    shape_a = w["shape_a"] if shape_a is None else shape_a
    shape_b = w["shape_b"] if shape_b is None else shape_b
    g = generator(5, salt)
    A = normal_f32(shape_a, g)
    B = symmetric_unit_f32(shape_b, g)
    return A, B


def random_points(batch, m, n, count, salt=0, edges=True):
    """(count, 3) int64 array of (b, i, j) output coordinates, plus the
    corners of every batch's matrix when `edges` is set."""
    g = generator(99, salt)
    b = torch.randint(0, batch, (count,), generator=g)
    i = torch.randint(0, m, (count,), generator=g)
    j = torch.randint(0, n, (count,), generator=g)
    pts = torch.stack([b, i, j], dim=1)
    if edges:
        extra = []
        for bb in sorted({0, batch - 1}):
            for ii in sorted({0, m - 1}):
                for jj in sorted({0, n - 1}):
                    extra.append((bb, ii, jj))
        pts = torch.cat([pts, torch.tensor(extra, dtype=torch.int64)], dim=0)
    return pts.to(torch.int64)


LABELS = string.ascii_lowercase + string.ascii_uppercase


def grid_network(rows, cols, bond, salt=0, integer=None):
    """A rows x cols square-lattice tensor network: the tensor of site (r, c)
    has one axis per bond at that site, in the order up, left, down, right
    (those that exist), every bond has extent `bond` and its own label, and
    entries are N(0, 1) float32 (or integers uniform on [-integer, integer]
    stored as float32 when `integer` is given).

    The contraction order sweeps the sites row by row: step t joins the
    running result with site t + 1.  A step keeps the labels that are still
    shared with later sites (every bond belongs to exactly two sites, so
    these are the labels found in one of the two operands only), the running
    result's first, in its order, then the new site's.  The last step leaves
    no label: a scalar.

    Returns dict(subs, shapes, tensors, steps) with steps as
    (lhs_slot, rhs_slot, out_subscript); slots 0..n-1 are the sites in
    row-major order and slot n + s is the result of step s.
    """
    nh, nv = rows * (cols - 1), (rows - 1) * cols
    if rows * cols < 2:
        raise ValueError("a network needs at least two sites")
    if nh + nv > len(LABELS):
        raise ValueError("more bonds than single-letter labels")

    def hb(r, c):  # bond between (r, c) and (r, c + 1)
        return LABELS[r * (cols - 1) + c]

    def vb(r, c):  # bond between (r, c) and (r + 1, c)
        return LABELS[nh + r * cols + c]

    subs = []
    for r in range(rows):
        for c in range(cols):
            s = ""
            if r > 0:
                s += vb(r - 1, c)
            if c > 0:
                s += hb(r, c - 1)
            if r < rows - 1:
                s += vb(r, c)
            if c < cols - 1:
                s += hb(r, c)
            subs.append(s)
    g = generator(6, salt)
    shapes = [tuple([bond] * len(s)) for s in subs]
    if integer is None:
        tensors = [normal_f32(sh, g) for sh in shapes]
    else:
        tensors = [int_uniform_f32(sh, -integer, integer, g) for sh in shapes]
    n = len(subs)
    steps = []
    cur, cur_sub = 0, subs[0]
    for t in range(1, n):
        new = subs[t]
        out = "".join([c for c in cur_sub if c not in new] + [c for c in new if c not in cur_sub])
        steps.append((cur, t, out))
        cur, cur_sub = n + len(steps) - 1, out
    return dict(subs=subs, shapes=shapes, tensors=tensors, steps=steps)
