"""Parity of the HIP permute and diagonal / trace gather with the CPU oracle
(bit-exact), through every kernel path (copy, tiled, runs, flat, naive,
reduce)."""
import itertools

import numpy as np
import pytest
import torch

from gpu_util import DEV, assert_bits_equal, assert_equal, device_copy
from tropical_semiring_tensor_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    from tropical_semiring_tensor_amd import binding
    binding.tropical_init(0)
    return binding


def launches(tb):
    return dict(tb.tropical_get_stats()["launches"])


def delta(before, after):
    return {k: after[k] - before[k] for k in after if after[k] != before[k]}


SHAPES = [(7,), (5, 9), (64, 64), (65, 130), (3, 1, 70, 2), (2, 3, 4, 5, 6), (33, 2, 65),
          (4, 1, 1, 9, 2, 3)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_permute_all_perms(tb, orc, shape):
    g = torch.Generator().manual_seed(len(shape) * 100 + shape[0])
    x = torch.randn(shape, generator=g)
    xd = x.to(DEV)
    perms = list(itertools.permutations(range(len(shape))))
    if len(perms) > 40:
        perms = perms[:: len(perms) // 40]
    for p in perms:
        out = tb.tropical_permute(xd, p)
        torch.cuda.synchronize()
        assert_bits_equal(out.cpu().numpy(), orc.permute(x.numpy(), p), f"permute {shape} {p}")


def test_permute_paths_and_pairs(tb, orc):
    g = torch.Generator().manual_seed(3)
    x = torch.randn(6, 70, 130, generator=g)
    idx = torch.randint(0, 1000, (6, 70, 130), generator=g, dtype=torch.int32)
    xd, idd = x.to(DEV), idx.to(DEV)
    cases = {(0, 1, 2): "gather_copy", (1, 0, 2): "gather_copy", (0, 2, 1): "gather_tiled",
             (2, 1, 0): "gather_tiled"}
    for p, path in cases.items():
        before = launches(tb)
        out, out2 = tb.tropical_permute(xd, p, x2=idd)
        torch.cuda.synchronize()
        assert delta(before, launches(tb)) == {path: 1}, (p, delta(before, launches(tb)))
        assert_bits_equal(out.cpu().numpy(), orc.permute(x.numpy(), p), f"pair value {p}")
        assert_equal(out2.cpu().numpy(), orc.permute(idx.numpy(), p), f"pair index {p}")


def test_permute_strided_input_and_naive(tb, orc, monkeypatch):
    g = torch.Generator().manual_seed(4)
    base = torch.randn(10, 90, 80, generator=g)
    view = base[1:9:2, 3:80:3, ::2]     # no unit stride: naive path
    vd = device_copy(view)
    before = launches(tb)
    out = tb.tropical_permute(vd, (2, 0, 1))
    torch.cuda.synchronize()
    assert delta(before, launches(tb)) == {"gather_naive": 1}
    assert_bits_equal(out.cpu().numpy(), orc.permute(view.numpy(), (2, 0, 1)), "strided naive")
    # unaligned copy path
    v2 = base[:, 1:, 1:]
    out = tb.tropical_permute(device_copy(v2), (1, 0, 2))
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), orc.permute(v2.numpy(), (1, 0, 2)), "unaligned copy")
    # the forced naive path gives the same bits
    x = torch.randn(5, 66, 70, generator=g)
    monkeypatch.setenv("TROPICAL_FORCE_NAIVE_PERMUTE", "1")
    before = launches(tb)
    out = tb.tropical_permute(x.to(DEV), (2, 1, 0))
    torch.cuda.synchronize()
    assert delta(before, launches(tb)) == {"gather_naive": 1}
    assert_bits_equal(out.cpu().numpy(), orc.permute(x.numpy(), (2, 1, 0)), "forced naive")


def test_permute_int32_and_scalar(tb, orc):
    x = torch.arange(2 * 3 * 4, dtype=torch.int32).reshape(2, 3, 4)
    out = tb.tropical_permute(x.to(DEV), (2, 0, 1))
    torch.cuda.synchronize()
    assert_equal(out.cpu().numpy(), orc.permute(x.numpy(), (2, 0, 1)), "int32")
    s = torch.tensor(3.5)
    out = tb.tropical_permute(s.to(DEV), ())
    torch.cuda.synchronize()
    assert out.item() == 3.5


DIAG_CASES = [
    ("iijb", "bij", (9, 9, 70, 5)),
    ("iijb", "ijb", (9, 9, 70, 5)),
    ("iaii", "ai", (6, 70, 6, 6)),
    ("ijij", "ij", (5, 7, 5, 7)),
    ("abc", "cab", (20, 30, 70)),
]


@pytest.mark.parametrize("inl,outl,shape", DIAG_CASES)
def test_diag(tb, orc, inl, outl, shape):
    g = torch.Generator().manual_seed(sum(shape))
    x = torch.randn(shape, generator=g)
    out = tb.tropical_diag_gather("max_plus", x.to(DEV), inl, outl)
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), orc.diag_gather("max_plus", x.numpy(), inl, outl),
                      f"{inl}->{outl}")


TRACE_CASES = [("iij", "j", (7, 7, 70)), ("iij", "ji", (7, 7, 9)), ("abj", "ja", (5, 6, 7)),
               ("iaib", "b", (4, 3, 4, 9)), ("ii", "", (6, 6))]


@pytest.mark.parametrize("sr,dt", [("max_plus", "f32"), ("min_plus", "f32"), ("max_mul", "f32"),
                                   ("max_plus", "i32"), ("min_plus", "i32"), ("max_mul", "i32")])
@pytest.mark.parametrize("inl,outl,shape", TRACE_CASES)
def test_trace_reduce(tb, orc, sr, dt, inl, outl, shape):
    g = torch.Generator().manual_seed(len(inl) * 7 + shape[0])
    if dt == "i32":
        x = torch.randint(-100, 100, shape, generator=g, dtype=torch.int32)
    else:
        x = torch.randint(-4, 5, shape, generator=g).float()
        x[torch.rand(shape, generator=g) < 0.1] = float("nan")
        x[torch.rand(shape, generator=g) < 0.1] = -0.0
    out = tb.tropical_diag_gather(sr, x.to(DEV), inl, outl)
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), orc.diag_gather(sr, x.numpy(), inl, outl),
                      f"{sr} {dt} {inl}->{outl}")


SLICE_CASES = [
    ("ijk", "ij", (33, 20, 70)),     # reduced axis contiguous: a slice's lanes are neighbours
    ("ijk", "jk", (300, 7, 9)),      # reduced axis outermost: lanes along the outputs
    ("ijk", "ik", (5, 300, 9)),
    ("ii", "", (700, 700)),          # one output, a long diagonal
    ("iaib", "ab", (40, 3, 40, 5)),  # a diagonal reduced
    ("abcd", "d", (6, 7, 8, 9)),     # three reduced axes
]


@pytest.mark.parametrize("slices", [None, 1, 2, 4, 8, 16, 64, 256])
@pytest.mark.parametrize("sr,dt", [("max_plus", "f32"), ("min_plus", "f32"), ("min_plus", "i32")])
def test_reduce_slices(tb, orc, monkeypatch, slices, sr, dt):
    """A reduction split into slices merged by (strictly better, or equal
    with an earlier position): the same bits as the sequential scan for
    every slice count and both lane layouts -- ties of +0 / -0 and of equal
    values, NaN, and values equal to the zero element (which never win)."""
    if slices:
        monkeypatch.setenv("TROPICAL_REDUCE_SLICES", str(slices))
    for inl, outl, shape in SLICE_CASES:
        g = torch.Generator().manual_seed(sum(shape) + len(inl))
        if dt == "i32":
            x = torch.randint(-3, 4, shape, generator=g, dtype=torch.int32)
        else:
            x = torch.randint(-3, 4, shape, generator=g).float()
            u = torch.rand(shape, generator=g)
            x[u < 0.1] = -0.0
            x[(u >= 0.1) & (u < 0.15)] = float("nan")
            x[(u >= 0.15) & (u < 0.2)] = float("-inf") if sr == "max_plus" else float("inf")
        out = tb.tropical_diag_gather(sr, x.to(DEV), inl, outl)
        torch.cuda.synchronize()
        assert_bits_equal(out.cpu().numpy(), orc.diag_gather(sr, x.numpy(), inl, outl),
                          f"{sr} {dt} {inl}->{outl} slices={slices}")
    # the reductions' winners feed the routed argmax of a contraction
    g = torch.Generator().manual_seed(17)
    A = torch.randint(-2, 3, (4, 300, 50), generator=g).float()
    B = torch.randint(-2, 3, (50, 20, 3), generator=g).float()
    if dt == "i32":
        A, B = A.to(torch.int32), B.to(torch.int32)
    C, I = tb.tropical_contract_pair("abj,jcd->bc", sr, A.to(DEV), B.to(DEV))
    torch.cuda.synchronize()
    Cr, Ir = orc.contract_pair("abj,jcd->bc", sr, A.numpy(), B.numpy())
    assert_bits_equal(C.cpu().numpy(), Cr, f"routed {sr} {dt} slices={slices}")
    assert_equal(I.cpu().numpy(), Ir, f"routed argmax {sr} {dt} slices={slices}")


def test_workload5_diag_full(tb, orc):
    A, _ = inputs.einsum_operands()
    out = tb.tropical_diag_gather("max_plus", A.to(DEV), "iijb", "bij")
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), orc.diag_gather("max_plus", A.numpy(), "iijb", "bij"),
                      "workload 5 diagonal")


def test_workload5_permutes_full(tb, orc):
    _, B = inputs.einsum_operands(shape_a=(1, 1, 256, 32))
    out = tb.tropical_permute(B.to(DEV), (2, 1, 0))
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), orc.permute(B.numpy(), (2, 1, 0)), "workload 5 B permute")
    g = torch.Generator().manual_seed(55)
    C = torch.randn(32, 128, 256, generator=g)
    I = torch.randint(0, 256, (32, 128, 256), generator=g, dtype=torch.int32)
    oc, oi = tb.tropical_permute(C.to(DEV), (0, 2, 1), x2=I.to(DEV))
    torch.cuda.synchronize()
    assert_bits_equal(oc.cpu().numpy(), orc.permute(C.numpy(), (0, 2, 1)), "workload 5 C permute")
    assert_equal(oi.cpu().numpy(), orc.permute(I.numpy(), (0, 2, 1)), "workload 5 argmax permute")


VEC_TILED = [
    ((5, 36, 44), (0, 2, 1)),    # P = 36 -> 32-wide tiles, partial along P
    ((3, 20, 48), (0, 2, 1)),    # P = 20 -> 16-wide tiles
    ((2, 100, 72), (0, 2, 1)),   # P = 100 -> 64-wide tiles, partial along P and Q
    ((128, 12, 8), (2, 1, 0)),   # batch axis between P and Q
    ((4, 8, 260, 16), (3, 1, 0, 2)),
    ((33, 64, 64), (0, 2, 1)),
]


@pytest.mark.parametrize("shape,perm", VEC_TILED, ids=[str(s) for s, _ in VEC_TILED])
def test_permute_vectorised_tiles(tb, orc, shape, perm):
    g = torch.Generator().manual_seed(sum(shape))
    x = torch.randn(shape, generator=g)
    i = torch.randint(-1000, 1000, shape, generator=g, dtype=torch.int32)
    before = launches(tb)
    out, out2 = tb.tropical_permute(x.to(DEV), perm, x2=i.to(DEV))
    torch.cuda.synchronize()
    assert delta(before, launches(tb)) == {"gather_tiled": 1}
    assert_bits_equal(out.cpu().numpy(), orc.permute(x.numpy(), perm), f"vec tiled {shape} {perm}")
    assert_equal(out2.cpu().numpy(), orc.permute(i.numpy(), perm), f"vec tiled pair {shape} {perm}")


VEC_COPY = [((7, 12, 3, 8), (1, 2, 0, 3)), ((9, 5, 4), (1, 0, 2)), ((3, 1000, 12), (1, 0, 2)),
            ((2, 3, 4, 5, 8), (4, 3, 2, 1, 0)[::-1]), ((6, 7, 16), (1, 0, 2))]


@pytest.mark.parametrize("shape,perm", VEC_COPY, ids=[str(s) for s, _ in VEC_COPY])
def test_permute_vectorised_copy(tb, orc, shape, perm):
    g = torch.Generator().manual_seed(len(shape) + shape[0])
    x = torch.randn(shape, generator=g)
    out = tb.tropical_permute(x.to(DEV), perm)
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), orc.permute(x.numpy(), perm), f"vec copy {shape} {perm}")


WIDE = [torch.float64, torch.complex64, torch.complex128, torch.int64]


def wide_tensor(shape, dt, g):
    x = torch.randn(shape, generator=g, dtype=torch.float64) * 1000
    if dt.is_complex:
        x = x + 1j * torch.randn(shape, generator=g, dtype=torch.float64)
    return x.to(dt)


@pytest.mark.parametrize("dt", WIDE, ids=lambda d: str(d).replace("torch.", ""))
@pytest.mark.parametrize("shape", [(5, 9), (65, 130), (3, 1, 70, 2), (2, 3, 4, 5, 6), (33, 2, 65)],
                         ids=lambda s: "x".join(map(str, s)))
def test_permute_wide_elements(tb, orc, dt, shape):
    """8- and 16-byte elements (f64, c32, c64, i64) through the same kernels."""
    g = torch.Generator().manual_seed(sum(shape))
    x = wide_tensor(shape, dt, g)
    xd = x.to(DEV)
    perms = list(itertools.permutations(range(len(shape))))
    if len(perms) > 24:
        perms = perms[:: len(perms) // 24]
    for p in perms:
        out = tb.tropical_permute(xd, p)
        torch.cuda.synchronize()
        assert out.dtype == dt
        assert_bits_equal(out.cpu().numpy(), orc.permute(x.numpy(), p), f"{dt} permute {shape} {p}")
    # a strided view of the same tensor
    v = x[(slice(None, None, 2),) + (slice(None),) * (len(shape) - 1)]
    vd = device_copy(v)
    p = tuple(reversed(range(len(shape))))
    out = tb.tropical_permute(vd, p)
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), orc.permute(v.numpy(), p), f"{dt} strided view {shape}")


def test_permute_wide_pairs_unaligned_and_rank8(tb, orc):
    g = torch.Generator().manual_seed(8)
    # value (float64) and index (int64) moved with one mapping, every path
    x = wide_tensor((6, 70, 130), torch.float64, g)
    idx = torch.randint(0, 1 << 40, (6, 70, 130), generator=g, dtype=torch.int64)
    xd, idd = x.to(DEV), idx.to(DEV)
    for p in ((0, 1, 2), (1, 0, 2), (0, 2, 1), (2, 1, 0)):
        out, out2 = tb.tropical_permute(xd, p, x2=idd)
        torch.cuda.synchronize()
        assert_bits_equal(out.cpu().numpy(), orc.permute(x.numpy(), p), f"f64 pair value {p}")
        assert_equal(out2.cpu().numpy(), orc.permute(idx.numpy(), p), f"i64 pair index {p}")
    # complex64 starting 8 bytes into an allocation (not 16-byte aligned)
    base = wide_tensor((1 + 40 * 33,), torch.complex64, g).to(DEV)
    xv = base[1:].view(40, 33)
    out = tb.tropical_permute(xv, (1, 0))
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), orc.permute(xv.cpu().numpy(), (1, 0)), "c64 unaligned")
    # rank 8: axes that merge fit the kernels; eight axes that stay apart
    # (every axis moved, the element words apart from all) do not
    x8 = wide_tensor((2, 3, 2, 3, 2, 3, 2, 3), torch.float64, g)
    x8d = x8.to(DEV)
    p = (1, 2, 3, 4, 5, 6, 7, 0)
    out = tb.tropical_permute(x8d, p)
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), orc.permute(x8.numpy(), p), "rank 8 f64")
    with pytest.raises(tb.TropicalError) as e:
        tb.tropical_permute(x8d, (7, 6, 5, 4, 3, 2, 1, 0))
    assert e.value.status == tb.UNSUPPORTED
    p = (7, 6, 5, 4, 3, 2, 1, 0)
    out = tb.tropical_permute(x8.to(torch.float32).to(DEV), p)  # 4-byte elements: 8 axes fit
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), orc.permute(x8.to(torch.float32).numpy(), p), "rank 8 f32")
    with pytest.raises(tb.TropicalError) as e:
        tb.tropical_permute(torch.zeros(4, 4, dtype=torch.float16, device=DEV), (1, 0))
    assert e.value.status == tb.UNSUPPORTED


@pytest.mark.parametrize("R", [2, 4, 8, 16])
@pytest.mark.parametrize("dims", [(6, 50, 37), (1, 300, 65), (3, 7, 129)], ids=lambda d: "x".join(map(str, d)))
def test_permute_runs_path(tb, orc, R, dims):
    """A short contiguous last axis (a run of R words) whose neighbour in the
    output is not its neighbour in the input: the runs path transposes
    whole runs through LDS.  Ragged tiles, pairs and unaligned views."""
    b, p_, q_ = dims
    g = torch.Generator().manual_seed(R * 1000 + p_)
    x = torch.randn(b, p_, q_, R, generator=g)
    idx = torch.randint(-10 ** 6, 10 ** 6, (b, p_, q_, R), generator=g, dtype=torch.int32)
    xd, idd = x.to(DEV), idx.to(DEV)
    perm = (0, 2, 1, 3)
    before = launches(tb)
    out, out2 = tb.tropical_permute(xd, perm, x2=idd)
    torch.cuda.synchronize()
    assert delta(before, launches(tb)) == {"gather_tiled": 1}
    assert_bits_equal(out.cpu().numpy(), orc.permute(x.numpy(), perm), f"runs R={R} {dims}")
    assert_equal(out2.cpu().numpy(), orc.permute(idx.numpy(), perm), f"runs pair R={R} {dims}")
    # the run axis moved to the front is not a run any more; the batch
    # axis last is the other transpose of the runs
    for perm in ((2, 0, 1, 3), (1, 2, 0, 3)):
        out = tb.tropical_permute(xd, perm)
        torch.cuda.synchronize()
        assert_bits_equal(out.cpu().numpy(), orc.permute(x.numpy(), perm), f"runs R={R} {dims} {perm}")
    # one word into the allocation: 4-byte aligned only (word accesses)
    base = torch.randn(1 + x.numel(), generator=g)
    xv = base[1:].view(x.shape)
    xvd = base.to(DEV)[1:].view(x.shape)
    out = tb.tropical_permute(xvd, (0, 2, 1, 3))
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), orc.permute(xv.numpy(), (0, 2, 1, 3)), f"runs unaligned R={R}")


def test_runs_path_in_contraction_describe(tb, monkeypatch):
    # the lattice network's boundary gather: a 16-word run (bond 16) whose
    # neighbour moves from the front to the end.  The runs tile (32 runs
    # along the moved axis) is half in range for its 16, so the flat tile
    # takes it; with the flat path off it is the runs path.  (By default the
    # GEMM reads this operand in place with a two-level k: the gather is
    # asked for here.)
    monkeypatch.setenv("TROPICAL_NO_KRUN_FOLD", "1")
    desc = tb.tropical_contract_pair_describe("vwxyze,veAf->wxyzAf", (16,) * 6, (16,) * 4)
    assert "A=gather:flat" in desc, desc
    monkeypatch.setenv("TROPICAL_FLAT_PATH", "0")
    desc = tb.tropical_contract_pair_describe("vwxyze,veAf->wxyzAf", (16,) * 6, (16,) * 4)
    assert "A=gather:runs" in desc, desc


# (shape, perm) whose transpose plane has a small extent on one side
FLAT = [
    ((3001, 2), (1, 0)),          # small P (the read-contiguous axis), ragged Q
    ((2, 3001), (1, 0)),          # small Q (the write-contiguous axis)
    ((5, 999, 3), (0, 2, 1)),     # odd small extent: odd LDS rows
    ((5, 3, 999), (0, 2, 1)),
    ((700, 6, 7), (2, 1, 0)),     # P = 7 with a batch axis between P and Q
    ((16, 2, 2050), (0, 2, 1)),
    ((9, 4, 1500), (2, 0, 1)),    # Q = 4 whose rows are apart in the output
    ((3, 5, 11, 300), (0, 3, 2, 1)),
    # batched transposes of small matrices: tiles of several whole blocks
    ((999, 8, 8), (0, 2, 1)),
    ((4097, 2, 2), (0, 2, 1)),
    ((777, 2, 3), (0, 2, 1)),
    ((333, 5, 6, 7), (0, 3, 1, 2)),
    ((16, 16, 16, 16, 16), (0, 1, 2, 4, 3)),
    ((3, 1500, 4, 4), (0, 1, 3, 2)),
    # the block transposed in place with the axis outside it moved: blocks
    # contiguous in the input only / in the output only
    ((16, 16, 16, 16, 16), (2, 0, 1, 4, 3)),
    ((8, 8, 60, 3, 4), (2, 0, 1, 4, 3)),
    ((40, 6, 5), (1, 2, 0)),
]


@pytest.mark.parametrize("mode", ["auto", "force", "0"])
@pytest.mark.parametrize("shape,perm", FLAT, ids=[f"{s}{p}" for s, p in FLAT])
def test_permute_flat_path(tb, orc, monkeypatch, mode, shape, perm):
    """The flat-tile transpose (the small extent whole in each tile) against
    the oracle, with a paired int32 tensor and an unaligned view; the same
    shapes with the path forced on for any valid tile, and switched off."""
    if mode != "auto":
        monkeypatch.setenv("TROPICAL_FLAT_PATH", mode)
    g = torch.Generator().manual_seed(sum(shape) + len(perm))
    x = torch.randn(shape, generator=g)
    idx = torch.randint(-10 ** 6, 10 ** 6, shape, generator=g, dtype=torch.int32)
    out, out2 = tb.tropical_permute(x.to(DEV), perm, x2=idx.to(DEV))
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), orc.permute(x.numpy(), perm), f"flat {shape} {perm}")
    assert_equal(out2.cpu().numpy(), orc.permute(idx.numpy(), perm), f"flat pair {shape} {perm}")
    base = torch.randn(1 + x.numel(), generator=g)
    xv = base[1:].view(shape)
    out = tb.tropical_permute(base.to(DEV)[1:].view(shape), perm)
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), orc.permute(xv.numpy(), perm), f"flat unaligned {shape} {perm}")


@pytest.mark.parametrize("dt", [torch.float64, torch.complex64, torch.complex128],
                         ids=lambda d: str(d).replace("torch.", ""))
@pytest.mark.parametrize("shape,perm", [((3001, 2), (1, 0)), ((2, 3001), (1, 0)), ((7, 3, 501), (2, 1, 0)),
                                        ((4, 640, 5), (0, 2, 1)), ((1001, 4, 4), (0, 2, 1)),
                                        ((555, 3, 2), (0, 2, 1))], ids=lambda v: str(v))
def test_permute_flat_path_wide_elements(tb, orc, dt, shape, perm):
    """Wide elements on the flat path: each element's words stay together
    (2 or 4 words per element), pairs with an int64 index."""
    g = torch.Generator().manual_seed(sum(shape))
    x = wide_tensor(shape, dt, g)
    idx = torch.randint(0, 1 << 40, shape, generator=g, dtype=torch.int64)
    if dt.itemsize == 8:
        out, out2 = tb.tropical_permute(x.to(DEV), perm, x2=idx.to(DEV))
        torch.cuda.synchronize()
        assert_equal(out2.cpu().numpy(), orc.permute(idx.numpy(), perm), f"{dt} flat pair {shape}")
    else:
        out = tb.tropical_permute(x.to(DEV), perm)
        torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), orc.permute(x.numpy(), perm), f"{dt} flat {shape} {perm}")


def test_flat_path_is_taken(tb, orc, monkeypatch):
    """The planner's choice shows in the contraction description, and the
    small-bond gather moves the same bits with the path on or off."""
    d = tb.tropical_contract_pair_describe("aib,ajb->bij", (2, 64, 512), (2, 64, 512))
    assert "A=gather:flat" in d, d
    g = torch.Generator().manual_seed(5)
    A = torch.randn(2, 64, 512, generator=g)
    B = torch.randn(2, 64, 512, generator=g)
    Ad, Bd = A.to(DEV), B.to(DEV)
    C1, I1 = tb.tropical_contract_pair("aib,ajb->bij", "max_plus", Ad, Bd, argmax=True)
    monkeypatch.setenv("TROPICAL_FLAT_PATH", "0")
    C0, I0 = tb.tropical_contract_pair("aib,ajb->bij", "max_plus", Ad, Bd, argmax=True)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int32), C0.view(torch.int32)) and torch.equal(I1, I0)
    Co, Io = orc.contract_pair("aib,ajb->bij", "max_plus", A.numpy(), B.numpy())
    assert_bits_equal(C1.cpu().numpy(), Co, "flat contraction value")
    assert_equal(I1.cpu().numpy(), Io, "flat contraction argmax")


MANY_AXES = [(4,) * 7, (8,) * 5, (2, 4, 8, 16, 8, 2), (3, 5, 2, 7, 4, 6), (2,) * 8]


@pytest.mark.parametrize("mode", ["auto", "force", "0"])
@pytest.mark.parametrize("shape", MANY_AXES, ids=lambda s: "x".join(map(str, s)))
def test_permute_many_small_axes(tb, orc, monkeypatch, mode, shape):
    """Tensor-network shapes (many axes of small bond): the flat tile's
    sides are groups of axes (contiguous in the input on one side, in the
    output on the other); random permutations, a paired int32 tensor, f64."""
    if mode != "auto":
        monkeypatch.setenv("TROPICAL_FLAT_PATH", mode)
    g = torch.Generator().manual_seed(len(shape) * 31 + shape[0])
    x = torch.randn(shape, generator=g)
    idx = torch.randint(-10 ** 6, 10 ** 6, shape, generator=g, dtype=torch.int32)
    x64 = wide_tensor(shape, torch.float64, g)
    xd, idd, x64d = x.to(DEV), idx.to(DEV), x64.to(DEV)
    rng = np.random.default_rng(len(shape))
    for _ in range(10):
        perm = tuple(int(v) for v in rng.permutation(len(shape)))
        out, out2 = tb.tropical_permute(xd, perm, x2=idd)
        torch.cuda.synchronize()
        assert_bits_equal(out.cpu().numpy(), orc.permute(x.numpy(), perm), f"{shape} {perm}")
        assert_equal(out2.cpu().numpy(), orc.permute(idx.numpy(), perm), f"pair {shape} {perm}")
        if len(shape) < 8:  # (8 axes apart plus the element's words exceed the 8 kernel axes)
            o64 = tb.tropical_permute(x64d, perm)
            torch.cuda.synchronize()
            assert_bits_equal(o64.cpu().numpy(), orc.permute(x64.numpy(), perm), f"f64 {shape} {perm}")


# reductions with many outputs along an input-contiguous last axis: four
# adjacent outputs per thread with 16-byte loads (TROPICAL_REDUCE_VEC=0
# keeps one output per thread); both against the oracle
VEC_TRACE_CASES = [("iij", "j", (7, 7, 72)), ("ijk", "jk", (300, 8, 16)), ("ijk", "ik", (5, 300, 12)),
                   ("iaib", "ab", (40, 3, 40, 8)), ("abcd", "cd", (6, 7, 8, 12)), ("iij", "j", (64, 64, 8192))]


@pytest.mark.parametrize("vec", [True, False])
@pytest.mark.parametrize("sr,dt", [("max_plus", "f32"), ("min_plus", "f32"), ("max_mul", "f32"),
                                   ("max_plus", "i32"), ("min_plus", "i32"), ("max_mul", "i32")])
def test_trace_reduce_vec(tb, orc, monkeypatch, vec, sr, dt):
    if not vec:
        monkeypatch.setenv("TROPICAL_REDUCE_VEC", "0")
    for inl, outl, shape in VEC_TRACE_CASES:
        g = torch.Generator().manual_seed(sum(shape) + len(inl))
        if dt == "i32":
            x = torch.randint(-3, 4, shape, generator=g, dtype=torch.int32)
        else:
            x = torch.randint(-3, 4, shape, generator=g).float()
            u = torch.rand(shape, generator=g)
            x[u < 0.1] = -0.0
            x[(u >= 0.1) & (u < 0.15)] = float("nan")
            x[(u >= 0.15) & (u < 0.2)] = float("-inf") if sr != "min_plus" else float("inf")
        out = tb.tropical_diag_gather(sr, x.to(DEV), inl, outl)
        torch.cuda.synchronize()
        assert_bits_equal(out.cpu().numpy(), orc.diag_gather(sr, x.numpy(), inl, outl),
                          f"{sr} {dt} {inl}->{outl} {shape} vec={vec}")
    # winners of a vectorised pre-pass reduction route a contraction's argmax
    A = torch.randint(-2, 3, (5, 40, 52), generator=g).float()
    B = torch.randint(-2, 3, (52, 24), generator=g).float()
    if dt == "i32":
        A, B = A.to(torch.int32), B.to(torch.int32)
    if sr == "max_mul":
        A, B = A.abs(), B.abs()
    C, I = tb.tropical_contract_pair("abj,jk->bk", sr, A.to(DEV), B.to(DEV))
    torch.cuda.synchronize()
    Cr, Ir = orc.contract_pair("abj,jk->bk", sr, A.numpy(), B.numpy())
    assert_bits_equal(C.cpu().numpy(), Cr, f"routed {sr} {dt} vec={vec}")
    assert_equal(I.cpu().numpy(), Ir, f"routed argmax {sr} {dt} vec={vec}")
