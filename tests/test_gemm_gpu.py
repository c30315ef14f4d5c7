"""Parity of the HIP tropical GEMM with the CPU oracle: bit-exact values and
exact argmax indices (tolerance 0), over semirings, dtypes, layouts, ragged
sizes, K around the 16-term chunk and 256-term LDS block, special values,
and the four GEMM workloads at full size."""
import zlib

import numpy as np
import pytest
import torch

import golden_io as gio
from gpu_util import DEV, assert_bits_equal, assert_equal, gpu_gemm
from tropical_semiring_tensor_amd import inputs

pytestmark = pytest.mark.gpu

I32_INF = 1 << 30
PAIRS = [("max_plus", "f32"), ("min_plus", "f32"), ("max_mul", "f32"),
         ("max_plus", "i32"), ("min_plus", "i32"), ("max_mul", "i32")]


@pytest.fixture(scope="module")
def tb():
    from tropical_semiring_tensor_amd import binding
    binding.tropical_init(0)
    return binding


@pytest.fixture(autouse=True, params=["auto", "wide", "narrow", "global", "general"])
def gemm_setting(request, monkeypatch):
    """Every test under every argmax kernel setting: the host picks the
    global-resolve kernel (two-slice ring, argmax resolved once per tile
    from global memory) for K > 256, else the narrow one (K-block 256,
    loads ahead, one workgroup per CU) for fewer than two tiles per CU and
    the wide one (float: K-block 128, 4 waves per SIMD) otherwise; "wide",
    "narrow" and "global" force one for any shape.  "general": the automatic
    choice with the instances whose operand layouts are fixed at compile
    time switched off (their general counterparts then run the same
    shapes)."""
    if request.param == "general":
        monkeypatch.setenv("TROPICAL_GEMM_FIXED_LAYOUT", "0")
    elif request.param != "auto":
        monkeypatch.setenv("TROPICAL_GEMM_SETTING", request.param)
    return request.param


def make(sr, dt, b, m, k, n, seed, ties=True, a_col=False, b_col=False):
    g = torch.Generator().manual_seed(seed)
    if dt == "i32":
        A = torch.randint(-50, 51, (b, m, k), generator=g, dtype=torch.int32)
        B = torch.randint(-50, 51, (b, k, n), generator=g, dtype=torch.int32)
        z = I32_INF if sr == "min_plus" else -I32_INF
        A[torch.rand(A.shape, generator=g) < 0.15] = z
        B[torch.rand(B.shape, generator=g) < 0.15] = z
    elif sr == "max_mul":
        if ties:
            A = torch.randint(0, 9, (b, m, k), generator=g).float() * 0.125
            B = torch.randint(0, 9, (b, k, n), generator=g).float() * 0.25
        else:
            A = torch.rand(b, m, k, generator=g)
            B = torch.rand(b, k, n, generator=g)
    else:
        if ties:
            A = torch.randint(-8, 9, (b, m, k), generator=g).float()
            B = torch.randint(-8, 9, (b, k, n), generator=g).float()
        else:
            A = torch.randn(b, m, k, generator=g)
            B = torch.randn(b, k, n, generator=g)
    if a_col:
        A = A.transpose(1, 2).contiguous().transpose(1, 2)
    if b_col:
        B = B.transpose(1, 2).contiguous().transpose(1, 2)
    return A, B


def check(tb, orc, sr, A, B, what, c_layout="row", argmax=True):
    C, I = gpu_gemm(tb, sr, A, B, argmax=argmax, c_layout=c_layout)
    Cr, Ir = orc.gemm(sr, A.numpy(), B.numpy(), argmax=argmax)
    assert_bits_equal(C, Cr, what + " C")
    if argmax:
        assert_equal(I, Ir, what + " argmax")


SHAPES = [(1, 1, 1, 1), (2, 3, 7, 5), (1, 64, 64, 64), (3, 65, 17, 63), (1, 130, 33, 70),
          (2, 127, 255, 129), (1, 70, 300, 90), (1, 33, 600, 40), (1, 17, 513, 200)]


@pytest.mark.parametrize("sr,dt", PAIRS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ragged_row_major(tb, orc, sr, dt, shape):
    b, m, k, n = shape
    A, B = make(sr, dt, b, m, k, n, seed=zlib.crc32(repr((sr, dt, shape)).encode()) % 10000)
    check(tb, orc, sr, A, B, f"{sr} {dt} {shape}")


@pytest.mark.parametrize("sr,dt", PAIRS)
@pytest.mark.parametrize("a_col,b_col", [(False, True), (True, False), (True, True)])
def test_layouts(tb, orc, sr, dt, a_col, b_col):
    A, B = make(sr, dt, 2, 97, 300, 75, seed=11, a_col=a_col, b_col=b_col)
    check(tb, orc, sr, A, B, f"{sr} {dt} a_col={a_col} b_col={b_col}")


@pytest.mark.parametrize("sr,dt", PAIRS)
@pytest.mark.parametrize("n", [1, 5, 16])
@pytest.mark.parametrize("b_col", [False, True])
def test_at_most_16_columns(tb, orc, sr, dt, n, b_col):
    """Products with at most 16 columns: each thread computes one 16-column
    group (the 64 x 64 tile's other 48 columns would be padding), with B
    row-major (the fixed-layout form) or column-major (the general one),
    over more tiles than two per CU, with and without argmax."""
    A, B = make(sr, dt, 8, 4100, 200, n, seed=n * 7 + b_col, b_col=b_col)
    check(tb, orc, sr, A, B, f"{sr} {dt} n={n} b_col={b_col}")
    check(tb, orc, sr, A, B, f"{sr} {dt} n={n} b_col={b_col} value only", argmax=False)


def test_at_most_16_columns_many_tiles_per_workgroup(tb, orc, monkeypatch):
    monkeypatch.setenv("TROPICAL_GEMM_MAX_WORKGROUPS", "8")
    for sr in ("max_plus", "max_mul"):
        A, B = make(sr, "f32", 3, 1000, 140, 16, seed=3)
        check(tb, orc, sr, A, B, f"{sr} n=16, 8 workgroups")


@pytest.mark.parametrize("k", [1, 2, 15, 16, 17, 31, 32, 255, 256, 257, 511, 512, 513, 1000])
def test_k_around_chunk_and_block(tb, orc, k):
    for sr in ("max_plus", "min_plus"):
        A, B = make(sr, "f32", 1, 40, k, 72, seed=k, ties=True)
        check(tb, orc, sr, A, B, f"{sr} k={k} ties")
        A, B = make(sr, "f32", 1, 40, k, 72, seed=k + 1, ties=False)
        check(tb, orc, sr, A, B, f"{sr} k={k} normal")


def test_increasing_terms_resolve_every_block(tb, orc):
    # every later term is larger: the best improves in every chunk of every block
    k = 800
    A = torch.arange(k, dtype=torch.float32).repeat(1, 70, 1) * 0.5
    B = torch.arange(k, dtype=torch.float32)[:, None].repeat(1, 1, 66) * 0.25
    A = A + torch.arange(70, dtype=torch.float32)[None, :, None]
    check(tb, orc, "max_plus", A, B, "increasing max-plus")
    check(tb, orc, "min_plus", -A, -B, "decreasing min-plus")


def test_all_ties(tb, orc):
    A = torch.zeros(2, 66, 300)
    B = torch.zeros(2, 300, 67)
    check(tb, orc, "max_plus", A, B, "all zero ties")
    check(tb, orc, "max_mul", A + 1, B + 1, "all one ties")


def special_matrix(shape, g, kinds):
    base = torch.randint(-4, 5, shape, generator=g).float()
    r = torch.rand(shape, generator=g)
    vals = {"inf": float("inf"), "-inf": float("-inf"), "nan": float("nan"), "-0": -0.0, "0": 0.0,
            "den": 1e-45, "-den": -3e-45}
    edges = np.linspace(0, 0.5, len(kinds) + 1)
    for i, kind in enumerate(kinds):
        base[(r >= edges[i]) & (r < edges[i + 1])] = vals[kind]
    return base


@pytest.mark.parametrize("sr", ["max_plus", "min_plus", "max_mul"])
def test_special_values(tb, orc, sr):
    g = torch.Generator().manual_seed(5)
    kinds = ["inf", "-inf", "nan", "-0", "0", "den", "-den"]
    A = special_matrix((2, 70, 290), g, kinds)
    B = special_matrix((2, 290, 68), g, kinds)
    check(tb, orc, sr, A, B, f"special {sr}")


def test_signed_zero_first_winner(tb, orc):
    # every term is -0 or +0; the first one decides the sign of C
    g = torch.Generator().manual_seed(9)
    A = torch.where(torch.rand(1, 64, 64, generator=g) < 0.5, -0.0, 0.0)
    B = torch.full((1, 64, 64), -0.0)
    check(tb, orc, "max_plus", A, B, "signed zeros")
    check(tb, orc, "min_plus", A, B, "signed zeros min")


def test_int32_saturation(tb, orc):
    g = torch.Generator().manual_seed(13)
    big = torch.tensor([2 ** 31 - 1, -(2 ** 31), I32_INF, -I32_INF, 0, 1, -1], dtype=torch.int32)
    A = big[torch.randint(0, 7, (1, 65, 100), generator=g)]
    B = big[torch.randint(0, 7, (1, 100, 66), generator=g)]
    for sr in ("max_plus", "min_plus"):
        check(tb, orc, sr, A, B, f"saturation {sr}")


def test_golden_fixtures(tb):
    for case in gio.load("gemm_3x3.json")["cases"] + gio.load("special_values.json")["cases"]:
        A = torch.from_numpy(gio.array(case["A"], case["dtype"]))
        B = torch.from_numpy(gio.array(case["B"], case["dtype"]))
        C, I = gpu_gemm(tb, case["semiring"], A, B)
        assert_bits_equal(C[0], gio.array(case["C"], case["dtype"]), case["name"])
        assert_equal(I[0], np.array(case["argmax"]), case["name"])


def test_k_zero_and_empty(tb, orc):
    for sr, dt in PAIRS:
        dtype = torch.float32 if dt == "f32" else torch.int32
        A = torch.zeros(2, 5, 0, dtype=dtype)
        B = torch.zeros(2, 0, 7, dtype=dtype)
        C, I = gpu_gemm(tb, sr, A, B)
        Cr, Ir = orc.gemm(sr, A.numpy(), B.numpy())
        assert_bits_equal(C, Cr, f"k=0 {sr} {dt}")
        assert_equal(I, Ir, f"k=0 {sr} {dt}")
    # zero-sized outputs enqueue nothing
    Cd = torch.empty(3, 0, 4, device=DEV)
    tb.tropical_gemm_strided_batched("max_plus", torch.empty(3, 0, 5, device=DEV),
                                     torch.empty(3, 5, 4, device=DEV), Cd)


def test_no_argmax_and_column_major_c(tb, orc):
    A, B = make("max_plus", "f32", 2, 70, 100, 90, seed=21, ties=False)
    check(tb, orc, "max_plus", A, B, "no argmax", argmax=False)
    check(tb, orc, "max_plus", A, B, "column-major C", c_layout="col")


def test_strided_views_and_unaligned(tb, orc):
    g = torch.Generator().manual_seed(17)
    big = torch.randint(-5, 6, (3, 90, 160), generator=g).float()
    A = big[:, 1:80:1, 3:150:1]          # unaligned base, row stride 160
    A2 = big[:, ::2, ::2]                # no unit stride at all
    Bbig = torch.randint(-5, 6, (3, 200, 100), generator=g).float()
    B = Bbig[:, 5:152, 1:70]             # k = 147 rows to match A
    check(tb, orc, "max_plus", A, B, "unaligned views")
    B2 = Bbig[:, ::2, ::3][:, :80, :]    # k = 80 to match A2's 80 columns
    check(tb, orc, "min_plus", A2, B2, "non-unit strides")
    # batch stride larger than m * k (padding between batch entries)
    P = torch.randint(-5, 6, (3, 40, 50), generator=g).float()
    check(tb, orc, "max_plus", P[:, :30, :20], P[:, :20, :33], "padded batches")
    # broadcast batch: stride 0 on B
    Bb = torch.randint(-5, 6, (1, 20, 33), generator=g).float().expand(3, 20, 33)
    check(tb, orc, "max_plus", P[:, :30, :20], Bb, "batch stride 0")


def test_simple_kernel_and_no_swizzle(tb, orc, monkeypatch):
    A, B = make("max_plus", "f32", 3, 70, 130, 66, seed=31)
    monkeypatch.setenv("TROPICAL_FORCE_SIMPLE_GEMM", "1")
    check(tb, orc, "max_plus", A, B, "simple kernel")
    Ai, Bi = make("min_plus", "i32", 2, 33, 70, 40, seed=32)
    check(tb, orc, "min_plus", Ai, Bi, "simple kernel i32")
    monkeypatch.delenv("TROPICAL_FORCE_SIMPLE_GEMM")
    monkeypatch.setenv("TROPICAL_NO_XCD_SWIZZLE", "1")
    check(tb, orc, "max_plus", A, B, "no swizzle")
    monkeypatch.delenv("TROPICAL_NO_XCD_SWIZZLE")
    # the 64-bit tile decode (taken when a grid has 2^31 tiles or more),
    # with and without split K
    monkeypatch.setenv("TROPICAL_GEMM_COORD64", "1")
    check(tb, orc, "max_plus", A, B, "64-bit tile decode")
    A2, B2 = make("min_plus", "f32", 2, 40, 3000, 50, seed=33)
    C, I = gpu_gemm_ws(tb, "min_plus", A2, B2)
    Cr, Ir = orc.gemm("min_plus", A2.numpy(), B2.numpy())
    assert_bits_equal(C, Cr, "64-bit tile decode, split K")
    assert_equal(I, Ir, "64-bit tile decode, split K argmax")
    monkeypatch.delenv("TROPICAL_GEMM_COORD64")


@pytest.mark.parametrize("coord64", [False, True])
@pytest.mark.parametrize("rows", ["default", "1", "3", "8"])
def test_tile_orders(tb, orc, monkeypatch, coord64, rows):
    # grouped raster (groups of 3, 4 or 8 tile-rows, the last one shorter)
    # and plain row-by-row order, with the 32- and 64-bit tile decodes:
    # tile-row counts 1, 3, 5, 7, 9 and several batch entries, every output
    # written once
    if coord64:
        monkeypatch.setenv("TROPICAL_GEMM_COORD64", "1")
    if rows == "1":
        monkeypatch.setenv("TROPICAL_GEMM_ROW_RASTER", "1")
    elif rows != "default":
        monkeypatch.setenv("TROPICAL_GEMM_GROUP_ROWS", rows)
    for shape in ((3, 40, 70, 500), (2, 130, 90, 200), (1, 300, 40, 190), (2, 450, 33, 70), (1, 520, 20, 600)):
        A, B = make("max_plus", "f32", *shape, seed=sum(shape))
        check(tb, orc, "max_plus", A, B, f"tile order {shape} coord64={coord64} rows={rows}")
    A, B = make("min_plus", "i32", 1, 300, 2000, 100, seed=9)
    C, I = gpu_gemm_ws(tb, "min_plus", A, B)
    Cr, Ir = orc.gemm("min_plus", A.numpy(), B.numpy())
    assert_bits_equal(C, Cr, "tile order split K")
    assert_equal(I, Ir, "tile order split K argmax")


# ---------------------------------------------------------------------------
# the four GEMM workloads at full size, in the launch configuration that the
# benchmark times

def test_workload1_full(tb, orc):
    A, B = inputs.gemm_operands(1)
    check(tb, orc, "max_plus", A, B, "workload 1")


def test_workload2_full(tb, orc):
    A, B = inputs.gemm_operands(2)
    check(tb, orc, "max_plus", A, B, "workload 2")


# Oracle results of workloads 3 and 4 at full size, computed once per test
# session (they do not depend on the kernel setting under test).  The oracle
# is handed B with k as its unit-stride axis: the same values, so the same
# definition, but its k loop then streams both operands.
_FULL_REF = {}


def _full_reference(orc, w):
    if w not in _FULL_REF:
        spec = inputs.WORKLOADS[w]
        A, B = inputs.gemm_operands(w)
        Bk = B.transpose(1, 2).contiguous().transpose(1, 2)
        Cr, Ir = orc.gemm(spec["semiring"], A.numpy(), Bk.numpy())
        _FULL_REF[w] = (A, B, Cr, Ir)
    return _FULL_REF[w]


def test_workload3_full(tb, orc):
    # min-plus int32 4096^3 with 20% 2^30 sentinels: every output and every
    # argmin against the oracle, bit for bit
    A, B, Cr, Ir = _full_reference(orc, 3)
    C, I = gpu_gemm(tb, "min_plus", A, B)
    assert_equal(C, Cr, "workload 3 C")
    assert_equal(I, Ir, "workload 3 argmin")


def test_workload4_full(tb, orc):
    # max-mul float32 16 x 2048^3 with column-major B: every output and
    # every argmax against the oracle, bit for bit
    A, B, Cr, Ir = _full_reference(orc, 4)
    C, I = gpu_gemm(tb, "max_mul", A, B)
    assert_bits_equal(C, Cr, "workload 4 C")
    assert_equal(I, Ir, "workload 4 argmax")


def test_workload3_reduced_full_check(tb, orc):
    A, B = inputs.gemm_operands(3, m=300, n=260, k=1100)
    check(tb, orc, "min_plus", A, B, "workload 3 recipe, 300x260x1100")


def test_workload4_reduced_full_check(tb, orc):
    A, B = inputs.gemm_operands(4, batch=3, m=200, n=150, k=700)
    check(tb, orc, "max_mul", A, B, "workload 4 recipe, 3x200x150x700")


@pytest.mark.parametrize("argmax", [True, False])
def test_many_tiles_per_workgroup(tb, orc, monkeypatch, argmax):
    """A grid capped at 8 persistent workgroups: each one walks many output
    tiles in turn, so the next tile's first slice is fetched while the
    previous tile resolves its argmax and stores, and every per-tile reset
    (running values, chunk records, K offsets) is exercised; int32 and
    float32 workload recipes, every output compared."""
    monkeypatch.setenv("TROPICAL_GEMM_MAX_WORKGROUPS", "8")
    A, B = inputs.gemm_operands(3, m=300, n=260, k=1100)
    check(tb, orc, "min_plus", A, B, "workload 3 recipe, 8 workgroups", argmax=argmax)
    A, B = inputs.gemm_operands(4, batch=3, m=200, n=150, k=700)
    check(tb, orc, "max_mul", A, B, "workload 4 recipe, 8 workgroups", argmax=argmax)
    A, B = inputs.gemm_operands(2, batch=5, m=130, n=200, k=256)
    check(tb, orc, "max_plus", A, B, "workload 2 recipe, 8 workgroups", argmax=argmax)
    for sr in ("min_plus", "max_plus"):
        name, (b, m, k, n), bad_k, rows, in_b = LIMIT_CASES[-1]
        Ai, Bi = limit_case(sr, 3, 200, k, 150, seed=41, bad_k=bad_k, bad_rows=rows, in_b=in_b)
        check(tb, orc, sr, Ai, Bi, f"int32 limits {sr} {name}, 8 workgroups", argmax=argmax)


# ---------------------------------------------------------------------------
# value-only launches (no argmax output) run their own kernel: same parity bar

VO_SHAPES = [(1, 1, 1, 1), (2, 3, 7, 5), (3, 65, 17, 63), (2, 127, 255, 129), (1, 33, 600, 40)]


@pytest.mark.parametrize("sr,dt", PAIRS)
@pytest.mark.parametrize("shape", VO_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_value_only_ragged(tb, orc, sr, dt, shape):
    b, m, k, n = shape
    A, B = make(sr, dt, b, m, k, n, seed=zlib.crc32(repr(("vo", sr, dt, shape)).encode()) % 10000)
    check(tb, orc, sr, A, B, f"value only {sr} {dt} {shape}", argmax=False)


@pytest.mark.parametrize("a_col,b_col", [(False, True), (True, False)])
def test_value_only_layouts(tb, orc, a_col, b_col):
    for sr, dt in PAIRS:
        A, B = make(sr, dt, 2, 97, 300, 75, seed=12, a_col=a_col, b_col=b_col)
        check(tb, orc, sr, A, B, f"value only {sr} {dt} a_col={a_col} b_col={b_col}", argmax=False)


def test_value_only_special_values_and_signed_zeros(tb, orc):
    g = torch.Generator().manual_seed(6)
    kinds = ["inf", "-inf", "nan", "-0", "0", "den", "-den"]
    A = special_matrix((2, 70, 290), g, kinds)
    B = special_matrix((2, 290, 68), g, kinds)
    for sr in ("max_plus", "min_plus", "max_mul"):
        check(tb, orc, sr, A, B, f"value only special {sr}", argmax=False)
    Z = torch.where(torch.rand(1, 64, 64, generator=g) < 0.5, -0.0, 0.0)
    Bz = torch.full((1, 64, 64), -0.0)
    for sr in ("max_plus", "min_plus"):
        check(tb, orc, sr, Z, Bz, f"value only signed zeros {sr}", argmax=False)


def test_value_only_workload2_full(tb, orc):
    A, B = inputs.gemm_operands(2)
    check(tb, orc, "max_plus", A, B, "workload 2 value only", argmax=False)


# ---------------------------------------------------------------------------
# split K (tropical_gemm_strided_batched_ws): few output tiles, long K
# ---------------------------------------------------------------------------

def gpu_gemm_ws(tb, sr, A, B, argmax=True, workspace=None):
    from gpu_util import device_copy
    Ad, Bd = device_copy(A), device_copy(B)
    b, m, _ = A.shape
    n = B.shape[2]
    C = torch.empty(b, m, n, dtype=A.dtype, device=DEV)
    I = torch.empty(b, m, n, dtype=torch.int32, device=DEV) if argmax else None
    tb.tropical_gemm_strided_batched_ws(sr, Ad, Bd, C, I, workspace=workspace)
    torch.cuda.synchronize()
    return C.cpu().numpy(), (I.cpu().numpy() if argmax else None)


SPLIT_SHAPES = [(1, 64, 8192, 64), (1, 17, 5000, 33), (3, 70, 3000, 50), (1, 1, 20000, 1),
                (2, 64, 4096, 130), (1, 5, 1024, 3), (1, 3, 700, 2), (1, 64, 65536, 64),
                # tiny products: ranges of 64 terms (K = 256 on one tile; a ragged last range)
                (1, 1, 256, 1), (1, 16, 256, 16), (2, 100, 300, 70)]


@pytest.mark.parametrize("sr,dt", PAIRS)
@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_split_k_matches_oracle(tb, orc, sr, dt, shape):
    b, m, k, n = shape
    assert tb.tropical_gemm_workspace_size(m, n, k, b) > 0, "this shape should split"
    A, B = make(sr, dt, b, m, k, n, seed=zlib.crc32(repr((sr, dt, shape)).encode()) % 10000,
                b_col=(shape[0] == 2))
    Cr, Ir = orc.gemm(sr, A.numpy(), B.numpy())
    before = dict(tb.tropical_get_stats()["launches"])
    C, I = gpu_gemm_ws(tb, sr, A, B)
    after = tb.tropical_get_stats()["launches"]
    assert after["gemm_splitk_merge"] - before["gemm_splitk_merge"] == 1
    assert_bits_equal(C, Cr, f"split {sr} {dt} {shape} C")
    assert_equal(I, Ir, f"split {sr} {dt} {shape} argmax")
    C, _ = gpu_gemm_ws(tb, sr, A, B, argmax=False)
    assert_bits_equal(C, Cr, f"split value-only {sr} {dt} {shape} C")


def test_split_k_ties_signed_zeros_and_nan_across_ranges(tb, orc):
    k = 8192
    # every term equal: the winner is k = 0, in the first range
    A = torch.zeros(1, 40, k)
    B = torch.zeros(1, k, 30)
    C, I = gpu_gemm_ws(tb, "max_plus", A, B)
    assert (I == 0).all()
    # the maximum 0 first reached as -0 in the last range and as +0 in an
    # earlier one, or the other way round: C has the first winner's bits
    for first, later in ((-0.0, 0.0), (0.0, -0.0)):
        A = torch.full((1, 8, k), -5.0)
        B = torch.full((1, k, 8), -0.0)
        A[0, :, 3000] = first
        A[0, :, k - 10] = later
        C, I = gpu_gemm_ws(tb, "max_plus", A, B)
        Cr, Ir = orc.gemm("max_plus", A.numpy(), B.numpy())
        assert_bits_equal(C, Cr, f"signed zero {first} then {later}")
        assert_equal(I, Ir, "signed zero argmax")
        assert (I == 3000).all()
    # NaN and +-inf scattered over the ranges
    g = torch.Generator().manual_seed(12)
    kinds = ["inf", "-inf", "nan", "-0", "0"]
    for sr in ("max_plus", "min_plus", "max_mul"):
        A = special_matrix((1, 30, k), g, kinds)
        B = special_matrix((1, k, 20), g, kinds)
        C, I = gpu_gemm_ws(tb, sr, A, B)
        Cr, Ir = orc.gemm(sr, A.numpy(), B.numpy())
        assert_bits_equal(C, Cr, f"special split {sr}")
        assert_equal(I, Ir, f"special split {sr} argmax")


def test_split_k_workspace_rules(tb, orc):
    A, B = make("max_plus", "f32", 1, 64, 8192, 64, seed=3)
    need = tb.tropical_gemm_workspace_size(64, 64, 8192, 1)
    assert need > 0
    # large grids and short K do not split (a large grid gets room for the
    # domain flags of the int32 float mode instead); a tiny product splits
    # into ranges of 64 terms, the others into whole 256-term blocks
    assert tb.tropical_gemm_workspace_size(256, 256, 4096, 64) == 4 * 256
    assert tb.tropical_gemm_workspace_size(64, 64, 100, 1) == 0
    assert tb.tropical_gemm_workspace_size(64, 64, 500, 1) == 2 * 4 * 64 * 64 * 4  # 4 ranges of 128
    assert tb.tropical_gemm_workspace_size(64, 64, 65536, 1) == 2 * 4 * 64 * 64 * 256  # 256 ranges of 256
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = torch.empty(1, 64, 64, device=DEV)
    with pytest.raises(tb.TropicalError) as e:
        tb.tropical_gemm_strided_batched_ws("max_plus", Ad, Bd, C,
                                            workspace=torch.empty(need - 4, dtype=torch.uint8, device=DEV))
    assert e.value.status == tb.WORKSPACE_TOO_SMALL
    # a larger workspace is fine; no workspace means no split
    Cr, Ir = orc.gemm("max_plus", A.numpy(), B.numpy())
    I = torch.empty(1, 64, 64, dtype=torch.int32, device=DEV)
    tb.tropical_gemm_strided_batched_ws("max_plus", Ad, Bd, C, I,
                                        workspace=torch.empty(need + 4096, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert_bits_equal(C.cpu().numpy(), Cr, "larger workspace")
    before = dict(tb.tropical_get_stats()["launches"])
    tb.tropical_gemm_strided_batched("max_plus", Ad, Bd, C, I)
    torch.cuda.synchronize()
    assert tb.tropical_get_stats()["launches"]["gemm_splitk_merge"] == before["gemm_splitk_merge"]
    assert_bits_equal(C.cpu().numpy(), Cr, "no workspace")
    assert_equal(I.cpu().numpy(), Ir, "no workspace argmax")


def test_int32_max_mul_saturation_and_ties(tb, orc):
    """int32 max-mul: products beyond the int32 range clamp (many terms
    then tie at INT32_MAX and the first one wins); negative and zero
    products never beat the zero element 0."""
    g = torch.Generator().manual_seed(77)
    b, m, k, n = 2, 70, 600, 66
    A = torch.randint(-3, 4, (b, m, k), generator=g, dtype=torch.int32)
    B = torch.randint(-3, 4, (b, k, n), generator=g, dtype=torch.int32)
    big = torch.tensor([46341, -46341, 65536, 1 << 30, -(1 << 30)], dtype=torch.int32)
    for X in (A, B):
        sel = torch.rand(X.shape, generator=g) < 0.1
        X[sel] = big[torch.randint(0, 5, (int(sel.sum()),), generator=g)]
    check(tb, orc, "max_mul", A, B, "int32 max-mul saturation")
    check(tb, orc, "max_mul", -A.abs(), B.abs(), "int32 max-mul all non-positive")


# ---------------------------------------------------------------------------
# int32 operands near the limits of the saturating ring: non-negative
# min-plus data with the 2^30 sentinel and values up to INT32_MAX (sums past
# 2^31 that saturate and must not win), max-plus data in [-2^30, 2^30), and
# values that break either pattern placed at 16-term chunk, 32- and 64-term
# slice and 256-term block boundaries, in some tiles and rows only.
# ---------------------------------------------------------------------------

LIMIT_POOL = {
    # non-negative pool for min-plus: sums reach 2^32 - 2, past INT32_MAX
    "min_plus": [0, 1, 2, 3, 5, 1000, I32_INF, I32_INF + 7, 2 ** 31 - 1, 2 ** 31 - 2, I32_INF - 1],
    # in-range pool for max-plus: [-2^30, 2^30 - 1]
    "max_plus": [-I32_INF, -(I32_INF - 1), -5, -1, 0, 1, 3, I32_INF - 1, I32_INF - 2],
}
LIMIT_BREAKERS = {
    "min_plus": [-1, -I32_INF, -(2 ** 31)],
    "max_plus": [I32_INF, -I32_INF - 1, 2 ** 31 - 1, -(2 ** 31)],
}


def limit_case(sr, b, m, k, n, seed, bad_k=(), bad_rows=None, in_b=False):
    g = torch.Generator().manual_seed(seed)
    pool = torch.tensor(LIMIT_POOL[sr], dtype=torch.int64)
    # mostly small values (ties), some from the whole pool
    lo = -2 if sr == "max_plus" else 0
    A = torch.randint(lo, lo + 4, (b, m, k), generator=g)
    B = torch.randint(lo, lo + 4, (b, k, n), generator=g)
    A = torch.where(torch.rand(b, m, k, generator=g) < 0.3, pool[torch.randint(0, len(pool), (b, m, k), generator=g)], A)
    B = torch.where(torch.rand(b, k, n, generator=g) < 0.3, pool[torch.randint(0, len(pool), (b, k, n), generator=g)], B)
    A, B = A.to(torch.int32), B.to(torch.int32)
    brk = LIMIT_BREAKERS[sr]
    for t, kk in enumerate(bad_k):
        v = brk[t % len(brk)]
        if in_b:
            cols = bad_rows if bad_rows is not None else range(n)
            for j in cols:
                B[:, kk, j] = v
        else:
            rows = bad_rows if bad_rows is not None else range(m)
            for i in rows:
                A[:, i, kk] = v
    return A, B


LIMIT_CASES = [
    # (name, (b, m, k, n), bad k positions, rows / columns that get them, in B)
    ("clean", (2, 70, 300, 90), (), None, False),
    ("first_term", (1, 70, 300, 90), (0,), [5], False),
    ("slice3_some_rows", (1, 130, 300, 70), (200,), [3, 100], False),
    ("vo_slice_edges", (1, 64, 260, 64), (31, 32, 63, 64), [0], True),
    ("last_term", (2, 65, 257, 66), (256,), [64], True),
    ("every_block", (1, 40, 700, 40), (255, 256, 511), None, False),
]


@pytest.mark.parametrize("sr", ["min_plus", "max_plus"])
@pytest.mark.parametrize("case", LIMIT_CASES, ids=lambda c: c[0])
def test_int32_limit_patterns(tb, orc, sr, case):
    name, (b, m, k, n), bad_k, rows, in_b = case
    A, B = limit_case(sr, b, m, k, n, seed=zlib.crc32(repr((sr, name)).encode()) % 10000,
                     bad_k=bad_k, bad_rows=rows, in_b=in_b)
    check(tb, orc, sr, A, B, f"int32 limits {sr} {name}")
    check(tb, orc, sr, A, B, f"int32 limits {sr} {name} value only", argmax=False)


@pytest.mark.parametrize("sr", ["min_plus", "max_plus"])
def test_int32_limit_patterns_split_k(tb, orc, sr):
    # long K over few tiles: split-K ranges, with a pattern-breaking value inside one range
    for bad_k in ((), (1500,), (0, 3999)):
        A, B = limit_case(sr, 1, 17, 4000, 33, seed=71 + len(bad_k), bad_k=bad_k, bad_rows=[0, 16])
        assert tb.tropical_gemm_workspace_size(17, 33, 4000, 1) > 0
        Cr, Ir = orc.gemm(sr, A.numpy(), B.numpy())
        C, I = gpu_gemm_ws(tb, sr, A, B)
        assert_bits_equal(C, Cr, f"split int32 limits {sr} {bad_k} C")
        assert_equal(I, Ir, f"split int32 limits {sr} {bad_k} argmax")
        C, _ = gpu_gemm_ws(tb, sr, A, B, argmax=False)
        assert_bits_equal(C, Cr, f"split int32 limits {sr} {bad_k} value-only C")



# ---------------------------------------------------------------------------
# float mode of int32 max-plus / min-plus (tropical_gemm_strided_batched_ws
# and the contraction paths, whose workspace holds the domain pre-pass's
# flags): min-plus data in [0, 2^23) or [2^30, 2^31), max-plus data in
# (-2^23, 2^23) are computed in float; one value outside sends the product to
# the int32 kernel.  Either way every output and argmax matches the oracle.
# ---------------------------------------------------------------------------

FM_POOL = {
    "min_plus": [0, 1, 2, 3, 999, 2 ** 23 - 2, 2 ** 23 - 1, I32_INF, I32_INF + 5, 2 ** 31 - 1],
    "max_plus": [-(2 ** 23) + 1, -(2 ** 23) + 2, -5, -1, 0, 1, 3, 2 ** 23 - 2, 2 ** 23 - 1],
}
FM_OUTSIDE = {
    "min_plus": [-1, 2 ** 23, I32_INF - 1, -(2 ** 31)],
    "max_plus": [2 ** 23, -(2 ** 23), I32_INF, -I32_INF, 2 ** 31 - 1],
}
FM_SLOTS = 256  # domain flags at the start of the workspace


def fm_case(sr, b, m, k, n, seed, outside=None, in_b=False, b_col=False):
    g = torch.Generator().manual_seed(seed)
    pool = torch.tensor(FM_POOL[sr], dtype=torch.int64)
    lo = -2 if sr == "max_plus" else 0
    A = torch.randint(lo, lo + 5, (b, m, k), generator=g)
    B = torch.randint(lo, lo + 5, (b, k, n), generator=g)
    A = torch.where(torch.rand(b, m, k, generator=g) < 0.2, pool[torch.randint(0, len(pool), (b, m, k), generator=g)], A)
    B = torch.where(torch.rand(b, k, n, generator=g) < 0.2, pool[torch.randint(0, len(pool), (b, k, n), generator=g)], B)
    A, B = A.to(torch.int32), B.to(torch.int32)
    if outside is not None:
        X = B if in_b else A
        pos = tuple(int(torch.randint(0, d, (1,), generator=g)) for d in X.shape)
        X[pos] = outside
    if b_col:
        B = B.transpose(1, 2).contiguous().transpose(1, 2)
    return A, B


def gpu_gemm_fm(tb, sr, A, B, argmax=True):
    """The product through the workspace call; returns (C, I, flags)."""
    from gpu_util import device_copy
    Ad, Bd = device_copy(A), device_copy(B)
    b, m, k = A.shape
    n = B.shape[2]
    ws = torch.zeros(max(4, tb.tropical_gemm_workspace_size_strided(Ad, Bd, argmax)), dtype=torch.uint8, device=DEV)
    C = torch.empty(b, m, n, dtype=torch.int32, device=DEV)
    I = torch.empty(b, m, n, dtype=torch.int32, device=DEV) if argmax else None
    tb.tropical_gemm_strided_batched_ws(sr, Ad, Bd, C, I, workspace=ws)
    torch.cuda.synchronize()
    flags = ws[:4 * FM_SLOTS].view(torch.int32).cpu().numpy() if ws.numel() >= 4 * FM_SLOTS else None
    return C.cpu().numpy(), (I.cpu().numpy() if argmax else None), flags


@pytest.mark.parametrize("sr", ["min_plus", "max_plus"])
@pytest.mark.parametrize("outside", [None, 0, 1, 2, 3], ids=lambda o: "inside" if o is None else f"outside{o}")
@pytest.mark.parametrize("argmax", [True, False])
def test_int32_float_mode(tb, orc, monkeypatch, sr, outside, argmax):
    monkeypatch.setenv("TROPICAL_GEMM_INT_FLOAT", "1")  # at any size
    # (no split-K, whose partials would take the workspace: these products
    # are small enough for ranges of 64 terms otherwise)
    monkeypatch.setenv("TROPICAL_SPLITK_TINY", "0")
    for shape, in_b, b_col in (((2, 130, 480, 90), False, False), ((1, 70, 500, 130), True, True),
                               ((3, 65, 17, 63), False, True)):
        v = None if outside is None else FM_OUTSIDE[sr][outside % len(FM_OUTSIDE[sr])]
        A, B = fm_case(sr, *shape, seed=sum(shape) + (outside or 0), outside=v, in_b=in_b, b_col=b_col)
        C, I, flags = gpu_gemm_fm(tb, sr, A, B, argmax)
        assert flags is not None
        # the pre-pass saw what the data holds
        assert (flags == 0).all() if v is None else (flags != 0).any(), (shape, v)
        Cr, Ir = orc.gemm(sr, A.numpy(), B.numpy(), argmax=argmax)
        assert_equal(C, Cr, f"float mode {sr} {shape} outside={v} C")
        if argmax:
            assert_equal(I, Ir, f"float mode {sr} {shape} outside={v} argmax")


def test_int32_float_mode_off_and_sizes(tb, orc, monkeypatch):
    # never taken with the knob at 0 (no workspace asked for small products
    # either, split-K ranges of 64 terms off); taken for large ones without
    # the knob
    monkeypatch.setenv("TROPICAL_SPLITK_TINY", "0")
    monkeypatch.setenv("TROPICAL_GEMM_INT_FLOAT", "0")
    assert tb.tropical_gemm_workspace_size(130, 90, 480, 2) == 0
    A, B = fm_case("min_plus", 2, 130, 480, 90, seed=5)
    C, I, flags = gpu_gemm_fm(tb, "min_plus", A, B)
    assert flags is None
    Cr, Ir = orc.gemm("min_plus", A.numpy(), B.numpy())
    assert_equal(C, Cr, "knob 0 C")
    assert_equal(I, Ir, "knob 0 argmax")
    monkeypatch.delenv("TROPICAL_GEMM_INT_FLOAT")
    assert tb.tropical_gemm_workspace_size(130, 90, 480, 2) == 0
    assert tb.tropical_gemm_workspace_size(4096, 4096, 4096, 1) == 4 * FM_SLOTS


def test_workload3_full_float_mode(tb, orc):
    # workload 3 (min-plus int32 4096^3, U{1..1000} with 20% 2^30) is in the
    # float domain: through the workspace call, every output against the oracle
    A, B, Cr, Ir = _full_reference(orc, 3)
    C, I, flags = gpu_gemm_fm(tb, "min_plus", A, B)
    assert flags is not None and (flags == 0).all()
    assert_equal(C, Cr, "workload 3 float mode C")
    assert_equal(I, Ir, "workload 3 float mode argmin")


def test_int32_float_mode_in_contractions(tb, orc, monkeypatch):
    monkeypatch.setenv("TROPICAL_GEMM_INT_FLOAT", "1")
    monkeypatch.setenv("TROPICAL_SPLITK_TINY", "0")  # (else these split into 64-term ranges)
    for sr, outside in (("min_plus", None), ("max_plus", None), ("min_plus", -1), ("max_plus", 2 ** 23)):
        A, B = fm_case(sr, 3, 70, 300, 50, seed=61, outside=outside)
        for spec in ("bij,bjk->bik", "bij,bjk->kbi"):
            C, I = tb.tropical_contract_pair(spec, sr, A.to(DEV), B.to(DEV))
            torch.cuda.synchronize()
            Cr, Ir = orc.contract_pair(spec, sr, A.numpy(), B.numpy())
            assert_equal(C.cpu().numpy(), Cr, f"contraction {spec} {sr} outside={outside} C")
            assert_equal(I.cpu().numpy(), Ir, f"contraction {spec} {sr} outside={outside} argmax")
