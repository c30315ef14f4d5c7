"""The short-K GEMM kernel (K <= 16; 192..256 columns and at least 32768
rows in all, or 128..191 columns and at least 65536 rows): B held in registers, rows of A streamed.  Every case is compared
bit for bit with the oracle, values and argmax, over semirings, dtypes,
operand layouts, ragged rows, K at its ends, special values and int32
limits; the same products with the kernel switched off give the same
bits."""
import pytest
import torch

from gpu_util import DEV, assert_bits_equal, assert_equal, device_copy

pytestmark = pytest.mark.gpu

I32_INF = 1 << 30
PAIRS = [("max_plus", "f32"), ("min_plus", "f32"), ("max_mul", "f32"),
         ("max_plus", "i32"), ("min_plus", "i32"), ("max_mul", "i32")]


@pytest.fixture(scope="module")
def tb():
    from tropical_semiring_tensor_amd import binding
    binding.tropical_init(0)
    return binding


def make(sr, dt, b, m, k, n, seed):
    g = torch.Generator().manual_seed(seed)
    if dt == "i32":
        A = torch.randint(-20, 21, (b, m, k), generator=g, dtype=torch.int32)
        B = torch.randint(-20, 21, (b, k, n), generator=g, dtype=torch.int32)
        if sr == "max_mul":
            A, B = A.abs(), B.abs()
        z = {"max_plus": -I32_INF, "min_plus": I32_INF, "max_mul": 0}[sr]
        A[torch.rand(A.shape, generator=g) < 0.1] = z
        B[torch.rand(B.shape, generator=g) < 0.1] = z
        return A, B
    if sr == "max_mul":
        return (torch.randint(0, 9, (b, m, k), generator=g).float() * 0.125,
                torch.randint(0, 9, (b, k, n), generator=g).float() * 0.25)
    return (torch.randint(-6, 7, (b, m, k), generator=g).float(),
            torch.randint(-6, 7, (b, k, n), generator=g).float())


def gemm(tb, sr, A, B, argmax=True):
    Ad, Bd = device_copy(A), device_copy(B)
    b, m, _ = A.shape
    n = B.shape[2]
    C = torch.empty(b, m, n, dtype=A.dtype, device=DEV)
    I = torch.empty(b, m, n, dtype=torch.int32, device=DEV) if argmax else None
    tb.tropical_gemm_strided_batched(sr, Ad, Bd, C, I)
    torch.cuda.synchronize()
    return C.cpu().numpy(), (I.cpu().numpy() if argmax else None)


def check(tb, orc, sr, A, B, what, argmax=True):
    C, I = gemm(tb, sr, A, B, argmax)
    Cr, Ir = orc.gemm(sr, A.numpy(), B.numpy(), argmax=argmax)
    if A.dtype == torch.int32:
        assert_equal(C, Cr, what + " C")
    else:
        assert_bits_equal(C, Cr, what + " C")
    if argmax:
        assert_equal(I, Ir, what + " argmax")


SHAPES = [(1, 32768, 16, 256), (1, 32801, 1, 196), (2, 16411, 15, 252), (3, 11000, 2, 200),
          # 128..191 columns: two rows per wave's lane groups
          (1, 65600, 8, 132), (2, 32800, 3, 128)]


@pytest.mark.parametrize("argmax", [True, False], ids=["argmax", "value_only"])
@pytest.mark.parametrize("sr,dt", PAIRS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_short_k_matches_oracle(tb, orc, sr, dt, shape, argmax):
    b, m, k, n = shape
    A, B = make(sr, dt, b, m, k, n, seed=sum(shape) + len(sr))
    check(tb, orc, sr, A, B, f"{sr} {dt} {shape}", argmax=argmax)


@pytest.mark.parametrize("layout", ["colA", "colB", "colA_colB", "strided"])
def test_short_k_layouts(tb, orc, layout):
    b, m, k, n = 2, 16400, 16, 256
    A, B = make("max_plus", "f32", b, m, k, n, seed=3)
    if "colA" in layout:
        A = A.transpose(1, 2).contiguous().transpose(1, 2)
    if "colB" in layout:
        B = B.transpose(1, 2).contiguous().transpose(1, 2)
    if layout == "strided":  # every other row of a larger A, every other k of a larger B
        A = make("max_plus", "f32", b, 2 * m, k, n, seed=4)[0][:, ::2]
        B = torch.cat([B, B], dim=1)[:, ::2]
    check(tb, orc, "max_plus", A, B, layout)
    check(tb, orc, "max_plus", A, B, layout + " value only", argmax=False)


def test_short_k_special_values_and_signed_zeros(tb, orc):
    g = torch.Generator().manual_seed(9)
    b, m, k, n = 1, 32768, 16, 256
    vals = torch.tensor([0.0, -0.0, 1.0, -1.0, float("inf"), float("-inf"), float("nan")])
    for sr in ("max_plus", "min_plus", "max_mul"):
        A = vals[torch.randint(0, len(vals), (b, m, k), generator=g)]
        B = vals[torch.randint(0, len(vals), (b, k, n), generator=g)]
        check(tb, orc, sr, A, B, f"{sr} special values")


def test_short_k_int32_saturation(tb, orc):
    g = torch.Generator().manual_seed(10)
    b, m, k, n = 1, 32768, 16, 256
    big = torch.tensor([2 ** 31 - 1, -2 ** 31, 2 ** 30, -2 ** 30, 1, -1, 0], dtype=torch.int32)
    A = big[torch.randint(0, len(big), (b, m, k), generator=g)]
    B = big[torch.randint(0, len(big), (b, k, n), generator=g)]
    for sr in ("max_plus", "min_plus"):
        check(tb, orc, sr, A, B, f"{sr} int32 limits")


def test_short_k_same_bits_as_the_tiled_kernel(tb, orc, monkeypatch):
    A, B = make("min_plus", "f32", 1, 65536, 16, 256, seed=12)
    C1, I1 = gemm(tb, "min_plus", A, B)
    monkeypatch.setenv("TROPICAL_GEMM_SMALLK", "0")
    C2, I2 = gemm(tb, "min_plus", A, B)
    assert_bits_equal(C1, C2, "short-K vs tiled C")
    assert_equal(I1, I2, "short-K vs tiled argmax")
    # sampled rows of the full product against the oracle
    rows = torch.randint(0, 65536, (64,), generator=torch.Generator().manual_seed(13))
    Cr, Ir = orc.gemm("min_plus", A[:, rows].numpy(), B.numpy())
    assert_bits_equal(C1[:, rows.numpy()], Cr, "sampled rows C")
    assert_equal(I1[:, rows.numpy()], Ir, "sampled rows argmax")


def test_two_level_k_through_a_contraction(tb, orc):
    """K = 2 x 8 read with a two-level k (the running result of a lattice
    network), 256 columns."""
    spec = "vwe,veA->wA"
    g = torch.Generator().manual_seed(14)
    A = torch.randint(-6, 7, (2, 32800, 8), generator=g).float()
    B = torch.randint(-6, 7, (2, 8, 256), generator=g).float()
    assert "A=fold:krun8" in tb.tropical_contract_pair_describe(spec, A.shape, B.shape)
    C, I = tb.tropical_contract_pair(spec, "max_plus", A.to(DEV), B.to(DEV))
    torch.cuda.synchronize()
    Cr, Ir = orc.contract_pair(spec, "max_plus", A.numpy(), B.numpy())
    assert_bits_equal(C.cpu().numpy(), Cr, "two-level k C")
    assert_equal(I.cpu().numpy(), Ir, "two-level k argmax")
