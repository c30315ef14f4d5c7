"""Operands copied transposed into the workspace: an argmax product with
K > 256 (a multiple of 4) copies a row-major B (when A is read along k) and
a column-major A, and then reads both operands along k, as for a row-major
A and a column-major B.  Each case is compared bit for bit with
the oracle, and the copy is checked to hold B with k as its unit-stride
axis (so the path under test ran); a workspace of the split / float-mode
size gets no copy and the same bits.  Small integer entries make ties
common, so the first-winner order along k is exercised."""
import pytest
import torch

from gpu_util import DEV, assert_bits_equal, assert_equal

pytestmark = pytest.mark.gpu

BT_OFF = 1024  # the copy follows the int32 float mode's flags
FM_SLOTS = 256

# (semiring, dtype, batch, m, k, n): more than 256 output tiles, so never
# split along K; ragged m and n, K not a multiple of 16 or 64
CASES = [
    ("max_plus", "f32", 43, 130, 260, 90),
    ("min_plus", "f32", 43, 130, 260, 90),
    ("max_mul", "f32", 43, 130, 260, 90),
    ("max_plus", "i32", 43, 130, 260, 90),
    ("min_plus", "i32", 43, 130, 260, 90),
    ("max_plus", "f32", 11, 260, 1028, 300),
    ("min_plus", "i32", 11, 260, 1028, 300),
    ("max_mul", "i32", 43, 130, 260, 90),
]


@pytest.fixture(scope="module")
def tb():
    from tropical_semiring_tensor_amd import binding
    binding.tropical_init(0)
    return binding


def operands(sr, dt, b, m, k, n, seed):
    g = torch.Generator().manual_seed(seed)
    if dt == "i32":
        A = torch.randint(-20, 21, (b, m, k), generator=g, dtype=torch.int32)
        B = torch.randint(-20, 21, (b, k, n), generator=g, dtype=torch.int32)
        if sr == "min_plus":
            A, B = A.abs(), B.abs()
            B[torch.rand(B.shape, generator=g) < 0.2] = 1 << 30
        if sr == "max_mul":
            A, B = A.abs(), B.abs()
        return A, B
    if sr == "max_mul":
        return (torch.randint(1, 9, (b, m, k), generator=g).float() * 0.125,
                torch.randint(1, 9, (b, k, n), generator=g).float() * 0.25)
    return (torch.randint(-6, 7, (b, m, k), generator=g).float(),
            torch.randint(-6, 7, (b, k, n), generator=g).float())


def copy_bytes(b, k, n):
    return BT_OFF + -(-(b * k * n * 4) // 256) * 256


def run(tb, sr, Ad, Bd, ws, argmax=True):
    b, m, _ = Ad.shape
    n = Bd.shape[2]
    C = torch.empty(b, m, n, dtype=Ad.dtype, device=DEV)
    I = torch.empty(b, m, n, dtype=torch.int32, device=DEV) if argmax else None
    tb.tropical_gemm_strided_batched_ws(sr, Ad, Bd, C, I, workspace=ws)
    torch.cuda.synchronize()
    return C, I


def copy_of_b(ws, b, k, n):
    return ws[BT_OFF:BT_OFF + b * k * n * 4].view(torch.int32).view(b, n, k).cpu()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "_".join(map(str, c)))
def test_transposed_copy_matches_oracle(tb, orc, monkeypatch, case):
    sr, dt, b, m, k, n = case
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "1")  # at any size
    A, B = operands(sr, dt, b, m, k, n, seed=b + m + k + n)
    Ad, Bd = A.to(DEV), B.to(DEV)
    nb = tb.tropical_gemm_workspace_size_strided(Ad, Bd)
    assert nb == max(tb.tropical_gemm_workspace_size(m, n, k, b), copy_bytes(b, k, n))
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    C, I = run(tb, sr, Ad, Bd, ws)
    assert torch.equal(copy_of_b(ws, b, k, n), B.view(torch.int32).transpose(1, 2))
    Cr, Ir = orc.gemm(sr, A.numpy(), B.numpy())
    assert_bits_equal(C.cpu().numpy(), Cr, f"{case} C")
    assert_equal(I.cpu().numpy(), Ir, f"{case} argmax")
    # the split / float-mode workspace and no workspace: no copy, same bits
    small = torch.zeros(max(4, tb.tropical_gemm_workspace_size(m, n, k, b)), dtype=torch.uint8, device=DEV)
    C2, I2 = run(tb, sr, Ad, Bd, small)
    C3 = torch.empty_like(C)
    I3 = torch.empty_like(I)
    tb.tropical_gemm_strided_batched(sr, Ad, Bd, C3, I3)
    torch.cuda.synchronize()
    for Cx, Ix in ((C2, I2), (C3, I3)):
        assert torch.equal(Cx.view(torch.int32), C.view(torch.int32)) and torch.equal(Ix, I)


@pytest.mark.parametrize("sr", ["min_plus", "max_plus"])
def test_transposed_copy_with_int32_float_mode(tb, orc, monkeypatch, sr):
    """The float mode's flags (the workspace's first KiB) and the copy side
    by side: the data lie in the float-exact domain, so the float-mode
    kernel computes, reading the copy."""
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "1")
    monkeypatch.setenv("TROPICAL_GEMM_INT_FLOAT", "1")
    b, m, k, n = 43, 130, 260, 90
    A, B = operands(sr, "i32", b, m, k, n, seed=3)
    Ad, Bd = A.to(DEV), B.to(DEV)
    ws = torch.full((tb.tropical_gemm_workspace_size_strided(Ad, Bd),), 7, dtype=torch.uint8, device=DEV)
    C, I = run(tb, sr, Ad, Bd, ws)
    assert (ws[:4 * FM_SLOTS].view(torch.int32) == 0).all()
    assert torch.equal(copy_of_b(ws, b, k, n), B.transpose(1, 2))
    Cr, Ir = orc.gemm(sr, A.numpy(), B.numpy())
    assert_equal(C.cpu().numpy(), Cr, f"{sr} float mode C")
    assert_equal(I.cpu().numpy(), Ir, f"{sr} float mode argmax")


def test_no_copy_without_argmax_or_with_the_knob_off(tb, orc, monkeypatch):
    b, m, k, n = 43, 130, 260, 90
    A, B = operands("max_plus", "f32", b, m, k, n, seed=4)
    Ad, Bd = A.to(DEV), B.to(DEV)
    Cr, _ = orc.gemm("max_plus", A.numpy(), B.numpy(), argmax=False)
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "1")
    ws = torch.zeros(copy_bytes(b, k, n), dtype=torch.uint8, device=DEV)
    C, _ = run(tb, "max_plus", Ad, Bd, ws, argmax=False)  # value only
    assert not ws.any()
    assert_bits_equal(C.cpu().numpy(), Cr, "value only")
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "0")
    C, I = run(tb, "max_plus", Ad, Bd, ws)
    assert not ws.any()
    assert_bits_equal(C.cpu().numpy(), Cr, "knob 0")



def test_transposed_copy_of_a_broadcast_b(tb, orc, monkeypatch):
    """B shared by every batch entry (batch stride 0): the copy holds one
    transposed B per entry, and the results match the oracle."""
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "1")
    b, m, k, n = 43, 130, 260, 90
    A, B = operands("max_plus", "f32", b, m, k, n, seed=5)
    B1 = B[:1].contiguous()
    Ad, Bd = A.to(DEV), B1.to(DEV).expand(b, k, n)
    assert Bd.stride(0) == 0
    ws = torch.zeros(tb.tropical_gemm_workspace_size_strided(Ad, Bd), dtype=torch.uint8, device=DEV)
    C, I = run(tb, "max_plus", Ad, Bd, ws)
    assert torch.equal(copy_of_b(ws, b, k, n), B1.expand(b, k, n).view(torch.int32).transpose(1, 2))
    Cr, Ir = orc.gemm("max_plus", A.numpy(), B1.expand(b, k, n).contiguous().numpy())
    assert_bits_equal(C.cpu().numpy(), Cr, "broadcast B C")
    assert_equal(I.cpu().numpy(), Ir, "broadcast B argmax")


@pytest.mark.parametrize("b_col", [False, True], ids=["rowB", "colB"])
@pytest.mark.parametrize("sr,dt", [("max_plus", "f32"), ("min_plus", "i32"), ("max_mul", "f32")])
def test_transposed_copy_of_a_column_major_a(tb, orc, monkeypatch, sr, dt, b_col):
    """A column-major A (i unit-stride) is copied as (batch, m, k) after B's
    copy (when B is row-major, it is copied too): both then read along k."""
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "1")
    b, m, k, n = 43, 130, 264, 90
    A, B = operands(sr, dt, b, m, k, n, seed=21 + b_col)
    Ad = A.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    Bd = B.transpose(1, 2).contiguous().to(DEV).transpose(1, 2) if b_col else B.to(DEV)
    a_off = BT_OFF if b_col else copy_bytes(b, k, n)
    nb = tb.tropical_gemm_workspace_size_strided(Ad, Bd)
    assert nb == a_off + -(-(b * m * k * 4) // 256) * 256
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    C, I = run(tb, sr, Ad, Bd, ws)
    a_copy = ws[a_off:a_off + b * m * k * 4].view(torch.int32).view(b, m, k).cpu()
    assert torch.equal(a_copy, A.view(torch.int32))
    if not b_col:
        assert torch.equal(copy_of_b(ws, b, k, n), B.view(torch.int32).transpose(1, 2))
    Cr, Ir = orc.gemm(sr, A.numpy(), B.numpy())
    if dt == "i32":
        assert_equal(C.cpu().numpy(), Cr, f"{sr} column-major A C")
    else:
        assert_bits_equal(C.cpu().numpy(), Cr, f"{sr} column-major A C")
    assert_equal(I.cpu().numpy(), Ir, f"{sr} column-major A argmax")


def test_value_only_copies_a_column_major_a(tb, orc, monkeypatch):
    """Without an argmax output only a column-major A is copied (a row-major
    B is read in place)."""
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "1")
    b, m, k, n = 43, 130, 264, 90
    A, B = operands("min_plus", "f32", b, m, k, n, seed=31)
    Ad = A.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    Bd = B.to(DEV)
    nb = tb.tropical_gemm_workspace_size_strided(Ad, Bd, with_argmax=False)
    assert nb == copy_bytes(b, k, m)
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    C, _ = run(tb, "min_plus", Ad, Bd, ws, argmax=False)
    assert torch.equal(ws[BT_OFF:BT_OFF + b * m * k * 4].view(torch.int32).view(b, m, k).cpu(), A.view(torch.int32))
    Cr, _ = orc.gemm("min_plus", A.numpy(), B.numpy(), argmax=False)
    assert_bits_equal(C.cpu().numpy(), Cr, "value only, column-major A")
