"""Contractions with a long K: the GEMM reads both operands along k.  An
operand that would be read with its free index at unit stride is gathered
with k at unit stride instead (the left one in (batch, rows, contracted)
order, the right one in (batch, cols, contracted) order, ":kcol" in the
plan).  Each case is compared bit for bit with the oracle's decomposed
pipeline, values and argmax, including an argmax routed through a pre-pass
reduction of the gathered operand (its winners then lie in the gathered
order) and a product taken as B (x) A.  Small integer entries make ties
common."""
import pytest
import torch

from gpu_util import DEV, assert_bits_equal, assert_equal

pytestmark = pytest.mark.gpu

# (spec, shape A, shape B, what the plan reads): more than 256 output tiles
# (never split along K), K = 260 or 264
CASES = [
    ("ij,jk->ik", (1100, 260), (260, 1000), "A=fold B=gather:tiled:kcol"),
    ("bij,bjk->bik", (3, 700, 264), (3, 264, 650), "A=fold B=gather:flat:kcol"),
    ("ij,jkl->ik", (1100, 260), (260, 1000, 3), "A=fold B=gather:reduce:kcol"),  # B's l reduced: winners routed
    ("ji,kj->ki", (260, 1100), (1000, 260), "A=gather:tiled:kcol B=fold"),  # taken as B (x) A
    ("jil,kj->ki", (260, 1100, 2), (1000, 260), "A=gather:reduce:kcol B=fold"),  # ... with A's l reduced
    ("ji,kj->ik", (260, 1100), (1000, 260), "A=gather:tiled B=fold"),  # A gathered along k
    ("ji,jk->ik", (260, 1100), (260, 1000), "A=gather:tiled B=gather:tiled:kcol"),  # both
    ("bjil,bjk->bik", (2, 264, 700, 2), (2, 264, 650), "A=gather:reduce B=gather:flat:kcol"),  # A reduced
]


@pytest.fixture(scope="module")
def tb():
    from tropical_semiring_tensor_amd import binding
    binding.tropical_init(0)
    return binding


def operands(sr, sa, sb, seed):
    g = torch.Generator().manual_seed(seed)
    if sr == "max_mul":
        return (torch.randint(1, 9, sa, generator=g).float() * 0.125,
                torch.randint(1, 9, sb, generator=g).float() * 0.25)
    return torch.randint(-6, 7, sa, generator=g).float(), torch.randint(-6, 7, sb, generator=g).float()


@pytest.mark.parametrize("sr", ["max_plus", "min_plus", "max_mul"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_right_operand_gathered_along_k(tb, orc, monkeypatch, sr, case):
    spec, sa, sb, how = case
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "1")  # at any size
    desc = tb.tropical_contract_pair_describe(spec, sa, sb)
    assert how in desc, desc
    A, B = operands(sr, sa, sb, seed=sum(sa) + sum(sb))
    for argmax in (True, False):
        C, I = tb.tropical_contract_pair(spec, sr, A.to(DEV), B.to(DEV), argmax=argmax)
        torch.cuda.synchronize()
        Cr, Ir = orc.contract_pair(spec, sr, A.numpy(), B.numpy(), argmax=argmax)
        assert_bits_equal(C.cpu().numpy(), Cr, f"{spec} {sr} C")
        if argmax:
            assert_equal(I.cpu().numpy(), Ir, f"{spec} {sr} argmax")


def test_same_bits_as_the_row_major_read(tb, orc, monkeypatch):
    spec, sa, sb = "ij,jk->ik", (1100, 264), (264, 1000)
    A, B = operands("max_plus", sa, sb, seed=9)
    Ad, Bd = A.to(DEV), B.to(DEV)
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "1")
    C1, I1 = tb.tropical_contract_pair(spec, "max_plus", Ad, Bd)
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "0")
    assert "B=fold" in tb.tropical_contract_pair_describe(spec, sa, sb)
    C2, I2 = tb.tropical_contract_pair(spec, "max_plus", Ad, Bd)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32)) and torch.equal(I1, I2)


def test_allocation_free_call_gathers_along_k_too(tb, monkeypatch):
    """The allocation-free call runs the same plan from its own scratch."""
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "1")
    for spec, sa, sb in (("ji,jk->ik", (260, 1100), (260, 1000)), ("ij,jk->ik", (1100, 264), (264, 1000))):
        A, B = operands("max_plus", sa, sb, seed=11)
        Ad, Bd = A.to(DEV), B.to(DEV)
        Cw, Iw = tb.tropical_contract_pair(spec, "max_plus", Ad, Bd)
        C = torch.full(Cw.shape, -7.0, device=DEV)
        I = torch.full(Cw.shape, -7, dtype=torch.int32, device=DEV)
        tb.tropical_contract_pair_noalloc(spec, "max_plus", Ad, Bd, C, I)
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int32), Cw.view(torch.int32)) and torch.equal(I, Iw), spec


@pytest.mark.parametrize("float_mode", ["0", "1"])
@pytest.mark.parametrize("sr", ["max_plus", "min_plus", "max_mul"])
def test_int32_operands_gathered_along_k(tb, orc, monkeypatch, sr, float_mode):
    """int32 operands gathered along k, with the int32 kernel or (max-plus,
    min-plus) the float mode, whose flags share the GEMM's workspace."""
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "1")
    monkeypatch.setenv("TROPICAL_GEMM_INT_FLOAT", float_mode)
    spec, sa, sb = "ji,jk->ik", (260, 1100), (260, 1000)
    assert "A=gather:tiled B=gather:tiled:kcol" in tb.tropical_contract_pair_describe(spec, sa, sb)
    g = torch.Generator().manual_seed(41)
    lo = 0 if sr != "max_plus" else -9
    A = torch.randint(lo, 10, sa, generator=g, dtype=torch.int32)
    B = torch.randint(lo, 10, sb, generator=g, dtype=torch.int32)
    C, I = tb.tropical_contract_pair(spec, sr, A.to(DEV), B.to(DEV))
    torch.cuda.synchronize()
    Cr, Ir = orc.contract_pair(spec, sr, A.numpy(), B.numpy())
    assert_equal(C.cpu().numpy(), Cr, f"{sr} int32 C")
    assert_equal(I.cpu().numpy(), Ir, f"{sr} int32 argmax")
