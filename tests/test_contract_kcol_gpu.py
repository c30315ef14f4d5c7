"""Contractions with a long K: the GEMM's right operand is gathered with k
at unit stride (":kcol" in the plan) where it would otherwise be read with
its free index at unit stride, so that the product reads both operands
along k.  Each case is compared bit for bit with the oracle's decomposed
pipeline, values and argmax, including an argmax routed through a pre-pass
reduction of the gathered operand (its winners then lie in the gathered
order) and a product taken as B (x) A.  Small integer entries make ties
common."""
import pytest
import torch

from gpu_util import DEV, assert_bits_equal, assert_equal

pytestmark = pytest.mark.gpu

# (spec, shape A, shape B, operand gathered along k): more than 256 output
# tiles (never split along K), K = 260 or 264
CASES = [
    ("ij,jk->ik", (1100, 260), (260, 1000), "B"),
    ("bij,bjk->bik", (3, 700, 264), (3, 264, 650), "B"),
    ("ij,jkl->ik", (1100, 260), (260, 1000, 3), "B"),      # B's l reduced: winners routed
    ("ji,kj->ki", (260, 1100), (1000, 260), "A"),          # taken as B (x) A
    ("jil,kj->ki", (260, 1100, 2), (1000, 260), "A"),      # ... with A's l reduced
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
    spec, sa, sb, side = case
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "1")  # at any size
    desc = tb.tropical_contract_pair_describe(spec, sa, sb)
    assert f"{side}=gather:" in desc and ":kcol" in desc, desc
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
