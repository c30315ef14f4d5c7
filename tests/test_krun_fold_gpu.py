"""Operands read in place with a two-level k: the contracted labels lie on
both sides of the free ones (e.g. the running result of a lattice network,
whose first and last axes are contracted with the next site), so k =
outer index * run + inner index with the inner labels at unit stride.  The
GEMM reads such an operand without a gathered copy.  Every case is compared
bit for bit with the oracle's decomposed pipeline, under each GEMM setting
and the element-wise kernel; small integer entries make ties common, so the
first-winner order along the split k is exercised."""
import pytest
import torch

from gpu_util import DEV, assert_bits_equal, assert_equal

pytestmark = pytest.mark.gpu

# (spec, shapes, GEMM operand read with a two-level k, run)
KRUN_SPECS = [
    # the lattice-network step, ragged K (48) against the 32-term slices
    ("vwxyze,veAf->wxyzAf", [(3, 5, 4, 3, 7, 16), (3, 16, 6, 5)], "A", 16),
    ("vwe,veA->wA", [(5, 70, 8), (5, 8, 66)], "A", 8),
    ("vwe,veA->wA", [(9, 70, 4), (9, 4, 66)], "A", 4),
    # a run of two inner labels, an outer group of two labels
    ("vwef,vefA->wA", [(3, 33, 2, 8), (3, 2, 8, 40)], "A", 16),
    ("uvwe,uveA->wA", [(2, 3, 65, 16), (2, 3, 16, 20)], "A", 16),
    # the GEMM's right operand, both operands, the B (x) A orientation
    ("wke,kAe->wA", [(70, 6, 16), (6, 66, 16)], "B", 16),
    ("vwe,vAe->wA", [(5, 70, 16), (5, 66, 16)], "AB", 16),
    ("vwe,vAe->Aw", [(5, 70, 16), (5, 66, 16)], "AB", 16),
    # a batch label
    ("bvwe,bveA->bwA", [(3, 4, 40, 8), (3, 4, 8, 50)], "A", 8),
    # K = 640: the global resolve re-reads quads through the two-level k
    ("vwe,vAe->wA", [(40, 70, 16), (40, 66, 16)], "AB", 16),
    # K = 4096 on one output tile: split into K ranges
    ("vwe,vAe->wA", [(256, 8, 16), (256, 8, 16)], "AB", 16),
]
KNOBS = [None, ("TROPICAL_GEMM_SETTING", "wide"), ("TROPICAL_GEMM_SETTING", "narrow"),
         ("TROPICAL_GEMM_SETTING", "global"), ("TROPICAL_FORCE_SIMPLE_GEMM", "1"),
         ("TROPICAL_GEMM_FIXED_LAYOUT", "0")]


@pytest.fixture(scope="module")
def tb():
    from tropical_semiring_tensor_amd import binding
    binding.tropical_init(0)
    return binding


def operands(sr, sa, sb, seed, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    if dtype == torch.int32:
        return (torch.randint(-9, 10, sa, generator=g, dtype=torch.int32),
                torch.randint(-9, 10, sb, generator=g, dtype=torch.int32))
    if sr == "max_mul":
        return (torch.randint(1, 9, sa, generator=g).float() * 0.125,
                torch.randint(1, 9, sb, generator=g).float() * 0.25)
    return (torch.randint(-6, 7, sa, generator=g).float(), torch.randint(-6, 7, sb, generator=g).float())


def check(tb, orc, spec, sr, A, B, what, argmax=True):
    C, I = tb.tropical_contract_pair(spec, sr, A.to(DEV), B.to(DEV), argmax=argmax)
    torch.cuda.synchronize()
    Cr, Ir = orc.contract_pair(spec, sr, A.numpy(), B.numpy(), argmax=argmax)
    if A.dtype == torch.int32:
        assert_equal(C.cpu().numpy(), Cr, what)
    else:
        assert_bits_equal(C.cpu().numpy(), Cr, what)
    if argmax:
        assert_equal(I.cpu().numpy(), Ir, what + " argmax")


@pytest.mark.parametrize("knob", KNOBS, ids=lambda k: "auto" if k is None else f"{k[0]}={k[1]}")
@pytest.mark.parametrize("sr", ["max_plus", "min_plus", "max_mul"])
@pytest.mark.parametrize("case", range(len(KRUN_SPECS)))
def test_two_level_k(tb, orc, monkeypatch, knob, sr, case):
    spec, shapes, side, run = KRUN_SPECS[case]
    if knob is not None:
        monkeypatch.setenv(*knob)
    desc = tb.tropical_contract_pair_describe(spec, shapes[0], shapes[1])
    for s in side:
        assert f"{s}=fold:krun{run}" in desc, desc
    A, B = operands(sr, shapes[0], shapes[1], seed=case * 7 + len(sr))
    check(tb, orc, spec, sr, A, B, f"{spec} {shapes[0]} {sr} {knob}")


@pytest.mark.parametrize("sr", ["max_plus", "min_plus", "max_mul"])
@pytest.mark.parametrize("case", [0, 4, 6, 9])
def test_two_level_k_int32_and_value_only(tb, orc, sr, case):
    spec, shapes, _, _ = KRUN_SPECS[case]
    A, B = operands(sr, shapes[0], shapes[1], seed=case + 100, dtype=torch.int32)
    check(tb, orc, spec, sr, A, B, f"{spec} i32 {sr}")
    A, B = operands(sr, shapes[0], shapes[1], seed=case + 200)
    check(tb, orc, spec, sr, A, B, f"{spec} value only {sr}", argmax=False)


def test_two_level_k_matches_the_gathered_operand(tb, orc, monkeypatch):
    """The lattice-network step at bond 16 (a 64 MiB running result): the
    in-place read and the gathered copy give the same bits, and a sample of
    outputs matches the oracle."""
    spec = "vwxyze,veAf->wxyzAf"
    g = torch.Generator().manual_seed(5)
    A = torch.randn((16,) * 6, generator=g)
    B = torch.randn((16,) * 4, generator=g)
    Ad, Bd = A.to(DEV), B.to(DEV)
    assert "A=fold:krun16" in tb.tropical_contract_pair_describe(spec, A.shape, B.shape)
    C1, I1 = tb.tropical_contract_pair(spec, "max_plus", Ad, Bd)
    monkeypatch.setenv("TROPICAL_NO_KRUN_FOLD", "1")
    assert "A=gather" in tb.tropical_contract_pair_describe(spec, A.shape, B.shape)
    C2, I2 = tb.tropical_contract_pair(spec, "max_plus", Ad, Bd)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32)) and torch.equal(I1, I2)
    # sampled outputs against the definition: C[w..f] = max over (v, e)
    An = A.numpy()
    Bn = B.numpy()
    c1, i1 = C1.cpu().numpy(), I1.cpu().numpy()
    rs = torch.Generator().manual_seed(6)
    idx = torch.randint(0, 16, (300, 6), generator=rs).numpy()
    for w, x, y, z, a, f in idx:
        terms = (An[:, w, x, y, z, :] + Bn[:, :, a, f]).reshape(-1)  # (v, e) row-major = k
        k = int(terms.argmax())
        assert c1[w, x, y, z, a, f] == terms[k] and i1[w, x, y, z, a, f] == k
