"""Parity of tropical_contract_pair with the oracle's decomposed pipeline
(bit-exact values and argmax), the full workload-5 einsum, and the
device-residency counters (no host syncs, no copies, one module load)."""
import numpy as np
import pytest
import torch

import golden_io as gio
from gpu_util import DEV, assert_bits_equal, assert_equal, device_copy
from tropical_semiring_tensor_amd import inputs

pytestmark = pytest.mark.gpu

SPECS = [
    ("iijb,kjb->bki", [(9, 9, 40, 3), (70, 40, 3)]),
    ("ij,jk->ik", [(70, 130), (130, 66)]),
    ("ij,jk->ki", [(70, 130), (130, 66)]),
    ("bij,bjk->bki", [(3, 65, 90), (3, 90, 70)]),
    ("abcd,cdbe->ea", [(5, 3, 20, 4), (20, 4, 3, 33)]),
    ("ijk,jl->lik", [(13, 40, 6), (40, 70)]),
    ("ij,jj->ij", [(30, 44), (44, 44)]),
    ("ab,ab->ab", [(30, 40), (30, 40)]),
    ("ab,cd->abcd", [(7, 9), (6, 5)]),
    ("kjb,iijb->bik", [(70, 40, 3), (9, 9, 40, 3)]),
    ("bij,bjk->bik", [(4, 70, 300), (4, 300, 66)]),
    # output (batch, B-side, A-side): taken as B (x) A (also "abcd,cdbe->ea"
    # above, with three contracted labels)
    ("xcb,bcy->yx", [(66, 5, 7), (7, 5, 70)]),
    ("iijb,kjb->kbi", [(9, 9, 40, 3), (70, 40, 3)]),
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
    return (torch.randint(-6, 7, sa, generator=g).float(), torch.randint(-6, 7, sb, generator=g).float())


@pytest.mark.parametrize("sr", ["max_plus", "min_plus", "max_mul"])
@pytest.mark.parametrize("spec,shapes", SPECS, ids=[s for s, _ in SPECS])
def test_specs(tb, orc, sr, spec, shapes):
    A, B = operands(sr, shapes[0], shapes[1], seed=len(spec))
    C, I = tb.tropical_contract_pair(spec, sr, A.to(DEV), B.to(DEV))
    torch.cuda.synchronize()
    Cr, Ir = orc.contract_pair(spec, sr, A.numpy(), B.numpy())
    assert_bits_equal(C.cpu().numpy(), Cr, f"{spec} {sr}")
    assert_equal(I.cpu().numpy(), Ir, f"{spec} {sr} argmax")


def test_int32_and_strided_operands(tb, orc):
    g = torch.Generator().manual_seed(8)
    A = torch.randint(0, 100, (9, 9, 40, 3), generator=g, dtype=torch.int32)
    Bbig = torch.randint(0, 100, (70, 50, 3), generator=g, dtype=torch.int32)
    B = Bbig[:, 5:45, :]  # non-contiguous operand
    for sr in ("min_plus", "max_plus", "max_mul"):
        C, I = tb.tropical_contract_pair("iijb,kjb->bki", sr, A.to(DEV), device_copy(B))
        torch.cuda.synchronize()
        Cr, Ir = orc.contract_pair("iijb,kjb->bki", sr, A.numpy(), B.numpy())
        assert_equal(C.cpu().numpy(), Cr, f"i32 {sr}")
        assert_equal(I.cpu().numpy(), Ir, f"i32 {sr} argmax")
    # a column-major operand that is read in place
    Ac = torch.randint(0, 100, (4, 60, 50), generator=g, dtype=torch.int32)
    Bc = torch.randint(0, 100, (4, 70, 50), generator=g, dtype=torch.int32).transpose(1, 2)
    d = tb.tropical_contract_pair_describe("bij,bjk->bik", Ac.shape, Bc.shape, Ac.stride(), Bc.stride())
    assert "B=fold" in d
    C, I = tb.tropical_contract_pair("bij,bjk->bik", "min_plus", Ac.to(DEV), device_copy(Bc))
    torch.cuda.synchronize()
    Cr, Ir = orc.contract_pair("bij,bjk->bik", "min_plus", Ac.numpy(), Bc.numpy())
    assert_equal(C.cpu().numpy(), Cr, "folded column-major B")
    assert_equal(I.cpu().numpy(), Ir, "folded column-major B argmax")


def test_pre_pass_reduction_values(tb, orc):
    g = torch.Generator().manual_seed(9)
    A = torch.randint(-5, 6, (6, 6, 40), generator=g).float()
    B = torch.randint(-5, 6, (40, 7, 9), generator=g).float()
    for spec in ("iij,jkl->k", "aij,jkl->ik"):
        for sr in ("max_plus", "min_plus"):
            Ad = A.to(DEV) if spec.startswith("iij") else A[:, :, :].to(DEV)
            C, I = tb.tropical_contract_pair(spec, sr, Ad, B.to(DEV), argmax=None)
            torch.cuda.synchronize()
            assert I is None
            Cr, _ = orc.contract_pair(spec, sr, A.numpy(), B.numpy(), argmax=False)
            assert_bits_equal(C.cpu().numpy(), Cr, f"{spec} {sr}")


# specs with labels reduced in the pre-pass: on A, on B, on both, with a
# batch label, a repeated label, and in the B (x) A orientation
ROUTE_SPECS = [
    ("iij,jkl->k", (6, 6, 40), (40, 7, 9)),
    ("aij,jkl->ik", (5, 6, 40), (40, 7, 9)),
    ("abj,jcd->bc", (4, 30, 50), (50, 20, 3)),
    ("zaij,zjk->zki", (3, 4, 20, 33), (3, 33, 25)),
    ("ij,jkl->ki", (70, 65), (65, 3, 66)),
    ("xabj,jbcy->bca", (2, 5, 17, 40), (40, 17, 6, 3)),
]


@pytest.mark.parametrize("sr,dt", [("max_plus", "f32"), ("min_plus", "f32"), ("max_mul", "f32"),
                                   ("max_plus", "i32"), ("min_plus", "i32"), ("max_mul", "i32")])
@pytest.mark.parametrize("spec,sa,sb", ROUTE_SPECS, ids=[r[0] for r in ROUTE_SPECS])
def test_argmax_routed_through_pre_pass_reductions(tb, orc, sr, dt, spec, sa, sb):
    """The argmax continues over the reduced labels: the product's k, then
    the reductions' winners at that k.  Small integers make ties common."""
    g = torch.Generator().manual_seed(len(spec) * 13 + sa[0])
    if dt == "i32":
        A = torch.randint(-9, 10, sa, generator=g, dtype=torch.int32)
        B = torch.randint(-9, 10, sb, generator=g, dtype=torch.int32)
    elif sr == "max_mul":
        A = torch.randint(0, 5, sa, generator=g).float() * 0.5
        B = torch.randint(0, 5, sb, generator=g).float() * 0.25
    else:
        A = torch.randint(-4, 5, sa, generator=g).float()
        B = torch.randint(-4, 5, sb, generator=g).float()
    C, I = tb.tropical_contract_pair(spec, sr, A.to(DEV), B.to(DEV))
    torch.cuda.synchronize()
    Cr, Ir = orc.contract_pair(spec, sr, A.numpy(), B.numpy())
    assert_bits_equal(C.cpu().numpy(), Cr, f"{spec} {sr} {dt}")
    assert_equal(I.cpu().numpy(), Ir, f"{spec} {sr} {dt} argmax")


def test_routed_argmax_index_range_and_k0(tb, orc):
    # a zero-extent contracted label: nothing wins, every index is 0
    A = torch.zeros(5, 0, 3)
    B = torch.zeros(0, 4)
    C, I = tb.tropical_contract_pair("ijr,jk->ik", "max_plus", A.to(DEV), B.to(DEV))
    torch.cuda.synchronize()
    Cr, Ir = orc.contract_pair("ijr,jk->ik", "max_plus", A.numpy(), B.numpy())
    assert_bits_equal(C.cpu().numpy(), Cr, "K = 0 with a reduction")
    assert (I == 0).all()
    # contracted x reduced extents beyond int32: only values can be asked
    # for (the check is on sizes, before any pointer is looked at)
    import ctypes
    z = ctypes.c_void_p(0)
    st = tb.lib().tropical_contract_pair(b"ijr,jk->ik", 0, 0, z, tb._i64([1, 1 << 16, 1 << 16]), None, z,
                                         tb._i64([1 << 16, 1]), None, z, ctypes.c_void_p(16), z, 0, None)
    assert st == tb.INVALID_ARGUMENT and "int32" in tb.tropical_last_error()


def test_golden_einsum(tb):
    gdata = gio.load("einsum_iijb_kjb_bki.json")
    A = np.zeros(gdata["A_shape"], dtype=np.float32)
    for e in gdata["A_entries"]:
        A[tuple(e["index"])] = gio.f32(e["value"])
    B = gio.nested(gdata["B"], "f32")
    C, I = tb.tropical_contract_pair(gdata["spec"], gdata["semiring"], torch.from_numpy(A).to(DEV),
                                     torch.from_numpy(B).to(DEV))
    torch.cuda.synchronize()
    assert_bits_equal(C.cpu().numpy(), gio.nested(gdata["out"], "f32"), "golden einsum")
    assert_equal(I.cpu().numpy(), np.array(gdata["argmax"]), "golden einsum argmax")


def test_workspace_too_small(tb):
    A = torch.zeros(4, 4, 5, 2, device=DEV)
    B = torch.zeros(6, 5, 2, device=DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(tb.TropicalError) as e:
        tb.tropical_contract_pair("iijb,kjb->bki", "max_plus", A, B, workspace=ws)
    assert e.value.status == tb.WORKSPACE_TOO_SMALL


def test_workload5_full(tb, orc):
    A, B = inputs.einsum_operands()
    Ad, Bd = A.to(DEV), B.to(DEV)
    tb.tropical_reset_stats()
    C, I = tb.tropical_contract_pair("iijb,kjb->bki", "max_plus", Ad, Bd)
    torch.cuda.synchronize()
    st = tb.tropical_get_stats()
    # diag gather and B permute in one paired launch of the tiled gather,
    # then the GEMM taken as B (x) A straight into (b, k, i): two launches,
    # no output permute
    assert st["launches_total"] == 2, st
    assert st["launches"]["gather_tiled"] == 1 and st["launches"]["gemm_tiled"] == 1, st
    Cr, Ir = orc.contract_pair("iijb,kjb->bki", "max_plus", A.numpy(), B.numpy())
    assert_bits_equal(C.cpu().numpy(), Cr, "workload 5")
    assert_equal(I.cpu().numpy(), Ir, "workload 5 argmax")


def test_contract_long_contraction_splits_k(tb, orc):
    """A narrow product with a long contracted extent is split along K
    inside the pairwise driver (its workspace holds the partials)."""
    spec = "ikl,klj->ji"
    g = torch.Generator().manual_seed(31)
    A = torch.randn(24, 64, 150, generator=g)
    B = torch.randn(64, 150, 40, generator=g)
    desc = tb.tropical_contract_pair_describe(spec, A.shape, B.shape)
    assert "splitK" in desc, desc
    for sr in ("max_plus", "min_plus"):
        C, I = tb.tropical_contract_pair(spec, sr, A.to(DEV), B.to(DEV))
        torch.cuda.synchronize()
        Cr, Ir = orc.contract_pair(spec, sr, A.numpy(), B.numpy())
        assert_bits_equal(C.cpu().numpy(), Cr, f"{spec} {sr}")
        assert_equal(I.cpu().numpy(), Ir, f"{spec} {sr} argmax")


@pytest.mark.parametrize("paired", [True, False])
def test_paired_pre_pass_gathers(tb, orc, monkeypatch, paired):
    """Both operands permuted or diagonal-gathered by the tiled kernel: one
    paired launch (workgroups split between the two jobs in proportion to
    their tiles) or two launches, with the same results.  Shapes give the
    two jobs very different tile counts, the same and different tile widths
    (which falls back to two launches), a routed argmax through reductions
    (two tensors per job), and grids past the resident cap."""
    if not paired:
        monkeypatch.setenv("TROPICAL_NO_PAIRED_GATHER", "1")
    g = torch.Generator().manual_seed(41)
    cases = [
        ("iijb,kjb->bki", (40, 40, 64, 8), (96, 64, 8)),
        ("abc,cbd->adb", (64, 48, 32), (32, 48, 128)),
        ("jib,kjb->bik", (256, 64, 12), (8, 256, 12)),
        ("ijb,jkb->bik", (512, 512, 4), (512, 256, 4)),
        ("iirb,kjrb->bki", (20, 20, 3, 8), (48, 36, 3, 8)),
    ]
    for spec, sa, sb in cases:
        A = torch.randint(-9, 10, sa, generator=g).float()
        B = torch.randint(-9, 10, sb, generator=g).float()
        Ad, Bd = A.to(DEV), B.to(DEV)
        C, I = tb.tropical_contract_pair(spec, "max_plus", Ad, Bd)
        torch.cuda.synchronize()
        Cr, Ir = orc.contract_pair(spec, "max_plus", A.numpy(), B.numpy())
        assert_bits_equal(C.cpu().numpy(), Cr, f"{spec} paired={paired}")
        assert_equal(I.cpu().numpy(), Ir, f"{spec} paired={paired} argmax")
