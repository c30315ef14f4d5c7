"""The allocation-free pairwise contraction (tropical_contract_pair_noalloc)
through the C ABI, against tropical_contract_pair with a caller workspace:
bit-identical values and argmax on calls in a row on one device, each later
one smaller than the one before (the library's scratch still holds the
previous call's contents), over specs that use every part of the scratch;
and the size limit, rejected before anything is enqueued."""
import pytest
import torch

from gpu_util import DEV, assert_bits_equal, assert_equal
from tropical_semiring_tensor_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    from tropical_semiring_tensor_amd import binding
    binding.tropical_init(0)
    return binding


def both(tb, spec, sr, A, B, argmax=True):
    """(C, I) of the workspace call and of the allocation-free call."""
    Cw, Iw = tb.tropical_contract_pair(spec, sr, A, B, argmax=argmax)
    C = torch.full(Cw.shape, -7, dtype=A.dtype, device=DEV)
    I = torch.full(Cw.shape, -7, dtype=torch.int32, device=DEV) if argmax else None
    tb.tropical_contract_pair_noalloc(spec, sr, A, B, C, I)
    torch.cuda.synchronize()
    got = (C.cpu().numpy(), I.cpu().numpy() if argmax else None)
    want = (Cw.cpu().numpy(), Iw.cpu().numpy() if argmax else None)
    return got, want


def check(tb, spec, sr, A, B, what, argmax=True):
    ws = tb.tropical_contract_pair_workspace_size(spec, A.shape, B.shape)
    assert ws <= tb.NOALLOC_SCRATCH_BYTES, f"{what}: needs {ws} bytes"
    (C, I), (Cw, Iw) = both(tb, spec, sr, A, B, argmax)
    assert_bits_equal(C, Cw, what + " C")
    if argmax:
        assert_equal(I, Iw, what + " argmax")
    return ws


def test_noalloc_matches_workspace_call_in_a_row(tb):
    # workload 5's einsum at full size (diagonal gather and permute into
    # 12 MiB of scratch), then the same spec smaller
    A, B = inputs.einsum_operands()
    ws1 = check(tb, "iijb,kjb->bki", "max_plus", A.to(DEV), B.to(DEV), "workload 5")
    A, B = inputs.einsum_operands(shape_a=(40, 40, 100, 8), shape_b=(70, 100, 8), salt=1)
    ws2 = check(tb, "iijb,kjb->bki", "max_plus", A.to(DEV), B.to(DEV), "workload 5 recipe, smaller")
    assert 0 < ws2 < ws1
    # an output permute (value and argmax through the scratch), smaller again
    g = torch.Generator().manual_seed(3)
    A = torch.randint(-20, 21, (6, 50, 70), generator=g, dtype=torch.int32)
    B = torch.randint(-20, 21, (6, 70, 30), generator=g, dtype=torch.int32)
    ws3 = check(tb, "bij,bjk->kbi", "min_plus", A.to(DEV), B.to(DEV), "int32 output permute")
    assert 0 < ws3 < ws2
    # value only, smaller still
    ws4 = check(tb, "bij,bjk->kbi", "max_mul", A.abs().float().to(DEV) * 0.5, B.abs().float().to(DEV) * 0.25,
                "max-mul value only", argmax=False)
    assert 0 < ws4 <= ws3


def test_noalloc_split_k_and_routed_argmax(tb):
    # a long narrow product (split-K partials in the scratch), then a
    # pre-pass reduction whose winners route the argmax (winners in the
    # scratch), each checked against the workspace call
    g = torch.Generator().manual_seed(4)
    A = torch.randn(40, 6000, generator=g)
    B = torch.randn(6000, 24, generator=g)
    ws = check(tb, "ij,jk->ik", "max_plus", A.to(DEV), B.to(DEV), "split K")
    assert "splitK" in tb.tropical_contract_pair_describe("ij,jk->ik", A.shape, B.shape)
    A = torch.randint(-9, 10, (30, 20, 12), generator=g).float()
    B = torch.randint(-9, 10, (20, 25), generator=g).float()
    ws2 = check(tb, "ijr,jk->ik", "max_plus", A.to(DEV), B.to(DEV), "reduced label, routed argmax")
    assert 0 < ws2 < ws


def test_noalloc_rejects_beyond_its_limit(tb):
    # a batched product whose output permute needs 2 x 32 MiB of scratch:
    # rejected with the limit in the message, and nothing is written
    spec = "bij,bjk->ikb"
    A = torch.zeros(2, 2048, 8, device=DEV)
    B = torch.zeros(2, 8, 2048, device=DEV)
    desc = tb.tropical_contract_pair_describe(spec, A.shape, B.shape)
    assert int(desc.rsplit("workspace=", 1)[1]) > tb.NOALLOC_SCRATCH_BYTES, desc
    C = torch.full((2048, 2048, 2), 5.0, device=DEV)
    I = torch.full((2048, 2048, 2), 5, dtype=torch.int32, device=DEV)
    with pytest.raises(tb.TropicalError) as e:
        tb.tropical_contract_pair_noalloc(spec, "max_plus", A, B, C, I)
    assert e.value.status == tb.WORKSPACE_TOO_SMALL
    assert str(tb.NOALLOC_SCRATCH_BYTES) in str(e.value)
    torch.cuda.synchronize()
    assert (C == 5.0).all() and (I == 5).all()
    # the same spec within the limit still works afterwards
    A = torch.randn(3, 64, 48, device=DEV)
    B = torch.randn(3, 48, 80, device=DEV)
    (Cn, In), (Cw, Iw) = both(tb, spec, "max_plus", A, B)
    assert_bits_equal(Cn, Cw, "after a rejected call C")
    assert_equal(In, Iw, "after a rejected call argmax")
