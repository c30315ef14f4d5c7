"""Parity of the HIP backward (winner routing) with the CPU oracle: the
gradients must be bit-identical, since both add each bin's terms in the
same ascending order.  The argmax fed to both sides comes from the oracle's
forward; the upstream gradient is N(0, 1), so any change of summation
order would show."""
import zlib

import numpy as np
import pytest
import torch

from gpu_util import DEV, assert_bits_equal, device_copy
from tropical_semiring_tensor_amd import inputs

pytestmark = pytest.mark.gpu

PAIRS = [("max_plus", "f32"), ("min_plus", "f32"), ("max_mul", "f32"),
         ("max_plus", "i32"), ("min_plus", "i32")]


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
    elif sr == "max_mul":
        A = torch.randint(1, 9, (b, m, k), generator=g).float() * 0.125
        B = torch.randint(1, 9, (b, k, n), generator=g).float() * 0.25
    else:
        A = torch.randint(-8, 9, (b, m, k), generator=g).float()
        B = torch.randint(-8, 9, (b, k, n), generator=g).float()
    G = torch.randn(b, m, n, generator=g)
    return A, B, G


def run_both(tb, orc, sr, A, B, I, G, k, what, grad_a=True, grad_b=True):
    mul = sr == "max_mul"
    Ad = device_copy(A) if mul else None
    Bd = device_copy(B) if mul else None
    ga, gb = tb.tropical_gemm_backward(sr, device_copy(I), device_copy(G), Ad, Bd, k=k,
                                       grad_a=grad_a, grad_b=grad_b)
    torch.cuda.synchronize()
    ra, rb = orc.gemm_backward(sr, I.numpy(), G.numpy(), A.numpy() if mul else None,
                               B.numpy() if mul else None, k=k, grad_a=grad_a is not None,
                               grad_b=grad_b is not None)
    if grad_a is not None:
        assert_bits_equal(ga.cpu().numpy(), ra, what + " grad_a")
    if grad_b is not None:
        assert_bits_equal(gb.cpu().numpy(), rb, what + " grad_b")


SHAPES = [(1, 1, 1, 1), (2, 3, 7, 5), (3, 65, 17, 63), (2, 127, 255, 129), (1, 33, 600, 40),
          (1, 70, 64, 300)]


@pytest.mark.parametrize("sr,dt", PAIRS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_ragged(tb, orc, sr, dt, shape):
    b, m, k, n = shape
    A, B, G = operands(sr, dt, b, m, k, n, seed=zlib.crc32(repr((sr, dt, shape)).encode()) % 10000)
    _, I = orc.gemm(sr, A.numpy(), B.numpy())
    run_both(tb, orc, sr, A, B, torch.from_numpy(I), G, k, f"{sr} {dt} {shape}")


def test_backward_hub_and_patterns(tb, orc):
    # every output routes to k = 0 (one bin takes all items), and striped
    # patterns with many equal keys inside one 64-item chunk
    b, m, k, n = 2, 40, 70, 300
    g = torch.Generator().manual_seed(3)
    G = torch.randn(b, m, n, generator=g)
    A = torch.rand(b, m, k, generator=g) + 0.5
    B = torch.rand(b, k, n, generator=g) + 0.5
    for name, I in (("all_zero", torch.zeros(b, m, n, dtype=torch.int32)),
                    ("j_mod_3", (torch.arange(n) % 3).to(torch.int32).expand(b, m, n).contiguous()),
                    ("i_mod_5", (torch.arange(m) % 5).to(torch.int32)[:, None].expand(b, m, n).contiguous()),
                    ("last_k", torch.full((b, m, n), k - 1, dtype=torch.int32))):
        for sr in ("max_plus", "max_mul"):
            run_both(tb, orc, sr, A, B, I, G, k, f"{name} {sr}")


def test_backward_bins_beyond_one_lds_chunk(tb, orc):
    # k above the 4096 bins one wave holds in LDS: the bins go in chunks
    b, m, k, n = 1, 9, 9000, 70
    g = torch.Generator().manual_seed(4)
    I = torch.randint(0, k, (b, m, n), generator=g, dtype=torch.int32)
    G = torch.randn(b, m, n, generator=g)
    A = torch.rand(b, m, k, generator=g)
    B = torch.rand(b, k, n, generator=g)
    for sr in ("min_plus", "max_mul"):
        run_both(tb, orc, sr, A, B, I, G, k, f"k=9000 {sr}")


def test_backward_out_of_range_argmax_routes_nothing(tb, orc):
    b, m, k, n = 2, 20, 33, 50
    g = torch.Generator().manual_seed(5)
    I = torch.randint(-40, 80, (b, m, n), generator=g, dtype=torch.int32)
    G = torch.randn(b, m, n, generator=g)
    run_both(tb, orc, "max_plus", None, None, I, G, k, "out-of-range keys")


def test_backward_strided_views_and_one_sided(tb, orc):
    b, m, k, n = 3, 45, 60, 70
    A, B, _ = operands("max_mul", "f32", b, m, k, n, seed=6)
    _, I = orc.gemm("max_mul", A.numpy(), B.numpy())
    g = torch.Generator().manual_seed(7)
    # argmax and G as transposed views with equal strides; column-major A / B
    It = torch.from_numpy(I).transpose(1, 2).contiguous().transpose(1, 2)
    Gt = torch.randn(b, n, m, generator=g).transpose(1, 2)
    Ac = A.transpose(1, 2).contiguous().transpose(1, 2)
    Bc = B.transpose(1, 2).contiguous().transpose(1, 2)
    run_both(tb, orc, "max_mul", Ac, Bc, It, Gt, k, "strided views")
    run_both(tb, orc, "max_mul", A, B, torch.from_numpy(I), Gt.contiguous(), k, "grad_a only", grad_b=None)
    run_both(tb, orc, "max_plus", A, B, torch.from_numpy(I), Gt.contiguous(), k, "grad_b only", grad_a=None)
    # outputs written into strided (column-major) destination views
    Id, Gd = device_copy(torch.from_numpy(I)), device_copy(Gt.contiguous())
    ga = torch.empty(b, k, m, device=DEV).transpose(1, 2)
    gb = torch.empty(b, n, k, device=DEV).transpose(1, 2)
    tb.tropical_gemm_backward("max_plus", Id, Gd, k=k, grad_a=ga, grad_b=gb)
    torch.cuda.synchronize()
    ra, rb = orc.gemm_backward("max_plus", I, Gt.contiguous().numpy(), k=k)
    assert_bits_equal(ga.cpu().numpy(), ra, "column-major grad_a")
    assert_bits_equal(gb.cpu().numpy(), rb, "column-major grad_b")


@pytest.mark.parametrize("knob", [None, "TROPICAL_BACKWARD_NO_PAIR", "TROPICAL_BACKWARD_LANE", "TROPICAL_BACKWARD_WAVE",
                                  "TROPICAL_BACKWARD_SPLIT", "TROPICAL_BACKWARD_RANGE", "TROPICAL_BACKWARD_STAGED"])
def test_backward_denormal_zero_and_inf_gradients(tb, orc, monkeypatch, knob):
    """Bins summed from denormal gradients, +0 / -0 mixes (a bin of only
    -0.0 items is +0.0, since sums start at +0.0), exact cancellations to
    zero and infinities: each kernel form's adds must round and keep
    denormals exactly as the oracle's sequential float32 loop does."""
    if knob:
        # (the staged form is the default; its knob set to 0 turns it off)
        monkeypatch.setenv(knob, "0" if knob == "TROPICAL_BACKWARD_STAGED" else "1")
    b, m, k, n = 2, 64, 40, 200
    g = torch.Generator().manual_seed(81)
    I = torch.randint(0, k, (b, m, n), generator=g, dtype=torch.int32)
    I[:, :, ::3] = 5   # one hub bin per row
    coin = torch.rand(b, m, n, generator=g) < 0.5
    cases = {
        "denormal": (torch.rand(b, m, n, generator=g) - 0.5) * 2e-38,
        "smallest denormals": torch.where(coin, 1e-45, -1.4e-45),
        "signed zeros": torch.where(coin, 0.0, -0.0),
        "cancelling": torch.where(coin, 1.5e-38, -1.5e-38),
        "infinities": torch.where(torch.rand(b, m, n, generator=g) < 0.02, float("inf"),
                                  torch.randn(b, m, n, generator=g)),
    }
    A = torch.rand(b, m, k, generator=g) * 1e-20
    B = torch.rand(b, k, n, generator=g) * 1e-20
    for name, G in cases.items():
        run_both(tb, orc, "max_plus", None, None, I, G, k, f"{knob} {name}")
    # max-mul: the weight products themselves underflow into denormals
    run_both(tb, orc, "max_mul", A, B, I, cases["denormal"] * 1e18, k, f"{knob} max_mul denormal")


@pytest.mark.parametrize("pair", [True, False])
@pytest.mark.parametrize("items", [3, 15, 16, 17, 32, 33, 64, 100])
def test_backward_staged_pieces(tb, orc, monkeypatch, items, pair):
    """The staged form's pieces of 16 items: fewer than one piece, exactly
    one, two and four, and a ragged last piece; both gradients in one
    launch and one launch each; bin counts that leave
    waves with no range (k = 2), ranges of one bin (k = 4), ranges of four
    (k = 16: the 16-byte output stores), a ragged last range (k = 129) and
    full ranges (k = 256); segments across batch entries and not a
    multiple of 64 or of 4; contiguous (grad_a) and strided (grad_b)
    items, both weights."""
    if not pair:
        monkeypatch.setenv("TROPICAL_BACKWARD_NO_PAIR", "1")
    g = torch.Generator().manual_seed(items)
    b, m, n = 3, items, items   # grad_a walks n items per row, grad_b m per column
    for k in (2, 4, 16, 129, 256):
        I = torch.randint(0, k, (b, m, n), generator=g, dtype=torch.int32)
        G = torch.randn(b, m, n, generator=g)
        A = torch.rand(b, m, k, generator=g) + 0.5
        B = torch.rand(b, k, n, generator=g) + 0.5
        for sr in ("max_plus", "max_mul"):
            run_both(tb, orc, sr, A, B, I, G, k, f"staged items={items} k={k} {sr}")


def test_backward_errors(tb):
    I = torch.zeros(1, 4, 5, dtype=torch.int32, device=DEV)
    G = torch.zeros(1, 4, 5, device=DEV)
    with pytest.raises(tb.TropicalError) as e:
        tb.tropical_gemm_backward("max_mul", I, G, k=3)   # max-mul needs A and B
    assert e.value.status == tb.INVALID_ARGUMENT
    with pytest.raises(tb.TropicalError) as e:
        tb.tropical_gemm_backward("max_plus", I.cpu(), G.cpu(), k=3)
    assert e.value.status == tb.NOT_DEVICE_MEMORY
    # k = 0 writes nothing; m = 0 (whose empty views have NULL data
    # pointers) reads nothing and writes grad_b as zeros
    tb.tropical_gemm_backward("max_plus", I, G, k=0)
    _, gb = tb.tropical_gemm_backward("max_plus", I[:, :0], G[:, :0], k=3, grad_a=None)
    torch.cuda.synchronize()
    assert (gb == 0).all() and gb.shape == (1, 3, 5)


def test_backward_workload2_full(tb, orc):
    A, B = inputs.gemm_operands(2)
    _, I = orc.gemm("max_plus", A.numpy(), B.numpy())
    G = torch.randn(A.shape[0], A.shape[1], B.shape[2], generator=torch.Generator().manual_seed(22))
    run_both(tb, orc, "max_plus", A, B, torch.from_numpy(I), G, A.shape[2], "workload 2 backward")


def test_backward_maxmul_workload4_recipe(tb, orc):
    A, B = inputs.gemm_operands(4, batch=2, m=300, n=260, k=700)
    _, I = orc.gemm("max_mul", A.numpy(), B.numpy())
    G = torch.randn(2, 300, 260, generator=torch.Generator().manual_seed(23))
    run_both(tb, orc, "max_mul", A, B, torch.from_numpy(I), G, 700, "workload 4 recipe backward")


@pytest.mark.parametrize("knob", [None, "TROPICAL_BACKWARD_NO_PAIR", "TROPICAL_BACKWARD_LANE", "TROPICAL_BACKWARD_WAVE",
                                  "TROPICAL_BACKWARD_SPLIT", "TROPICAL_BACKWARD_RANGE", "TROPICAL_BACKWARD_STAGED"])
def test_backward_every_kernel_form(tb, orc, monkeypatch, knob):
    """The same gradients from the staged form (the default: both
    gradients in one launch; with TROPICAL_BACKWARD_NO_PAIR one launch
    each), the 16-lanes-per-segment form, the lane-per-segment form, the
    wave-per-segment form, the 64-bin range form and the choice among them
    without the staged form, over hub-heavy and uniform argmaxes, both
    weights."""
    if knob:
        # (the staged form is the default; its knob set to 0 turns it off)
        monkeypatch.setenv(knob, "0" if knob == "TROPICAL_BACKWARD_STAGED" else "1")
    b, m, k, n = 3, 70, 200, 130
    g = torch.Generator().manual_seed(61)
    G = torch.randn(b, m, n, generator=g)
    A = torch.rand(b, m, k, generator=g) + 0.5
    B = torch.rand(b, k, n, generator=g) + 0.5
    hub = torch.where(torch.rand(b, m, n, generator=g) < 0.8, 3, torch.randint(0, k, (b, m, n), generator=g))
    for name, I in (("uniform", torch.randint(0, k, (b, m, n), generator=g, dtype=torch.int32)),
                    ("hub", hub.to(torch.int32))):
        for sr in ("max_plus", "max_mul"):
            run_both(tb, orc, sr, A, B, I, G, k, f"{knob} {name} {sr}")
    # bins not a multiple of the 16 lanes, and fewer bins than lanes
    for kk in (37, 5):
        I = torch.randint(0, kk, (b, m, n), generator=g, dtype=torch.int32)
        run_both(tb, orc, "min_plus", None, None, I, G, kk, f"{knob} k={kk}")
