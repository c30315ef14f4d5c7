"""Helpers for the GPU parity tests (HIP path vs the CPU oracle)."""
import numpy as np
import torch

DEV = torch.device("cuda:0")


def bits(a):
    return np.ascontiguousarray(a).view(np.int32)


def assert_bits_equal(got, want, what=""):
    got = np.ascontiguousarray(got)
    want = np.ascontiguousarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    g, w = bits(got), bits(want)
    if not np.array_equal(g, w):
        bad = np.argwhere(g != w)
        pos = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {pos}: "
                             f"got {got[pos]!r} want {want[pos]!r}")


def assert_equal(got, want, what=""):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        pos = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {pos}: "
                             f"got {got[pos]!r} want {want[pos]!r}")


def gpu_gemm(tb, sr, A, B, argmax=True, c_layout="row"):
    """Run the HIP GEMM on CPU tensors A (b,m,k), B (b,k,n) (any strides:
    the device copies keep the same strides).  Returns numpy (C, I)."""
    if A.dim() == 2:
        A = A.unsqueeze(0)
    if B.dim() == 2:
        B = B.unsqueeze(0)
    Ad = device_copy(A)
    Bd = device_copy(B)
    batch, m, _ = Ad.shape
    n = Bd.shape[2]
    if c_layout == "row":
        C = torch.empty(batch, m, n, dtype=A.dtype, device=DEV)
        I = torch.empty(batch, m, n, dtype=torch.int32, device=DEV) if argmax else None
    else:  # column-major C / argmax
        C = torch.empty(batch, n, m, dtype=A.dtype, device=DEV).transpose(1, 2)
        I = torch.empty(batch, n, m, dtype=torch.int32, device=DEV).transpose(1, 2) if argmax else None
    tb.tropical_gemm_strided_batched(sr, Ad, Bd, C, I)
    torch.cuda.synchronize()
    return C.cpu().numpy(), (I.cpu().numpy() if argmax else None)


def device_copy(t):
    """Copy a CPU tensor to the GPU preserving its strides (incl. views)."""
    if t.is_contiguous():
        return t.to(DEV)
    storage_elems = t.untyped_storage().nbytes() // t.element_size()
    flat = torch.empty(storage_elems, dtype=t.dtype)
    flat.copy_(torch.as_strided(t, (storage_elems,), (1,), 0))
    dflat = flat.to(DEV)
    return torch.as_strided(dflat, t.shape, t.stride(), t.storage_offset())
