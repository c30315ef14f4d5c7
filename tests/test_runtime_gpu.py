"""Runtime behaviour on the GPU: one module load per device, pointer and
extent checks, caller streams, and the module-load failure path."""
import os
import subprocess
import sys
import textwrap

import pytest
import torch

from gpu_util import DEV

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def tb():
    from tropical_semiring_tensor_amd import binding
    binding.tropical_init(0)
    return binding


def test_module_loaded_once(tb):
    before = tb.tropical_get_stats()["module_loads"]
    A = torch.randn(2, 70, 80, device=DEV)
    B = torch.randn(2, 80, 90, device=DEV)
    for sr in ("max_plus", "min_plus", "max_mul"):
        for _ in range(3):
            tb.tropical_gemm_strided_batched(sr, A, B, torch.empty(2, 70, 90, device=DEV))
    tb.tropical_permute(A, (2, 0, 1))
    tb.tropical_diag_gather("max_plus", torch.randn(5, 5, 3, device=DEV), "iij", "j")
    tb.tropical_contract_pair("bij,bjk->bki", "max_plus", A, B)
    torch.cuda.synchronize()
    st = tb.tropical_get_stats()
    assert st["module_loads"] == before == 1


def test_host_and_pinned_pointers_rejected(tb):
    A = torch.randn(1, 8, 8)
    Bd = torch.randn(1, 8, 8, device=DEV)
    Cd = torch.empty(1, 8, 8, device=DEV)
    with pytest.raises(tb.TropicalError) as e:
        tb.tropical_gemm_strided_batched("max_plus", A, Bd, Cd)
    assert e.value.status == tb.NOT_DEVICE_MEMORY
    Ap = torch.randn(1, 8, 8).pin_memory()
    with pytest.raises(tb.TropicalError) as e:
        tb.tropical_gemm_strided_batched("max_plus", Ap, Bd, Cd)
    assert e.value.status == tb.NOT_DEVICE_MEMORY
    with pytest.raises(tb.TropicalError) as e:
        tb.tropical_permute(torch.randn(4, 5), (1, 0), out=torch.empty(5, 4, device=DEV))
    assert e.value.status == tb.NOT_DEVICE_MEMORY


def test_extent_past_allocation_rejected(tb):
    """Strides that reach past the end of the allocation are refused on the
    host (nothing is launched)."""
    import ctypes
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    raw = torch.empty(16 * 2 ** 20, device=DEV)          # a fresh 64 MiB allocation
    B = torch.randn(1, 8192, 8, device=DEV)
    C = torch.empty(1, 4096, 8, device=DEV)
    torch.cuda.synchronize()
    before = tb.tropical_get_stats()["launches_total"]
    L = tb.lib()
    # A claimed as (1, 4096, 8192) row-major: 128 MiB from the same base
    st = L.tropical_gemm_strided_batched(0, 0, ctypes.c_void_p(raw.data_ptr()),
                                         tb.trop_strides(8192, 1, 4096 * 8192),
                                         ctypes.c_void_p(B.data_ptr()), tb.trop_strides(8, 1, 8192 * 8),
                                         ctypes.c_void_p(C.data_ptr()), tb.trop_strides(8, 1, 4096 * 8),
                                         None, 4096, 8, 8192, 1, None)
    assert st == tb.INVALID_ARGUMENT
    assert "allocation" in tb.tropical_last_error()
    assert tb.tropical_get_stats()["launches_total"] == before


def test_side_stream(tb, orc):
    A = torch.randint(-5, 6, (4, 70, 90)).float()
    B = torch.randint(-5, 6, (4, 90, 66)).float()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Ad, Bd = A.to(DEV, non_blocking=False), B.to(DEV)
        C = torch.empty(4, 70, 66, device=DEV)
        I = torch.empty(4, 70, 66, dtype=torch.int32, device=DEV)
        tb.tropical_gemm_strided_batched("max_plus", Ad, Bd, C, I, stream=s)
    s.synchronize()
    Cr, Ir = orc.gemm("max_plus", A.numpy(), B.numpy())
    assert (C.cpu().numpy() == Cr).all() and (I.cpu().numpy() == Ir).all()


def test_module_load_failure_is_not_cached():
    code = textwrap.dedent("""
        import os, sys, torch
        sys.path.insert(0, %r)
        os.environ["TROPICAL_CODE_OBJECT"] = "/nonexistent/tropical.co"
        from tropical_semiring_tensor_amd import binding as tb
        torch.cuda.init()
        try:
            tb.tropical_init(0)
            print("UNEXPECTED_OK")
        except tb.TropicalError as e:
            assert e.status == tb.HIP_ERROR, e
            print("FAILED_AS_EXPECTED", tb.tropical_get_stats()["module_loads"])
        del os.environ["TROPICAL_CODE_OBJECT"]
        tb.tropical_init(0)
        A = torch.randn(1, 4, 4, device="cuda")
        C = torch.empty(1, 4, 4, device="cuda")
        tb.tropical_gemm_strided_batched("max_plus", A, A, C)
        torch.cuda.synchronize()
        print("RECOVERED", tb.tropical_get_stats()["module_loads"])
    """ % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=180)
    assert out.returncode == 0, out.stderr
    assert "FAILED_AS_EXPECTED 0" in out.stdout, out.stdout
    assert "RECOVERED 1" in out.stdout, out.stdout


@pytest.mark.parametrize("setting", ["wide", "narrow"])
def test_gemm_graph_capture_replays_both_settings(tb, monkeypatch, setting):
    """The argmax GEMM captured in a HIP graph, in both kernel settings (the
    wide one spills a few registers to scratch): every replay, with eager
    work and synchronisations between them, gives the eager result."""
    monkeypatch.setenv("TROPICAL_GEMM_SETTING", setting)
    g = torch.Generator().manual_seed(41)
    A = torch.randn(8, 256, 300, generator=g).to(DEV)
    B = torch.randn(8, 300, 256, generator=g).to(DEV)
    C0 = torch.empty(8, 256, 256, device=DEV)
    I0 = torch.empty(8, 256, 256, dtype=torch.int32, device=DEV)
    tb.tropical_gemm_strided_batched("max_plus", A, B, C0, I0)
    torch.cuda.synchronize()
    C = torch.empty_like(C0)
    I = torch.empty_like(I0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        tb.tropical_gemm_strided_batched("max_plus", A, B, C, I, stream=s)
    for rep in range(3):
        C.fill_(0.0)
        I.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int32), C0.view(torch.int32)), f"replay {rep}"
        assert torch.equal(I, I0), f"replay {rep} argmax"
