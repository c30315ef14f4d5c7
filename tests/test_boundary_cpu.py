"""The C-ABI library on the CPU: it loads, exports what include/tropical.h
declares, and its host-only logic (argument checks, spec parsing, planning,
workspace sizing) behaves as documented.  No kernel is launched here."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tropical.h")


@pytest.fixture(scope="module")
def tb():
    from tropical_semiring_tensor_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from tropical_semiring_tensor_amd.csrc import build
        build.build()
    binding.lib()
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"TROP_API\s+[\w\s\*]+?\b(tropical_\w+)\s*\(", text)))


def test_header_declares_the_four_operations():
    fns = declared_functions()
    for f in ("tropical_gemm_strided_batched", "tropical_permute", "tropical_diag_gather",
              "tropical_contract_pair"):
        assert f in fns


def test_library_exports_every_declared_symbol(tb):
    fns = declared_functions()
    assert len(fns) >= 10
    for f in fns:
        assert hasattr(tb.lib(), f), f
    out = subprocess.run(["nm", "-D", "--defined-only", tb.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)", out))
    assert set(fns) == exported, f"exported {sorted(exported)} vs declared {fns}"


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "tropical.h"\nint main(void){trop_strides s={1,2,3};'
                   'return (int)sizeof(s) + (int)TROP_OK;}\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-c",
                    str(src), "-o", str(tmp_path / "use.o")], check=True)


def test_code_object_is_gfx950_only():
    from tropical_semiring_tensor_amd.csrc import build
    co = os.path.join(build.BUILD, "tropical_kernels.co")
    if not os.path.exists(co):
        build.build()
    data = open(co, "rb").read()
    assert data[:4] == b"\x7fELF"
    assert b"gfx950" in data
    for other in (b"gfx90a", b"gfx942", b"gfx1100"):
        assert other not in data


def _status(tb, fn, *args):
    return getattr(tb.lib(), fn)(*args)


def test_gemm_argument_errors_before_any_device_call(tb):
    L = tb.lib()
    s = tb.trop_strides(1, 1, 1)
    nul = ctypes.c_void_p(0)
    # unknown semiring / dtype, negative sizes and strides
    assert L.tropical_gemm_strided_batched(7, 0, nul, s, nul, s, nul, s, nul, 1, 1, 1, 1, nul) == tb.INVALID_ARGUMENT
    assert "semiring" in tb.tropical_last_error()
    assert L.tropical_gemm_strided_batched(0, 9, nul, s, nul, s, nul, s, nul, 1, 1, 1, 1, nul) == tb.INVALID_ARGUMENT
    assert L.tropical_gemm_strided_batched(0, 0, nul, s, nul, s, nul, s, nul, -1, 1, 1, 1, nul) == tb.INVALID_ARGUMENT
    neg = tb.trop_strides(-1, 1, 1)
    assert L.tropical_gemm_strided_batched(0, 0, nul, neg, nul, s, nul, s, nul, 1, 1, 1, 1, nul) == tb.INVALID_ARGUMENT
    assert L.tropical_gemm_strided_batched(0, 0, nul, s, nul, s, nul, s, nul, 1, 1, 2 ** 31, 1, nul) == tb.INVALID_ARGUMENT
    # the strided workspace query: NULL bytes, negative sizes and strides
    nb = ctypes.c_size_t(0)
    assert L.tropical_gemm_workspace_size_strided(s, s, 1, 4, 4, 4, 1, None) == tb.INVALID_ARGUMENT
    assert L.tropical_gemm_workspace_size_strided(s, s, 1, 4, -4, 4, 1, ctypes.byref(nb)) == tb.INVALID_ARGUMENT
    assert L.tropical_gemm_workspace_size_strided(s, neg, 1, 4, 4, 4, 1, ctypes.byref(nb)) == tb.INVALID_ARGUMENT
    assert "stride" in tb.tropical_last_error()
    assert L.tropical_gemm_workspace_size_strided(s, s, 1, 4, 4, 4, 1, ctypes.byref(nb)) == tb.OK and nb.value == 0
    # sizes near the int64 limit: answered without overflow (no split, K >= 2^31 is no call's)
    big = 2 ** 62
    assert L.tropical_gemm_workspace_size(big, 1, 2 ** 62, 1, ctypes.byref(nb)) == tb.OK
    assert L.tropical_gemm_workspace_size_strided(s, s, 1, big, big, big, big, ctypes.byref(nb)) == tb.OK
    # an empty output is a no-op before any pointer is looked at
    assert L.tropical_gemm_strided_batched(0, 0, nul, s, nul, s, nul, s, nul, 0, 5, 5, 3, nul) == tb.OK
    assert L.tropical_gemm_strided_batched(1, 1, nul, s, nul, s, nul, s, nul, 4, 4, 4, 0, nul) == tb.OK
    assert tb.tropical_last_error() == ""


def test_permute_argument_errors(tb):
    L = tb.lib()
    shape = tb._i64([2, 3])
    strides = tb._i64([3, 1])
    arr = (ctypes.c_void_p * 2)(0, 0)
    assert L.tropical_permute(4, 2, shape, strides, tb._i32([0, 0]), 1, arr, arr, None) == tb.INVALID_ARGUMENT
    assert "permutation" in tb.tropical_last_error()
    assert L.tropical_permute(4, 2, shape, strides, tb._i32([1, 2]), 1, arr, arr, None) == tb.INVALID_ARGUMENT
    assert L.tropical_permute(4, 2, shape, strides, tb._i32([1, 0]), 3, arr, arr, None) == tb.INVALID_ARGUMENT
    for eb in (1, 2, 12, 32):
        assert L.tropical_permute(eb, 2, shape, strides, tb._i32([1, 0]), 1, arr, arr, None) == tb.UNSUPPORTED
    # 8- and 16-byte elements are moved as 4-byte words; eight output axes
    # that stay apart, plus the element's words, exceed the 8 kernel axes
    s8, t8 = tb._i64([2, 3] * 4), tb._i64([648, 216, 108, 36, 18, 6, 3, 1])
    rev = tb._i32(list(range(7, -1, -1)))
    for eb in (8, 16):
        assert L.tropical_permute(eb, 8, s8, t8, rev, 1, arr, arr, None) == tb.UNSUPPORTED
        assert L.tropical_permute(eb, 2, tb._i64([0, 3]), strides, tb._i32([1, 0]), 1, arr, arr, None) == tb.OK
    assert L.tropical_permute(4, 9, shape, strides, tb._i32([1, 0]), 1, arr, arr, None) == tb.INVALID_ARGUMENT
    # zero-size output: no-op
    assert L.tropical_permute(4, 2, tb._i64([0, 3]), strides, tb._i32([1, 0]), 1, arr, arr, None) == tb.OK


def test_diag_argument_errors(tb):
    L = tb.lib()
    nul = ctypes.c_void_p(0)
    # repeated label with mismatched extents
    st = L.tropical_diag_gather(0, 0, 2, tb._i64([3, 4]), tb._i64([4, 1]), tb._i32([1, 1]), 1,
                                tb._i32([1]), nul, nul, None)
    assert st == tb.INVALID_ARGUMENT and "extent" in tb.tropical_last_error()
    # output label missing from the input, or repeated in the output
    assert L.tropical_diag_gather(0, 0, 2, tb._i64([3, 3]), tb._i64([3, 1]), tb._i32([1, 1]), 1,
                                  tb._i32([2]), nul, nul, None) == tb.INVALID_ARGUMENT
    assert L.tropical_diag_gather(0, 0, 2, tb._i64([3, 4]), tb._i64([4, 1]), tb._i32([1, 2]), 2,
                                  tb._i32([1, 1]), nul, nul, None) == tb.INVALID_ARGUMENT
    # the int32 max-mul backward is not defined (checked before any device call)
    z = tb.trop_strides(0, 0, 0)
    assert L.tropical_gemm_backward(2, 1, nul, z, nul, z, nul, nul, z, nul, z, nul, z, 1, 1, 1, 1,
                                    nul) == tb.UNSUPPORTED


def test_gemm_workspace_policy(tb, monkeypatch):
    """Split-K and float-mode workspace sizes (host only).  Partials are two
    arrays (values, argmax) of ranges x batch x m x n words, each rounded up
    to 256 bytes."""
    def parts(ranges, b, m, n):
        one = -(-(ranges * b * m * n * 4) // 256) * 256
        return 2 * one
    ws = tb.tropical_gemm_workspace_size
    # a large grid: no split, room for the int32 float mode's 256 flags
    assert ws(256, 256, 4096, 64) == 4 * 256
    # one tile, K = 65536: 256 ranges of 256 (not tiny: 256 (tile, block) pairs)
    assert ws(64, 64, 65536, 1) == parts(256, 1, 64, 64)
    # tiny products (at most 64 (tile, 256-term block) pairs): ranges of 64 terms
    assert ws(64, 64, 500, 1) == parts(4, 1, 64, 64)  # 4 ranges of 128 (ceil(500/7) -> 128)
    assert ws(1, 1, 256, 1) == parts(4, 1, 1, 1)
    assert ws(4096, 16, 256, 1) == parts(4, 1, 4096, 16)  # 64 tiles
    assert ws(64, 64, 100, 1) == 0  # K < 128
    assert ws(4096, 64, 256, 2) == 0  # 128 tiles: neither tiny nor few enough to split
    monkeypatch.setenv("TROPICAL_SPLITK_TINY", "0")
    assert ws(64, 64, 500, 1) == 0 and ws(1, 1, 256, 1) == 0
    assert ws(64, 64, 65536, 1) == parts(256, 1, 64, 64)


def test_gemm_workspace_with_transposed_b(tb, monkeypatch):
    """The strided size query (host only): room for transposed copies of a
    row-major B (1 KiB in, batch x k x n words rounded up to 256 bytes) and
    of a column-major A (after it, batch x m x k words) for an argmax
    product with K >= 512 and a multiple of 4, at least 256 rows and 2^30
    terms, not split; else the plain size (the knob at 1: K > 256 at any
    size)."""
    def t(*shape, col=False):
        x = torch.empty(*shape, device="meta")
        return x.transpose(1, 2).contiguous().transpose(1, 2) if col else x

    def copy(b, k, n):
        return 1024 + -(-(b * k * n * 4) // 256) * 256
    ws = tb.tropical_gemm_workspace_size_strided
    assert ws(t(1, 4096, 4096), t(1, 4096, 4096)) == copy(1, 4096, 4096)
    assert ws(t(16, 2048, 2048), t(16, 2048, 2048)) == copy(16, 2048, 2048)
    # no copy: column-major B, column-major A, no argmax, K <= 256 or not a
    # multiple of 4, fewer than 256 rows or 2^30 terms, a split product
    assert ws(t(16, 2048, 2048), t(16, 2048, 2048, col=True)) == tb.tropical_gemm_workspace_size(2048, 2048, 2048, 16)
    # a column-major A is copied too (after B's copy), also beside a column-major B
    assert ws(t(1, 4096, 4096, col=True), t(1, 4096, 4096)) == copy(1, 4096, 4096) + 4096 * 4096 * 4
    assert ws(t(1, 4096, 4096, col=True), t(1, 4096, 4096, col=True)) == copy(1, 4096, 4096)
    assert ws(t(2, 1000, 2048, col=True), t(2, 2048, 600, col=True)) == copy(2, 2048, 1000)
    assert ws(t(1, 4096, 4096), t(1, 4096, 4096), with_argmax=False) == 4 * 256
    # without an argmax only a column-major A is copied
    assert ws(t(1, 4096, 4096, col=True), t(1, 4096, 4096), with_argmax=False) == copy(1, 4096, 4096)
    assert ws(t(64, 256, 256), t(64, 256, 256)) == 0
    assert ws(t(1, 4096, 4094), t(1, 4094, 4096)) == 4 * 256
    assert ws(t(64, 128, 1024), t(64, 1024, 2048)) == 4 * 256  # 128 rows: the float-mode flags only
    assert ws(t(1, 256, 512), t(1, 512, 4160)) == 0  # 260 tiles, 2^29 terms
    assert ws(t(1, 4096, 300), t(1, 300, 4096)) == 4 * 256  # K = 300
    assert ws(t(1, 64, 65536), t(1, 65536, 64)) == tb.tropical_gemm_workspace_size(64, 64, 65536, 1)
    # the knob: 1 at any size (not split), 0 never
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "1")
    assert ws(t(43, 130, 260), t(43, 260, 90)) == copy(43, 260, 90)
    assert ws(t(1, 64, 65536), t(1, 65536, 64)) == tb.tropical_gemm_workspace_size(64, 64, 65536, 1)
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "0")
    assert ws(t(1, 4096, 4096), t(1, 4096, 4096)) == 4 * 256


def test_contract_plan_gathers_b_along_k_for_long_k(tb, monkeypatch):
    """A long-K contraction whose operands would be read with their free
    index at unit stride gathers them with k at unit stride (the workspace
    holds the copies); one already read along k stays in place."""
    d = tb.tropical_contract_pair_describe("ij,jk->ik", (2048, 2048), (2048, 2048))
    assert "A=fold B=gather:tiled:kcol" in d and "workspace=16778240" in d, d
    assert "B=fold" in tb.tropical_contract_pair_describe("ij,kj->ik", (2048, 2048), (2048, 2048))
    # a left operand read with its free index at unit stride is gathered along k too
    d = tb.tropical_contract_pair_describe("ji,jk->ik", (2048, 2048), (2048, 2048))
    assert "A=gather:tiled B=gather:tiled:kcol" in d, d
    assert "A=gather:tiled B=fold" in tb.tropical_contract_pair_describe("ji,kj->ik", (2048, 2048), (2048, 2048))
    # split along K (few tiles), K <= 256, or the knob at 0: in place
    assert "B=fold" in tb.tropical_contract_pair_describe("ij,jk->ik", (1024, 1024), (1024, 1024))
    assert "B=fold" in tb.tropical_contract_pair_describe("bij,bjk->bik", (64, 256, 256), (64, 256, 256))
    monkeypatch.setenv("TROPICAL_GEMM_B_TRANSPOSE", "0")
    assert "B=fold" in tb.tropical_contract_pair_describe("ij,jk->ik", (2048, 2048), (2048, 2048))
    assert "A=fold B=fold" in tb.tropical_contract_pair_describe("ji,jk->ik", (2048, 2048), (2048, 2048))


def test_contract_plan_config5(tb):
    d = tb.tropical_contract_pair_describe("iijb,kjb->bki", (128, 128, 256, 32), (256, 256, 32))
    assert "batch=b left=i right=k contracted=j" in d
    # the output order is (batch, B-side, A-side): the product is taken as
    # B (x) A and lands in (b, k, i) with no output permute
    assert "gemm B(x)A batch=32 m=256 n=128 k=256" in d
    assert "A=gather:tiled" in d and "B=gather:tiled" in d and "out=direct" in d
    ws = tb.tropical_contract_pair_workspace_size("iijb,kjb->bki", (128, 128, 256, 32), (256, 256, 32))
    assert ws == 4 * (32 * 128 * 256 + 32 * 256 * 256)
    # the canonical order keeps A (x) B and permutes the output
    d = tb.tropical_contract_pair_describe("iijb,kjb->kbi", (128, 128, 256, 32), (256, 256, 32))
    assert "gemm A(x)B batch=32 m=128 n=256 k=256" in d and "out=permute:" in d


def test_contract_plan_folds_canonical_operands(tb):
    d = tb.tropical_contract_pair_describe("bij,bjk->bik", (4, 5, 6), (4, 6, 7))
    assert "A=fold" in d and "B=fold" in d and "out=direct" in d and "workspace=0" in d
    # a column-major B (k unit-stride) is read in place too
    d = tb.tropical_contract_pair_describe("bij,bjk->bik", (4, 5, 6), (4, 6, 7), (30, 6, 1), (42, 1, 6))
    assert "B=fold" in d
    # a label reduced in the pre-pass forces the gather
    d = tb.tropical_contract_pair_describe("aij,jk->ik", (3, 4, 5), (5, 6))
    assert "reduceA=a" in d and "A=gather:reduce" in d


def test_contract_plan_two_level_k(tb, monkeypatch):
    # the lattice-network step: the running result's first and last axes
    # are contracted, the GEMM reads it in place with runs of 16 along k
    d = tb.tropical_contract_pair_describe("vwxyze,veAf->wxyzAf", (16,) * 6, (16,) * 4)
    assert "gemm A(x)B batch=1 m=65536 n=256 k=256" in d and "A=fold:krun16 B=fold" in d, d
    # runs of two inner labels; the right operand; both, swapped
    assert "A=fold:krun16" in tb.tropical_contract_pair_describe("vwef,vefA->wA", (3, 5, 2, 8), (3, 2, 8, 4))
    assert "B=fold:krun8" in tb.tropical_contract_pair_describe("wke,kAe->wA", (7, 6, 8), (6, 5, 8))
    d = tb.tropical_contract_pair_describe("vwe,vAe->Aw", (5, 7, 4), (5, 6, 4))
    assert "B(x)A" in d and "A=fold:krun4 B=fold:krun4" in d, d
    # runs of 2 or 32 elements, or an inner label off the unit stride, are gathered
    assert "A=gather" in tb.tropical_contract_pair_describe("vwe,veA->wA", (5, 7, 2), (5, 2, 6))
    assert "A=gather" in tb.tropical_contract_pair_describe("vwe,veA->wA", (5, 7, 32), (5, 32, 6))
    assert "A=gather" in tb.tropical_contract_pair_describe("vwe,veA->wA", (5, 7, 16), (5, 16, 6),
                                                            (1, 5, 35), None)
    # (with the inner label at unit stride the axis order does not matter)
    assert "A=fold:krun16" in tb.tropical_contract_pair_describe("vew,veA->wA", (5, 16, 7), (5, 16, 6),
                                                                 (16 * 7, 1, 16), None)
    monkeypatch.setenv("TROPICAL_NO_KRUN_FOLD", "1")
    d = tb.tropical_contract_pair_describe("vwxyze,veAf->wxyzAf", (16,) * 6, (16,) * 4)
    assert "A=gather" in d, d


def test_contract_plan_flat_gather_for_a_small_bond(tb):
    # A (a=2, i=64, b=512): its canonical (b, i, a) order is a transpose of a
    # 512 x 2 plane, where a fixed 64-wide tile would be 2/64 in range; B's
    # (b, a*j) plane is 512 x 128 and keeps the 64 x 64 tiles
    d = tb.tropical_contract_pair_describe("aib,ajb->bij", (2, 64, 512), (2, 64, 512))
    assert "A=gather:flat" in d and "B=gather:tiled" in d, d


@pytest.mark.parametrize("spec,err", [
    ("ij,jk", tb_err := "INVALID"), ("ij->i", "INVALID"), ("ij,jk->iq", "INVALID"),
    ("i1,jk->ik", "INVALID"), ("ij,jk->ii", "INVALID"), ("ij,j,k->ik", "INVALID"),
])
def test_contract_spec_errors(tb, spec, err):
    with pytest.raises(tb.TropicalError) as e:
        tb.tropical_contract_pair_describe(spec, (2, 3), (3, 4))
    assert e.value.status == tb.INVALID_ARGUMENT


def test_contract_extent_mismatch(tb):
    with pytest.raises(tb.TropicalError):
        tb.tropical_contract_pair_describe("ij,jk->ik", (2, 3), (4, 5))


def test_stats_counters_are_consistent(tb):
    s = tb.tropical_get_stats()
    assert set(s["launches"]) == set(tb.KERNEL_FAMILIES)
    # every launch is counted once overall and once in its family
    assert s["launches_total"] == sum(s["launches"].values())
    tb.tropical_reset_stats()
    s = tb.tropical_get_stats()
    assert s["launches_total"] == 0 and not any(s["launches"].values())


# ---------------------------------------------------------------------------
# contraction trees (host-side planning only)
# ---------------------------------------------------------------------------

def _grid_plan(tb, rows=5, cols=5, bond=16, sr="max_plus"):
    import torch
    from tropical_semiring_tensor_amd import inputs
    net = inputs.grid_network(rows, cols, bond)
    return net, tb.tropical_tree_plan_create(sr, torch.float32, net["subs"], net["shapes"], net["steps"])


def _parse_tree_description(text):
    """(step, result offset or None, result bytes, scratch offset or None,
    scratch bytes) per step line of tropical_tree_describe."""
    rows = []
    for line in text.splitlines():
        m = re.match(r"step (\d+): \S+->(\w*) result=(ws@(\d+)|out)( scratch=ws@(\d+))?;.*workspace=(\d+)$", line)
        if m:
            rows.append((int(m.group(1)), m.group(2), int(m.group(4)) if m.group(4) else None,
                         int(m.group(6)) if m.group(6) else None, int(m.group(7))))
    return rows


def test_tree_plan_workspace_is_liveness_packed(tb):
    net, plan = _grid_plan(tb)
    text = tb.tropical_tree_describe(plan)
    rows = _parse_tree_description(text)
    assert len(rows) == len(net["steps"]) == 24
    n = len(net["subs"])
    last_use = {}
    for s, (lhs, rhs, _) in enumerate(net["steps"]):
        for slot in (lhs, rhs):
            if slot >= n:
                last_use[slot - n] = s
    bufs = []  # (first, last, begin, end)
    for s, out, r_off, x_off, x_bytes in rows:
        elems = 16 ** len(out)
        if r_off is not None:
            bufs.append((s, last_use[s], r_off, r_off + elems * 4))
        if x_off is not None:
            bufs.append((s, s, x_off, x_off + x_bytes))
    ws = tb.tropical_tree_workspace_size(plan)
    for i, a in enumerate(bufs):
        assert a[3] <= ws
        for b in bufs[i + 1:]:
            if a[0] <= b[1] and b[0] <= a[1]:  # lifetimes meet
                assert a[3] <= b[2] or b[3] <= a[2], f"live buffers overlap: {a} {b}"
    results = int(re.search(r"results=(\d+)", text).group(1))
    # 19 of the 23 intermediates are 64 MiB or 4 MiB; liveness keeps two
    # results and one scratch buffer resident at a time
    assert results > 700 << 20 and ws < 256 << 20


def test_tree_step_info_and_plan_reuse(tb):
    net, plan = _grid_plan(tb, 3, 4, 5)
    for s, (_, _, out) in enumerate(net["steps"]):
        sub, shape = tb.tropical_tree_step_info(plan, s)
        assert sub == out and shape == [5] * len(out)
    with pytest.raises(tb.TropicalError):
        tb.tropical_tree_step_info(plan, len(net["steps"]))
    tb.tropical_tree_plan_destroy(plan)
    tb.tropical_tree_plan_destroy(plan)  # second destroy is a no-op


@pytest.mark.parametrize("case", [
    "bad_slot", "future_slot", "unused_result", "extent_mismatch", "bad_label", "bad_semiring", "long_sub",
    "no_steps"])
def test_tree_plan_errors(tb, case):
    import torch
    subs, shapes = ["ab", "bc", "cd"], [(2, 3), (3, 4), (4, 5)]
    steps = [(0, 1, "ac"), (3, 2, "ad")]
    sr, dt = "max_plus", torch.float32
    if case == "bad_slot":
        steps = [(0, -1, "ac"), (3, 2, "ad")]
    elif case == "future_slot":
        steps = [(0, 4, "ac"), (3, 2, "ad")]
    elif case == "unused_result":
        steps = [(0, 1, "ac"), (1, 2, "bd")]
    elif case == "extent_mismatch":
        shapes = [(2, 3), (3, 4), (5, 5)]
    elif case == "bad_label":
        steps = [(0, 1, "a1"), (3, 2, "ad")]
    elif case == "bad_semiring":
        sr = 7
    elif case == "long_sub":
        subs, shapes = ["abcdefghi", "bc", "cd"], [(1,) * 9, (1, 4), (4, 5)]
    elif case == "no_steps":
        steps = []
    want = tb.INVALID_ARGUMENT
    with pytest.raises(tb.TropicalError) as e:
        tb.tropical_tree_plan_create(sr, dt, subs, shapes, steps)
    assert e.value.status == want
    if case in ("extent_mismatch", "future_slot", "unused_result"):
        assert "step" in str(e.value)
