"""Parity of the HIP contraction-tree executor with the CPU oracle.

Every step of a tree is a pairwise contraction, so the oracle's tree (its
pairwise steps in the same order) and the device tree must agree bit for bit
in the result and in every step's argmax, at the benchmark's network size
too (the oracle's tree takes ~15-30 s there).  That network is further
checked against the device's own pairwise calls, each step's sampled outputs
against the oracle's brute-force einsum, and the winner routing against the
result.
"""
import numpy as np
import pytest
import torch

from gpu_util import DEV, assert_bits_equal, assert_equal, device_copy
from tropical_semiring_tensor_amd import inputs

pytestmark = pytest.mark.gpu

PAIRS = [("max_plus", torch.float32), ("min_plus", torch.float32), ("max_mul", torch.float32),
         ("max_plus", torch.int32), ("min_plus", torch.int32), ("max_mul", torch.int32)]


@pytest.fixture(scope="module")
def tb():
    from tropical_semiring_tensor_amd import binding
    binding.tropical_init(0)
    return binding


def cast_inputs(sr, dt, tensors, seed):
    """The network's N(0, 1) tensors as the semiring / dtype needs them."""
    g = torch.Generator().manual_seed(seed)
    out = []
    for t in tensors:
        if dt == torch.int32:
            out.append(torch.randint(-50, 51, t.shape, generator=g, dtype=torch.int32))
        elif sr == "max_mul":
            out.append(t.abs() + 0.25)
        else:
            out.append(t.clone())
    return out


def run_both(tb, orc, sr, dt, subs, xs, steps, argmax=True, strides_views=None, what=""):
    shapes = [tuple(x.shape) for x in xs]
    dev_in = [device_copy(x) for x in xs]
    strides = [tuple(x.stride()) if not x.is_contiguous() else None for x in xs]
    plan = tb.tropical_tree_plan_create(sr, dt, subs, shapes, steps,
                                        strides=strides if any(s is not None for s in strides) else None)
    out, ams = tb.tropical_tree_run(plan, dev_in, argmax=argmax)
    torch.cuda.synchronize()
    ref, rams = orc.contract_tree(sr, [x.numpy() for x in xs], subs, steps,
                                  argmax=argmax if isinstance(argmax, bool) else [bool(a) for a in argmax])
    assert_bits_equal(out.cpu().numpy(), ref, what + " result")
    for s, (a, r) in enumerate(zip(ams, rams)):
        if r is None:
            assert a is None
        else:
            assert_equal(a.cpu().numpy(), r, f"{what} argmax of step {s}")
    return plan


@pytest.mark.parametrize("sr,dt", PAIRS, ids=lambda p: str(p).replace("torch.", ""))
@pytest.mark.parametrize("grid", [(2, 3, 3), (3, 3, 4), (4, 4, 3), (3, 5, 5)], ids=lambda g: "x".join(map(str, g)))
def test_tree_grid_networks(tb, orc, sr, dt, grid):
    rows, cols, bond = grid
    net = inputs.grid_network(rows, cols, bond, salt=rows * 100 + cols * 10 + bond)
    xs = cast_inputs(sr, dt, net["tensors"], seed=rows + cols + bond)
    run_both(tb, orc, sr, dt, net["subs"], xs, net["steps"], what=f"grid {grid} {sr}")


# a tree with repeated labels (diagonal pre-pass), batch labels, a swapped
# (B (x) A) step, an input read by two steps and a non-scalar result
TREE = dict(subs=["aab", "bcz", "cdz", "dez", "ea"],
            shapes=[(7, 7, 33), (33, 20, 5), (20, 9, 5), (9, 70, 5), (70, 7)],
            steps=[(0, 1, "zac"), (5, 2, "zda"), (6, 3, "zea"), (7, 4, "az"), (8, 4, "ze")])


@pytest.mark.parametrize("sr,dt", PAIRS, ids=lambda p: str(p).replace("torch.", ""))
def test_tree_labels_batch_diag_and_shared_input(tb, orc, sr, dt):
    g = torch.Generator().manual_seed(11)
    xs = cast_inputs(sr, dt, [torch.randn(s, generator=g) for s in TREE["shapes"]], seed=12)
    run_both(tb, orc, sr, dt, TREE["subs"], xs, TREE["steps"], what=f"labelled tree {sr}")


def test_tree_strided_inputs_and_partial_argmax(tb, orc):
    g = torch.Generator().manual_seed(13)
    xs = [torch.randn(s, generator=g) for s in TREE["shapes"]]
    # column-major and sliced views as inputs
    xs[1] = torch.randn(5, 20, 33, generator=g).permute(2, 1, 0)
    xs[4] = torch.randn(70, 14, generator=g)[:, ::2]
    for flags in ([True, False, True, False, True], [False] * 5):
        run_both(tb, orc, "max_plus", torch.float32, TREE["subs"], xs, TREE["steps"], argmax=flags,
                 what=f"strided inputs, argmax {flags}")


def test_tree_reduction_label(tb, orc):
    # f is in one tensor only and not in the result: reduced in its step's
    # pre-pass
    subs, steps = ["ab", "bcf", "cd"], [(0, 1, "ac"), (3, 2, "ad")]
    g = torch.Generator().manual_seed(14)
    xs = [torch.randn(s, generator=g) for s in ((30, 40), (40, 50, 6), (50, 20))]
    run_both(tb, orc, "min_plus", torch.float32, subs, xs, steps, argmax=[False, True], what="reduced label")
    # its argmax continues over the reduced label (routed through the pre-pass)
    run_both(tb, orc, "min_plus", torch.float32, subs, xs, steps, argmax=True, what="routed reduced label")


def test_tree_workspace_reuse_across_runs_and_streams(tb, orc):
    net = inputs.grid_network(3, 4, 6, salt=3)
    plan = tb.tropical_tree_plan_create("max_plus", torch.float32, net["subs"], net["shapes"], net["steps"])
    nbytes = tb.tropical_tree_workspace_size(plan)
    ws = torch.full((nbytes // 4 + 1,), float("nan"), device=DEV).view(torch.uint8)
    s = torch.cuda.Stream()
    results = []
    for salt, stream in ((4, None), (5, s), (4, s)):
        xs = inputs.grid_network(3, 4, 6, salt=salt)["tensors"]
        with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
            out, ams = tb.tropical_tree_run(plan, [x.to(DEV) for x in xs], argmax=True, workspace=ws,
                                            stream=stream)
        torch.cuda.synchronize()
        ref, rams = orc.contract_tree("max_plus", [x.numpy() for x in xs], net["subs"], net["steps"])
        assert_bits_equal(out.cpu().numpy(), ref, f"run with salt {salt}")
        for a, r in zip(ams, rams):
            assert_equal(a.cpu().numpy(), r, f"argmax, salt {salt}")
        results.append(out.cpu())
    assert torch.equal(results[0], results[2])
    with pytest.raises(tb.TropicalError) as e:
        tb.tropical_tree_run(plan, [x.to(DEV) for x in net["tensors"]], workspace=ws[: nbytes - 4])
    assert e.value.status == tb.WORKSPACE_TOO_SMALL


def test_tree_stays_on_device(tb, monkeypatch):
    """Counters of one run: kernels only -- no host synchronisation, no copy."""
    net = inputs.grid_network(4, 4, 4, salt=6)
    plan = tb.tropical_tree_plan_create("max_plus", torch.float32, net["subs"], net["shapes"], net["steps"])
    xs = [x.to(DEV) for x in net["tensors"]]
    ws = torch.empty(tb.tropical_tree_workspace_size(plan), dtype=torch.uint8, device=DEV)
    out = torch.empty((), device=DEV)
    ams = [torch.empty(tb.tropical_tree_step_info(plan, s)[1], dtype=torch.int32, device=DEV)
           for s in range(len(net["steps"]))]
    torch.cuda.synchronize()
    desc = tb.tropical_tree_describe(plan)
    # (a step split along K adds its merge launch)
    gathers = desc.count("gather:") + desc.count("permute:") + desc.count("splitK")
    tb.tropical_reset_stats()
    tb.tropical_tree_run(plan, xs, out=out, argmax=ams, workspace=ws)
    st = tb.tropical_get_stats()
    torch.cuda.synchronize()
    # a step whose two operands both take the tiled gather runs them in one
    # launch; with pairing off every gather is its own launch
    assert st["launches_total"] <= len(net["steps"]) + gathers
    paired = [a.clone() for a in ams]
    monkeypatch.setenv("TROPICAL_NO_PAIRED_GATHER", "1")
    tb.tropical_reset_stats()
    tb.tropical_tree_run(plan, xs, out=out, argmax=ams, workspace=ws)
    st = tb.tropical_get_stats()
    torch.cuda.synchronize()
    assert st["launches_total"] == len(net["steps"]) + gathers
    for a, b in zip(paired, ams):
        assert torch.equal(a, b)


def test_tree_zero_extent_bond(tb, orc):
    # a bond of extent 0: every sum over it is empty (K = 0), so the first
    # step fills its result with the zero element, and so is the scalar
    subs, steps = ["ab", "bc", "ca"], [(0, 1, "ac"), (3, 2, "")]
    shapes = [(3, 0), (0, 4), (4, 3)]
    xs = [torch.zeros(s) for s in shapes]
    for sr, zero in (("max_plus", -np.inf), ("min_plus", np.inf), ("max_mul", 0.0)):
        plan = tb.tropical_tree_plan_create(sr, torch.float32, subs, shapes, steps)
        out, _ = tb.tropical_tree_run(plan, [x.to(DEV) for x in xs])
        torch.cuda.synchronize()
        ref, _ = orc.contract_tree(sr, [x.numpy() for x in xs], subs, steps, argmax=False)
        assert_bits_equal(out.cpu().numpy(), ref, f"zero-extent bond {sr}")
        assert out.item() == zero


def test_tree_graph_capture_replays(tb, orc):
    """The run only enqueues kernels, so it can be captured in a HIP graph;
    replays are checked one by one against the eager result."""
    net = inputs.grid_network(3, 3, 8, salt=7)
    plan = tb.tropical_tree_plan_create("max_plus", torch.float32, net["subs"], net["shapes"], net["steps"])
    xs = [x.to(DEV) for x in net["tensors"]]
    ws = torch.empty(tb.tropical_tree_workspace_size(plan), dtype=torch.uint8, device=DEV)
    out = torch.empty((), device=DEV)
    ams = [torch.empty(tb.tropical_tree_step_info(plan, s)[1], dtype=torch.int32, device=DEV)
           for s in range(len(net["steps"]))]
    eager, eager_ams = tb.tropical_tree_run(plan, xs, argmax=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        tb.tropical_tree_run(plan, xs, out=out, argmax=ams, workspace=ws, stream=s)
    for rep in range(3):
        out.fill_(0.0)
        for a in ams:
            a.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        for a, e in zip(ams, eager_ams):
            assert torch.equal(a, e), f"replay {rep} argmax"


def _brute_points(orc, sr, la, lb, out, A, B, points, argmax):
    """Sampled outputs of one step by the oracle's brute-force einsum: the
    operands are sliced at each output position, leaving the contracted
    labels (in left-operand order), and contracted to a scalar."""
    con = []
    for c in la:
        if c in lb and c not in out and c not in con:
            con.append(c)
    vals, args = [], []
    for pos in points:
        fix = dict(zip(out, pos))
        sa = tuple(fix.get(c, slice(None)) for c in la)
        sb = tuple(fix.get(c, slice(None)) for c in lb)
        ra = "".join(c for c in la if c not in fix)
        rb = "".join(c for c in lb if c not in fix)
        C, I = orc.einsum_brute(sr, f"{ra},{rb}->", np.ascontiguousarray(A[sa]), np.ascontiguousarray(B[sb]),
                                sum_order=con, argmax=argmax)
        vals.append(C.reshape(()))
        args.append(I.reshape(()) if argmax else None)
    return vals, args


def test_tree_benchmark_network_full_size(tb, orc):
    """The 5 x 5 lattice with bond 16 (64 MiB intermediates) as the benchmark
    runs it: the result and every step's argmax equal the oracle's tree bit
    for bit; the tree equals the device's own pairwise calls bit for bit,
    sampled outputs of every step equal the oracle's brute force, and
    following the argmax from the result down to the inputs recomputes the
    result exactly (the same additions in the same order)."""
    net = inputs.grid_network(5, 5, 16)
    subs, steps = list(net["subs"]), net["steps"]
    xs = [x.to(DEV) for x in net["tensors"]]
    plan = tb.tropical_tree_plan_create("max_plus", torch.float32, subs, net["shapes"], steps)
    out, ams = tb.tropical_tree_run(plan, xs, argmax=True)
    torch.cuda.synchronize()
    ref, rams = orc.contract_tree("max_plus", [x.numpy() for x in net["tensors"]], list(net["subs"]), steps,
                                  argmax=True)
    assert_bits_equal(out.cpu().numpy(), ref, "5x5 bond-16 network result")
    for s, r in enumerate(rams):
        assert_equal(ams[s].cpu().numpy(), r, f"5x5 bond-16 network argmax of step {s}")
    # the same steps through tropical_contract_pair, keeping intermediates
    slots = list(xs)
    for s, (l, r, o) in enumerate(steps):
        C, I = tb.tropical_contract_pair(f"{subs[l]},{subs[r]}->{o}", "max_plus", slots[l], slots[r])
        slots.append(C)
        subs.append(o)
        assert torch.equal(I, ams[s]), f"step {s} argmax vs pairwise call"
    torch.cuda.synchronize()
    assert torch.equal(out, slots[-1])
    host = [t.cpu().numpy() for t in slots]
    rng = np.random.default_rng(21)
    n = len(net["subs"])
    for s, (l, r, o) in enumerate(steps):
        R = host[n + s]
        pts = [tuple(int(rng.integers(0, e)) for e in R.shape) for _ in range(12)]
        pts.append(tuple(e - 1 for e in R.shape))
        vals, args = _brute_points(orc, "max_plus", subs[l], subs[r], o, host[l], host[r], pts, True)
        am = ams[s].cpu().numpy()
        for p, v, a in zip(pts, vals, args):
            assert_bits_equal(R[p], v, f"step {s} at {p}")
            assert am[p] == a, f"step {s} argmax at {p}: {am[p]} vs {a}"
    # winner routing: recompute the result along the argmax path
    ams_h = [a.cpu().numpy() for a in ams]

    def routed(slot, assign):
        if slot < n:
            return host[slot][tuple(assign[c] for c in subs[slot])]
        s = slot - n
        l, r, o = steps[s]
        con = []
        for c in subs[l]:
            if c in subs[r] and c not in o and c not in con:
                con.append(c)
        code = int(ams_h[s][tuple(assign[c] for c in o)])
        for c in reversed(con):
            assign[c] = code % 16
            code //= 16
        return np.float32(routed(l, assign) + routed(r, assign))

    assert_bits_equal(np.float32(routed(len(slots) - 1, {})), out.cpu().numpy(), "routed result")
