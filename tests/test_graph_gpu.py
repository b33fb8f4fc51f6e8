"""The kernels captured in a HIP graph: every replay matches the eager result
bitwise.

The library launches on the caller's stream and records no memset or host
work into it, so a caller may capture its calls.  Replays run with eager
work and synchronisations between them, on inputs changed between replays
(the graph reads its buffers at replay time), and each replay is checked
against an eager call on the same inputs.
"""
import pytest

import workloads
from tests.test_parity_gpu import _as, _bits, _rr, _say, softmax_input

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rr = _rr()
    rr.lib()
    yield


def test_graph_replays_match_eager():
    rr = _rr()
    M, H = 64, 4096
    x = _as(workloads.random_rows(M, H, seed=1), "bf16").cuda()
    r0 = _as(workloads.random_rows(M, H, seed=2), "bf16").cuda()
    g = _as(workloads.gamma_vector(H, seed=3), "bf16").cuda()
    res = r0.clone()
    y = torch.empty_like(x)
    s = softmax_input(40, 152064, seed=4, dt="bf16").cuda()          # the split path, with workspace
    sy = torch.empty(s.shape, dtype=torch.float32, device="cuda")
    ws = rr.softmax_workspace(s, torch.float32)
    c = softmax_input(300, 4096, seed=5, dt="f32").cuda()            # causal rule, log output
    cy = torch.empty_like(c)
    opts = rr.make_softmax_opts(log_output=True, causal_period=300, causal_offset=3796)

    def step():
        rr.rr_fused_add_rmsnorm(y, res, x, g, 1e-6)
        rr.rr_softmax_rows(sy, s, ws)
        rr.rr_softmax_rows_ex(cy, c, opts)

    def eager_reference():
        """Outputs of one eager step from the current inputs, leaving them as they were."""
        keep = res.clone()
        step()
        torch.cuda.synchronize()
        out = (y.clone(), res.clone(), sy.clone(), cy.clone())
        res.copy_(keep)
        return out

    step()                       # warm-up outside the capture
    torch.cuda.synchronize()
    res.copy_(r0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for k in range(4):
        _say(f"graph replay {k}")
        # new inputs in place: the replay must read them
        x.copy_(_as(workloads.random_rows(M, H, seed=10 + k), "bf16").cuda())
        res.copy_(r0)
        s.mul_(0.5)
        c.add_(1.0)
        ref = eager_reference()
        y.zero_()
        sy.zero_()
        cy.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, what in zip((y, res, sy, cy), ref, ("fused y", "residual", "split softmax", "causal log")):
            assert torch.equal(_bits(got), _bits(want)), f"replay {k}: {what}"
        torch.cuda.synchronize()


def test_graph_replays_of_cut_rows_match_eager():
    """The cut-row kernels captured: a softmax of few odd-width rows (the
    split, with its workspace), a packed one, and a LayerNorm over rows of an
    odd width, replayed on changed inputs and checked bitwise against eager
    calls."""
    rr = _rr()
    s1 = softmax_input(4, 152065, seed=21, dt="bf16").cuda()         # split, rows cut at aligned addresses
    y1 = torch.empty(s1.shape, dtype=torch.float32, device="cuda")
    ws = rr.softmax_workspace(s1, torch.float32)
    s2 = softmax_input(256, 50257, seed=22, dt="bf16").cuda()        # packed, cut
    y2 = torch.empty(s2.shape, dtype=torch.float32, device="cuda")
    M, H = 100, 4097
    x = _as(workloads.random_rows(M, H, seed=23), "bf16").cuda()
    g = _as(workloads.gamma_vector(H, seed=24), "bf16").cuda()
    b = _as(workloads.gamma_vector(H, seed=25) - 1.0, "bf16").cuda()
    y3 = torch.empty_like(x)
    for t, N in ((s1, 152065), (s2, 50257)):
        assert rr.rr_query_plan(rr.RR_OP_SOFTMAX, t.shape[0], N, rr.RR_BF16, rr.RR_F32, 2)["row_shift"] == 1
    assert rr.rr_query_plan(rr.RR_OP_LAYERNORM, M, H, rr.RR_BF16, rr.RR_BF16, 2)["row_shift"] == 1

    def step():
        rr.rr_softmax_rows(y1, s1, ws)
        rr.rr_softmax_rows(y2, s2, None)
        rr.rr_layernorm(y3, x, g, b, 1e-5)

    def eager_reference():
        step()
        torch.cuda.synchronize()
        return (y1.clone(), y2.clone(), y3.clone())

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for k in range(4):
        _say(f"cut-row graph replay {k}")
        s1.mul_(0.5)
        s2.add_(0.25)
        x.copy_(_as(workloads.random_rows(M, H, seed=30 + k), "bf16").cuda())
        ref = eager_reference()
        for t in (y1, y2, y3):
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, what in zip((y1, y2, y3), ref, ("cut split softmax", "cut packed softmax", "cut layernorm")):
            assert torch.equal(_bits(got), _bits(want)), f"replay {k}: {what}"


def test_graph_replays_of_the_no_allocation_call_and_a_forced_one_kernel_split():
    """The no-allocation entry point on a split row (its (m, d) slots in the
    library's static scratch, no workspace argument) and the one-kernel
    split forced in the diagnostics build, captured: the one-kernel form
    stays one kernel in the graph, its slot tags coming from per-row epochs
    that each replay reads and advances on the device.  Between replays the
    graph's slots hold the previous replay's pairs (the eager references use
    workspaces of their own), so a replay that took a stale pair for a fresh
    one would be off; replays on changed inputs equal eager calls bit for
    bit."""
    rr = _rr()
    s1 = softmax_input(24, 152064, seed=41, dt="bf16").cuda()
    y1 = torch.empty(s1.shape, dtype=torch.float32, device="cuda")
    s2 = softmax_input(16, 65536, seed=42, dt="f32").cuda()
    y2 = torch.empty_like(s2)
    ws2 = rr.softmax_workspace(s2, torch.float32)
    assert rr.rr_query_plan(rr.RR_OP_SOFTMAX, 24, 152064, rr.RR_BF16, rr.RR_F32)["variant_name"] == "split"

    def eager_reference():
        r1 = torch.empty_like(y1)
        r2 = torch.empty_like(y2)
        rr.rr_softmax_rows(r1, s1, rr.softmax_workspace(s1, torch.float32))
        rr.rr_softmax_rows(r2, s2, rr.softmax_workspace(s2, torch.float32))
        torch.cuda.synchronize()
        return r1, r2

    with rr.forced_variant(rr.RR_VARIANT_SPLIT_ONE_KERNEL):
        def step():
            rr.rr_softmax_rows_strided_noalloc(y1, s1)
            rr.rr_softmax_rows(y2, s2, ws2)
        step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
    for k in range(4):
        _say(f"no-allocation / one-kernel graph replay {k}")
        s1.mul_(0.75)
        s2.add_(0.5)
        ref = eager_reference()
        y1.zero_()
        y2.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, what in zip((y1, y2), ref, ("no-allocation split", "forced one-kernel split")):
            assert torch.equal(_bits(got), _bits(want)), f"replay {k}: {what}"
