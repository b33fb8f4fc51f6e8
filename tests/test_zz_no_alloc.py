"""GPU test of the no-allocation softmax entry point.

rr_softmax_rows_strided_noalloc takes its split-row (m, d) slots from the
library's static scratch array instead of a workspace argument.  Called
through the C ABI, its output must equal, bit for bit, that of
rr_softmax_rows_strided with a workspace from torch (the same kernels and
plans), and the oracle within the softmax bars.  Two calls follow each other
on the shared array, the second on a smaller input (rows cut at aligned
addresses, another dtype pair), then a shape that needs no workspace.  (The
refusal of a split larger than the array is a host test in
tests/test_abi_host.py.)
"""
import numpy as np
import pytest

import oracle
from tests import compare

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _rr():
    import row_reduction_rmsnorm_amd as rr
    return rr


def _dt(t):
    rr = _rr()
    return rr.RR_F32 if t.dtype == torch.float32 else rr.RR_BF16


def _noalloc(y, x):
    rr = _rr()
    M, N = x.shape
    st = rr.raw_softmax_rows_strided_noalloc(y.data_ptr(), N, x.data_ptr(), N, M, N, _dt(x), _dt(y), None,
                                             torch.cuda.current_stream().cuda_stream)
    rr.check(st, "rr_softmax_rows_strided_noalloc")


def _with_workspace(y, x):
    rr = _rr()
    M, N = x.shape
    nb = rr.rr_softmax_rows_ex_workspace_bytes(M, N, _dt(x), _dt(y))
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None
    st = rr.raw_softmax_rows_strided(y.data_ptr(), N, x.data_ptr(), N, M, N, _dt(x), _dt(y), None,
                                     ws.data_ptr() if ws is not None else None, nb,
                                     torch.cuda.current_stream().cuda_stream)
    rr.check(st, "rr_softmax_rows_strided")
    return nb


def _input(M, N, seed, dt):
    rng = np.random.default_rng(seed)
    x = (3.0 * rng.standard_normal((M, N), dtype=np.float32)).astype(np.float32)
    for r in range(M):
        x[r, rng.choice(N, 4, replace=False)] = rng.uniform(20.0, 30.0, 4).astype(np.float32)
    t = torch.from_numpy(x)
    return t.to(torch.bfloat16) if dt == "bf16" else t


def _case(M, N, din, dout, seed, expect_split):
    rr = _rr()
    x_cpu = _input(M, N, seed, din)
    odt = torch.float32 if dout == "f32" else torch.bfloat16
    plan = rr.rr_query_plan(rr.RR_OP_SOFTMAX, M, N, _dt(x_cpu), rr.RR_F32 if dout == "f32" else rr.RR_BF16,
                            aligned16=1 if (N * x_cpu.element_size()) % 16 == 0 else 2)
    assert (plan["variant_name"] == "split") == expect_split, plan
    print(f"[no-alloc] M={M} N={N} {din}->{dout} plan={plan['variant_name']} "
          f"chunks={plan['chunks_per_row']}", flush=True)
    x = x_cpu.cuda()
    y_ref = torch.full((M, N), float("nan"), dtype=odt, device="cuda")
    nb = _with_workspace(y_ref, x)
    assert (nb > 0) == expect_split
    y = torch.full((M, N), float("nan"), dtype=odt, device="cuda")
    _noalloc(y, x)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32 if dout == "f32" else torch.int16),
                       y_ref.view(torch.int32 if dout == "f32" else torch.int16)), \
        "no-allocation call differs from the call with a workspace"
    xf = compare.to_f64(x_cpu)
    compare.check_softmax(y.cpu(), xf, oracle.softmax(xf), f"no-alloc {M}x{N} {din}->{dout}")


def test_noalloc_equals_workspace_call_twice_then_smaller():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    # few long rows: the split path, slots in the static scratch array
    _case(40, 152064, "bf16", "f32", seed=11, expect_split=True)
    # a second, smaller call on the same array: rows cut at aligned addresses
    _case(6, 70001, "f32", "bf16", seed=12, expect_split=True)
    # a shape that needs no slots at all
    _case(64, 1024, "f32", "f32", seed=13, expect_split=False)

