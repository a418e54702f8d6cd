"""Calls captured in a HIP graph (torch.cuda.graph) and replayed: every replay,
on fresh operands written into the captured buffers, must give the bits of an
eager call on the same operands (deterministic modes) or stay within the
oracle's tolerance (atomic modes).  The library's workspace is allocated by an
eager call before the capture; a call enqueues kernels only (no memset nodes),
and the Stream-K turnstile's flags clear themselves after use, so the epoch
fixed at capture time serves every replay."""
import pytest
import torch

from oracle import gemm as og
from workloads import WORKLOADS, make_operands

from gpu_util import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_work_amd as dg

    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return dg


CASES = [
    ("c3-turnstile", "c3_wavequant", "heuristic", 0, False, 0),
    ("c1-two-pass", "c1_sk32", "streamk", 32, False, 0),
    ("c1-turnstile", "c1_sk32", "streamk", 32, False, "IN_LAUNCH"),
    ("c2a-last-arriver", "c2a_m96_s8", "splitk", 8, False, "IN_LAUNCH"),
    ("c2a-two-pass", "c2a_m96_s8", "splitk", 8, False, 0),
    ("c5-atomic", "c5_longk_fp16", "streamk", 0, True, 0),
    ("hybrid", "x1_hybrid", "heuristic", 0, False, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(dg, case):
    cid, name, mode, splits, atomic, debug = case
    w = WORKLOADS[name]
    dbg = dg.GEMM_DEBUG_IN_LAUNCH if debug == "IN_LAUNCH" else 0
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    c = torch.empty((w.M, w.N), dtype=torch.float32, device=DEV)
    call = lambda out: dg.gemm_tensors(a, b, out, b_layout=w.b_layout, mode=mode, splits=splits, atomic=atomic,
                                       debug=dbg)
    call(c)                      # eager: allocates the workspace outside the capture
    torch.cuda.synchronize()
    assert dg.gemm_sync_status() == 0
    g = torch.cuda.CUDAGraph()
    say(f"  capture {cid}")
    with torch.cuda.graph(g):
        call(c)
    rows = sorted({0, 1, w.M // 2, w.M - 1})
    for r in range(4):
        A2, B2 = make_operands(w, seed=50 + r)
        a.copy_(A2.to(DEV))
        b.copy_(B2.to(DEV))
        c.fill_(7.0)
        say(f"  replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
        ce = torch.full_like(c, 7.0)
        call(ce)                 # eager work between the replays, on the same operands
        torch.cuda.synchronize()
        if not atomic:
            assert torch.equal(c.view(torch.int32), ce.view(torch.int32)), f"replay {r} differs from eager"
        C, S = og.ref_gemm(A2, B2, w.M, w.N, w.K, w.b_layout, w.dtype, rows=rows)
        ok, worst, idx = og.within_tolerance(c.cpu().numpy()[rows], C, S)
        assert ok, f"replay {r}: worst ratio {worst} at {idx}"
    del g


# the refused call enqueues nothing, so torch reports the captured graph as empty
@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_capture_refuses_workspace_growth(dg):
    # with no library workspace yet, a captured call would have to allocate one:
    # it is refused (GEMM_ERR_WORKSPACE), nothing is captured, and the same call
    # works eagerly afterwards
    w = WORKLOADS["c1_sk32"]
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    torch.cuda.synchronize()
    dg.gemm_release()
    c = torch.full((w.M, w.N), 7.0, dtype=torch.float32, device=DEV)
    g = torch.cuda.CUDAGraph()
    status = None
    say("  capture with an empty library workspace")
    with torch.cuda.graph(g):
        try:
            dg.gemm_tensors(a, b, c, mode="streamk", splits=32)
        except dg.GemmError as e:
            status = e.status
    assert status == dg.GEMM_ERR_WORKSPACE, dg.gemm_last_error()
    del g
    torch.cuda.synchronize()
    assert torch.all(c == 7.0), "a refused call must not touch C"
    dg.gemm_tensors(a, b, c, mode="streamk", splits=32)
    assert dg.gemm_sync_status() == 0
    C, S = og.ref_gemm(A, B, w.M, w.N, w.K, w.b_layout, w.dtype)
    ok, worst, idx = og.within_tolerance(c.cpu().numpy(), C, S)
    assert ok, f"worst ratio {worst} at {idx}"


def test_graph_replays_after_workspace_grows(dg):
    # a graph captured on a small library workspace keeps replaying correctly
    # after a larger eager call has grown the workspace (the outgrown blocks are
    # retired, not freed)
    small = WORKLOADS["c1_sk32"]
    A, B = make_operands(small)
    a, b = A.to(DEV), B.to(DEV)
    torch.cuda.synchronize()
    dg.gemm_release()
    c = torch.empty((small.M, small.N), dtype=torch.float32, device=DEV)
    call = lambda out: dg.gemm_tensors(a, b, out, mode="streamk", splits=32, debug=dg.GEMM_DEBUG_IN_LAUNCH)
    call(c)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(c)
    # grow both blocks: 65 x 65 = 4225 tiles need more Split-K counters than the
    # first control block holds (4096), and S = 2 partials of 8320 x 8320 fp32
    # (554 MB) more data than the Stream-K slots took
    big = WORKLOADS["c1_sk32"].with_(name="grow", M=8320, N=8320, K=128)
    A2, B2 = make_operands(big)
    c2 = torch.empty((big.M, big.N), dtype=torch.float32, device=DEV)
    say("  eager call that grows the workspace")
    dg.gemm_tensors(A2.to(DEV), B2.to(DEV), c2, mode="splitk", splits=2, debug=dg.GEMM_DEBUG_IN_LAUNCH)
    assert dg.gemm_sync_status() == 0
    rows = [0, 4160, 8319]
    C2, S2 = og.ref_gemm(A2, B2, big.M, big.N, big.K, big.b_layout, big.dtype, rows=rows)
    ok, worst, idx = og.within_tolerance(c2.cpu().numpy()[rows], C2, S2)
    assert ok, f"growing call: worst ratio {worst} at {idx}"
    del c2
    for r in range(3):
        A3, B3 = make_operands(small, seed=70 + r)
        a.copy_(A3.to(DEV))
        b.copy_(B3.to(DEV))
        c.fill_(7.0)
        say(f"  replay {r} after growth")
        g.replay()
        torch.cuda.synchronize()
        assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
        ce = torch.full_like(c, 7.0)
        call(ce)
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int32), ce.view(torch.int32)), f"replay {r} differs from eager"
        C, S = og.ref_gemm(A3, B3, small.M, small.N, small.K, small.b_layout, small.dtype)
        ok, worst, idx = og.within_tolerance(c.cpu().numpy(), C, S)
        assert ok, f"replay {r}: worst ratio {worst} at {idx}"
    del g
