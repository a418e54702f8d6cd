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
