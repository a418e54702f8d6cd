"""gemm_ex_noalloc, the entry point that allocates nothing (its workspace is the
library's fixed per-device scratch array), against gemm_ex on the library
workspace, called through the C ABI on the same operands: bit-identical for the
deterministic merges, within the oracle's bound |C - C_ref| <= 1e-4 sum|a||b|
for the atomic ones.  Each case makes two gemm_ex_noalloc calls in a row on one
stream, the second with a smaller problem, so the second runs on what the first
left in the array (flags, counters, partials)."""
import pytest
import torch

from oracle import gemm as og
from workloads import WORKLOADS, make_operands

from gpu_util import guarded_output, guards_intact, oracle_full, say, tile_row_sample

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_work_amd as dg

    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return dg


# (workload, mode, splits, atomic, merge): merge "plan", "two_pass" or "in_launch"
PAIRS = [
    # turnstile Stream-K (16 MiB of slots), then two-pass Stream-K on 32 short units
    (("c3_wavequant", "heuristic", 0, False, "plan"), ("c1_sk32", "streamk", 32, False, "plan")),
    # two-pass Stream-K (32 MiB of slots), then two-pass Split-K S = 8
    (("c5_longk_fp16", "streamk", 0, False, "two_pass"), ("c2a_m96_s8", "splitk", 8, False, "plan")),
    # the hybrid (768 data-parallel tiles first), then the last arriver of Split-K S = 2
    (("x1_hybrid", "heuristic", 0, False, "plan"), ("c2b_m256_s2", "splitk", 2, False, "in_launch")),
    # last-arriver Split-K S = 8, then a turnstile on 7 units over ragged tiles
    (("c2a_m96_s8", "splitk", 8, False, "in_launch"), ("c1_sk32@300x200x320", "streamk", 7, False, "in_launch")),
    # atomic Stream-K, then atomic Split-K
    (("c5_longk_fp16", "streamk", 0, True, "plan"), ("c2a_m96_s8", "splitk", 8, True, "plan")),
]


def _workload(spec):
    if "@" in spec:
        name, shape = spec.split("@")
        M, N, K = map(int, shape.split("x"))
        return WORKLOADS[name].with_(name=spec, M=M, N=N, K=K)
    return WORKLOADS[spec]


def _kw(dg, w, mode, splits, atomic, merge):
    return dict(b_layout=w.b_layout, mode=mode, splits=splits, atomic=atomic, two_pass=merge == "two_pass",
                debug=dg.GEMM_DEBUG_IN_LAUNCH if merge == "in_launch" else 0)


def _operands(w):
    if w.M * w.N >= 1 << 21:
        A, B, _, _ = oracle_full(w)   # the large ones are also checked in full below
        return A, B
    return make_operands(w)


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0][0]}-then-{p[1][0]}")
def test_noalloc_matches_gemm_ex(dg, pair):
    calls = []
    for spec, mode, splits, atomic, merge in pair:
        w = _workload(spec)
        A, B = _operands(w)
        a, b = A.to(DEV), B.to(DEV)
        kw = _kw(dg, w, mode, splits, atomic, merge)
        ref = torch.full((w.M, w.N), 7.0, dtype=torch.float32, device=DEV)
        dg.gemm_tensors(a, b, ref, **kw)                 # gemm_ex, library workspace
        calls.append((w, A, B, a, b, kw, ref))
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    outs = []
    for w, A, B, a, b, kw, ref in calls:                 # two gemm_ex_noalloc calls in a row
        full, c = guarded_output(w.M, w.N, DEV)
        say(f"  gemm_ex_noalloc {w.name} {w.M}x{w.N}x{w.K} {kw}")
        dg.gemm_tensors(a, b, c, noalloc=True, **kw)
        outs.append((full, c))
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    for (w, A, B, a, b, kw, ref), (full, c) in zip(calls, outs):
        assert guards_intact(full, w.M, w.N), "guard band overwritten"
        if not kw["atomic"]:
            assert torch.equal(c.view(torch.int32), ref.view(torch.int32)), f"{w.name}: bits differ from gemm_ex"
        else:
            rows = tile_row_sample(w.M, seed=9) if w.M > 256 else None
            for out in (c, ref):
                C, S = og.ref_gemm(A, B, w.M, w.N, w.K, w.b_layout, w.dtype, rows=rows)
                got = out.cpu().numpy()
                ok, worst, idx = og.within_tolerance(got if rows is None else got[rows], C, S)
                say(f"    atomic {w.name}: worst err/bound {worst:.3e}")
                assert ok, f"{w.name}: worst ratio {worst} at {idx}"


def test_noalloc_refuses_beyond_its_array(dg):
    # Split-K partials [4, 2048, 2048] fp32 (64 MiB) exceed the array: refused, C untouched
    w = WORKLOADS["c1_sk32"].with_(name="too-big", M=2048, N=2048, K=2048)
    a = torch.zeros((w.M, w.K), dtype=torch.bfloat16, device=DEV)
    b = torch.zeros((w.K, w.N), dtype=torch.bfloat16, device=DEV)
    full, c = guarded_output(w.M, w.N, DEV)
    with pytest.raises(dg.GemmError) as ei:
        dg.gemm_tensors(a, b, c, mode="splitk", splits=4, noalloc=True)
    assert ei.value.status == dg.GEMM_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(c == 7.0) and guards_intact(full, w.M, w.N)
    # the same problem at S = 2 (32 MiB of partials) fits and matches gemm_ex
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    ref = torch.empty((w.M, w.N), dtype=torch.float32, device=DEV)
    dg.gemm_tensors(a, b, ref, mode="splitk", splits=2)
    dg.gemm_tensors(a, b, c, mode="splitk", splits=2, noalloc=True)
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    assert torch.equal(c.view(torch.int32), ref.view(torch.int32))
    assert guards_intact(full, w.M, w.N)
