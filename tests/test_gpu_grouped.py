"""GPU parity of grouped calls (gemm_grouped: problems of one K and their own M
and N, decomposed as one call) through the C ABI: every problem against the
fp64 oracle on every element, the schedule trace against the simulator's
grouped reading, the bits of deterministic merges over runs and unit orders,
the zero-partial control, and problems left empty."""
import numpy as np
import pytest
import torch

from oracle import gemm as og
from oracle import schedule as sch
from workloads import WORKLOADS, make_operands

from gpu_util import GUARD, NGUARD, POISON, decode_trace, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_work_amd as dg

    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return dg


def _problems(shapes, K, layout, dtype, seed=300):
    """Per-problem seeded operands and guarded outputs (C poisoned with 7, a guard
    band of 11 behind each C)."""
    base = WORKLOADS["c1_sk32"]
    dist = dict(dist="uniform", low=-1.0, high=1.0) if dtype == "bf16" else dict(dist="uniform", low=-0.5, high=0.5)
    out = []
    for i, (M, N) in enumerate(shapes):
        w = base.with_(name=f"group{i}", M=max(M, 1), N=max(N, 8), K=max(K, 8), b_layout=layout, dtype=dtype,
                       **dist)
        A, B = make_operands(w, seed=seed + i)
        if K == 0:
            A = A[:, :0]
            B = B[:0] if layout == "kn" else B[:, :0]
        if M == 0:
            A = A[:0]
        if N == 0:
            B = B[:, :0] if layout == "kn" else B[:0]
        full = torch.full((M * N + NGUARD,), POISON, dtype=torch.float32, device=DEV)
        full[M * N:] = GUARD
        out.append(dict(M=M, N=N, w=w, A=A, B=B, a=A.to(DEV).contiguous(), b=B.to(DEV).contiguous(),
                        full=full, c=full[: M * N].view(M, N)))
    return out


def _run(dg, probs, layout, **kw):
    say(f"  grouped {[(p['M'], p['N']) for p in probs]} layout={layout} {kw}")
    dg.gemm_grouped_tensors([(p["a"], p["b"], p["c"]) for p in probs], b_layout=layout, **kw)
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    for i, p in enumerate(probs):
        assert bool(torch.all(p["full"][p["M"] * p["N"]:] == GUARD)), f"problem {i}: guard band overwritten"


def _check(probs, K, layout, dtype):
    worst = 0.0
    for i, p in enumerate(probs):
        if p["M"] == 0 or p["N"] == 0:
            continue
        C, S = og.ref_gemm(p["A"], p["B"], p["M"], p["N"], K, layout, dtype)
        ok, ratio, idx = og.within_tolerance(p["c"].cpu().numpy().astype(np.float64), C, S)
        worst = max(worst, ratio)
        assert ok, f"problem {i} ({p['M']}x{p['N']}): worst ratio {ratio} at {idx}"
    say(f"    worst err/bound over {len(probs)} problems = {worst:.3e}")


SETS = {
    "ragged": [(96, 512), (0, 512), (300, 1024), (1, 8), (130, 136)],
    "experts": [(64 * i + 17, 1024) for i in range(8)],            # ragged batch sizes through one projection
    "big-and-small": [(1024, 1024), (128, 128), (33, 200), (256, 512)],
}

# (mode, splits, extra)
PATHS = [
    ("heuristic", 0, {}),
    ("dp", 0, {}),
    ("splitk", 4, {}),                          # the planner's merge
    ("splitk", 4, {"debug": "IN_LAUNCH"}),      # last arriver
    ("splitk", 8, {"debug": "SPLITK_BANDS"}),   # row bands
    ("splitk", 2, {"atomic": True}),
    ("streamk", 0, {}),
    ("streamk", 37, {"debug": "IN_LAUNCH"}),    # turnstile
    ("streamk", 37, {"two_pass": True}),
    ("streamk", 0, {"atomic": True}),
]


def _kw(dg, extra):
    kw = dict(extra)
    if "debug" in kw:
        kw["debug"] = {"IN_LAUNCH": dg.GEMM_DEBUG_IN_LAUNCH, "SPLITK_BANDS": dg.GEMM_DEBUG_SPLITK_BANDS}[kw["debug"]]
    return kw


@pytest.mark.parametrize("path", PATHS, ids=lambda p: f"{p[0]}{p[1]}-" + "-".join(f"{k}{v}" for k, v in p[2].items()))
@pytest.mark.parametrize("set_name,layout,dtype", [("ragged", "nk", "bf16"), ("experts", "kn", "fp16"),
                                                    ("big-and-small", "kn", "bf16")])
def test_grouped_parity(dg, set_name, layout, dtype, path):
    mode, splits, extra = path
    shapes = SETS[set_name]
    if layout == "kn" and any(N % 8 for _, N in shapes):
        pytest.fail("test set breaks the [K,N] layout's N % 8 requirement")
    K = 1024
    probs = _problems(shapes, K, layout, dtype)
    _run(dg, probs, layout, mode=mode, splits=splits, **_kw(dg, extra))
    _check(probs, K, layout, dtype)


@pytest.mark.parametrize("mode,splits", [("heuristic", 0), ("splitk", 4), ("streamk", 0)])
def test_grouped_skinny_tiles(dg, mode, splits):
    shapes = SETS["experts"]
    K = 2048
    probs = _problems(shapes, K, "nk", "bf16", seed=400)
    _run(dg, probs, "nk", mode=mode, splits=splits, tile="64x128")
    _check(probs, K, "nk", "bf16")


@pytest.mark.parametrize("set_name,mode,splits", [("ragged", "streamk", 37), ("experts", "heuristic", 0),
                                                  ("big-and-small", "splitk", 4), ("ragged", "dp", 0)])
def test_grouped_trace_matches_simulator(dg, set_name, mode, splits):
    shapes = SETS[set_name]
    K = 1024
    cus = dg.gemm_num_cus()
    lw = dg.layout_word("nk", "bf16")
    p = dg.gemm_plan_grouped(shapes, K, lw, dg.mode_word(mode), splits, cus)
    tr = torch.zeros(p.trace_ints, dtype=torch.int32, device=DEV)
    probs = _problems(shapes, K, "nk", "bf16")
    _run(dg, probs, "nk", mode=mode, splits=splits, trace=tr)
    got = decode_trace(tr)
    s = sch.plan_schedule_grouped(shapes, K, mode, splits, cus)
    assert dg.DECISION_NAMES[got["decision"]] == s.kind
    assert got["segments"] == sorted(x.as_tuple() for x in s.segments)
    groups = sch.tile_groups(s.segments)
    assert got["folds"] == {t: [owner] + peers for t, (owner, peers) in groups.items()}
    assert np.all(got["coverage"] == 1), "every (tile, k) pair must run exactly once"


@pytest.mark.parametrize("mode,splits,extra", [("streamk", 0, {}), ("splitk", 8, {}), ("splitk", 4, {})])
def test_grouped_bit_identical_over_runs_and_unit_order(dg, mode, splits, extra):
    shapes = SETS["experts"]
    K = 2048
    probs = _problems(shapes, K, "nk", "bf16")
    _run(dg, probs, "nk", mode=mode, splits=splits, **extra)
    ref = [p["c"].clone() for p in probs]
    for r in range(9):
        for p in probs:
            p["c"].fill_(POISON)
        kw = dict(extra)
        if r == 8 and mode == "streamk":   # the last run in reversed unit order
            n = dg.gemm_plan_grouped(shapes, K, dg.layout_word("nk", "bf16"), dg.mode_word(mode), splits,
                                     dg.gemm_num_cus()).sk_units
            kw["unit_perm"] = torch.arange(n - 1, -1, -1, dtype=torch.int32, device=DEV)
        _run(dg, probs, "nk", mode=mode, splits=splits, **kw)
        for i, p in enumerate(probs):
            assert torch.equal(p["c"].view(torch.int32), ref[i].view(torch.int32)), f"run {r}: problem {i} differs"


@pytest.mark.parametrize("mode,splits,extra", [("streamk", 0, {}), ("splitk", 4, {}), ("splitk", 8, {}),
                                               ("streamk", 0, {"atomic": True})])
def test_grouped_zero_partial_control(dg, mode, splits, extra):
    import dense_gemm_work_amd as dgm

    shapes = SETS["experts"]
    K = 2048
    probs = _problems(shapes, K, "nk", "bf16")
    _run(dg, probs, "nk", mode=mode, splits=splits, debug=dgm.GEMM_DEBUG_ZERO_PARTIAL, **extra)
    with pytest.raises(AssertionError):
        _check(probs, K, "nk", "bf16")
    _run(dg, probs, "nk", mode=mode, splits=splits, **extra)
    _check(probs, K, "nk", "bf16")


def test_grouped_k_zero_and_all_empty(dg):
    probs = _problems([(96, 512), (0, 64), (40, 8)], 0, "nk", "bf16")
    _run(dg, probs, "nk")
    for p in probs:
        assert torch.all(p["c"] == 0.0)
    probs = _problems([(0, 512), (64, 0)], 256, "nk", "bf16")
    _run(dg, probs, "nk")   # nothing to do: no launch, guards intact


@pytest.mark.parametrize("mode,splits,tile", [("heuristic", 0, "128x128"), ("heuristic", 0, "64x128")])
def test_grouped_expert_layer_full_size(dg, mode, splits, tile):
    """The grouped bench workload (8 problems, 2048 tokens, 4096 -> 2048) at its
    full size, every element of every problem against the oracle."""
    from workloads import GROUPED, make_group_operands

    gw = GROUPED["x4_grouped"]
    As, B = make_group_operands(gw)
    b = B.to(DEV)
    probs = []
    for g, (A, M) in enumerate(zip(As, gw.Ms)):
        full = torch.full((M * gw.N + NGUARD,), POISON, dtype=torch.float32, device=DEV)
        full[M * gw.N:] = GUARD
        probs.append(dict(M=M, N=gw.N, A=A, B=B[g], a=A.to(DEV), b=b[g], full=full,
                          c=full[: M * gw.N].view(M, gw.N)))
    _run(dg, probs, gw.b_layout, mode=mode, splits=splits, tile=tile)
    for p in probs:
        assert not bool(torch.any(p["c"] == POISON)), "an output element was never written"
    _check(probs, gw.K, gw.b_layout, gw.dtype)



@pytest.mark.parametrize("mode,splits,tile", [("streamk", 0, "128x128"), ("splitk", 4, "128x128"),
                                              ("dp", 0, "64x128"), ("streamk", 0, "64x128")])
def test_grouped_ragged_k(dg, mode, splits, tile):
    """K not a multiple of the 64-wide iteration: the last iteration of every
    tile is zero-filled beyond K, in every problem."""
    K = 1000
    probs = _problems(SETS["ragged"], K, "nk", "bf16", seed=500)
    _run(dg, probs, "nk", mode=mode, splits=splits, tile=tile)
    _check(probs, K, "nk", "bf16")


@pytest.mark.parametrize("mode,splits", [("heuristic", 0), ("splitk", 4), ("streamk", 37)])
def test_grouped_graph_replays_match_eager(dg, mode, splits):
    """A grouped call captured in a HIP graph (its problem table is written by a
    kernel, no memset or host copy): every replay on fresh operands gives the
    bits of an eager call, with eager work between the replays."""
    shapes = SETS["experts"]
    K = 1024
    probs = _problems(shapes, K, "kn", "fp16", seed=600)
    triples = [(p["a"], p["b"], p["c"]) for p in probs]
    call = lambda outs: dg.gemm_grouped_tensors([(a, b, o) for (a, b, _), o in zip(triples, outs)],
                                                b_layout="kn", mode=mode, splits=splits)
    call([p["c"] for p in probs])           # eager: allocates the workspace outside the capture
    torch.cuda.synchronize()
    assert dg.gemm_sync_status() == 0
    g = torch.cuda.CUDAGraph()
    say(f"  capture grouped {mode}{splits}")
    with torch.cuda.graph(g):
        call([p["c"] for p in probs])
    for r in range(3):
        fresh = _problems(shapes, K, "kn", "fp16", seed=700 + 10 * r)
        for p, q in zip(probs, fresh):
            p["a"].copy_(q["a"])
            p["b"].copy_(q["b"])
            p["c"].fill_(POISON)
            p["A"], p["B"] = q["A"], q["B"]
        say(f"  replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
        eager = [torch.full_like(p["c"], POISON) for p in probs]
        call(eager)                          # eager work between the replays, on the same operands
        torch.cuda.synchronize()
        for i, (p, e) in enumerate(zip(probs, eager)):
            assert torch.equal(p["c"].view(torch.int32), e.view(torch.int32)), f"replay {r}: problem {i} differs"
        _check(probs, K, "kn", "fp16")
    del g
