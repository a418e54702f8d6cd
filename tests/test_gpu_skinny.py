"""GPU parity of the skinny 64 x 128 tile (GEMM_TILE_64x128: the CUTLASS guide's
"Tile Size Selection", tall/skinny tab, recommends 64-row tiles when N is much
larger than M; the book chapter names small-M products as Split-K's case),
through the C ABI, on every decomposition and merge: values against the fp64
oracle (|C - C_ref| <= 1e-4 sum|a||b| on every element), the kernels' trace
against the simulator's schedule for 64-row tiles, bit identity over runs and
across the deterministic merges, the zero-partial control, and the fused
epilogue where it applies."""
import numpy as np
import pytest
import torch

from oracle import epilogue as oe
from oracle import gemm as og
from workloads import WORKLOADS, make_epilogue_inputs, make_operands

from gpu_util import (GUARD, NGUARD, check_against_oracle, check_full, decode_trace, expected_trace,
                      guarded_output, guards_intact, oracle_full, poison_rows, say)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SKINNY = "64x128"


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_work_amd as dg

    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return dg


def _w(M, N, K, layout="kn", dtype="bf16", name="skinny"):
    dist = dict(dist="uniform", low=-1.0, high=1.0) if dtype == "bf16" else dict(dist="uniform", low=-0.5, high=0.5)
    return WORKLOADS["c1_sk32"].with_(name=name, M=M, N=N, K=K, b_layout=layout, dtype=dtype, **dist)


def run_skinny(dg, w, A, B, mode, splits=0, **kw):
    a, b = A.to(DEV), B.to(DEV)
    full, c = guarded_output(w.M, w.N, DEV)
    say(f"  skinny {w.name} {w.M}x{w.N}x{w.K} {w.dtype} {w.b_layout} mode={mode} splits={splits} {kw}")
    dg.gemm_tensors(a, b, c, b_layout=w.b_layout, mode=mode, splits=splits, tile=SKINNY, **kw)
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    assert guards_intact(full, w.M, w.N), "guard band overwritten"
    return c


SMALL = [   # (M, N, K, layout, dtype)
    (64, 256, 512, "kn", "bf16"),
    (96, 512, 2048, "nk", "bf16"),     # the second tile row half empty
    (1, 8, 8, "kn", "bf16"),
    (33, 200, 328, "nk", "fp16"),      # ragged M, N and K
    (130, 136, 1024, "kn", "bf16"),    # three tile rows, the last with 2 rows
    (128, 100, 2048, "nk", "fp16"),    # N not a multiple of 8 (scalar fold paths)
]

# (mode, splits, extra arguments)
PATHS = [
    ("dp", 0, {}),
    ("splitk", 4, {}),                                   # the planner's merge
    ("splitk", 4, {"debug": "IN_LAUNCH"}),               # last arriver
    ("splitk", 4, {"debug": "SPLITK_BANDS"}),            # row bands
    ("splitk", 2, {"two_pass": True}),
    ("splitk", 8, {"atomic": True}),
    ("streamk", 7, {}),
    ("streamk", 7, {"debug": "IN_LAUNCH"}),              # turnstile
    ("streamk", 5, {"two_pass": True}),
    ("streamk", 6, {"atomic": True}),
    ("heuristic", 0, {}),
]


def _kw(dg, extra):
    kw = dict(extra)
    if "debug" in kw:
        kw["debug"] = {"IN_LAUNCH": dg.GEMM_DEBUG_IN_LAUNCH, "SPLITK_BANDS": dg.GEMM_DEBUG_SPLITK_BANDS}[kw["debug"]]
    return kw


def _fits(M, N, K, mode, splits):
    ipt = -(-K // 64)
    return mode != "splitk" or (ipt % splits == 0)


# every (shape, path) pair where Split-K's S divides the k-iterations
SMALL_CASES = [(shape, path) for shape in SMALL for path in PATHS if _fits(*shape[:3], path[0], path[1])]


@pytest.mark.parametrize("shape,path", SMALL_CASES,
                         ids=["x".join(map(str, c[0][:3])) + f"-{c[0][3]}-{c[0][4]}-{c[1][0]}{c[1][1]}-"
                              + "-".join(f"{k}{v}" for k, v in c[1][2].items()) for c in SMALL_CASES])
def test_skinny_small_shapes(dg, shape, path):
    M, N, K, layout, dtype = shape
    mode, splits, extra = path
    w = _w(M, N, K, layout, dtype)
    A, B = make_operands(w)
    c = run_skinny(dg, w, A, B, mode, splits, **_kw(dg, extra))
    ok, worst, idx = check_against_oracle(c, A, B, w)
    say(f"    worst err/bound = {worst:.3e} at {idx}")
    assert ok, f"outside tolerance: worst ratio {worst} at {idx}"
    assert not poison_rows(c), "an output element was never written"


@pytest.mark.parametrize("name,mode,splits,extra", [
    ("c2a_m96_s8", "splitk", 8, {}),
    ("c2b_m256_s2", "splitk", 2, {}),
    ("c2a_m96_s8", "splitk", 8, {"atomic": True}),
    ("c1_sk32", "streamk", 32, {}),
    ("c1_sk32", "streamk", 32, {"atomic": True}),
    ("c1_sk32", "dp", 0, {}),
])
def test_skinny_config_shapes_full(dg, name, mode, splits, extra):
    w = WORKLOADS[name]
    A, B, _, _ = oracle_full(w)
    c = run_skinny(dg, w, A, B, mode, splits, **extra)
    ok, worst, idx = check_full(c, w)
    say(f"    worst err/bound = {worst:.3e} at {idx} (all {w.M * w.N} elements)")
    assert ok, f"outside tolerance: worst ratio {worst} at {idx}"
    if name.startswith("c2"):
        assert torch.all(c[0] == 0.0), "A row 0 is zero, so C row 0 must be exactly zero"


@pytest.mark.parametrize("atomic", [False, True])
def test_skinny_longk_fp16_full(dg, atomic):
    # 1536^2 x 16384 fp16 on 64x128 tiles (288 tiles x 256 iterations over 256
    # units), both fixup modes; every element
    w = WORKLOADS["c5_longk_fp16"]
    A, B, _, _ = oracle_full(w)
    c = run_skinny(dg, w, A, B, "streamk", 0, atomic=atomic)
    ok, worst, idx = check_full(c, w)
    say(f"    worst err/bound = {worst:.3e} at {idx} (all {w.M * w.N} elements)")
    assert ok, f"outside tolerance: worst ratio {worst} at {idx}"


def test_skinny_decode_batch(dg):
    # the book chapter's skinny case: a 128-row batch through a 4096-wide
    # projection (64 tiles of 64 x 128); the rule's choice and Split-K S = 4
    w = _w(128, 4096, 4096, "nk", "bf16", name="decode128")
    A, B = make_operands(w)
    C, S = og.ref_gemm(A, B, w.M, w.N, w.K, w.b_layout, w.dtype)
    for mode, splits in (("heuristic", 0), ("splitk", 4)):
        c = run_skinny(dg, w, A, B, mode, splits)
        ok, worst, idx = og.within_tolerance(c.cpu().numpy().astype(np.float64), C, S)
        say(f"    {mode}: worst err/bound = {worst:.3e} at {idx}")
        assert ok, f"{mode}: outside tolerance: worst ratio {worst} at {idx}"


def test_skinny_hybrid_full_size(dg):
    # 4096x4224x4096 on 64x128 tiles: 64 x 33 = 2112 tiles = 8 full waves + a
    # 64-tile tail, so the rule keeps 7 waves data-parallel and runs Stream-K over
    # the last 320 tiles, all in one persistent launch; every element
    w = WORKLOADS["x1_hybrid"]
    p = dg.gemm_plan(w.M, w.N, w.K, 0, dg.mode_word("heuristic", tile=SKINNY), 0, 256)
    assert dg.DECISION_NAMES[p.decision] == "StreamK" and (p.dp_tiles, p.sk_tiles) == (1792, 320)
    A, B, _, _ = oracle_full(w)
    c = run_skinny(dg, w, A, B, "heuristic")
    ok, worst, idx = check_full(c, w)
    say(f"    worst err/bound = {worst:.3e} at {idx} (all {w.M * w.N} elements)")
    assert ok, f"outside tolerance: worst ratio {worst} at {idx}"


TRACE = [   # (M, N, K, mode, splits)
    (96, 512, 2048, "splitk", 8),
    (128, 4096, 4096, "splitk", 4),
    (256, 512, 2048, "streamk", 32),
    (300, 200, 328, "streamk", 7),
    (64, 128, 128, "streamk", 6),     # more units than iterations
    (130, 136, 1024, "dp", 0),
    (128, 4096, 4096, "heuristic", 0),
]


@pytest.mark.parametrize("case", TRACE, ids=lambda c: "x".join(map(str, c[:3])) + f"-{c[3]}{c[4]}")
def test_skinny_trace_matches_simulator(dg, case):
    M, N, K, mode, splits = case
    cus = dg.gemm_num_cus()
    p = dg.gemm_plan(M, N, K, 0, dg.mode_word(mode, tile=SKINNY), splits, cus)
    tr = torch.zeros(p.trace_ints, dtype=torch.int32, device=DEV)
    w = _w(M, N, K)
    A, B = make_operands(w)
    full, c = guarded_output(M, N, DEV)
    say(f"  skinny trace {M}x{N}x{K} {mode} splits={splits}")
    dg.gemm_tensors(A.to(DEV), B.to(DEV), c, mode=mode, splits=splits, tile=SKINNY, trace=tr)
    assert dg.gemm_sync_status() == 0
    got = decode_trace(tr)
    s, segs, folds = expected_trace(M, N, K, mode, splits, cus, bm=64)
    assert dg.DECISION_NAMES[got["decision"]] == s.kind
    assert got["segments"] == segs
    assert got["folds"] == folds
    assert np.all(got["coverage"] == 1), "every (tile, k) pair must run exactly once"


@pytest.mark.parametrize("name,mode,splits", [("c2a_m96_s8", "splitk", 8), ("c2b_m256_s2", "splitk", 2),
                                              ("c1_sk32", "streamk", 32)])
def test_skinny_bit_identical_10_runs(dg, name, mode, splits):
    w = WORKLOADS[name]
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    c0 = torch.empty((w.M, w.N), dtype=torch.float32, device=DEV)
    say(f"  skinny 10 runs {name} {mode} S={splits}")
    dg.gemm_tensors(a, b, c0, b_layout=w.b_layout, mode=mode, splits=splits, tile=SKINNY)
    for _ in range(9):
        c = torch.full((w.M, w.N), 7.0, dtype=torch.float32, device=DEV)
        dg.gemm_tensors(a, b, c, b_layout=w.b_layout, mode=mode, splits=splits, tile=SKINNY)
        assert torch.equal(c.view(torch.int32), c0.view(torch.int32))
    assert dg.gemm_sync_status() == 0


@pytest.mark.parametrize("M,N", [(96, 512), (200, 392)])
def test_skinny_splitk_merges_agree(dg, M, N):
    # row bands, last arriver and second kernel add the partials in split order:
    # the same bits
    w = WORKLOADS["c2a_m96_s8"].with_(M=M, N=N)
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    outs = []
    for kw in (dict(debug=dg.GEMM_DEBUG_SPLITK_BANDS), dict(debug=dg.GEMM_DEBUG_IN_LAUNCH), dict(two_pass=True)):
        say(f"  skinny Split-K merges {M}x{N} {kw}")
        full, c = guarded_output(w.M, w.N, DEV)
        dg.gemm_tensors(a, b, c, b_layout=w.b_layout, mode="splitk", splits=8, tile=SKINNY, **kw)
        outs.append((full, c))
    assert dg.gemm_sync_status() == 0
    for f, _ in outs:
        assert guards_intact(f, w.M, w.N)
    for _, c in outs[1:]:
        assert torch.equal(outs[0][1].view(torch.int32), c.view(torch.int32))
    ok, worst, idx = check_against_oracle(outs[0][1], A, B, w)
    assert ok, f"outside tolerance: worst ratio {worst} at {idx}"


def test_skinny_streamk_two_pass_equals_turnstile(dg):
    w = WORKLOADS["c1_sk32"]
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    outs = []
    for kw in (dict(debug=dg.GEMM_DEBUG_IN_LAUNCH), dict(two_pass=True)):
        say(f"  skinny Stream-K turnstile / two-pass {kw}")
        c = torch.full((w.M, w.N), 7.0, dtype=torch.float32, device=DEV)
        dg.gemm_tensors(a, b, c, mode="streamk", splits=32, tile=SKINNY, **kw)
        outs.append(c)
    assert dg.gemm_sync_status() == 0
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))


@pytest.mark.parametrize("name,mode,splits,extra", [
    ("c2a_m96_s8", "splitk", 8, {}),
    ("c2b_m256_s2", "splitk", 2, {}),
    ("c2a_m96_s8", "splitk", 8, {"atomic": True}),
    ("c1_sk32", "streamk", 32, {}),
    ("c1_sk32", "streamk", 32, {"two_pass": True}),
])
def test_skinny_zero_partial_control(dg, name, mode, splits, extra):
    w = WORKLOADS[name]
    A, B, _, _ = oracle_full(w)
    for control in (True, False):
        c = run_skinny(dg, w, A, B, mode, splits, debug=dg.GEMM_DEBUG_ZERO_PARTIAL if control else 0, **extra)
        ok, worst, _ = check_full(c, w)
        say(f"    control={control}: worst err/bound = {worst:.3e}")
        assert ok != control


@pytest.mark.parametrize("mode,splits,extra", [
    ("dp", 0, {}), ("splitk", 8, {}), ("splitk", 8, {"two_pass": True}), ("splitk", 8, {"atomic": True}),
    # 8 tiles x 32 iterations: 12 units split every tile over at most three (the turnstile), 24 units over
    # four (the second kernel adds them), 20 units with atomics
    ("streamk", 12, {}), ("streamk", 24, {}), ("streamk", 12, {"two_pass": True}), ("streamk", 20, {"atomic": True}),
    ("heuristic", 0, {})])
def test_skinny_epilogue(dg, mode, splits, extra):
    w = _w(96, 512, 2048, "nk", "bf16", name="skinny-epi")
    A, B = make_operands(w)
    alpha, beta, act = 0.75, -0.5, "gelu"
    c_in, bias = make_epilogue_inputs(w.M, w.N)
    full = torch.full((w.M * w.N + NGUARD,), GUARD, dtype=torch.float32, device=DEV)
    full[: w.M * w.N] = c_in.reshape(-1).to(DEV)
    c = full[: w.M * w.N].view(w.M, w.N)
    say(f"  skinny epilogue {mode} S={splits} {extra}")
    dg.gemm_tensors(A.to(DEV), B.to(DEV), c, b_layout=w.b_layout, mode=mode, splits=splits, tile=SKINNY,
                    alpha=alpha, beta=beta, bias=bias.to(DEV), act=act, **extra)
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    assert bool(torch.all(full[w.M * w.N:] == GUARD)), "guard band overwritten"
    P, S = og.ref_gemm(A, B, w.M, w.N, w.K, w.b_layout, w.dtype)
    c0 = c_in.numpy().astype(np.float64)
    b64 = bias.numpy().astype(np.float64)
    D, _ = oe.epilogue_ref(P, c0, alpha, beta, b64, act)
    bound = oe.epilogue_bound(S, P, c0, alpha, beta, b64, act)
    ok, worst, idx = oe.within_bound(c.cpu().numpy().astype(np.float64), D, bound)
    say(f"    worst err/bound = {worst:.3e} at {idx}")
    assert ok, f"outside the epilogue bound: worst ratio {worst} at {idx}"


def test_skinny_streamk_epilogue_is_deterministic(dg):
    # the turnstile and the second kernel give the same bits with the epilogue,
    # in any unit order, run after run
    w = _w(96, 512, 2048, "nk", "bf16", name="skinny-epi-bits")
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    c_in, bias = make_epilogue_inputs(w.M, w.N)
    epi = dict(alpha=0.75, beta=-0.5, bias=bias.to(DEV), act="relu")
    outs = []
    for extra in ({}, {"two_pass": True}, {}, {"unit_perm": torch.arange(11, -1, -1, dtype=torch.int32, device=DEV)}):
        c = c_in.to(DEV).clone()
        dg.gemm_tensors(a, b, c, b_layout=w.b_layout, mode="streamk", splits=12, tile=SKINNY, **epi, **extra)
        assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
        outs.append(c.view(torch.int32).clone())
    for o in outs[1:]:
        assert torch.equal(outs[0], o)


@pytest.mark.parametrize("name,mode,splits,extra", [
    ("c1_sk32", "streamk", 32, {"debug": "IN_LAUNCH"}),   # turnstile owners reading their peers' flags
    ("c2a_m96_s8", "splitk", 8, {}),                      # row bands in the launch
    ("c2b_m256_s2", "splitk", 2, {}),                     # second kernel
])
def test_skinny_graph_replays_match_eager(dg, name, mode, splits, extra):
    w = WORKLOADS[name]
    kw = _kw(dg, extra)
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    c = torch.empty((w.M, w.N), dtype=torch.float32, device=DEV)
    call = lambda out: dg.gemm_tensors(a, b, out, b_layout=w.b_layout, mode=mode, splits=splits, tile=SKINNY, **kw)
    call(c)                      # eager: the workspace exists before the capture
    torch.cuda.synchronize()
    assert dg.gemm_sync_status() == 0
    g = torch.cuda.CUDAGraph()
    say(f"  capture skinny {name} {mode} S={splits} {extra}")
    with torch.cuda.graph(g):
        call(c)
    for r in range(3):
        A2, B2 = make_operands(w, seed=60 + r)
        a.copy_(A2.to(DEV))
        b.copy_(B2.to(DEV))
        c.fill_(7.0)
        say(f"  replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
        ce = torch.full_like(c, 7.0)
        call(ce)                 # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int32), ce.view(torch.int32)), f"replay {r} differs from eager"
        ok, worst, idx = check_against_oracle(c, A2, B2, w)
        assert ok, f"replay {r}: worst ratio {worst} at {idx}"
    del g


@pytest.mark.parametrize("mode,splits,extra", [("splitk", 4, {}), ("streamk", 40, {"debug": "IN_LAUNCH"}),
                                               ("heuristic", 0, {})])
def test_skinny_batched(dg, mode, splits, extra):
    # three entries of 96x512x2048 (B [N,K]) at a padded stride of C
    w = _w(96, 512, 2048, "nk", "bf16", name="skinny-batched")
    batch, pad = 3, 20
    As, Bs = zip(*(make_operands(w, seed=200 + e) for e in range(batch)))
    A, B = torch.stack(As), torch.stack(Bs)
    stride = (w.M * w.N + 3) // 4 * 4 + pad
    full = torch.full((batch * stride + NGUARD,), GUARD, dtype=torch.float32, device=DEV)
    c = torch.as_strided(full, (batch, w.M, w.N), (stride, w.N, 1))
    c.fill_(7.0)
    say(f"  skinny batched {mode} S={splits} {extra}")
    dg.gemm_tensors(A.to(DEV), B.to(DEV), c, b_layout="nk", mode=mode, splits=splits, tile=SKINNY, **_kw(dg, extra))
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    mask = torch.ones_like(full, dtype=torch.bool)
    for e in range(batch):
        mask[e * stride: e * stride + w.M * w.N] = False
    assert bool(torch.all(full[mask] == GUARD)), "a pad or the guard band was overwritten"
    for e in range(batch):
        ok, worst, idx = check_against_oracle(c[e], As[e], Bs[e], w)
        assert ok, f"entry {e}: worst ratio {worst} at {idx}"
