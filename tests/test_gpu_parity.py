"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle and the
schedule simulator.

Bar (per element): |C_gpu - C_ref| <= 1e-4 * sum_k |a_ik||b_kj|, outputs that
start poisoned at 7 are all overwritten, and 64 trailing guard elements keep
their value 11.  Schedules (segments, fold order, coverage) must equal the
simulator's exactly.  Deterministic modes must be bit-identical across runs
and unit orders."""
import numpy as np
import pytest
import torch

from oracle import gemm as og
from workloads import WORKLOADS, make_operands

from gpu_util import (POISON, check_against_oracle, check_full, decode_trace, expected_trace, guarded_output,
                      guards_intact, oracle_full, poison_rows, sample_rows, say, tile_row_sample)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_work_amd as dg

    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return dg


DEV = "cuda:0"


def run(dg, w, mode=None, splits=None, atomic=None, A=None, B=None, **kw):
    mode = w.mode if mode is None else mode
    splits = w.splits if splits is None else splits
    atomic = w.atomic if atomic is None else atomic
    if A is None:
        A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    full, c = guarded_output(w.M, w.N, DEV)
    say(f"  gemm {w.name} {w.M}x{w.N}x{w.K} {w.dtype} {w.b_layout} mode={mode} splits={splits} atomic={atomic}")
    dg.gemm_tensors(a, b, c, b_layout=w.b_layout, mode=mode, splits=splits, atomic=atomic, **kw)
    st = dg.gemm_sync_status()
    assert st == 0, dg.gemm_last_error()
    assert guards_intact(full, w.M, w.N), "guard band overwritten"
    return A, B, c


def assert_parity(c, A, B, w, rows=None):
    """Elementwise bound on every row, or on a row sample joined by every row
    that still holds the fill value somewhere (an element never written fails
    there; a product that happens to equal the fill value passes)."""
    if rows is not None:
        rows = sorted(set(rows) | set(poison_rows(c)))
    ok, worst, idx = check_against_oracle(c, A, B, w, rows=rows)
    say(f"    worst err/bound = {worst:.3e} at {idx}" + ("" if rows is None else f" ({len(rows)} rows)"))
    assert ok, f"outside tolerance: worst ratio {worst} at {idx}"


def assert_parity_full(c, w):
    """Every element against the session's cached full-size oracle."""
    ok, worst, idx = check_full(c, w)
    say(f"    worst err/bound = {worst:.3e} at {idx} (all {w.M * w.N} elements)")
    assert ok, f"outside tolerance: worst ratio {worst} at {idx}"


# ---------------------------------------------------------------------------
# Layout probe: identity A makes C equal B exactly, so any mistake in the
# MFMA operand/result layout shows up as a permutation.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("b_layout", ["kn", "nk"])
def test_identity_layout(dg, b_layout):
    M = N = K = 128
    A = torch.eye(M, K, dtype=torch.bfloat16)
    vals = (torch.arange(K * N) % 251 - 125).to(torch.float32).view(K, N)
    B = vals.to(torch.bfloat16) if b_layout == "kn" else vals.t().contiguous().to(torch.bfloat16)
    w = WORKLOADS["c1_sk32"].with_(name="identity", M=M, N=N, K=K, b_layout=b_layout)
    _, _, c = run(dg, w, mode="dp", splits=0, A=A, B=B)
    assert torch.equal(c.cpu(), vals), "MFMA layout mismatch"


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------
def test_c1_streamk_32_units(dg):
    w = WORKLOADS["c1_sk32"]
    A, B, c = run(dg, w)
    assert_parity(c, A, B, w)


@pytest.mark.parametrize("name", ["c2a_m96_s8", "c2b_m256_s2"])
def test_c2_splitk(dg, name):
    w = WORKLOADS[name]
    A, B, c = run(dg, w)
    assert_parity(c, A, B, w)
    assert torch.all(c[0] == 0), "row 0 of A is zero, so row 0 of C must be exactly zero"


def test_c3_heuristic_streamk(dg):
    # every element of the headline workload against the full fp64 product
    w = WORKLOADS["c3_wavequant"]
    p = dg.gemm_plan(w.M, w.N, w.K, 0, dg.GEMM_HEURISTIC, 0, 256)
    assert (dg.DECISION_NAMES[p.decision], p.sk_units, p.sk_tiles) == ("StreamK", 256, 272)
    A, B, _, _ = oracle_full(w)
    _, _, c = run(dg, w, A=A, B=B)
    assert_parity_full(c, w)


def test_x1_hybrid_full_size(dg):
    # the heuristic's hybrid regime at full size: 3 data-parallel waves + Stream-K,
    # every element
    w = WORKLOADS["x1_hybrid"]
    p = dg.gemm_plan(w.M, w.N, w.K, 0, dg.GEMM_HEURISTIC, 0, 256)
    assert dg.DECISION_NAMES[p.decision] == "StreamK" and p.dp_tiles == 768 and p.sk_tiles == 288
    assert p.sk_units == 256 and p.q == 72 and p.big == 0
    A, B, _, _ = oracle_full(w)
    _, _, c = run(dg, w, A=A, B=B)
    assert_parity_full(c, w)


def test_x3_decode_heuristic_full_size(dg):
    # the book chapter's skinny case: a 128-row batch through a 4096-wide
    # projection (32 tiles); the rule picks Split-K S = 8 over 256 workgroups,
    # partials added by the second kernel; every element
    w = WORKLOADS["x3_decode"]
    p = dg.gemm_plan(w.M, w.N, w.K, dg.layout_word(w.b_layout, w.dtype), dg.GEMM_HEURISTIC, 0, 256)
    assert (dg.DECISION_NAMES[p.decision], p.splits, p.tiles, p.two_pass) == ("SplitK", 8, 32, 1)
    A, B, _, _ = oracle_full(w)
    _, _, c = run(dg, w, A=A, B=B)
    assert_parity_full(c, w)


def test_c4_heuristic_dp(dg):
    # 8192^3 (1.1 Tflop of fp64): one random row inside every 128-row tile row,
    # plus every row that still holds the fill value
    w = WORKLOADS["c4_large_dp"]
    p = dg.gemm_plan(w.M, w.N, w.K, 0, dg.GEMM_HEURISTIC, 0, 256)
    assert dg.DECISION_NAMES[p.decision] == "DataParallel"
    A, B, c = run(dg, w)
    # a row holding the fill value joins the sample (an exact 7.0 is a legitimate
    # product here: about 0.4 are expected among the 2^26 outputs)
    assert_parity(c, A, B, w, rows=tile_row_sample(w.M, seed=4))


@pytest.mark.parametrize("M,N,K,layout,cus", [
    (4096, 4096, 320, "kn", 0),      # 1024 tiles -> 256 groups, odd iteration count
    (4000, 4064, 200, "kn", 0),      # ragged M, N and K (K % 64 = 8)
    (4096, 4096, 192, "nk", 0),      # B [N,K]
    (1024, 1024, 512, "kn", 16),     # 64 tiles on 16 CUs
    (2900, 4000, 256, "kn", 0),      # 23 x 32 tiles: the last group row hangs over the edge of M
])
def test_dp_tile_groups(dg, M, N, K, layout, cus):
    # data-parallel launches whose 2x2 tile groups finish in fewer tile times run
    # them one per workgroup; checked against the oracle and against one-tile
    # workgroups
    w = WORKLOADS["c4_large_dp"].with_(name="dp_groups", M=M, N=N, K=K, b_layout=layout)
    A, B, c = run(dg, w, mode="dp", splits=0, num_cus=cus)
    rows = sample_rows(M, 12) + [M - 2, M - 129]
    assert_parity(c, A, B, w, rows=sorted(set(rows)))
    _, c_tile = guarded_output(M, N, DEV)
    dg.gemm_tensors(A.to(DEV), B.to(DEV), c_tile, b_layout=layout, mode="dp", splits=0, num_cus=cus,
                    debug=dg.GEMM_DEBUG_TILE_DP)
    assert dg.gemm_sync_status() == 0
    assert_parity(c_tile, A, B, w, rows=sorted(set(rows)))


@pytest.mark.parametrize("atomic", [False, True])
def test_c5_streamk_fp16(dg, atomic):
    # both fixup modes, every element against the full fp64 product
    w = WORKLOADS["c5_longk_fp16"]
    A, B, _, _ = oracle_full(w)
    _, _, c = run(dg, w, A=A, B=B, atomic=atomic)
    assert_parity_full(c, w)


# ---------------------------------------------------------------------------
# Numerical control: with every partial written as zeros, each workload with
# split tiles must fail the oracle check, and pass again without the control
# (Metal split-K note, "Contract and numerical coverage")
# ---------------------------------------------------------------------------
ZERO_PARTIAL_CASES = [   # (workload, merge kind, extra gemm_tensors arguments)
    ("c1_sk32", "two-pass (plan)", {}),
    ("c1_sk32", "turnstile", dict(debug_in_launch=True)),
    ("c2a_m96_s8", "two-pass (plan)", {}),
    ("c2a_m96_s8", "last arriver", dict(debug_in_launch=True)),
    ("c2a_m96_s8", "atomic", dict(atomic=True)),
    ("c2b_m256_s2", "two-pass (plan)", {}),
    ("c2b_m256_s2", "last arriver", dict(debug_in_launch=True)),
    ("c3_wavequant", "turnstile (plan)", {}),
    ("c3_wavequant", "two-pass", dict(two_pass=True)),
    ("c5_longk_fp16", "turnstile", {}),
    ("c5_longk_fp16", "two-pass", dict(two_pass=True)),
    ("c5_longk_fp16", "atomic", dict(atomic=True)),
]


@pytest.mark.parametrize("name,kind,extra", ZERO_PARTIAL_CASES, ids=lambda x: x if isinstance(x, str) else "")
def test_zero_partial_control_fails(dg, name, kind, extra):
    w = WORKLOADS[name]
    A, B, _, _ = oracle_full(w)
    a, b = A.to(DEV), B.to(DEV)
    extra = dict(extra)
    base_debug = dg.GEMM_DEBUG_IN_LAUNCH if extra.pop("debug_in_launch", False) else 0
    kw = dict(b_layout=w.b_layout, mode=w.mode, splits=w.splits, **extra)
    for control in (True, False):
        full, c = guarded_output(w.M, w.N, DEV)
        debug = base_debug | (dg.GEMM_DEBUG_ZERO_PARTIAL if control else 0)
        say(f"  zero-partial control={control} {name} {kind}")
        dg.gemm_tensors(a, b, c, debug=debug, **kw)
        assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
        assert guards_intact(full, w.M, w.N)
        ok, worst, idx = check_full(c, w)
        say(f"    worst err/bound = {worst:.3e} at {idx}")
        assert ok != control, ("the control must fail the check" if control else "the plain call must pass")


# ---------------------------------------------------------------------------
# Every decomposition and layout on small, ragged shapes (full comparison)
# ---------------------------------------------------------------------------
SMALL = [
    # (M, N, K, layout, dtype)
    (256, 256, 512, "kn", "bf16"),
    (300, 200, 320, "kn", "bf16"),     # ragged M and N tails
    (300, 200, 328, "nk", "bf16"),     # ragged K (not a multiple of 64)
    (130, 136, 72, "kn", "fp16"),
    (96, 100, 2048, "nk", "fp16"),     # N not a multiple of 8 ([N,K] layout allows it)
    (1, 8, 8, "kn", "bf16"),           # a single element row
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s[:3])) + f"-{s[3]}-{s[4]}")
@pytest.mark.parametrize("mode,splits,atomic", [
    ("dp", 0, False), ("splitk", 1, False), ("splitk", -1, False), ("streamk", 7, False),
    ("streamk", 3, True), ("streamk", 0, False), ("streamk", 1, False), ("heuristic", 0, False),
])
def test_small_shapes_all_modes(dg, shape, mode, splits, atomic):
    M, N, K, layout, dtype = shape
    ipt = -(-K // 64)
    if splits == -1:   # largest split factor dividing ipt (at most 8)
        splits = max(s for s in range(1, 9) if ipt % s == 0)
    dist = dict(dist="uniform", low=-1.0, high=1.0) if dtype == "bf16" else dict(dist="uniform", low=-0.5, high=0.5)
    w = WORKLOADS["c1_sk32"].with_(name="small", M=M, N=N, K=K, b_layout=layout, dtype=dtype, **dist)
    A, B, c = run(dg, w, mode=mode, splits=splits, atomic=atomic)
    assert_parity(c, A, B, w)


# (shape, S) pairs of SMALL[:5] and S in 2, 3, 5, 8, 10 where S divides the k-iterations
BAND_CASES = [(shape, S) for shape in SMALL[:5] for S in (2, 3, 5, 8, 10) if -(-shape[2] // 64) % S == 0]


@pytest.mark.parametrize("shape,splits", BAND_CASES,
                         ids=["x".join(map(str, c[0][:3])) + f"-{c[0][3]}-{c[0][4]}-s{c[1]}" for c in BAND_CASES])
def test_small_shapes_splitk_row_bands(dg, shape, splits):
    # the in-launch row-band merge at split factors from 2 to 10 (the last arriver
    # where N is not a multiple of 4), against the oracle and the second kernel's bits
    M, N, K, layout, dtype = shape
    dist = dict(dist="uniform", low=-1.0, high=1.0) if dtype == "bf16" else dict(dist="uniform", low=-0.5, high=0.5)
    w = WORKLOADS["c1_sk32"].with_(name="bands", M=M, N=N, K=K, b_layout=layout, dtype=dtype, **dist)
    A, B, c = run(dg, w, mode="splitk", splits=splits, debug=dg.GEMM_DEBUG_SPLITK_BANDS)
    assert_parity(c, A, B, w)
    _, _, c2 = run(dg, w, mode="splitk", splits=splits, two_pass=True, A=A, B=B)
    assert torch.equal(c.view(torch.int32), c2.view(torch.int32))


def _random_cases(n, seed=11):
    """Seeded random small problems: shape, layout, dtype, decomposition, merge mode
    and CU count (small CU counts make tile groups and hybrids appear)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        layout = str(rng.choice(["kn", "nk"]))
        M = int(rng.integers(1, 700))
        N = int(rng.integers(1, 90)) * 8 if layout == "kn" else int(rng.integers(1, 700))
        K = int(rng.integers(1, 40)) * 8
        dtype = str(rng.choice(["bf16", "fp16"]))
        mode = str(rng.choice(["dp", "splitk", "streamk", "heuristic"]))
        cus = int(rng.choice([0, 4, 16, 64]))
        ipt = -(-K // 64)
        splits, atomic, two_pass = 0, False, False
        if mode == "splitk":
            splits = int(rng.choice([s for s in range(1, 9) if ipt % s == 0]))
            merge = int(rng.integers(0, 3))
            atomic, two_pass = merge == 1, merge == 2
        elif mode == "streamk":
            splits = int(rng.integers(1, 40))
            atomic = bool(rng.integers(0, 2))
        cases.append((i, M, N, K, layout, dtype, mode, splits, atomic, two_pass, cus))
    return cases


@pytest.mark.parametrize("case", _random_cases(24), ids=lambda c: f"r{c[0]}")
def test_random_small_problems(dg, case):
    i, M, N, K, layout, dtype, mode, splits, atomic, two_pass, cus = case
    dist = dict(dist="uniform", low=-1.0, high=1.0) if dtype == "bf16" else dict(dist="uniform", low=-0.5, high=0.5)
    w = WORKLOADS["c1_sk32"].with_(name=f"random{i}", M=M, N=N, K=K, b_layout=layout, dtype=dtype, seed=100 + i,
                                   **dist)
    cap = dg.gemm_num_cus() if cus == 0 else cus
    if mode == "streamk" and splits > cap:
        splits = cap   # Stream-K units must all be resident
    A, B, c = run(dg, w, mode=mode, splits=splits, atomic=atomic, two_pass=two_pass, num_cus=cus)
    assert_parity(c, A, B, w)


def _medium_cases(n, seed=23):
    """Seeded random medium problems on the device's own CU count: enough tiles
    for hybrids (three of the twelve on 256 CUs), tile groups (two) and
    multi-wave plans to arise as they do in real calls (sampled rows against
    the oracle, every element written)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        layout = str(rng.choice(["kn", "nk"]))
        M = int(rng.integers(300, 6200))
        N = int(rng.integers(40, 780)) * 8
        K = int(rng.integers(8, 320)) * 8
        dtype = str(rng.choice(["bf16", "fp16"]))
        mode = str(rng.choice(["heuristic", "heuristic", "dp", "streamk", "splitk"]))
        ipt = -(-K // 64)
        splits, atomic = 0, False
        if mode == "splitk":
            splits = int(rng.choice([s for s in range(1, 9) if ipt % s == 0]))
        elif mode == "streamk":
            atomic = bool(rng.integers(0, 2))
        cases.append((i, M, N, K, layout, dtype, mode, splits, atomic))
    return cases


@pytest.mark.parametrize("case", _medium_cases(12), ids=lambda c: f"m{c[0]}")
def test_random_medium_problems(dg, case):
    i, M, N, K, layout, dtype, mode, splits, atomic = case
    dist = dict(dist="uniform", low=-1.0, high=1.0) if dtype == "bf16" else dict(dist="uniform", low=-0.5, high=0.5)
    w = WORKLOADS["c1_sk32"].with_(name=f"medium{i}", M=M, N=N, K=K, b_layout=layout, dtype=dtype, seed=300 + i,
                                   **dist)
    A, B, c = run(dg, w, mode=mode, splits=splits, atomic=atomic)
    # rows still holding the fill value join the sample: an element never
    # written fails there, a product that happens to equal it passes
    filled = torch.nonzero((c == POISON).any(dim=1)).flatten().tolist()[:64]
    assert_parity(c, A, B, w, rows=sorted(set(sample_rows(M, 12, seed=i)) | set(filled)))


def test_k_zero_writes_zeros(dg):
    full, c = guarded_output(64, 64, DEV)
    a = torch.empty((64, 0), dtype=torch.bfloat16, device=DEV)
    b = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    dg.gemm_tensors(a, b, c, mode="dp")
    torch.cuda.synchronize()
    assert torch.all(c == 0) and guards_intact(full, 64, 64)


def test_units_more_than_iterations(dg):
    # 2 tiles x 2 iterations over 6 units: two units have nothing to do
    w = WORKLOADS["c1_sk32"].with_(name="tiny", M=256, N=128, K=128)
    A, B, c = run(dg, w, mode="streamk", splits=6)
    assert_parity(c, A, B, w)


def test_hybrid_dp_plus_streamk(dg):
    # with 20 CUs planned, 66 tiles = 3 full waves + 6: two DP waves, Stream-K on the last 26 tiles
    w = WORKLOADS["c3_wavequant"].with_(name="hybrid", M=1408, N=768, K=1024)
    p = dg.gemm_plan(w.M, w.N, w.K, 0, dg.GEMM_HEURISTIC, 0, 20)
    assert dg.DECISION_NAMES[p.decision] == "StreamK" and p.dp_tiles == 40 and p.sk_tiles == 26
    A, B, c = run(dg, w, mode="heuristic", splits=0, num_cus=20)
    assert_parity(c, A, B, w)


# ---------------------------------------------------------------------------
# Schedule: the kernels' own trace equals the simulator, bit for bit
# ---------------------------------------------------------------------------
TRACE_CASES = [
    ("c1", 256, 512, 2048, "streamk", 32, 256, False),
    ("c3", 2048, 2176, 4096, "heuristic", 0, 256, False),
    ("c5", 1536, 1536, 16384, "streamk", 0, 256, False),
    ("c5-atomic", 1536, 1536, 16384, "streamk", 0, 256, True),
    ("c2a", 96, 512, 2048, "splitk", 8, 256, False),
    ("c2b", 256, 512, 2048, "splitk", 2, 256, False),
    ("ragged-7u", 300, 200, 320, "streamk", 7, 256, False),
    ("one-unit", 300, 200, 328, "streamk", 1, 256, False),   # every tile whole, one after another
    ("units-over-iterations", 256, 128, 128, "streamk", 6, 256, False),   # 4 iterations over 6 units
    ("hybrid", 1408, 768, 1024, "heuristic", 0, 20, False),
    ("dp", 640, 384, 256, "dp", 0, 256, False),
    ("dp-groups", 1024, 1024, 256, "dp", 0, 16, False),   # 2x2 tile groups (64 tiles, 16 CUs)
    ("dp-groups-odd", 1152, 1024, 128, "dp", 0, 8, False),   # 9 x 8 tiles: the last group row hangs over M
    ("x1-hybrid", 4096, 4224, 4096, "heuristic", 0, 256, False),   # 768 DP tiles + Stream-K over 288
]


@pytest.mark.parametrize("case", TRACE_CASES, ids=lambda c: c[0])
def test_trace_matches_simulator(dg, case):
    name, M, N, K, mode, splits, cus, atomic = case
    layout = "nk" if name in ("c2a", "c2b") else "kn"
    lw = dg.layout_word(layout, "bf16")
    p = dg.gemm_plan(M, N, K, lw, dg.mode_word(mode, atomic), splits, cus)
    tr = torch.zeros(p.trace_ints, dtype=torch.int32, device=DEV)
    w = WORKLOADS["c1_sk32"].with_(name=name, M=M, N=N, K=K, b_layout=layout)
    A, B = make_operands(w)
    full, c = guarded_output(M, N, DEV)
    say(f"  trace {name}")
    dg.gemm_tensors(A.to(DEV), B.to(DEV), c, b_layout=layout, mode=mode, splits=splits, atomic=atomic,
                    num_cus=cus, trace=tr)
    assert dg.gemm_sync_status() == 0
    got = decode_trace(tr)
    s, segs, folds = expected_trace(M, N, K, mode, splits, cus)
    assert got["segments"] == segs
    assert np.all(got["coverage"] == 1), "every (tile, k) pair must run exactly once"
    if not atomic:
        assert got["folds"] == folds
    else:
        for t, f in got["folds"].items():
            assert f == (folds[t] if len(folds[t]) == 1 else [])


# ---------------------------------------------------------------------------
# Determinism
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["c1_sk32", "c2a_m96_s8", "c2b_m256_s2", "c5_longk_fp16", "c3_wavequant"])
def test_deterministic_bit_identical_10_runs(dg, name):
    w = WORKLOADS[name]
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    c0 = torch.empty((w.M, w.N), dtype=torch.float32, device=DEV)
    say(f"  10 runs {name}")
    dg.gemm_tensors(a, b, c0, b_layout=w.b_layout, mode=w.mode, splits=w.splits)
    for _ in range(9):
        c = torch.full((w.M, w.N), 7.0, dtype=torch.float32, device=DEV)
        dg.gemm_tensors(a, b, c, b_layout=w.b_layout, mode=w.mode, splits=w.splits)
        assert torch.equal(c.view(torch.int32), c0.view(torch.int32))
    assert dg.gemm_sync_status() == 0


@pytest.mark.parametrize("order", ["reverse", "shuffle"])
def test_unit_order_does_not_change_bits(dg, order):
    w = WORKLOADS["c5_longk_fp16"]
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    ref = torch.empty((w.M, w.N), dtype=torch.float32, device=DEV)
    dg.gemm_tensors(a, b, ref, mode="streamk", splits=0)
    units = dg.gemm_plan(w.M, w.N, w.K, dg.GEMM_FP16, dg.GEMM_STREAMK, 0, dg.gemm_num_cus()).sk_units
    if order == "reverse":
        perm = torch.arange(units - 1, -1, -1, dtype=torch.int32)
    else:
        perm = torch.from_numpy(np.random.default_rng(5).permutation(units).astype(np.int32))
    c = torch.empty_like(ref)
    say(f"  perm {order}")
    dg.gemm_tensors(a, b, c, mode="streamk", splits=0, unit_perm=perm.to(DEV))
    assert dg.gemm_sync_status() == 0
    assert torch.equal(c.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("name,M,N", [("c2a_m96_s8", None, None), ("c2b_m256_s2", None, None),
                                      ("c1_sk32", None, None), ("c2a_m96_s8", 200, 392)])
def test_splitk_merges_agree(dg, name, M, N):
    # the deterministic merges add the partials in split order, so they give the
    # same bits: the row bands of a resident grid (the default here), the last
    # arriver (GEMM_DEBUG_IN_LAUNCH) and a second kernel (GEMM_TWO_PASS); atomics
    # into a zero-filled C are within tolerance
    w = WORKLOADS[name]
    if M is not None:
        w = w.with_(M=M, N=N)   # ragged tiles in M and N
    splits = w.splits if w.mode == "splitk" else 4
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    p = dg.gemm_plan(w.M, w.N, w.K, dg.layout_word(w.b_layout, w.dtype), dg.GEMM_SPLITK, splits, dg.gemm_num_cus())
    assert p.two_pass == (1 if splits < 8 else 0)
    say(f"  bands / last-arriver / two-pass / atomic Split-K {w.name} {w.M}x{w.N}x{w.K} S={splits}")
    outs = []
    for kw in (dict(debug=dg.GEMM_DEBUG_SPLITK_BANDS), dict(debug=dg.GEMM_DEBUG_IN_LAUNCH), dict(two_pass=True),
               dict(atomic=True)):
        full, c = guarded_output(w.M, w.N, DEV)
        dg.gemm_tensors(a, b, c, b_layout=w.b_layout, mode="splitk", splits=splits, **kw)
        outs.append((full, c))
    assert dg.gemm_sync_status() == 0
    for f, _ in outs:
        assert guards_intact(f, w.M, w.N)
    c0 = outs[0][1]
    for _, c in outs[1:3]:
        assert torch.equal(c0.view(torch.int32), c.view(torch.int32))
    assert_parity(c0, A, B, w)
    assert_parity(outs[3][1], A, B, w)


def test_splitk_two_pass_trace(dg):
    # the second kernel records the same fold order the in-launch fold does
    M, N, K, S = 96, 512, 2048, 8
    lw = dg.layout_word("nk", "bf16")
    p = dg.gemm_plan(M, N, K, lw, dg.mode_word("splitk", two_pass=True), S, 256)
    assert p.two_pass == 1 and p.atomic == 0
    w = WORKLOADS["c2a_m96_s8"]
    A, B = make_operands(w)
    tr = torch.zeros(p.trace_ints, dtype=torch.int32, device=DEV)
    _, c = guarded_output(M, N, DEV)
    dg.gemm_tensors(A.to(DEV), B.to(DEV), c, b_layout="nk", mode="splitk", splits=S, two_pass=True, trace=tr)
    assert dg.gemm_sync_status() == 0
    got = decode_trace(tr)
    _, segs, folds = expected_trace(M, N, K, "splitk", S, 256)
    assert got["segments"] == segs and got["folds"] == folds
    assert np.all(got["coverage"] == 1)


@pytest.mark.parametrize("name,mode,splits,M,N,K,cus", [
    ("c1_sk32", "streamk", 32, None, None, None, 0),
    ("c3_wavequant", "heuristic", 0, None, None, None, 0),
    ("c5_longk_fp16", "streamk", 0, None, None, None, 0),
    ("c1_sk32", "streamk", 7, 300, 200, 320, 0),          # ragged M and N, units crossing tile edges
    ("c1_sk32", "heuristic", 0, 1408, 768, 1024, 20),     # hybrid: DP tiles + Stream-K part
])
def test_streamk_two_pass_equals_turnstile(dg, name, mode, splits, M, N, K, cus):
    # a second kernel adding each split tile's partials in k order gives the
    # turnstile's bits
    w = WORKLOADS[name]
    if M is not None:
        w = w.with_(M=M, N=N, K=K)
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    say(f"  two-pass vs turnstile Stream-K {w.name} {w.M}x{w.N}x{w.K} units={splits} cus={cus}")
    full0, c0 = guarded_output(w.M, w.N, DEV)
    full1, c1 = guarded_output(w.M, w.N, DEV)
    dg.gemm_tensors(a, b, c0, b_layout=w.b_layout, mode=mode, splits=splits, num_cus=cus,
                    debug=dg.GEMM_DEBUG_IN_LAUNCH)
    dg.gemm_tensors(a, b, c1, b_layout=w.b_layout, mode=mode, splits=splits, num_cus=cus, two_pass=True)
    assert dg.gemm_sync_status() == 0
    assert guards_intact(full0, w.M, w.N) and guards_intact(full1, w.M, w.N)
    assert torch.equal(c0.view(torch.int32), c1.view(torch.int32))
    assert_parity(c1, A, B, w, rows=sample_rows(w.M, 16))


@pytest.mark.parametrize("M,N,K,units", [(256, 512, 2048, 32), (300, 200, 320, 7), (1536, 1536, 16384, 0)])
def test_streamk_two_pass_trace(dg, M, N, K, units):
    p = dg.gemm_plan(M, N, K, 0, dg.mode_word("streamk", two_pass=True), units, 256)
    assert p.two_pass == 1
    w = WORKLOADS["c1_sk32"].with_(M=M, N=N, K=K)
    A, B = make_operands(w)
    tr = torch.zeros(p.trace_ints, dtype=torch.int32, device=DEV)
    _, c = guarded_output(M, N, DEV)
    dg.gemm_tensors(A.to(DEV), B.to(DEV), c, mode="streamk", splits=units, two_pass=True, trace=tr)
    assert dg.gemm_sync_status() == 0
    got = decode_trace(tr)
    _, segs, folds = expected_trace(M, N, K, "streamk", units, 256)
    assert got["segments"] == segs and got["folds"] == folds
    assert np.all(got["coverage"] == 1)


def test_streamk_equals_splitk_bits_when_segments_coincide(dg):
    # 8 tiles x 32 iterations over 32 units = 4 segments of 8 per tile, the same k
    # ranges as Split-K with S = 4; both fold ((P0 + P1) + P2) + P3 in k order
    w = WORKLOADS["c1_sk32"]
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    c_sk = torch.empty((w.M, w.N), dtype=torch.float32, device=DEV)
    c_s4 = torch.empty_like(c_sk)
    c_dp = torch.empty_like(c_sk)
    dg.gemm_tensors(a, b, c_sk, mode="streamk", splits=32)
    dg.gemm_tensors(a, b, c_s4, mode="splitk", splits=4)
    dg.gemm_tensors(a, b, c_dp, mode="dp")
    torch.cuda.synchronize()
    assert torch.equal(c_sk.view(torch.int32), c_s4.view(torch.int32))
    # a different addition order is expected to change some bits against DP
    assert not torch.equal(c_sk.view(torch.int32), c_dp.view(torch.int32))


def test_atomic_mode_within_tolerance_over_runs(dg):
    w = WORKLOADS["c5_longk_fp16"].with_(M=512, N=512)   # 16 tiles, 3 contributors on some
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    for i in range(3):
        c = torch.full((w.M, w.N), 7.0, dtype=torch.float32, device=DEV)
        dg.gemm_tensors(a, b, c, mode="streamk", splits=0, atomic=True)
        assert_parity(c, A, B, w)


# ---------------------------------------------------------------------------
# Failure path: a wait that can never be satisfied ends at its spin limit
# ---------------------------------------------------------------------------
def test_bounded_wait_reports_timeout(dg):
    w = WORKLOADS["c1_sk32"].with_(name="timeout", M=256, N=256, K=512)
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    c = torch.empty((w.M, w.N), dtype=torch.float32, device=DEV)
    say("  forced timeout (contributors never raise flags, spin limit 2000 polls)")
    dg.gemm_tensors(a, b, c, mode="streamk", splits=12, spin_limit=2000,
                    debug=dg.GEMM_DEBUG_NO_PUBLISH | dg.GEMM_DEBUG_IN_LAUNCH)
    assert dg.gemm_sync_status() == dg.GEMM_ERR_TIMEOUT
    # the status is cleared and the next call is healthy
    full, c2 = guarded_output(w.M, w.N, DEV)
    dg.gemm_tensors(a, b, c2, mode="streamk", splits=12)
    assert dg.gemm_sync_status() == 0
    assert_parity(c2, A, B, w)


def test_capacity_refusal(dg):
    w = WORKLOADS["c1_sk32"]
    a = torch.zeros((w.M, w.K), dtype=torch.bfloat16, device=DEV)
    b = torch.zeros((w.K, w.N), dtype=torch.bfloat16, device=DEV)
    c = torch.full((w.M, w.N), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(dg.GemmError) as ei:
        dg.gemm_tensors(a, b, c, mode="streamk", splits=100000)
    assert ei.value.status == dg.GEMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(c == 7.0), "a refused call must not touch C"


def test_caller_workspace(dg):
    w = WORKLOADS["c1_sk32"]
    p = dg.gemm_plan(w.M, w.N, w.K, 0, dg.GEMM_STREAMK, 32, dg.gemm_num_cus())
    ws = torch.zeros(p.workspace_bytes // 4 + 64, dtype=torch.int32, device=DEV)
    A, B = make_operands(w)
    full, c = guarded_output(w.M, w.N, DEV)
    dg.gemm_tensors(A.to(DEV), B.to(DEV), c, mode="streamk", splits=32, workspace=ws)
    assert dg.gemm_sync_status() == 0
    assert_parity(c, A, B, w)
    small = torch.zeros(16, dtype=torch.int32, device=DEV)
    with pytest.raises(dg.GemmError) as ei:
        dg.gemm_tensors(A.to(DEV), B.to(DEV), c, mode="streamk", splits=32, workspace=small)
    assert ei.value.status == dg.GEMM_ERR_WORKSPACE


@pytest.mark.parametrize("M,N,K,cus", [(1408, 768, 1024, 20), (4096, 4224, 4096, 256)])
def test_hybrid_single_launch_equals_two_launches(dg, M, N, K, cus):
    # the persistent units run the hybrid's data-parallel tiles first, in the
    # Stream-K launch; GEMM_DEBUG_HYBRID_SPLIT runs them as a second launch.
    # Same tiles, same k order: the same bits, and the same trace.
    w = WORKLOADS["x1_hybrid"].with_(name="hybrid", M=M, N=N, K=K)
    p = dg.gemm_plan(M, N, K, 0, dg.GEMM_HEURISTIC, 0, cus)
    assert dg.DECISION_NAMES[p.decision] == "StreamK" and p.dp_tiles > 0
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    outs, traces = [], []
    for debug in (0, dg.GEMM_DEBUG_HYBRID_SPLIT):
        c = torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)
        tr = torch.zeros(p.trace_ints, dtype=torch.int32, device=DEV)
        say(f"  hybrid {M}x{N}x{K} cus={cus} debug={debug}")
        dg.gemm_tensors(a, b, c, num_cus=cus, trace=tr, debug=debug)
        assert dg.gemm_sync_status() == 0
        outs.append(c.cpu())
        traces.append(decode_trace(tr))
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    assert traces[0]["segments"] == traces[1]["segments"] and traces[0]["folds"] == traces[1]["folds"]
    assert np.all(traces[0]["coverage"] == 1)
    assert_parity(outs[0], A, B, w, rows=sample_rows(M, 8))


@pytest.mark.parametrize("M,N,K,mode", [(65536, 33024, 64, "heuristic"), (40960, 53248, 512, "streamk")])
def test_outputs_beyond_2_to_the_31_elements(dg, M, N, K, mode):
    # C holds more than 2^31 fp32 elements (8.6 / 8.7 GB): every output offset
    # past 2^31 must be formed in 64 bits; rows near the end are checked
    w = WORKLOADS["c1_sk32"].with_(name="large", M=M, N=N, K=K)
    assert M * N > 2 ** 31
    A, B = make_operands(w)
    c = torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)
    say(f"  large {M}x{N}x{K} {mode}")
    dg.gemm_tensors(A.to(DEV), B.to(DEV), c, mode=mode)
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    rows = [0, 1, M // 2, 2 ** 31 // N + 1, M - 129, M - 2, M - 1]
    got = c[torch.tensor(rows, device=DEV)].cpu().numpy().astype(np.float64)   # only the checked rows
    del c
    torch.cuda.empty_cache()
    C, S = og.ref_gemm(A, B, M, N, K, "kn", "bf16", rows=rows)
    ok, worst, idx = og.within_tolerance(got, C, S)
    say(f"    worst err/bound = {worst:.3e} at {idx}")
    assert ok, f"outside tolerance: worst ratio {worst} at {idx}"


# ---------------------------------------------------------------------------
# Flags and counters reset themselves: calls of every merge kind enqueued back
# to back on one stream and one library workspace, twice over with fresh
# operands, each checked against the oracle afterwards
# ---------------------------------------------------------------------------
def test_modes_interleaved_on_one_workspace(dg):
    inl = dg.GEMM_DEBUG_IN_LAUNCH
    seq = [  # (mode, splits, atomic, two_pass, debug)
        ("streamk", 7, False, False, inl), ("splitk", 4, False, False, inl), ("splitk", 4, False, True, 0),
        ("splitk", 3, False, False, dg.GEMM_DEBUG_SPLITK_BANDS), ("splitk", 8, False, False, 0),
        ("streamk", 5, True, False, 0), ("streamk", 9, False, True, 0), ("dp", 0, False, False, 0),
        ("splitk", 2, True, False, 0), ("heuristic", 0, False, False, 0), ("streamk", 3, False, False, inl),
    ]
    shapes = [(512, 384, 1024, "kn", "bf16"), (300, 200, 328, "nk", "fp16")]
    for rep in range(2):
        pending = []
        for si, (M, N, K, layout, dtype) in enumerate(shapes):
            dist = dict(dist="uniform", low=-1.0, high=1.0) if dtype == "bf16" else \
                dict(dist="uniform", low=-0.5, high=0.5)
            w = WORKLOADS["c1_sk32"].with_(name=f"seq{rep}-{si}", M=M, N=N, K=K, b_layout=layout, dtype=dtype,
                                           seed=500 + 10 * rep + si, **dist)
            A, B = make_operands(w)
            a, b = A.to(DEV), B.to(DEV)
            ipt = -(-K // 64)
            for mode, splits, atomic, two_pass, debug in seq:
                if mode == "splitk":
                    while ipt % splits:   # Split-K factors divide the k-iterations
                        splits -= 1
                full, c = guarded_output(M, N, DEV)
                say(f"  enqueue rep {rep} {w.name} {M}x{N}x{K} mode={mode} splits={splits} atomic={atomic} "
                    f"two_pass={two_pass} debug={debug}")
                dg.gemm_tensors(a, b, c, b_layout=layout, mode=mode, splits=splits, atomic=atomic,
                                two_pass=two_pass, debug=debug)
                pending.append((w, A, B, full, c, mode, splits))
        assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
        for w, A, B, full, c, mode, splits in pending:
            assert guards_intact(full, w.M, w.N), f"guard band overwritten ({w.name} {mode} {splits})"
            assert_parity(c, A, B, w)
