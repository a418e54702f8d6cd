"""GPU parity of the 256 x 128 Stream-K tile (GEMM_TILE_256x128; the tile shape
the book chapter's Case 4 names for CUTLASS's Stream-K example), through the C
ABI: values against the fp64 oracle (|C - C_ref| <= 1e-4 sum|a||b| on every
element), the kernels' trace against the simulator's schedule for 256-row tiles,
bit identity over runs, and the zero-partial control."""
import numpy as np
import pytest
import torch

from oracle import epilogue as oe
from oracle import gemm as og
from workloads import WORKLOADS, make_epilogue_inputs, make_operands

from gpu_util import (check_against_oracle, check_full, decode_trace, expected_trace, guarded_output,
                      guards_intact, oracle_full, say)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TALL = "256x128"


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_work_amd as dg

    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return dg


def run_tall(dg, w, A, B, units, atomic=False, **kw):
    a, b = A.to(DEV), B.to(DEV)
    full, c = guarded_output(w.M, w.N, DEV)
    say(f"  tall {w.name} {w.M}x{w.N}x{w.K} {w.dtype} {w.b_layout} units={units} atomic={atomic}")
    dg.gemm_tensors(a, b, c, b_layout=w.b_layout, mode="streamk", splits=units, atomic=atomic, tile=TALL, **kw)
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    assert guards_intact(full, w.M, w.N), "guard band overwritten"
    return c


SMALL = [   # (M, N, K, layout, dtype, units)
    (256, 256, 512, "kn", "bf16", 5),
    (300, 200, 328, "nk", "bf16", 7),      # ragged M, N and K
    (520, 136, 72, "kn", "fp16", 3),       # a 256-row tile with 8 rows, ragged K
    (96, 100, 2048, "nk", "fp16", 9),      # one tile, N not a multiple of 8
    (768, 384, 1024, "kn", "bf16", 12),
    (1, 8, 8, "kn", "bf16", 1),
    (512, 256, 128, "kn", "bf16", 6),      # more units than iterations
]


@pytest.mark.parametrize("atomic", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s[:3])) + f"-{s[3]}-{s[4]}-u{s[5]}")
def test_tall_small_shapes(dg, shape, atomic):
    M, N, K, layout, dtype, units = shape
    dist = dict(dist="uniform", low=-1.0, high=1.0) if dtype == "bf16" else dict(dist="uniform", low=-0.5, high=0.5)
    w = WORKLOADS["c1_sk32"].with_(name="tall-small", M=M, N=N, K=K, b_layout=layout, dtype=dtype, **dist)
    A, B = make_operands(w)
    c = run_tall(dg, w, A, B, units, atomic)
    ok, worst, idx = check_against_oracle(c, A, B, w)
    say(f"    worst err/bound = {worst:.3e} at {idx}")
    assert ok, f"outside tolerance: worst ratio {worst} at {idx}"


@pytest.mark.parametrize("name,atomic", [("c3_wavequant", False), ("c5_longk_fp16", False),
                                         ("c5_longk_fp16", True), ("x1_hybrid", False)])
def test_tall_full_size(dg, name, atomic):
    w = WORKLOADS[name]
    A, B, _, _ = oracle_full(w)
    c = run_tall(dg, w, A, B, 0, atomic)
    ok, worst, idx = check_full(c, w)
    say(f"    worst err/bound = {worst:.3e} at {idx} (all {w.M * w.N} elements)")
    assert ok, f"outside tolerance: worst ratio {worst} at {idx}"


TRACE = [   # (M, N, K, units)
    (2048, 2176, 4096, 256),
    (1536, 1536, 16384, 256),
    (300, 200, 328, 7),
    (512, 256, 128, 6),
    (300, 200, 328, 1),
]


@pytest.mark.parametrize("case", TRACE, ids=lambda c: "x".join(map(str, c)))
def test_tall_trace_matches_simulator(dg, case):
    M, N, K, units = case
    p = dg.gemm_plan(M, N, K, 0, dg.mode_word("streamk", tile=TALL), units, 256)
    tr = torch.zeros(p.trace_ints, dtype=torch.int32, device=DEV)
    w = WORKLOADS["c1_sk32"].with_(name="tall-trace", M=M, N=N, K=K)
    A, B = make_operands(w)
    full, c = guarded_output(M, N, DEV)
    say(f"  tall trace {M}x{N}x{K} units={units}")
    dg.gemm_tensors(A.to(DEV), B.to(DEV), c, mode="streamk", splits=units, tile=TALL, trace=tr)
    assert dg.gemm_sync_status() == 0
    got = decode_trace(tr)
    _, segs, folds = expected_trace(M, N, K, "streamk", units, 256, bm=256)
    assert got["segments"] == segs
    assert got["folds"] == folds
    assert np.all(got["coverage"] == 1), "every (tile, k) pair must run exactly once"


def test_tall_bit_identical_10_runs_and_unit_order(dg):
    w = WORKLOADS["c3_wavequant"]
    A, B, _, _ = oracle_full(w)
    a, b = A.to(DEV), B.to(DEV)
    c0 = torch.empty((w.M, w.N), dtype=torch.float32, device=DEV)
    dg.gemm_tensors(a, b, c0, mode="streamk", splits=0, tile=TALL)
    for _ in range(9):
        c = torch.full((w.M, w.N), 7.0, dtype=torch.float32, device=DEV)
        dg.gemm_tensors(a, b, c, mode="streamk", splits=0, tile=TALL)
        assert torch.equal(c.view(torch.int32), c0.view(torch.int32))
    perm = torch.arange(dg.gemm_num_cus() - 1, -1, -1, dtype=torch.int32, device=DEV)
    c = torch.empty_like(c0)
    dg.gemm_tensors(a, b, c, mode="streamk", splits=0, tile=TALL, unit_perm=perm)
    assert dg.gemm_sync_status() == 0
    assert torch.equal(c.view(torch.int32), c0.view(torch.int32)), "reversed unit order changed bits"


@pytest.mark.parametrize("name,atomic", [("c3_wavequant", False), ("c5_longk_fp16", True)])
def test_tall_zero_partial_control(dg, name, atomic):
    w = WORKLOADS[name]
    A, B, _, _ = oracle_full(w)
    for control in (True, False):
        c = run_tall(dg, w, A, B, 0, atomic, debug=dg.GEMM_DEBUG_ZERO_PARTIAL if control else 0)
        ok, worst, _ = check_full(c, w)
        say(f"    control={control}: worst err/bound = {worst:.3e}")
        assert ok != control


def _tall_epilogue(dg, w, A, B, units, atomic, alpha, beta, act, use_bias=True, **kw):
    c_in, bias = make_epilogue_inputs(w.M, w.N, seed=5)
    full, c = guarded_output(w.M, w.N, DEV)
    c.copy_(c_in.to(DEV))
    say(f"  tall epilogue {w.name} {w.M}x{w.N}x{w.K} units={units} atomic={atomic} "
        f"alpha={alpha} beta={beta} act={act} bias={use_bias}")
    dg.gemm_tensors(A.to(DEV), B.to(DEV), c, b_layout=w.b_layout, mode="streamk", splits=units, atomic=atomic,
                    tile=TALL, alpha=alpha, beta=beta, bias=bias.to(DEV) if use_bias else None, act=act, **kw)
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    assert guards_intact(full, w.M, w.N), "guard band overwritten"
    return c, c_in, bias


@pytest.mark.parametrize("atomic", [False, True])
@pytest.mark.parametrize("shape,epi", [
    ((300, 200, 328, "nk", "bf16", 7), (1.5, -0.75, "gelu", True)),     # ragged M, N and K
    ((520, 136, 72, "kn", "fp16", 3), (0.5, 0.0, "relu", True)),         # beta = 0: C_in is not read
    ((768, 384, 1024, "kn", "bf16", 12), (-1.0, 1.25, "none", False)),
], ids=["ragged", "beta0", "no-bias"])
def test_tall_epilogue(dg, shape, epi, atomic):
    M, N, K, layout, dtype, units = shape
    alpha, beta, act, use_bias = epi
    dist = dict(dist="uniform", low=-1.0, high=1.0) if dtype == "bf16" else dict(dist="uniform", low=-0.5, high=0.5)
    w = WORKLOADS["c1_sk32"].with_(name="tall-epi", M=M, N=N, K=K, b_layout=layout, dtype=dtype, **dist)
    A, B = make_operands(w)
    c, c_in, bias = _tall_epilogue(dg, w, A, B, units, atomic, alpha, beta, act, use_bias)
    P, S = og.ref_gemm(A, B, M, N, K, layout, dtype)
    c0 = c_in.numpy().astype(np.float64) if beta != 0.0 else None
    b64 = bias.numpy().astype(np.float64) if use_bias else None
    D, _ = oe.epilogue_ref(P, c0, alpha, beta, b64, act)
    ok, worst, idx = oe.within_bound(c.cpu().numpy().astype(np.float64), D,
                                     oe.epilogue_bound(S, P, c0, alpha, beta, b64, act))
    say(f"    worst err/bound = {worst:.3e} at {idx}")
    assert ok, f"outside the epilogue bound: worst ratio {worst} at {idx}"


def test_tall_epilogue_full_size_and_bits(dg):
    # every element of 1536^2 x 16384 with the epilogue, and the turnstile's bits
    # again on a second run and in reverse unit order
    w = WORKLOADS["c5_longk_fp16"]
    A, B, P, S = oracle_full(w)
    alpha, beta, act = 0.75, -0.5, "gelu"
    c, c_in, bias = _tall_epilogue(dg, w, A, B, 0, False, alpha, beta, act)
    c0, b64 = c_in.numpy().astype(np.float64), bias.numpy().astype(np.float64)
    D, _ = oe.epilogue_ref(P, c0, alpha, beta, b64, act)
    ok, worst, idx = oe.within_bound(c.cpu().numpy().astype(np.float64), D,
                                     oe.epilogue_bound(S, P, c0, alpha, beta, b64, act))
    say(f"    worst err/bound = {worst:.3e} at {idx}")
    assert ok, f"outside the epilogue bound: worst ratio {worst} at {idx}"
    units = dg.gemm_plan(w.M, w.N, w.K, dg.layout_word(w.b_layout, w.dtype), dg.mode_word("streamk", tile=TALL),
                         0, dg.gemm_num_cus()).sk_units
    perm = torch.arange(units - 1, -1, -1, dtype=torch.int32, device=DEV)
    for kw in ({}, {"unit_perm": perm}):
        again, _, _ = _tall_epilogue(dg, w, A, B, 0, False, alpha, beta, act, **kw)
        assert torch.equal(again.view(torch.int32), c.view(torch.int32))
