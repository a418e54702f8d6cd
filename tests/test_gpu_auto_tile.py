"""GEMM_TILE_AUTO on the GPU, through the C ABI: a call with tile "auto" runs the
plan of the tile the library picks (the same bits as a call that names that
tile), with and without a fused epilogue, and its output matches the fp64
oracle."""
import pytest
import torch

from workloads import WORKLOADS, make_epilogue_inputs, make_operands

from gpu_util import check_against_oracle, guarded_output, guards_intact, poison_rows, say, tile_row_sample

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# 144 tiles of 128 x 128 (more than half the CUs); 256 x 128 Stream-K units of 72 iterations
LONG_K = WORKLOADS["c5_longk_fp16"]

CASES = [   # (workload, the tile "auto" picks on a 256-CU MI355X)
    (WORKLOADS["c1_sk32"], "64x128"),
    (WORKLOADS["c2a_m96_s8"], "64x128"),
    (WORKLOADS["c2b_m256_s2"], "64x128"),
    (WORKLOADS["x3_decode"], "64x128"),
    (LONG_K, "256x128"),
]


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_work_amd as dg

    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return dg


def _call(dg, w, a, b, tile, start=None, **kw):
    full, c = guarded_output(w.M, w.N, DEV)
    if start is not None:
        c.copy_(start)
    mode = "streamk" if tile == "256x128" else w.mode
    dg.gemm_tensors(a, b, c, b_layout=w.b_layout, mode=mode, splits=w.splits, tile=tile, **kw)
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    assert guards_intact(full, w.M, w.N), "guard band overwritten"
    return c


@pytest.mark.parametrize("w,tile", CASES, ids=lambda x: x.name if hasattr(x, "name") else x)
def test_auto_runs_the_picked_tile(dg, w, tile):
    assert dg.gemm_num_cus() == 256, "the expected tiles assume 256 CUs"
    plan = dg.gemm_plan(w.M, w.N, w.K, dg.layout_word(w.b_layout, w.dtype), dg.mode_word(w.mode, tile="auto"),
                        w.splits, dg.gemm_num_cus())
    assert plan.bm == int(tile.split("x")[0])
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    say(f"  auto {w.name} {w.M}x{w.N}x{w.K} mode={w.mode} -> {tile}")
    c_auto = _call(dg, w, a, b, "auto")
    c_named = _call(dg, w, a, b, tile)
    assert not poison_rows(c_auto), "elements never written"
    assert torch.equal(c_auto.view(torch.int32), c_named.view(torch.int32)), "auto and the named tile differ"
    rows = None if w.M * w.N * w.K <= 2 ** 32 else tile_row_sample(w.M, bm=int(tile.split("x")[0]))
    ok, worst, idx = check_against_oracle(c_auto, A, B, w, rows=rows)
    say(f"    worst err/bound = {worst:.3e} at {idx}")
    assert ok, f"outside tolerance: worst ratio {worst} at {idx}"


@pytest.mark.parametrize("w,expect", [
    (LONG_K, "256x128"),
    (WORKLOADS["c1_sk32"], "64x128"),
    (WORKLOADS["c2a_m96_s8"], "64x128"),
], ids=["c5_longk_fp16", "c1_sk32", "c2a_m96_s8"])
def test_auto_with_an_epilogue(dg, w, expect):
    A, B = make_operands(w)
    a, b = A.to(DEV), B.to(DEV)
    c_in, bias = make_epilogue_inputs(w.M, w.N, seed=11)
    start = c_in.to(DEV)
    epi = dict(alpha=1.5, beta=-1.0, bias=bias.to(DEV), act="gelu")
    say(f"  auto + epilogue {w.name} {w.M}x{w.N}x{w.K} -> {expect}")
    c_auto = _call(dg, w, a, b, "auto", start, **epi)
    c_named = _call(dg, w, a, b, expect, start, **epi)
    # C starts at C_in here, so only the bits of the named tile's call (checked
    # against the oracle by the tile's own tests) tell a missed element
    assert torch.equal(c_auto.view(torch.int32), c_named.view(torch.int32)), "auto and the named tile differ"
