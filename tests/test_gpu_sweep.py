"""Seeded randomised sweeps through the C ABI: many small problems drawn over
every decomposition, merge, tile shape (the library's own choice included), B
layout, dtype, batch count, fused epilogue and CU count, plus grouped calls and
the no-allocation entry point.
Each call is checked against the fp64 oracle (every element; the epilogue
bound where one is fused), its guard band and the device status word, and a
deterministic call is run twice for the same bits.  Combinations the library
refuses (documented limits, e.g. 256-row tiles outside Stream-K) are counted,
not failed."""
import numpy as np
import pytest
import torch

from oracle import epilogue as oe
from oracle import gemm as og
from workloads import WORKLOADS, make_epilogue_inputs, make_operands

from gpu_util import GUARD, NGUARD, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_work_amd as dg

    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return dg


def _operands(M, N, K, layout, dtype, seed, batch=1):
    dist = dict(dist="uniform", low=-1.0, high=1.0) if dtype == "bf16" else dict(dist="uniform", low=-0.5, high=0.5)
    w = WORKLOADS["c1_sk32"].with_(name=f"sweep{seed}", M=M, N=N, K=K, b_layout=layout, dtype=dtype, seed=seed,
                                   batch=batch, **dist)
    return make_operands(w)


def _merge(rng):
    m = int(rng.integers(0, 3))
    return m == 1, m == 2          # atomic, two_pass


def test_sweep_single_and_batched(dg):
    rng = np.random.default_rng(2024)
    cap_dev = dg.gemm_num_cus()
    fails, ran, refused = [], 0, 0
    for i in range(300):
        layout = str(rng.choice(["kn", "nk"]))
        dtype = str(rng.choice(["bf16", "fp16"]))
        M = int(rng.integers(1, 700))
        N = int(rng.integers(1, 90)) * 8 if layout == "kn" else int(rng.integers(1, 700))
        K = int(rng.integers(0, 130)) * 8
        batch = int(rng.choice([1, 1, 1, 2, 3]))
        tile = str(rng.choice(["128x128", "128x128", "64x128", "256x128", "auto"]))
        mode = str(rng.choice(["dp", "splitk", "streamk", "heuristic", "streamk"]))
        cus = int(rng.choice([0, 0, 8, 32, 100]))
        cap = cap_dev if cus == 0 else cus
        ipt = -(-K // 64)
        splits, atomic, two_pass = 0, False, False
        if mode == "splitk" and ipt > 0:
            splits = int(rng.choice([s for s in range(1, 17) if ipt % s == 0]))
            atomic, two_pass = _merge(rng)
        elif mode == "splitk":
            mode = "dp"
        elif mode == "streamk":
            splits = int(rng.integers(0, min(cap, 300) + 1))
            atomic, two_pass = _merge(rng)
        elif mode == "heuristic":
            atomic, two_pass = _merge(rng)
        epi = None
        if rng.random() < 0.25:
            epi = (float(rng.choice([1.0, 1.5, -0.75])), float(rng.choice([0.0, 1.25, -1.0])),
                   bool(rng.integers(0, 2)), str(rng.choice(["none", "relu", "gelu"])))
        desc = (f"{i}: {M}x{N}x{K} batch {batch} {dtype} {layout} tile {tile} {mode} splits {splits} "
                f"atomic {atomic} two_pass {two_pass} cus {cus} epilogue {epi}")
        A, B = _operands(M, N, K, layout, dtype, 20000 + i, batch)
        shape = (batch, M, N) if batch > 1 else (M, N)
        if epi is not None:
            c_in, bias = make_epilogue_inputs(M, N, seed=7 + i)
            if epi[1] == 0.0:
                c_in = torch.full_like(c_in, float("nan"))     # beta = 0: C_in must not be read
            start = c_in.expand(*shape).contiguous()
        else:
            start = torch.full(shape, 7.0)
        n = start.numel()
        full = torch.full((n + NGUARD,), GUARD, dtype=torch.float32, device=DEV)
        full[:n] = start.reshape(-1).to(DEV)
        c = full[:n].view(*shape)
        kw = dict(b_layout=layout, mode=mode, splits=splits, atomic=atomic, two_pass=two_pass, num_cus=cus,
                  tile=tile)
        if epi is not None:
            kw.update(alpha=epi[0], beta=epi[1], bias=bias.to(DEV) if epi[2] else None, act=epi[3])
        a, b = A.to(DEV), B.to(DEV)
        try:
            dg.gemm_tensors(a, b, c, **kw)
        except dg.GemmError:
            refused += 1
            continue
        ran += 1
        problems = []
        if dg.gemm_sync_status() != 0:
            problems.append("device status")
        if not bool(torch.all(full[n:] == GUARD)):
            problems.append("guard band overwritten")
        got = c.detach().cpu().numpy().astype(np.float64).reshape(batch, M, N)
        for e in range(batch):
            P, S = og.ref_gemm(A[e] if batch > 1 else A, B[e] if batch > 1 else B, M, N, K, layout, dtype)
            if epi is None:
                ok, worst, idx = og.within_tolerance(got[e], P, S)
            else:
                c0 = c_in.numpy().astype(np.float64) if epi[1] != 0.0 else None
                b64 = bias.numpy().astype(np.float64) if epi[2] else None
                D, _ = oe.epilogue_ref(P, c0, epi[0], epi[1], b64, epi[3])
                ok, worst, idx = oe.within_bound(got[e], D, oe.epilogue_bound(S, P, c0, epi[0], epi[1], b64, epi[3]))
            if not ok:
                problems.append(f"entry {e}: worst err/bound {worst:.3e} at {idx}")
        if not atomic and not problems:
            first = c.clone()
            full[:n] = start.reshape(-1).to(DEV)
            dg.gemm_tensors(a, b, c, **kw)
            if dg.gemm_sync_status() != 0 or not torch.equal(first.view(torch.int32), c.view(torch.int32)):
                problems.append("a second run gave other bits")
        if problems:
            say(f"  FAIL {desc}: {problems}")
            fails.append(desc)
    say(f"  sweep: {ran} calls checked, {refused} refused by the library")
    assert ran >= 150, "the sweep ran too few calls"
    assert not fails, f"{len(fails)} failing calls, first: {fails[0]}"


def test_sweep_grouped_and_noalloc(dg):
    rng = np.random.default_rng(4048)
    cap_dev = dg.gemm_num_cus()
    fails, ran, refused = [], 0, 0
    for i in range(160):
        grouped = bool(rng.integers(0, 2))
        layout = str(rng.choice(["kn", "nk"]))
        dtype = str(rng.choice(["bf16", "fp16"]))
        mode = str(rng.choice(["dp", "splitk", "streamk", "heuristic"]))
        tile = str(rng.choice(["128x128", "64x128", "auto"]))
        atomic, two_pass = _merge(rng)
        K = int(rng.integers(1 if not grouped else 0, 200)) * 8
        ipt = -(-K // 64)
        splits = 0
        if mode == "splitk" and ipt > 0:
            splits = int(rng.choice([s for s in range(1, 9) if ipt % s == 0]))
        elif mode == "splitk":
            mode = "dp"
        elif mode == "streamk":
            splits = int(rng.integers(0, cap_dev + 1))
        if mode == "dp":
            atomic = two_pass = False
        try:
            if grouped:
                probs, ops = [], []
                for g in range(int(rng.integers(1, 9))):
                    M = 0 if rng.random() < 0.1 else int(rng.integers(1, 500))
                    N = int(rng.integers(1, 70)) * 8 if layout == "kn" else int(rng.integers(1, 500))
                    A, B = _operands(M, N, K, layout, dtype, 30000 + 10 * i + g)
                    probs.append((A.to(DEV), B.to(DEV), torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)))
                    ops.append((A, B, M, N))
                desc = (f"{i}: grouped, {len(probs)} problems K {K} {dtype} {layout} {mode} splits {splits} "
                        f"atomic {atomic} two_pass {two_pass} tile {tile}")
                dg.gemm_grouped_tensors(probs, b_layout=layout, mode=mode, splits=splits, atomic=atomic,
                                        two_pass=two_pass, tile=tile)
                problems = [] if dg.gemm_sync_status() == 0 else ["device status"]
                for g, ((A, B, M, N), (_, _, c)) in enumerate(zip(ops, probs)):
                    if M * N == 0:
                        continue
                    P, S = og.ref_gemm(A, B, M, N, K, layout, dtype)
                    ok, worst, idx = og.within_tolerance(c.cpu().numpy().astype(np.float64), P, S)
                    if not ok:
                        problems.append(f"problem {g}: worst err/bound {worst:.3e} at {idx}")
            else:
                M = int(rng.integers(1, 1200))
                N = int(rng.integers(1, 150)) * 8 if layout == "kn" else int(rng.integers(1, 1200))
                A, B = _operands(M, N, K, layout, dtype, 40000 + i)
                a, b = A.to(DEV), B.to(DEV)
                c1 = torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)
                c2 = torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)
                desc = (f"{i}: no-allocation {M}x{N}x{K} {dtype} {layout} {mode} splits {splits} atomic {atomic} "
                        f"two_pass {two_pass} tile {tile}")
                kw = dict(b_layout=layout, mode=mode, splits=splits, atomic=atomic, two_pass=two_pass, tile=tile)
                dg.gemm_tensors(a, b, c2, noalloc=True, **kw)
                dg.gemm_tensors(a, b, c1, **kw)
                problems = [] if dg.gemm_sync_status() == 0 else ["device status"]
                if not atomic and not torch.equal(c1.view(torch.int32), c2.view(torch.int32)):
                    problems.append("gemm_ex_noalloc bits differ from gemm_ex")
                P, S = og.ref_gemm(A, B, M, N, K, layout, dtype)
                ok, worst, idx = og.within_tolerance(c2.cpu().numpy().astype(np.float64), P, S)
                if not ok:
                    problems.append(f"worst err/bound {worst:.3e} at {idx}")
        except dg.GemmError:
            refused += 1
            continue
        ran += 1
        if problems:
            say(f"  FAIL {desc}: {problems}")
            fails.append(desc)
    say(f"  sweep: {ran} calls checked, {refused} refused by the library")
    assert ran >= 100, "the sweep ran too few calls"
    assert not fails, f"{len(fails)} failing calls, first: {fails[0]}"
