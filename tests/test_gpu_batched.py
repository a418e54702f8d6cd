"""GPU parity of batched calls (gemm_args_t.batch with element strides) through
the C ABI: every batch entry against the fp64 oracle, the schedule trace
against the simulator's batched plan, shared operands (stride 0), entries at
padded strides, the fused epilogue, and the bits of deterministic merges."""
import numpy as np
import pytest
import torch

from oracle import epilogue as oe
from oracle import gemm as og
from workloads import WORKLOADS, make_epilogue_inputs, make_operands

from gpu_util import GUARD, decode_trace, expected_trace, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
POISON = 7.0


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_work_amd as dg

    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return dg


def _workload(M, N, K, layout, dtype):
    return WORKLOADS["c1_sk32"].with_(name=f"batched_{M}x{N}x{K}", M=M, N=N, K=K, b_layout=layout, dtype=dtype)


def _operands(w, batch, share_b=False):
    """Per-entry operands from seeds 100 + b (B from entry 0 only when shared)."""
    As, Bs = [], []
    for b in range(batch):
        A, B = make_operands(w, seed=100 + b)
        As.append(A)
        Bs.append(B)
    A = torch.stack(As)
    B = Bs[0] if share_b else torch.stack(Bs)
    return A, B


def _strided_c(batch, M, N, pad):
    """A [batch, M, N] view whose entries are M*N (rounded up to 4) + pad elements
    apart inside a buffer poisoned with 7 and guarded (pads and tail) with 11."""
    stride = (M * N + 3) // 4 * 4 + pad      # entries 16-byte aligned
    full = torch.full((batch * stride + 64,), GUARD, dtype=torch.float32, device=DEV)
    c = torch.as_strided(full, (batch, M, N), (stride, N, 1))
    c.fill_(POISON)
    return full, c, stride


def _guards_ok(full, batch, M, N, stride):
    mask = torch.ones_like(full, dtype=torch.bool)
    for b in range(batch):
        mask[b * stride: b * stride + M * N] = False
    return bool(torch.all(full[mask] == GUARD))


def _check_entries(A, B, c, w, batch, share_b, rows=None):
    worst = 0.0
    for b in range(batch):
        Bb = B if share_b else B[b]
        C, S = og.ref_gemm(A[b], Bb, w.M, w.N, w.K, w.b_layout, w.dtype, rows=rows)
        got = c[b].detach().cpu().numpy().astype(np.float64)
        if rows is not None:
            got = got[np.asarray(rows)]
        ok, ratio, idx = og.within_tolerance(got, C, S)
        worst = max(worst, ratio)
        assert ok, f"batch entry {b}: worst ratio {ratio} at {idx}"
    say(f"    worst err/bound over {batch} entries = {worst:.3e}")


# (id, batch, M, N, K, layout, dtype, mode, splits, atomic, two_pass, debug, cus, share_b, pad)
CASES = [
    ("dp-ragged", 3, 300, 272, 320, "kn", "bf16", "dp", 0, False, False, 0, 0, False, 0),
    ("dp-groups", 2, 1024, 1024, 256, "kn", "bf16", "dp", 0, False, False, 0, 16, False, 0),
    ("dp-groups-padded", 3, 1000, 1000, 200, "nk", "fp16", "dp", 0, False, False, 0, 16, False, 40),
    ("splitk8-in-launch", 4, 96, 512, 2048, "nk", "bf16", "splitk", 8, False, False, "IN_LAUNCH", 0, False, 0),
    ("splitk8-two-pass", 4, 96, 512, 2048, "nk", "bf16", "splitk", 8, False, False, 0, 0, True, 0),
    ("splitk2-scalar", 3, 200, 130, 512, "nk", "bf16", "splitk", 2, False, True, 0, 0, False, 12),
    ("splitk4-atomic", 3, 256, 512, 2048, "kn", "bf16", "splitk", 4, True, False, 0, 0, False, 4),
    ("streamk-turnstile", 3, 256, 512, 2048, "kn", "bf16", "streamk", 40, False, False, "IN_LAUNCH", 0, False, 0),
    ("streamk-two-pass", 3, 256, 512, 2048, "kn", "bf16", "streamk", 100, False, True, 0, 0, False, 0),
    ("streamk-atomic", 2, 330, 200, 1000, "nk", "fp16", "streamk", 7, True, False, 0, 0, False, 8),
    ("heuristic", 6, 256, 512, 2048, "kn", "bf16", "heuristic", 0, False, False, 0, 0, True, 0),
    ("hybrid", 2, 640, 640, 2048, "kn", "bf16", "heuristic", 0, False, False, 0, 8, False, 0),
]


def _run(dg, case, trace=None, epi=None):
    _, batch, M, N, K, layout, dtype, mode, splits, atomic, two_pass, debug, cus, share_b, pad = case
    w = _workload(M, N, K, layout, dtype)
    A, B = _operands(w, batch, share_b)
    full, c, stride = _strided_c(batch, M, N, pad)
    kw = {}
    c_in = bias = None
    if epi is not None:
        alpha, beta, act = epi
        c_in, bias = make_epilogue_inputs(batch * M, N, seed=3)
        c_in = c_in.view(batch, M, N)
        c.copy_(c_in.to(DEV))
        kw = dict(alpha=alpha, beta=beta, bias=bias.to(DEV), act=act)
    say(f"  batched {case[0]} batch={batch} {M}x{N}x{K} {dtype} {layout} mode={mode} splits={splits} "
        f"atomic={atomic} two_pass={two_pass} pad={pad} share_b={share_b} epi={epi}")
    dg.gemm_tensors(A.to(DEV), B.to(DEV), c, b_layout=layout, mode=mode, splits=splits, atomic=atomic,
                    two_pass=two_pass, debug=dg.GEMM_DEBUG_IN_LAUNCH if debug == "IN_LAUNCH" else 0,
                    num_cus=cus, trace=trace, **kw)
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    assert _guards_ok(full, batch, M, N, stride), "a pad or the guard band was overwritten"
    return w, A, B, c, c_in, bias


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_batched_parity(dg, case):
    w, A, B, c, *_ = _run(dg, case)
    _check_entries(A, B, c, w, case[1], case[13])


@pytest.mark.parametrize("case", [c for c in CASES if c[0] in ("streamk-turnstile", "heuristic", "hybrid",
                                                              "splitk8-in-launch", "dp-groups")],
                         ids=lambda c: c[0])
def test_batched_trace_matches_simulator(dg, case):
    _, batch, M, N, K, layout, dtype, mode, splits, atomic, two_pass, debug, cus, share_b, pad = case
    lw = dg.layout_word(layout, dtype)
    p = dg.gemm_plan_batched(M, N, K, batch, lw, dg.mode_word(mode, atomic), splits, cus or 256)
    assert p.batch == batch and p.tiles == batch * p.tiles_m * p.tiles_n
    tr = torch.zeros(p.trace_ints, dtype=torch.int32, device=DEV)
    _run(dg, case, trace=tr)
    got = decode_trace(tr)
    s, segs, folds = expected_trace(M, N, K, mode, splits, cus or 256, batch=batch)
    assert dg.DECISION_NAMES[p.decision] == s.kind
    assert got["segments"] == segs
    assert np.all(got["coverage"] == 1), "every (tile, k) pair must run exactly once"
    assert got["folds"] == folds


@pytest.mark.parametrize("name", ["streamk-two-pass", "splitk8-in-launch", "dp-groups-padded", "streamk-atomic"])
def test_batched_epilogue(dg, name):
    case = {c[0]: c for c in CASES}[name]
    epi = (0.75, -0.5, "gelu")
    w, A, B, c, c_in, bias = _run(dg, case, epi=epi)
    batch, share_b = case[1], case[13]
    for b in range(batch):
        P, S = og.ref_gemm(A[b], B if share_b else B[b], w.M, w.N, w.K, w.b_layout, w.dtype)
        c0 = c_in[b].numpy().astype(np.float64)
        b64 = bias.numpy().astype(np.float64)
        D, _ = oe.epilogue_ref(P, c0, epi[0], epi[1], b64, epi[2])
        bound = oe.epilogue_bound(S, P, c0, epi[0], epi[1], b64, epi[2])
        ok, worst, idx = oe.within_bound(c[b].cpu().numpy().astype(np.float64), D, bound)
        assert ok, f"batch entry {b}: worst ratio {worst} at {idx}"


def test_batched_deterministic_repeat(dg):
    # a deterministic batched Stream-K call gives the same bits on a repeat
    case = {c[0]: c for c in CASES}["streamk-turnstile"]
    _, _, _, c1, *_ = _run(dg, case)
    _, _, _, c2, *_ = _run(dg, case)
    assert torch.equal(c1.contiguous().view(torch.int32), c2.contiguous().view(torch.int32))


def test_batched_rejects_bad_strides(dg):
    M, N, K = 128, 128, 64
    a = torch.zeros(2, M, K, dtype=torch.bfloat16, device=DEV)
    b = torch.zeros(2, K, N, dtype=torch.bfloat16, device=DEV)
    c = torch.zeros(2, M, N, dtype=torch.float32, device=DEV)
    args = dg.GemmArgs()
    args.A, args.B, args.C = a.data_ptr(), b.data_ptr(), c.data_ptr()
    args.M, args.N, args.K = M, N, K
    args.mode = dg.GEMM_DP
    args.batch = 2
    args.stride_a, args.stride_b, args.stride_c = M * K, K * N, M * N - 4    # entries of C overlap
    assert dg.gemm_ex(args) == dg.GEMM_ERR_INVALID
    args.stride_c = M * N + 2                                              # breaks 16-byte alignment
    assert dg.gemm_ex(args) == dg.GEMM_ERR_UNSUPPORTED


def test_batched_empty_k(dg):
    # K = 0 in a batch: the operands are empty tensors (torch gives them strides
    # that describe no layout) and every entry of C is the empty sum, 0, or with
    # the epilogue act(beta C_in + bias)
    M, N = 200, 136
    for layout in ("kn", "nk"):
        a = torch.empty(3, M, 0, dtype=torch.bfloat16, device=DEV)
        b = torch.empty((3, 0, N) if layout == "kn" else (3, N, 0), dtype=torch.bfloat16, device=DEV)
        c = torch.full((3, M, N), 7.0, dtype=torch.float32, device=DEV)
        say(f"  batched K = 0, {layout}")
        dg.gemm_tensors(a, b, c, b_layout=layout, mode="heuristic")
        assert dg.gemm_sync_status() == 0
        assert bool(torch.all(c == 0.0))
        c_in, bias = make_epilogue_inputs(M, N)
        c = c_in.to(DEV).expand(3, M, N).contiguous()
        dg.gemm_tensors(a, b, c, b_layout=layout, alpha=2.0, beta=-1.0, bias=bias.to(DEV), act="relu")
        assert dg.gemm_sync_status() == 0
        D, _ = oe.epilogue_ref(np.zeros((M, N)), c_in.numpy().astype(np.float64), 2.0, -1.0,
                               bias.numpy().astype(np.float64), "relu")
        for e in range(3):
            assert np.allclose(c[e].cpu().numpy(), D, rtol=0, atol=1e-6)


def test_x2_batched_workload(dg):
    # the benchmark's batched workload at full size: 5 x (1024x1024x2048), heuristic
    w = WORKLOADS["x2_batched"]
    p = dg.gemm_plan_batched(w.M, w.N, w.K, w.batch, 0, dg.GEMM_HEURISTIC, 0, 256)
    assert (dg.DECISION_NAMES[p.decision], p.sk_units, p.tiles, p.q) == ("StreamK", 256, 320, 40)
    A, B = make_operands(w)
    assert tuple(A.shape) == (5, 1024, 2048) and tuple(B.shape) == (5, 2048, 1024)
    full, c, stride = _strided_c(w.batch, w.M, w.N, 0)
    say("  x2_batched")
    dg.gemm_tensors(A.to(DEV), B.to(DEV), c, b_layout=w.b_layout)
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    assert _guards_ok(full, w.batch, w.M, w.N, stride)
    _check_entries(A, B, c, w, w.batch, False, rows=[0, 1, 127, 128, 511, 640, 1000, 1023])


def _random_batched_cases(n, seed=23):
    """Seeded random batched problems with random epilogues: shape, layout, dtype,
    batch, C padding, a shared B, decomposition, merge mode, CU count."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        layout = str(rng.choice(["kn", "nk"]))
        M = int(rng.integers(1, 400))
        N = int(rng.integers(1, 50)) * 8 if layout == "kn" else int(rng.integers(1, 400))
        K = int(rng.integers(1, 30)) * 8
        dtype = str(rng.choice(["bf16", "fp16"]))
        batch = int(rng.integers(1, 5))
        pad = int(rng.integers(0, 4)) * 4
        share_b = bool(rng.integers(0, 2))
        mode = str(rng.choice(["dp", "splitk", "streamk", "heuristic"]))
        cus = int(rng.choice([0, 4, 16]))
        ipt = -(-K // 64)
        splits, atomic, two_pass = 0, False, False
        if mode == "splitk":
            splits = int(rng.choice([s for s in range(1, 9) if ipt % s == 0]))
            merge = int(rng.integers(0, 3))
            atomic, two_pass = merge == 1, merge == 2
        elif mode == "streamk":
            splits = int(rng.integers(1, 24))
            atomic = bool(rng.integers(0, 2))
        kind = int(rng.integers(0, 5))
        epi = [None, (1.5, 0.0, "none"), (-0.5, 0.75, "relu"), (0.75, -1.25, "gelu"), (1.0, 1.0, "gelu")][kind]
        use_bias = bool(rng.integers(0, 2)) and epi is not None
        cases.append((i, M, N, K, layout, dtype, batch, pad, share_b, mode, splits, atomic, two_pass, cus, epi,
                      use_bias))
    return cases


@pytest.mark.parametrize("case", _random_batched_cases(20), ids=lambda c: f"rb{c[0]}")
def test_random_batched_epilogue(dg, case):
    i, M, N, K, layout, dtype, batch, pad, share_b, mode, splits, atomic, two_pass, cus, epi, use_bias = case
    dist = dict(dist="uniform", low=-1.0, high=1.0) if dtype == "bf16" else dict(dist="uniform", low=-0.5, high=0.5)
    w = WORKLOADS["c1_sk32"].with_(name=f"rb{i}", M=M, N=N, K=K, b_layout=layout, dtype=dtype, **dist)
    if mode == "streamk":
        splits = min(splits, dg.gemm_num_cus() if cus == 0 else cus)
    A, B = _operands(w, batch, share_b)
    if batch == 1:
        A = A[0]
    full, c, stride = _strided_c(batch, M, N, pad)
    c_in, bias = make_epilogue_inputs(batch * M, N, seed=200 + i)
    c_in = c_in.view(batch, M, N)
    kw = {}
    if epi is not None:
        c.copy_(c_in.to(DEV))
        kw = dict(alpha=epi[0], beta=epi[1], act=epi[2], bias=bias.to(DEV) if use_bias else None)
    cc = c if batch > 1 else c[0]
    say(f"  rb{i}: batch={batch} {M}x{N}x{K} {dtype} {layout} pad={pad} share_b={share_b} mode={mode} "
        f"splits={splits} atomic={atomic} two_pass={two_pass} cus={cus} epi={epi} bias={use_bias}")
    dg.gemm_tensors(A.to(DEV), B.to(DEV), cc, b_layout=layout, mode=mode, splits=splits, atomic=atomic,
                    two_pass=two_pass, num_cus=cus, **kw)
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    assert _guards_ok(full, batch, M, N, stride), "a pad or the guard band was overwritten"
    for b in range(batch):
        Ab = A if batch == 1 else A[b]
        Bb = B if share_b else B[b]
        P, S = og.ref_gemm(Ab, Bb, M, N, K, layout, dtype)
        got = c[b].cpu().numpy().astype(np.float64)
        if epi is None:
            ok, worst, idx = og.within_tolerance(got, P, S)
        else:
            c0 = c_in[b].numpy().astype(np.float64) if epi[1] != 0.0 else None
            b64 = bias.numpy().astype(np.float64) if use_bias else None
            D, _ = oe.epilogue_ref(P, c0, epi[0], epi[1], b64, epi[2])
            ok, worst, idx = oe.within_bound(got, D, oe.epilogue_bound(S, P, c0, epi[0], epi[1], b64, epi[2]))
        assert ok, f"entry {b}: worst ratio {worst} at {idx}"


def test_matmul_convenience(dg):
    # matmul allocates the fp32 output: 2-D, a batch with a shared B, and the epilogue
    w = _workload(200, 136, 256, "kn", "bf16")
    A, B = _operands(w, 3, share_b=True)
    out = dg.matmul(A.to(DEV), B.to(DEV))
    assert tuple(out.shape) == (3, 200, 136) and out.dtype == torch.float32
    _check_entries(A, B, out, w, 3, True)
    bias = torch.linspace(-1, 1, 136, device=DEV)
    one = dg.matmul(A[1].to(DEV), B.to(DEV), bias=bias, act="relu")
    P, S = og.ref_gemm(A[1], B, 200, 136, 256, "kn", "bf16")
    D, _ = oe.epilogue_ref(P, None, 1.0, 0.0, bias.cpu().numpy().astype(np.float64), "relu")
    ok, worst, idx = oe.within_bound(one.cpu().numpy().astype(np.float64), D,
                                     oe.epilogue_bound(S, P, None, 1.0, 0.0, bias.cpu().numpy().astype(np.float64),
                                                       "relu"))
    assert ok, worst
