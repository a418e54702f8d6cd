"""GPU parity of the fused epilogue C = act(alpha A.B + beta C + bias) through
the C ABI, on every decomposition and merge path, against the fp64 oracle
(oracle/epilogue.py over oracle/gemm.py's product).

Bar (per element): |D_gpu - D| <= epilogue_bound (the GEMM bound 1e-4 sum|a||b|
scaled by |alpha|, plus the epilogue's fp32 roundings, times the activation's
Lipschitz constant).  Deterministic merges must give the same bits on repeated
runs, and two-pass merges the same bits as in-launch ones."""
import numpy as np
import pytest
import torch

from oracle import epilogue as oe
from oracle import gemm as og
from workloads import WORKLOADS, make_epilogue_inputs, make_operands

from gpu_util import GUARD, NGUARD, sample_rows, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def dg():
    import dense_gemm_work_amd as dg

    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return dg


# epilogue variants: (alpha, beta, use bias, activation)
E_ALL = (0.75, -0.5, True, "gelu")
E_RELU_NOBETA = (-2.0, 0.0, False, "relu")
E_BIAS = (None, None, True, "none")
E_LINEAR = (1.5, 1.25, False, "none")


def _workload(M, N, K, layout="kn", dtype="bf16"):
    return WORKLOADS["c1_sk32"].with_(name=f"epi_{M}x{N}x{K}", M=M, N=N, K=K, b_layout=layout, dtype=dtype)


def run_epilogue(dg, w, epi, mode, splits=0, atomic=False, two_pass=False, debug=0, num_cus=0,
                 A=None, B=None):
    """Runs the call on a guarded output holding C_in; returns (A, B, c_in, bias, D)."""
    alpha, beta, use_bias, act = epi
    if A is None:
        A, B = make_operands(w)
    c_in, bias = make_epilogue_inputs(w.M, w.N)
    if beta == 0.0:
        c_in = torch.full_like(c_in, float("nan"))   # beta = 0: C_in must not be read
    full = torch.full((w.M * w.N + NGUARD,), GUARD, dtype=torch.float32, device=DEV)
    full[: w.M * w.N] = c_in.reshape(-1).to(DEV)
    c = full[: w.M * w.N].view(w.M, w.N)
    bias_d = bias.to(DEV) if use_bias else None
    say(f"  epilogue {w.name} {w.dtype} {w.b_layout} mode={mode} splits={splits} atomic={atomic} "
        f"two_pass={two_pass} debug={debug} cus={num_cus} epi={epi}")
    dg.gemm_tensors(A.to(DEV), B.to(DEV), c, b_layout=w.b_layout, mode=mode, splits=splits, atomic=atomic,
                    two_pass=two_pass, debug=debug, num_cus=num_cus, alpha=alpha, beta=beta, bias=bias_d,
                    act=act)
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    assert bool(torch.all(full[w.M * w.N:] == GUARD)), "guard band overwritten"
    return A, B, c_in, (bias if use_bias else None), c


def check(A, B, w, epi, c_in, bias, d_gpu, rows=None):
    alpha, beta, _, act = epi
    a = 1.0 if alpha is None else alpha
    b = 0.0 if beta is None else beta
    P, S = og.ref_gemm(A, B, w.M, w.N, w.K, w.b_layout, w.dtype, rows=rows)
    c0 = c_in.numpy().astype(np.float64)
    got = d_gpu.detach().cpu().numpy().astype(np.float64)
    if rows is not None:
        c0, got = c0[np.asarray(rows)], got[np.asarray(rows)]
    bias64 = None if bias is None else bias.numpy().astype(np.float64)
    D, _ = oe.epilogue_ref(P, c0 if b != 0.0 else None, a, b, bias64, act)
    bound = oe.epilogue_bound(S, P, c0 if b != 0.0 else None, a, b, bias64, act)
    ok, worst, idx = oe.within_bound(got, D, bound)
    say(f"    worst err/bound = {worst:.3e} at {idx}")
    assert ok, f"outside the epilogue bound: worst ratio {worst} at {idx}"


# (id, M, N, K, layout, dtype, mode, splits, atomic, two_pass, debug, num_cus)
CASES = [
    ("dp-ragged", 300, 272, 320, "kn", "bf16", "dp", 0, False, False, 0, 0),
    ("dp-groups", 1024, 1024, 256, "kn", "bf16", "dp", 0, False, False, 0, 16),
    ("dp-groups-ragged", 1000, 1000, 200, "nk", "fp16", "dp", 0, False, False, 0, 16),
    ("splitk4-in-launch", 256, 512, 2048, "kn", "bf16", "splitk", 4, False, False, "IN_LAUNCH", 0),
    ("splitk8-in-launch", 96, 512, 2048, "nk", "bf16", "splitk", 8, False, False, "IN_LAUNCH", 0),
    ("splitk8-two-pass", 96, 512, 2048, "nk", "bf16", "splitk", 8, False, False, 0, 0),
    ("splitk2-scalar-in-launch", 200, 130, 512, "nk", "bf16", "splitk", 2, False, False, "IN_LAUNCH", 0),
    ("splitk2-scalar-two-pass", 200, 130, 512, "nk", "bf16", "splitk", 2, False, True, 0, 0),
    ("splitk8-atomic", 96, 512, 2048, "nk", "bf16", "splitk", 8, True, False, 0, 0),
    ("streamk-turnstile", 256, 512, 2048, "kn", "bf16", "streamk", 32, False, False, "IN_LAUNCH", 0),
    ("streamk-two-pass", 256, 512, 2048, "kn", "bf16", "streamk", 32, False, False, 0, 0),
    ("streamk-atomic", 256, 512, 2048, "kn", "fp16", "streamk", 32, True, False, 0, 0),
    ("streamk-ragged", 330, 200, 1000, "nk", "bf16", "streamk", 7, False, False, 0, 0),
    ("hybrid", 640, 640, 2048, "kn", "bf16", "heuristic", 0, False, False, 0, 8),
    ("hybrid-atomic", 640, 640, 2048, "kn", "bf16", "heuristic", 0, True, False, 0, 8),
]


def _debug(dg, d):
    return dg.GEMM_DEBUG_IN_LAUNCH if d == "IN_LAUNCH" else 0


@pytest.mark.parametrize("epi", [E_ALL, E_RELU_NOBETA], ids=["all", "relu-beta0"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_epilogue_parity(dg, case, epi):
    _, M, N, K, layout, dtype, mode, splits, atomic, two_pass, debug, cus = case
    w = _workload(M, N, K, layout, dtype)
    A, B, c_in, bias, d = run_epilogue(dg, w, epi, mode, splits, atomic, two_pass, _debug(dg, debug), cus)
    if epi[1] == 0.0:
        assert bool(torch.isfinite(d).all()), "beta = 0 must not read C_in"
    check(A, B, w, epi, c_in, bias, d)


@pytest.mark.parametrize("epi", [E_BIAS, E_LINEAR], ids=["bias", "linear"])
@pytest.mark.parametrize("case", [c for c in CASES if c[0] in ("dp-groups", "splitk8-in-launch", "streamk-two-pass",
                                                              "streamk-atomic")],
                         ids=lambda c: c[0])
def test_epilogue_parts(dg, case, epi):
    _, M, N, K, layout, dtype, mode, splits, atomic, two_pass, debug, cus = case
    w = _workload(M, N, K, layout, dtype)
    A, B, c_in, bias, d = run_epilogue(dg, w, epi, mode, splits, atomic, two_pass, _debug(dg, debug), cus)
    check(A, B, w, epi, c_in, bias, d)


@pytest.mark.parametrize("epi", [E_ALL, E_RELU_NOBETA, E_BIAS], ids=["all", "relu-beta0", "bias"])
def test_epilogue_empty_sum(dg, epi):
    # K == 0: the product is zero, C = act(beta C_in + bias)
    w = _workload(130, 72, 0)
    A = torch.zeros(130, 0, dtype=torch.bfloat16)
    B = torch.zeros(0, 72, dtype=torch.bfloat16)
    A, B, c_in, bias, d = run_epilogue(dg, w, epi, "heuristic", A=A, B=B)
    check(A, B, w, epi, c_in, bias, d)


@pytest.mark.parametrize("act", ["gelu", "relu"])
def test_activation_sweep(dg, act):
    # K == 0 with alpha = beta = 1: C = act(C_in) over C_in from -12 to 12, the
    # activation alone against the oracle's exact one
    M, N = 64, 4096
    w = _workload(M, N, 0)
    c_in = torch.linspace(-12.0, 12.0, M * N, dtype=torch.float32).view(M, N)
    full = torch.full((M * N + NGUARD,), GUARD, dtype=torch.float32, device=DEV)
    full[: M * N] = c_in.reshape(-1).to(DEV)
    c = full[: M * N].view(M, N)
    say(f"  activation sweep {act}")
    dg.gemm_tensors(torch.zeros(M, 0, dtype=torch.bfloat16, device=DEV),
                    torch.zeros(0, N, dtype=torch.bfloat16, device=DEV), c, alpha=1.0, beta=1.0, act=act)
    assert dg.gemm_sync_status() == 0, dg.gemm_last_error()
    assert bool(torch.all(full[M * N:] == GUARD))
    c0 = c_in.numpy().astype(np.float64)
    zero = np.zeros_like(c0)
    D, _ = oe.epilogue_ref(zero, c0, 1.0, 1.0, None, act)
    bound = oe.epilogue_bound(zero, zero, c0, 1.0, 1.0, None, act)
    ok, worst, idx = oe.within_bound(c.cpu().numpy().astype(np.float64), D, bound)
    say(f"    worst err/bound = {worst:.3e} at {idx}")
    assert ok, f"activation outside the bound: worst ratio {worst} at {idx}"


def test_epilogue_deterministic_bits(dg):
    # same bits on repeated runs; two-pass merges give the in-launch merges' bits
    def bits(case, debug=0, two_pass=False):
        _, M, N, K, layout, dtype, mode, splits, atomic, _, _, cus = case
        w = _workload(M, N, K, layout, dtype)
        *_, d = run_epilogue(dg, w, E_ALL, mode, splits, atomic, two_pass, debug, cus)
        return d.cpu().clone()

    by = {c[0]: c for c in CASES}
    sk_in = bits(by["streamk-turnstile"], dg.GEMM_DEBUG_IN_LAUNCH)
    sk_2p = bits(by["streamk-turnstile"], two_pass=True)
    assert torch.equal(sk_in, sk_2p), "Stream-K two-pass epilogue differs from the turnstile"
    for _ in range(2):
        assert torch.equal(bits(by["streamk-turnstile"], dg.GEMM_DEBUG_IN_LAUNCH), sk_in)
    spk_in = bits(by["splitk8-in-launch"], dg.GEMM_DEBUG_IN_LAUNCH)
    spk_2p = bits(by["splitk8-in-launch"], two_pass=True)
    assert torch.equal(spk_in, spk_2p), "Split-K two-pass epilogue differs from the in-launch fold"
    sc_in = bits(by["splitk2-scalar-in-launch"], dg.GEMM_DEBUG_IN_LAUNCH)
    sc_2p = bits(by["splitk2-scalar-in-launch"], two_pass=True)
    assert torch.equal(sc_in, sc_2p)


def test_epilogue_wavequant_full_size(dg):
    # the 2048 x 2176 x 4096 Stream-K call with the whole epilogue, sampled rows
    w = WORKLOADS["c3_wavequant"]
    A, B, c_in, bias, d = run_epilogue(dg, w, E_ALL, "heuristic")
    check(A, B, w, E_ALL, c_in, bias, d, rows=sample_rows(w.M, 24))
