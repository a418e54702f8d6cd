"""Pins of the fp64 value oracle (oracle/ref_gemm.c) against facts that do not
come from the oracle itself: the bf16/fp16 format definitions, exact integer
arithmetic, closed forms, brute-force rational sums, numpy's float64 matmul,
and planted mistakes that every pin set must catch."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import build as obuild
from oracle import gemm as og
from workloads import WORKLOADS, make_operands, operand_bits


def _bits_of(values, dtype):
    td = torch.bfloat16 if dtype == "bf16" else torch.float16
    t = torch.tensor(values, dtype=torch.float32).to(td)
    return operand_bits(t).reshape(np.shape(values))


# -- format decoding (IEEE-754 binary16; bfloat16 = top half of binary32) ------
@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xBF80, -1.0), (0x4000, 2.0), (0x3F00, 0.5), (0x4049, 3.140625),
    (0x0000, 0.0), (0x0001, 2.0 ** -133), (0x0080, 2.0 ** -126), (0x7F7F, 3.3895313892515355e38),
    (0x3DCD, 0.10009765625),
])
def test_bf16_decode(bits, value):
    assert og.decode(np.array([bits], np.uint16), "bf16")[0] == value


@pytest.mark.parametrize("bits,value", [
    (0x3C00, 1.0), (0xC000, -2.0), (0x3800, 0.5), (0x0001, 2.0 ** -24), (0x0400, 2.0 ** -14),
    (0x7BFF, 65504.0), (0x3555, 0.333251953125), (0x8000, -0.0), (0x03FF, 1023 * 2.0 ** -24),
])
def test_fp16_decode(bits, value):
    assert og.decode(np.array([bits], np.uint16), "fp16")[0] == value


def test_decode_special_values():
    assert np.isinf(og.decode(np.array([0x7C00], np.uint16), "fp16")[0])
    assert np.isnan(og.decode(np.array([0x7E00], np.uint16), "fp16")[0])
    assert np.isinf(og.decode(np.array([0xFF80], np.uint16), "bf16")[0])


def test_decode_matches_torch_upcast_all_patterns():
    # every finite 16-bit pattern, against torch's own widening to float32 (exact)
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for dtype, td in (("bf16", torch.bfloat16), ("fp16", torch.float16)):
        vals = torch.from_numpy(allbits.view(np.int16)).view(td).float().double().numpy()
        sample = allbits[::97]
        got = og.decode(sample, dtype)
        ref = vals[::97]
        finite = np.isfinite(ref)
        assert np.array_equal(got[finite], ref[finite])


# -- exact integer arithmetic ----------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_small_integers_exact(dtype, layout):
    rng = np.random.default_rng(7)
    M, N, K = 5, 7, 11
    a = rng.integers(-8, 9, size=(M, K)).astype(np.float64)
    b = rng.integers(-8, 9, size=(K, N)).astype(np.float64)
    ab = _bits_of(a, dtype)
    bb = _bits_of(b if layout == "kn" else b.T.copy(), dtype)
    C, S = og.ref_gemm(ab, bb, M, N, K, layout, dtype)
    assert np.array_equal(C, a @ b)            # all integers: exact in fp64
    assert np.array_equal(S, np.abs(a) @ np.abs(b))


def test_brute_force_rationals_tiny():
    # pure-Python exact sum of products on a tiny case; fp64 accumulation of
    # exactly-representable products over 6 terms stays within 2 ulp
    rng = np.random.default_rng(3)
    M, N, K = 3, 4, 6
    a = rng.uniform(-1, 1, (M, K))
    b = rng.uniform(-1, 1, (K, N))
    ab, bb = _bits_of(a, "bf16"), _bits_of(b, "bf16")
    av = og.decode(ab, "bf16")
    bv = og.decode(bb, "bf16")
    C, S = og.ref_gemm(ab, bb, M, N, K, "kn", "bf16")
    for i in range(M):
        for j in range(N):
            exact = sum(Fraction(av[i, k]) * Fraction(bv[k, j]) for k in range(K))
            exact_abs = sum(abs(Fraction(av[i, k]) * Fraction(bv[k, j])) for k in range(K))
            assert abs(Fraction(C[i, j]) - exact) <= Fraction(2 ** -50) * exact_abs
            assert abs(Fraction(S[i, j]) - exact_abs) <= Fraction(2 ** -50) * exact_abs


# -- closed forms --------------------------------------------------------------
def test_all_ones_gives_k():
    M, N, K = 9, 13, 333
    ab = _bits_of(np.ones((M, K)), "bf16")
    bb = _bits_of(np.ones((K, N)), "bf16")
    C, S = og.ref_gemm(ab, bb, M, N, K, "kn", "bf16")
    assert np.all(C == K) and np.all(S == K)


def test_alternating_signs_cancel():
    M, N, K = 4, 6, 64
    a = np.tile((-1.0) ** np.arange(K), (M, 1))
    ab = _bits_of(a, "fp16")
    bb = _bits_of(np.full((N, K), 0.5), "fp16")       # nk layout
    C, S = og.ref_gemm(ab, bb, M, N, K, "nk", "fp16")
    assert np.all(C == 0.0) and np.all(S == K * 0.5)


def test_outer_product_closed_form():
    # rank-one A (rows r_i times one row v) against B columns: C_ij = r_i * (v . b_j)
    M, N, K = 6, 5, 32
    r = np.array([1, -2, 0.5, 4, -0.25, 8.0])
    v = np.arange(1, K + 1) % 7 - 3.0
    a = np.outer(r, v)
    b = (np.arange(K * N).reshape(K, N) % 5) - 2.0
    ab, bb = _bits_of(a, "bf16"), _bits_of(b, "bf16")
    C, _ = og.ref_gemm(ab, bb, M, N, K, "kn", "bf16")
    assert np.array_equal(C, np.outer(r, v @ b))


def test_skinny_workload_structure():
    # the skinny split-K operands: row 0 of C is exactly zero, S too; the last row is 4x
    w = WORKLOADS["c2a_m96_s8"].with_(K=256)
    A, B = make_operands(w)
    C, S = og.ref_gemm(A, B, w.M, w.N, w.K, "nk", "bf16")
    assert np.all(C[0] == 0.0) and np.all(S[0] == 0.0)
    assert np.all(S[1:] > 0.0)
    A1 = A.clone()
    A1[w.M - 1] = (A1[w.M - 1].float() / 4).to(torch.bfloat16)
    C1, _ = og.ref_gemm(A1, B, w.M, w.N, w.K, "nk", "bf16", rows=[w.M - 1])
    assert np.array_equal(C[w.M - 1], 4.0 * C1[0])


def test_abs_sum_bounds_value():
    w = WORKLOADS["c3_wavequant"].with_(M=64, N=96, K=512)
    A, B = make_operands(w)
    C, S = og.ref_gemm(A, B, w.M, w.N, w.K, "kn", "bf16")
    assert np.all(np.abs(C) <= S)


# -- library routine: numpy float64 matmul -------------------------------------
@pytest.mark.parametrize("name", ["c1_sk32", "c2a_m96_s8", "c2b_m256_s2"])
def test_matches_numpy_float64(name):
    w = WORKLOADS[name]
    A, B = make_operands(w)
    a = A.double().numpy()
    b = B.double().numpy()
    ref = a @ (b if w.b_layout == "kn" else b.T)
    C, S = og.ref_gemm(A, B, w.M, w.N, w.K, w.b_layout, w.dtype)
    assert np.all(np.abs(C - ref) <= 1e-12 * S + 1e-300)
    assert np.allclose(S, np.abs(a) @ np.abs(b if w.b_layout == "kn" else b.T), rtol=1e-13)


def test_fp16_workload_matches_numpy():
    w = WORKLOADS["c5_longk_fp16"].with_(M=48, N=80, K=4096)
    A, B = make_operands(w)
    ref = A.double().numpy() @ B.double().numpy()
    C, S = og.ref_gemm(A, B, w.M, w.N, w.K, "kn", "fp16")
    assert np.all(np.abs(C - ref) <= 1e-12 * S)


def test_row_sampling_matches_full():
    w = WORKLOADS["c1_sk32"]
    A, B = make_operands(w)
    C, S = og.ref_gemm(A, B, w.M, w.N, w.K, "kn", "bf16")
    rows = [0, 17, 255, 128]
    Cs, Ss = og.ref_gemm(A, B, w.M, w.N, w.K, "kn", "bf16", rows=rows)
    assert np.array_equal(Cs, C[rows]) and np.array_equal(Ss, S[rows])


def test_layout_transposition():
    w = WORKLOADS["c1_sk32"].with_(M=40, N=72, K=192)
    A, B = make_operands(w)
    Ckn, _ = og.ref_gemm(A, B, w.M, w.N, w.K, "kn", "bf16")
    Cnk, _ = og.ref_gemm(A, B.t().contiguous(), w.M, w.N, w.K, "nk", "bf16")
    assert np.array_equal(Ckn, Cnk)


def test_empty_and_degenerate():
    C, S = og.ref_gemm(np.zeros(0, np.uint16), np.zeros(0, np.uint16), 0, 4, 0, "kn", "bf16")
    assert C.shape == (0, 4)
    # K = 0: the empty sum
    C, S = og.ref_gemm(np.zeros(0, np.uint16), np.zeros(0, np.uint16), 3, 4, 0, "kn", "bf16")
    assert np.all(C == 0) and np.all(S == 0)
    with pytest.raises(ValueError):
        og.ref_gemm(np.zeros(6, np.uint16), np.zeros(6, np.uint16), 2, 3, 3, "kn", "bf16", rows=[5])


def test_tolerance_function():
    ref = np.array([[1.0, 0.0]])
    s = np.array([[10.0, 0.0]])
    assert og.within_tolerance(np.array([[1.0 + 9e-4, 0.0]]), ref, s)[0]
    assert not og.within_tolerance(np.array([[1.0 + 2e-3, 0.0]]), ref, s)[0]
    assert not og.within_tolerance(np.array([[1.0, 1e-30]]), ref, s)[0]     # S = 0 demands exact zero
    assert not og.within_tolerance(np.array([[np.nan, 0.0]]), ref, s)[0]


# -- planted mistakes: every one must be caught by the pins above ----------------
def _pins_pass(lib_file) -> bool:
    try:
        rng = np.random.default_rng(11)
        M, N, K = 5, 7, 11
        a = rng.integers(-8, 9, size=(M, K)).astype(np.float64)
        b = rng.integers(-8, 9, size=(K, N)).astype(np.float64)
        for dtype in ("bf16", "fp16"):
            for layout in ("kn", "nk"):
                ab = _bits_of(a, dtype)
                bb = _bits_of(b if layout == "kn" else b.T.copy(), dtype)
                C, S = og.ref_gemm(ab, bb, M, N, K, layout, dtype, lib_file=lib_file)
                if not (np.array_equal(C, a @ b) and np.array_equal(S, np.abs(a) @ np.abs(b))):
                    return False
        return True
    except Exception:
        return False


@pytest.mark.parametrize("mutation", [1, 2, 3, 4])
def test_planted_mistakes_are_caught(tmp_path, mutation):
    good = obuild.build(0, out_dir=tmp_path)
    assert _pins_pass(good)
    bad = obuild.build(mutation, out_dir=tmp_path)
    assert not _pins_pass(bad), f"planted mistake {mutation} slipped through the pins"
