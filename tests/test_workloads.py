"""Pins of the seeded input recipe (workloads/__init__.py), which the oracle and
the GPU path both consume: the draw order from one PCG64 stream, the rounding
to the 16-bit formats (checked against an integer round-to-nearest-even for
bf16 and numpy's float16 conversion for fp16), and the row edits applied after
rounding."""
import numpy as np
import pytest

from workloads import WORKLOADS, make_operands, operand_bits


def _bf16_rne_bits(x32: np.ndarray) -> np.ndarray:
    # round-to-nearest-even of the fp32 pattern to its top 16 bits (finite inputs)
    u = x32.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _draws(w, seed=None):
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    lead = (w.batch,) if w.batch > 1 else ()
    def draw(shape):
        if w.dist == "uniform":
            return rng.uniform(w.low, w.high, size=shape)
        return rng.standard_normal(size=shape) * w.scale
    a = draw(lead + (w.M, w.K))
    b = draw(lead + tuple(w.b_shape()))
    return a.astype(np.float32), b.astype(np.float32)


@pytest.mark.parametrize("name", ["c1_sk32", "c3_wavequant"])
def test_bf16_operands_are_the_rounded_draws(name):
    w = WORKLOADS[name].with_(M=40, N=24, K=72)
    A, B = make_operands(w)
    a32, b32 = _draws(w)
    assert np.array_equal(operand_bits(A), _bf16_rne_bits(a32))
    assert np.array_equal(operand_bits(B), _bf16_rne_bits(b32))


def test_fp16_operands_are_the_rounded_draws():
    w = WORKLOADS["c5_longk_fp16"].with_(M=33, N=40, K=64)
    A, B = make_operands(w)
    a32, b32 = _draws(w)
    assert np.array_equal(operand_bits(A), a32.astype(np.float16).view(np.uint16))
    assert np.array_equal(operand_bits(B), b32.astype(np.float16).view(np.uint16))


def test_skinny_rows_edited_after_rounding():
    w = WORKLOADS["c2a_m96_s8"].with_(K=128, N=32)
    A, B = make_operands(w)
    a32, _ = _draws(w)
    rounded = _bf16_rne_bits(a32).astype(np.uint32) << 16
    rounded = rounded.view(np.float32)
    got = A.float().numpy()
    assert np.all(got[0] == 0.0)
    assert np.array_equal(got[-1], 4.0 * rounded[-1])     # a power of two: exact
    assert np.array_equal(got[1:-1], rounded[1:-1])
    assert w.b_layout == "nk" and tuple(B.shape) == (w.N, w.K)


def test_batched_draws_all_of_a_before_b():
    w = WORKLOADS["x2_batched"].with_(M=16, N=24, K=32, batch=3)
    A, B = make_operands(w)
    a32, b32 = _draws(w)
    assert tuple(A.shape) == (3, 16, 32) and tuple(B.shape) == (3, 32, 24)
    assert np.array_equal(operand_bits(A), _bf16_rne_bits(a32))
    assert np.array_equal(operand_bits(B), _bf16_rne_bits(b32))


def test_seed_determines_the_operands():
    w = WORKLOADS["c1_sk32"].with_(M=20, N=16, K=24)
    A1, B1 = make_operands(w)
    A2, B2 = make_operands(w)
    A3, _ = make_operands(w, seed=w.seed + 1)
    assert np.array_equal(operand_bits(A1), operand_bits(A2))
    assert np.array_equal(operand_bits(B1), operand_bits(B2))
    assert not np.array_equal(operand_bits(A1), operand_bits(A3))


def test_grouped_draws_every_a_then_all_weights():
    from dataclasses import replace

    from workloads import GROUPED, make_group_operands

    gw = replace(GROUPED["x4_grouped"], Ms=(5, 0, 3), N=16, K=24)
    As, B = make_group_operands(gw)
    rng = np.random.Generator(np.random.PCG64(gw.seed))
    for M, A in zip(gw.Ms, As):
        a32 = rng.uniform(gw.low, gw.high, size=(M, gw.K)).astype(np.float32)
        assert tuple(A.shape) == (M, gw.K)
        assert np.array_equal(operand_bits(A), _bf16_rne_bits(a32))
    b32 = rng.uniform(gw.low, gw.high, size=(3, gw.N, gw.K)).astype(np.float32)
    assert tuple(B.shape) == (3, gw.N, gw.K)
    assert np.array_equal(operand_bits(B), _bf16_rne_bits(b32))
    assert gw.flops == 2 * 8 * 16 * 24


def test_grouped_workload_tile_count():
    from workloads import GROUPED

    gw = GROUPED["x4_grouped"]
    assert sum(-(-M // 128) for M in gw.Ms) * (gw.N // 128) == 304
    assert sum(gw.Ms) == 2048
