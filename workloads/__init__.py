"""Seeded synthetic operands for the DP / Split-K / Stream-K GEMM workloads.

This module only *makes inputs*: shapes, seeds, value distributions and the
rounding of fp64 draws to the 16-bit operand format.  It holds none of the GEMM
arithmetic, so both the CPU oracle (``oracle/``) and the HIP path
(``dense_gemm_work_amd``) can consume what it produces without sharing any of
the method's code.

Input recipe (the pages fix only the shapes, distributions and, for the first
workload, the seed; the rest is a stated reading):

* ``numpy.random.Generator(PCG64(seed))``; A is drawn first, then B, each as one
  float64 array in row-major order of its *stored* shape.
* Draws are cast to float32 and then rounded to nearest-even in bf16 or fp16
  (``torch.Tensor.to`` performs round-to-nearest-even).
* "Skinny split-K" operands additionally set A's first row to zero and scale
  its last row by 4 *after* rounding (4 is a power of two, so the scaling is
  exact).  This mirrors the Metal split-K benchmark note's fixture design
  (first input row zero, last row at four times the ordinary scale).

The five workloads below are the ones the performance and parity harness runs
(plus one beyond them, ``x1_hybrid``, for the heuristic's hybrid regime).
Row counts, tile counts and wave arithmetic for each are derived from 128x128
output tiles and 64-wide k-iterations, as the Split-K/Stream-K book chapter
uses throughout its worked cases.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_operands", "operand_bits", "get", "GroupedWorkload", "GROUPED",
           "make_group_operands"]


@dataclass(frozen=True)
class Workload:
    """One synthetic GEMM problem: ``C[M,N] = A[M,K] . op(B)`` in fp32."""

    name: str
    M: int
    N: int
    K: int
    dtype: str = "bf16"          # operand format: "bf16" or "fp16"
    b_layout: str = "kn"         # "kn": B stored [K,N]; "nk": B stored [N,K] (C = A.B^T)
    dist: str = "uniform"        # "uniform" (low, high) or "normal" (scale)
    low: float = -1.0
    high: float = 1.0
    scale: float = 1.0
    zero_first_row: bool = False  # A row 0 := 0 after rounding
    scale_last_row: float = 1.0   # A row M-1 *= this after rounding
    seed: int = 0
    mode: str = "heuristic"      # decomposition the workload is specified with
    splits: int = 0              # Split-K factor or Stream-K unit count (0 = one per CU)
    atomic: bool = False         # nondeterministic (atomic) fixup for Stream-K
    note: str = ""
    batch: int = 1               # independent products of this shape (operands [batch, ...])

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch

    def b_shape(self):
        return (self.K, self.N) if self.b_layout == "kn" else (self.N, self.K)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads (names used by tests and the benchmark).
WORKLOADS = {
    # Small Stream-K case: 8 tiles x 32 k-iterations, 32 units of 8 iterations.
    "c1_sk32": Workload("c1_sk32", 256, 512, 2048, "bf16", "kn", "uniform", -1.0, 1.0,
                        mode="streamk", splits=32,
                        note="8 tiles x 32 iters; Stream-K 32 units x 8 iters; deterministic fixup"),
    # Skinny Split-K with weights stored [N,K].
    "c2a_m96_s8": Workload("c2a_m96_s8", 96, 512, 2048, "bf16", "nk", "uniform", -1.0, 1.0,
                           zero_first_row=True, scale_last_row=4.0, mode="splitk", splits=8,
                           note="C = A.B^T, 8 splits, fp32 partials [S,M,N] reduced in k order"),
    "c2b_m256_s2": Workload("c2b_m256_s2", 256, 512, 2048, "bf16", "nk", "uniform", -1.0, 1.0,
                            zero_first_row=True, scale_last_row=4.0, mode="splitk", splits=2,
                            note="C = A.B^T, 2 splits"),
    # Wave-quantized: 16x17 = 272 tiles = one full 256-CU wave + 16-tile tail.
    "c3_wavequant": Workload("c3_wavequant", 2048, 2176, 4096, "bf16", "kn", "normal",
                             scale=0.1, mode="heuristic",
                             note="272 tiles on 256 CUs; heuristic must pick Stream-K"),
    # Large, data-parallel dominant: 4096 tiles = 16 full waves.
    "c4_large_dp": Workload("c4_large_dp", 8192, 8192, 8192, "bf16", "kn", "uniform", -1.0, 1.0,
                            mode="heuristic", note="16 full waves; heuristic must stay DP"),
    # Long-K, 144 tiles on 256 CUs, fp16, both fixup modes.
    "c5_longk_fp16": Workload("c5_longk_fp16", 1536, 1536, 16384, "fp16", "kn", "uniform", -0.5, 0.5,
                              mode="streamk", splits=0,
                              note="144 tiles x 256 iters; Stream-K 256 units; turnstile and atomic fixup"),
    # Beyond the five: the heuristic's hybrid regime.  32x33 = 1056 tiles = 4 full
    # waves + a 32-tile tail, so 3 waves stay data-parallel and the last 288 tiles
    # go to 256 Stream-K units of 72 iterations.
    "x1_hybrid": Workload("x1_hybrid", 4096, 4224, 4096, "bf16", "kn", "uniform", -1.0, 1.0,
                          mode="heuristic", note="1056 tiles; heuristic -> 768 DP tiles + Stream-K over 288"),
    # A wave-quantized batch: 5 x (1024x1024x2048) = 320 tiles (one full wave + a
    # 64-tile tail on 256 CUs) x 32 iterations.
    "x2_batched": Workload("x2_batched", 1024, 1024, 2048, "bf16", "kn", "uniform", -1.0, 1.0,
                           mode="heuristic", batch=5,
                           note="5 entries x 64 tiles x 32 iters; heuristic -> Stream-K, 256 units x 40 iterations"),
    # The book chapter's skinny case: a decode-time batch of 128 rows through a
    # 4096-wide projection, weights stored [N,K]: 32 tiles of 128x128 (64 of
    # 64x128) on 256 CUs, 64 iterations each.
    "x3_decode": Workload("x3_decode", 128, 4096, 4096, "bf16", "nk", "uniform", -1.0, 1.0,
                          mode="heuristic", note="32 tiles (64 of 64x128); heuristic -> Split-K"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


@dataclass(frozen=True)
class GroupedWorkload:
    """Problems of one K and one weight shape with their own row counts, run as
    one grouped call: an expert layer, where problem g multiplies the ``Ms[g]``
    tokens routed to expert g by that expert's own weights."""

    name: str
    Ms: tuple
    N: int
    K: int
    dtype: str = "bf16"
    b_layout: str = "nk"
    low: float = -1.0
    high: float = 1.0
    seed: int = 0
    note: str = ""

    @property
    def flops(self) -> int:
        return 2 * sum(self.Ms) * self.N * self.K

    def member(self, g: int) -> Workload:
        """Problem g as a single-problem workload (same distribution)."""
        return Workload(f"{self.name}[{g}]", self.Ms[g], self.N, self.K, self.dtype, self.b_layout, "uniform",
                        self.low, self.high)

    def b_shape(self):
        return (self.K, self.N) if self.b_layout == "kn" else (self.N, self.K)


GROUPED = {
    # 2048 tokens routed unevenly over 8 experts, each a 4096 -> 2048 projection
    # with weights stored [N,K]: 19 tile rows x 16 = 304 tiles of 128x128 (one
    # full wave on 256 CUs and a 48-tile tail), 64 iterations each.
    "x4_grouped": GroupedWorkload("x4_grouped", (448, 96, 320, 64, 512, 160, 256, 192), 2048, 4096,
                                  note="8 problems, 304 tiles; heuristic -> Stream-K over all of them"),
}


def make_group_operands(gw: GroupedWorkload, seed: Optional[int] = None):
    """Return ``([A_g], B)`` as CPU torch tensors in the workload's 16-bit dtype:
    ``A_g`` of shape ``[Ms[g], K]`` drawn in problem order, then every problem's
    weights as one ``[G, N, K]`` (layout "nk") or ``[G, K, N]`` array, all from
    one ``PCG64(seed)`` stream, uniform on [low, high), rounded as in
    ``make_operands``."""
    rng = np.random.Generator(np.random.PCG64(gw.seed if seed is None else seed))
    td = _torch_dtype(gw.dtype)
    As = [torch.from_numpy(rng.uniform(gw.low, gw.high, size=(M, gw.K)).astype(np.float32)).to(td).contiguous()
          for M in gw.Ms]
    b64 = rng.uniform(gw.low, gw.high, size=(len(gw.Ms),) + tuple(gw.b_shape()))
    B = torch.from_numpy(b64.astype(np.float32)).to(td).contiguous()
    return As, B


def _torch_dtype(dtype: str) -> torch.dtype:
    if dtype == "bf16":
        return torch.bfloat16
    if dtype == "fp16":
        return torch.float16
    raise ValueError(f"unknown operand dtype {dtype!r}")


def _draw(rng: np.random.Generator, w: Workload, shape) -> np.ndarray:
    if w.dist == "uniform":
        return rng.uniform(w.low, w.high, size=shape)
    if w.dist == "normal":
        return rng.standard_normal(size=shape) * w.scale
    raise ValueError(f"unknown distribution {w.dist!r}")


def make_operands(w: Workload, seed: Optional[int] = None):
    """Return ``(A, B)`` as CPU torch tensors in the workload's 16-bit dtype.

    A has shape ``[M, K]``; B has shape ``[K, N]`` (layout "kn") or ``[N, K]``
    (layout "nk"); with ``batch > 1`` both gain a leading batch dimension (all
    of A drawn before all of B).  Both are contiguous.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    td = _torch_dtype(w.dtype)
    lead = (w.batch,) if w.batch > 1 else ()
    a64 = _draw(rng, w, lead + (w.M, w.K))
    b64 = _draw(rng, w, lead + tuple(w.b_shape()))
    A = torch.from_numpy(a64.astype(np.float32)).to(td)
    del a64
    B = torch.from_numpy(b64.astype(np.float32)).to(td)
    del b64
    if w.M > 0 and w.zero_first_row:
        A[..., 0, :].zero_()
    if w.M > 0 and w.scale_last_row != 1.0:
        A[..., w.M - 1, :] = (A[..., w.M - 1, :].float() * w.scale_last_row).to(td)
    return A.contiguous(), B.contiguous()


def operand_bits(t: torch.Tensor) -> np.ndarray:
    """The raw 16-bit patterns of a bf16/fp16 CPU tensor as a numpy uint16 array."""
    if t.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("expected a bf16 or fp16 tensor")
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def make_epilogue_inputs(M: int, N: int, seed: int = 1):
    """Seeded fp32 inputs of the fused epilogue: the prior output ``C_in`` [M,N]
    and a per-column ``bias`` [N], both uniform on [-1, 1) (CPU torch tensors)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    c_in = torch.from_numpy(rng.uniform(-1.0, 1.0, size=(M, N)).astype(np.float32))
    bias = torch.from_numpy(rng.uniform(-1.0, 1.0, size=(N,)).astype(np.float32))
    return c_in.contiguous(), bias.contiguous()
