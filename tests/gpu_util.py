"""Shared helpers of the GPU tests: guarded output buffers, oracle comparison,
and decoding of the kernels' debug trace (layout in include/gemm.h)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import gemm as og
from oracle import schedule as sch

POISON = 7.0      # every output starts at 7 (Metal split-K note's fixture)
GUARD = 11.0      # 64 trailing guard elements start at 11
NGUARD = 64


def say(*a):
    print(*a, flush=True)


def guarded_output(M: int, N: int, dev):
    """An fp32 [M,N] view into a buffer with NGUARD trailing guard elements."""
    full = torch.full((M * N + NGUARD,), POISON, dtype=torch.float32, device=dev)
    full[M * N:] = GUARD
    return full, full[: M * N].view(M, N)


def guards_intact(full: torch.Tensor, M: int, N: int) -> bool:
    return bool(torch.all(full[M * N:] == GUARD).item())


def check_against_oracle(c_gpu: torch.Tensor, A, B, w, rows=None, tol=og.TOLERANCE):
    """Elementwise |C_gpu - C_ref| <= tol * sum|a||b| on all rows or a row sample."""
    C, S = og.ref_gemm(A, B, w.M, w.N, w.K, w.b_layout, w.dtype, rows=rows)
    got = c_gpu.detach().cpu().numpy().astype(np.float64)
    if rows is not None:
        got = got[np.asarray(rows)]
    ok, worst, idx = og.within_tolerance(got, C, S, tol)
    return ok, worst, idx


_ORACLE_CACHE: dict = {}


def oracle_full(w):
    """(A, B, C_ref, S) of a workload's seeded operands over every row, computed
    once per test session (the full-size products take a few seconds each)."""
    from workloads import make_operands

    if w not in _ORACLE_CACHE:
        A, B = make_operands(w)
        C, S = og.ref_gemm(A, B, w.M, w.N, w.K, w.b_layout, w.dtype)
        _ORACLE_CACHE[w] = (A, B, C, S)
    return _ORACLE_CACHE[w]


def check_full(c_gpu: torch.Tensor, w, tol=og.TOLERANCE):
    """Every element of C against the cached full-size oracle: (ok, worst ratio, index)."""
    _, _, C, S = oracle_full(w)
    got = c_gpu.detach().cpu().numpy().astype(np.float64)
    return og.within_tolerance(got, C, S, tol)


def poison_rows(c_gpu: torch.Tensor, limit: int = 64):
    """Rows of C that still hold the fill value somewhere (at most `limit`)."""
    return torch.nonzero((c_gpu == POISON).any(dim=1)).flatten().tolist()[:limit]


def tile_row_sample(M: int, seed: int = 0, bm: int = 128):
    """One random row inside every bm-row band of C, plus the first and last row."""
    rng = np.random.default_rng(seed)
    rows = {0, M - 1}
    for r0 in range(0, M, bm):
        rows.add(int(rng.integers(r0, min(M, r0 + bm))))
    return sorted(rows)


def sample_rows(M: int, n: int, seed: int = 0):
    """First, last, a ragged-tile row and n random rows (sorted, unique)."""
    rng = np.random.default_rng(seed)
    rows = {0, M - 1, (M - 1) // 128 * 128, min(M - 1, 127), min(M - 1, 128)}
    rows |= set(rng.integers(0, M, size=n).tolist())
    return sorted(r for r in rows if 0 <= r < M)


def decode_trace(tr: torch.Tensor):
    t = tr.cpu().numpy().astype(np.int64)
    magic, decision, workers, tiles, ipt, maxseg, maxfold, splits = t[:8]
    assert magic == 0x4B525453
    pos = 8
    segs = []
    for w in range(workers):
        rec = t[pos: pos + 1 + 4 * maxseg]
        n = rec[0]
        for i in range(n):
            tile, k0, k1, role = rec[1 + 4 * i: 5 + 4 * i]
            segs.append((w, int(tile), int(k0), int(k1), int(role)))
        pos += 1 + 4 * maxseg
    folds = {}
    for tile in range(tiles):
        rec = t[pos: pos + 1 + maxfold]
        folds[tile] = [int(x) for x in rec[1: 1 + rec[0]]]
        pos += 1 + maxfold
    cov = t[pos: pos + tiles * ipt].reshape(tiles, ipt) if ipt > 0 else np.zeros((tiles, 0))
    return dict(decision=int(decision), workers=int(workers), tiles=int(tiles), ipt=int(ipt),
                segments=sorted(segs), folds=folds, coverage=cov)


def expected_trace(M, N, K, mode, splits, cus, batch=1, bm=128):
    s = sch.plan_schedule(M, N, K, mode, splits, sms=cus, batch=batch, bm=bm)
    segs = sorted(x.as_tuple() for x in s.segments)
    groups = sch.tile_groups(s.segments)
    folds = {t: [owner] + peers for t, (owner, peers) in groups.items()}
    return s, segs, folds
