"""Python front end of the fp64 value oracle (``ref_gemm.c``).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the library.

``ref_gemm(A, B, b_layout, rows=None)`` returns ``(C, S)`` as float64 numpy
arrays, where ``C = sum_k a_ik b_kj`` and ``S = sum_k |a_ik| |b_kj|`` over the
exact values of the bf16/fp16 operands (Split-K/Stream-K book chapter, "The
boring rule": an fp64 reference with a K-scaled tolerance; Metal split-K note,
"Contract and numerical coverage": fp64 dot products over the dtype-rounded
inputs).  ``within_tolerance`` applies the elementwise bound
``|C_gpu - C| <= tol * S`` with ``tol = 1e-4``.
"""
from __future__ import annotations

import ctypes
import time
from pathlib import Path
from typing import Optional, Sequence

import numpy as np

from . import build as _build

_LIBS: dict = {}

TOLERANCE = 1e-4  # relative to S = sum_k |a||b|


def _load(mutation: int = 0, lib_file: Optional[Path] = None):
    key = (mutation, str(lib_file))
    if key in _LIBS:
        return _LIBS[key]
    path = Path(lib_file) if lib_file is not None else _build.lib_path(mutation)
    if not path.exists() or (lib_file is None and path.stat().st_mtime < _build.SRC.stat().st_mtime):
        path = _build.build(mutation, out_dir=path.parent)
    lib = ctypes.CDLL(str(path))
    lib.oracle_gemm_rows.restype = ctypes.c_int
    lib.oracle_gemm_rows.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
        ctypes.c_void_p,
    ]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_fp16_to_f64.restype = ctypes.c_double
    lib.oracle_fp16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_num_threads.restype = ctypes.c_int
    _LIBS[key] = lib
    return lib


def _bits(x) -> np.ndarray:
    """Accept a numpy uint16 array or a CPU torch bf16/fp16 tensor."""
    if isinstance(x, np.ndarray):
        if x.dtype != np.uint16:
            raise TypeError("numpy operands must be uint16 bit patterns")
        return np.ascontiguousarray(x)
    import torch  # local: keep the oracle importable without torch for pure-numpy use

    if isinstance(x, torch.Tensor):
        if x.dtype not in (torch.bfloat16, torch.float16):
            raise TypeError("torch operands must be bf16 or fp16")
        return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    raise TypeError(f"unsupported operand type {type(x)}")


def _dtype_code(dtype: str) -> int:
    return {"bf16": 0, "fp16": 1}[dtype]


def decode(bits: np.ndarray, dtype: str, mutation: int = 0) -> np.ndarray:
    """Exact fp64 values of bf16/fp16 bit patterns (element by element, through the C decoder)."""
    lib = _load(mutation)
    f = lib.oracle_fp16_to_f64 if dtype == "fp16" else lib.oracle_bf16_to_f64
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([f(int(h)) for h in flat], dtype=np.float64).reshape(np.shape(bits))


def ref_gemm(A, B, M: int, N: int, K: int, b_layout: str, dtype: str,
             rows: Optional[Sequence[int]] = None, with_abs: bool = True,
             mutation: int = 0, lib_file: Optional[Path] = None):
    """fp64 ``C`` (and ``S``) for the selected rows (all rows by default)."""
    lib = _load(mutation, lib_file)
    a = _bits(A).reshape(-1)
    b = _bits(B).reshape(-1)
    if a.size != M * K:
        raise ValueError("A has the wrong number of elements")
    if b.size != K * N:
        raise ValueError("B has the wrong number of elements")
    r = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    C = np.zeros((r.size, N), dtype=np.float64)
    S = np.zeros((r.size, N), dtype=np.float64) if with_abs else None
    rc = lib.oracle_gemm_rows(
        a.ctypes.data, b.ctypes.data, M, N, K, {"kn": 0, "nk": 1}[b_layout], _dtype_code(dtype),
        r.ctypes.data, r.size, C.ctypes.data, S.ctypes.data if S is not None else None)
    if rc != 0:
        raise ValueError("oracle_gemm_rows rejected its arguments")
    return C, S


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def within_tolerance(c_test: np.ndarray, c_ref: np.ndarray, s_ref: np.ndarray,
                     tol: float = TOLERANCE):
    """Elementwise ``|c_test - c_ref| <= tol * s_ref``; returns (ok, worst ratio, index)."""
    c_test = np.asarray(c_test, dtype=np.float64)
    err = np.abs(c_test - c_ref)
    bound = tol * s_ref
    bad = ~(err <= bound)          # also catches NaN
    if s_ref.size == 0:
        return True, 0.0, None
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0),
                         np.where(err == 0, 0.0, np.inf))
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    return (not bool(bad.any())), float(ratio[idx]), idx


def time_rows(A, B, M, N, K, b_layout, dtype, rows) -> float:
    """Wall seconds for the oracle on a row sample (C and S both computed)."""
    t0 = time.perf_counter()
    ref_gemm(A, B, M, N, K, b_layout, dtype, rows=rows, with_abs=True)
    return time.perf_counter() - t0
