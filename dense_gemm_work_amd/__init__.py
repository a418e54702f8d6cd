"""Python binding of the MI355X DP / Split-K / Stream-K GEMM library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libdgw_gemm.so`` (built in-tree by ``dense_gemm_work_amd/build.py``).
The functions carry the names of the C entry points in ``include/gemm.h``:

* ``gemm(A, B, C, M, N, K, layout, mode, splits)`` -- raw device pointers.
* ``gemm_ex(args)``, ``gemm_plan(...)``, ``gemm_plan_batched(...)``, ``gemm_workspace_size(...)``,
  ``gemm_unit_range(...)``,
  ``gemm_set_stream``, ``gemm_sync_status``, ``gemm_release``,
  ``gemm_last_error``, ``gemm_num_cus``, ``gemm_version``.

``gemm_tensors(a, b, c, ...)`` is the torch-facing convenience (``matmul(a, b)``
returns a new fp32 tensor): it checks the
tensors' device, dtype, shape and contiguity on the host, passes their data
pointers and torch's current HIP stream, and raises ``GemmError`` on a
negative status.  Importing this module fails loudly when the library has not
been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
from pathlib import Path
from typing import Optional

__all__ = [
    "GemmError", "GemmPlan", "GemmArgs", "GemmGroup", "gemm", "gemm_ex", "gemm_ex_noalloc", "gemm_grouped",
    "gemm_plan", "gemm_plan_batched", "gemm_plan_grouped", "group_array", "gemm_grouped_tensors",
    "gemm_workspace_size", "gemm_unit_range",
    "gemm_set_stream", "gemm_sync_status", "gemm_release", "gemm_last_error", "gemm_num_cus",
    "gemm_version", "gemm_tensors", "matmul", "plan_dict", "library_path",
]

_PKG = Path(__file__).resolve().parent
_LIB_PATH = _PKG / "libdgw_gemm.so"

# ---- constants (include/gemm.h) ------------------------------------------------
GEMM_OK = 0
GEMM_ERR_INVALID = -1
GEMM_ERR_UNSUPPORTED = -2
GEMM_ERR_WORKSPACE = -3
GEMM_ERR_HIP = -4
GEMM_ERR_TIMEOUT = -5

GEMM_B_KN = 0x00
GEMM_B_NK = 0x01
GEMM_BF16 = 0x00
GEMM_FP16 = 0x10

GEMM_HEURISTIC = 0x0
GEMM_DP = 0x1
GEMM_SPLITK = 0x2
GEMM_STREAMK = 0x3
GEMM_DETERMINISTIC = 0x000
GEMM_ATOMIC = 0x100
GEMM_TWO_PASS = 0x200
GEMM_TILE_128x128 = 0x0000
GEMM_TILE_256x128 = 0x1000
GEMM_TILE_64x128 = 0x2000
GEMM_TILE_AUTO = 0x3000
TILES = {"128x128": GEMM_TILE_128x128, "256x128": GEMM_TILE_256x128, "64x128": GEMM_TILE_64x128,
         "auto": GEMM_TILE_AUTO}

GEMM_EPI_ALPHA_BETA = 0x01
GEMM_EPI_BIAS = 0x02
GEMM_EPI_RELU = 0x10
GEMM_EPI_GELU = 0x20
ACTIVATIONS = {"none": 0, "relu": GEMM_EPI_RELU, "gelu": GEMM_EPI_GELU}

GEMM_DEBUG_NO_PUBLISH = 0x1
GEMM_DEBUG_IN_LAUNCH = 0x4
GEMM_DEBUG_TILE_DP = 0x8
GEMM_DEBUG_HYBRID_SPLIT = 0x10
GEMM_DEBUG_ZERO_PARTIAL = 0x20
GEMM_DEBUG_SPLITK_BANDS = 0x40

GEMM_BM = 128
GEMM_NOALLOC_MAX_BYTES = 32 * 1024 * 1024 + 256 * 1024   # gemm_ex_noalloc scratch per device
GEMM_BN = 128
GEMM_BK = 64

MODES = {"heuristic": GEMM_HEURISTIC, "dp": GEMM_DP, "splitk": GEMM_SPLITK, "streamk": GEMM_STREAMK}
DECISION_NAMES = {GEMM_DP: "DataParallel", GEMM_SPLITK: "SplitK", GEMM_STREAMK: "StreamK"}


class GemmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"gemm status {status}: {message}")
        self.status = status


class GemmPlan(ctypes.Structure):
    _fields_ = [
        ("decision", ctypes.c_int32), ("atomic", ctypes.c_int32),
        ("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64), ("tiles", ctypes.c_int64),
        ("ipt", ctypes.c_int64), ("full_waves", ctypes.c_int64), ("total_waves", ctypes.c_int64),
        ("tail", ctypes.c_int64), ("sk_tiles", ctypes.c_int64), ("sk_units", ctypes.c_int64),
        ("dp_tiles", ctypes.c_int64), ("q", ctypes.c_int64), ("big", ctypes.c_int64),
        ("splits", ctypes.c_int32), ("max_segments", ctypes.c_int32), ("max_fold", ctypes.c_int32),
        ("two_pass", ctypes.c_int32),
        ("workers", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64), ("trace_ints", ctypes.c_int64),
        ("batch", ctypes.c_int64),
    ]


class GemmArgs(ctypes.Structure):
    _fields_ = [
        ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("layout", ctypes.c_uint32), ("mode", ctypes.c_uint32), ("splits", ctypes.c_int32),
        ("num_cus", ctypes.c_int32), ("stream", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("unit_perm", ctypes.c_void_p),
        ("trace", ctypes.c_void_p), ("trace_ints", ctypes.c_int64),
        ("spin_limit", ctypes.c_uint32), ("debug", ctypes.c_uint32),
        ("timing", ctypes.c_void_p),
        ("epilogue", ctypes.c_uint32), ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
        ("bias", ctypes.c_void_p),
        ("batch", ctypes.c_int64), ("stride_a", ctypes.c_int64), ("stride_b", ctypes.c_int64),
        ("stride_c", ctypes.c_int64),
    ]


class GemmGroup(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64)]


GEMM_MAX_GROUPS = 64


def library_path() -> Path:
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7).
    # Loading torch first makes the library bind to that one; loading the
    # library first would bring in the system runtime as a second HIP runtime
    # in the process, and torch would then not see the GPU.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not _LIB_PATH.exists():
        raise ImportError(
            f"{_LIB_PATH} is not built; run __graft_entry__.build() (or python3 "
            "dense_gemm_work_amd/build.py) first -- there is no fallback implementation")
    lib = ctypes.CDLL(str(_LIB_PATH))
    i64, u32, i32, vp = ctypes.c_int64, ctypes.c_uint32, ctypes.c_int32, ctypes.c_void_p
    lib.gemm.restype = ctypes.c_int
    lib.gemm.argtypes = [vp, vp, vp, i64, i64, i64, u32, u32, i32]
    lib.gemm_ex.restype = ctypes.c_int
    lib.gemm_ex.argtypes = [ctypes.POINTER(GemmArgs)]
    lib.gemm_ex_noalloc.restype = ctypes.c_int
    lib.gemm_ex_noalloc.argtypes = [ctypes.POINTER(GemmArgs)]
    lib.gemm_plan.restype = ctypes.c_int
    lib.gemm_plan.argtypes = [i64, i64, i64, u32, u32, i32, i32, ctypes.POINTER(GemmPlan)]
    lib.gemm_workspace_size.restype = ctypes.c_int64
    lib.gemm_workspace_size.argtypes = [i64, i64, i64, i64, u32, u32, i32, i32]
    lib.gemm_plan_batched.restype = ctypes.c_int
    lib.gemm_plan_batched.argtypes = [i64, i64, i64, i64, u32, u32, i32, i32, ctypes.POINTER(GemmPlan)]
    lib.gemm_grouped.restype = ctypes.c_int
    lib.gemm_grouped.argtypes = [ctypes.POINTER(GemmArgs), ctypes.POINTER(GemmGroup), i32]
    lib.gemm_plan_grouped.restype = ctypes.c_int
    lib.gemm_plan_grouped.argtypes = [ctypes.POINTER(GemmGroup), i32, i64, u32, u32, i32, i32, ctypes.POINTER(GemmPlan)]
    lib.gemm_unit_range.restype = ctypes.c_int
    lib.gemm_unit_range.argtypes = [ctypes.POINTER(GemmPlan), i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.gemm_set_stream.restype = ctypes.c_int
    lib.gemm_set_stream.argtypes = [vp]
    lib.gemm_sync_status.restype = ctypes.c_int
    lib.gemm_sync_status.argtypes = [vp]
    lib.gemm_release.restype = None
    lib.gemm_release.argtypes = []
    lib.gemm_last_error.restype = ctypes.c_char_p
    lib.gemm_last_error.argtypes = []
    lib.gemm_num_cus.restype = ctypes.c_int32
    lib.gemm_num_cus.argtypes = []
    lib.gemm_version.restype = ctypes.c_int32
    lib.gemm_version.argtypes = []
    return lib


_lib = _load()


def _check(status: int) -> int:
    if status < 0:
        raise GemmError(status, gemm_last_error())
    return status


# ---- C entry points, same names ----------------------------------------------------
def gemm(A: int, B: int, C: int, M: int, N: int, K: int, layout: int, mode: int, splits: int) -> int:
    """Raw call on device pointers; returns the status (no exception)."""
    return _lib.gemm(A, B, C, M, N, K, layout, mode, splits)


def gemm_ex(args: GemmArgs) -> int:
    return _lib.gemm_ex(ctypes.byref(args))


def gemm_ex_noalloc(args: GemmArgs) -> int:
    """gemm_ex on the library's fixed per-device scratch array (no allocation)."""
    return _lib.gemm_ex_noalloc(ctypes.byref(args))


def gemm_plan(M: int, N: int, K: int, layout: int, mode: int, splits: int, num_cus: int) -> GemmPlan:
    p = GemmPlan()
    _check(_lib.gemm_plan(M, N, K, layout, mode, splits, num_cus, ctypes.byref(p)))
    return p


def gemm_plan_batched(M: int, N: int, K: int, batch: int, layout: int, mode: int, splits: int,
                      num_cus: int) -> GemmPlan:
    p = GemmPlan()
    _check(_lib.gemm_plan_batched(M, N, K, batch, layout, mode, splits, num_cus, ctypes.byref(p)))
    return p


def gemm_workspace_size(M: int, N: int, K: int, layout: int, mode: int, splits: int, num_cus: int,
                        batch: int = 1) -> int:
    return _check(int(_lib.gemm_workspace_size(M, N, K, batch, layout, mode, splits, num_cus)))


def _group_array(groups):
    """A ctypes array of GemmGroup from (A, B, C, M, N) tuples or GemmGroup items."""
    arr = (GemmGroup * max(len(groups), 1))()
    for i, g in enumerate(groups):
        arr[i] = g if isinstance(g, GemmGroup) else GemmGroup(*g)
    return arr


def gemm_grouped(common: GemmArgs, groups) -> int:
    """gemm_grouped(): ``groups`` a sequence of (A, B, C, M, N) (device addresses),
    or an array from ``group_array`` (built once, passed as it is)."""
    arr = groups if isinstance(groups, ctypes.Array) else _group_array(groups)
    return _lib.gemm_grouped(ctypes.byref(common), arr, len(groups))


def group_array(groups):
    """A reusable ctypes array of GemmGroup for gemm_grouped()."""
    return _group_array(groups)


def gemm_plan_grouped(shapes, K: int, layout: int, mode: int, splits: int, num_cus: int) -> GemmPlan:
    """gemm_plan_grouped() for problems of the given (M, N) shapes."""
    arr = _group_array([(None, None, None, M, N) for M, N in shapes])
    p = GemmPlan()
    _check(_lib.gemm_plan_grouped(arr, len(shapes), K, layout, mode, splits, num_cus, ctypes.byref(p)))
    return p


def gemm_unit_range(plan: GemmPlan, unit: int):
    b, e = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.gemm_unit_range(ctypes.byref(plan), unit, ctypes.byref(b), ctypes.byref(e)))
    return b.value, e.value


def gemm_set_stream(stream: Optional[int]) -> int:
    return _lib.gemm_set_stream(stream or None)


def gemm_sync_status(stream: Optional[int] = None) -> int:
    return _lib.gemm_sync_status(stream or None)


def gemm_release() -> None:
    _lib.gemm_release()


def gemm_last_error() -> str:
    return (_lib.gemm_last_error() or b"").decode()


def gemm_num_cus() -> int:
    return int(_lib.gemm_num_cus())


def gemm_version() -> int:
    return int(_lib.gemm_version())


# ---- helpers ---------------------------------------------------------------------------
def plan_dict(p: GemmPlan) -> dict:
    d = {name: getattr(p, name) for name, _ in GemmPlan._fields_}
    d["decision_name"] = DECISION_NAMES.get(p.decision, str(p.decision))
    return d


def layout_word(b_layout: str, dtype: str) -> int:
    lw = {"kn": GEMM_B_KN, "nk": GEMM_B_NK}[b_layout]
    return lw | {"bf16": GEMM_BF16, "fp16": GEMM_FP16}[dtype]


def mode_word(mode: str, atomic: bool = False, two_pass: bool = False, tile: str = "128x128") -> int:
    return MODES[mode] | (GEMM_ATOMIC if atomic else 0) | (GEMM_TWO_PASS if two_pass else 0) | TILES[tile]


def _matrix_strides(name: str, t, rows: int, cols: int):
    """(batch entries or None, element stride between entries) of a row-major
    matrix or a batch of them (``[rows, cols]`` or ``[batch, rows, cols]``)."""
    if t.dim() == 2:
        if tuple(t.shape) != (rows, cols):
            raise ValueError(f"{name} must be [{rows}, {cols}]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return None, 0
    if t.dim() != 3 or tuple(t.shape[1:]) != (rows, cols):
        raise ValueError(f"{name} must be [{rows}, {cols}] or [batch, {rows}, {cols}]")
    if rows * cols == 0:
        # an empty entry (K == 0 operands, an empty C) is never read or written:
        # its strides carry no layout (torch gives such tensors arbitrary ones)
        return t.shape[0], 0
    if (cols > 1 and t.stride(2) != 1) or (rows > 1 and t.stride(1) != cols):
        raise ValueError(f"{name}: every batch entry must be a contiguous row-major matrix")
    return t.shape[0], (t.stride(0) if t.shape[0] > 1 else 0)


def gemm_tensors(a, b, c, b_layout: str = "kn", mode: str = "heuristic", splits: int = 0,
                 atomic: bool = False, num_cus: int = 0, unit_perm=None, trace=None,
                 workspace=None, spin_limit: int = 0, debug: int = 0, timing=None,
                 stream=None, two_pass: bool = False, alpha: Optional[float] = None,
                 beta: Optional[float] = None, bias=None, act: str = "none", noalloc: bool = False,
                 tile: str = "128x128") -> None:
    """``c[M,N] = a[M,K] . b`` (b [K,N]) or ``a . b^T`` (b [N,K]) on torch tensors.

    Batched: c ``[batch, M, N]``; a and b ``[batch, ...]`` or 2-D (one matrix
    shared by every entry); each entry a contiguous row-major matrix, entries at
    any stride (the tensors' own).
    With ``alpha``/``beta``/``bias``/``act`` the call fuses the epilogue
    ``c = act(alpha a.b + beta c + bias)`` (bias: contiguous fp32 [N] device tensor;
    act: "none", "relu" or "gelu").
    a, b: bf16/fp16 tensors on one HIP device; c: fp32.
    unit_perm / trace / workspace / timing: optional int32 / int32 / any-dtype / int64
    device tensors (see gemm_args_t in include/gemm.h).
    Enqueues on ``stream`` (a torch.cuda.Stream) or torch's current stream.
    ``noalloc``: call gemm_ex_noalloc (no workspace argument allowed).
    ``tile``: "128x128", "256x128" (Stream-K only), "64x128" or "auto" (the library
    picks one of them, GEMM_TILE_AUTO).
    """
    import torch

    if c.dim() not in (2, 3) or a.dim() not in (2, 3) or b.dim() not in (2, 3):
        raise ValueError("a, b and c must be 2-D (or 3-D batches)")
    if a.dtype not in (torch.bfloat16, torch.float16) or b.dtype != a.dtype:
        raise TypeError("a and b must both be bf16 or both fp16")
    if c.dtype != torch.float32:
        raise TypeError("c must be fp32")
    for name, t in (("a", a), ("b", b), ("c", c)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
    if not (a.device == b.device == c.device):
        raise ValueError("a, b and c must be on one device")
    M, K = a.shape[-2], a.shape[-1]
    if b_layout == "kn":
        N = b.shape[-1]
        b_rows, b_cols = K, N
    elif b_layout == "nk":
        N = b.shape[-2]
        b_rows, b_cols = N, K
    else:
        raise ValueError("b_layout must be 'kn' or 'nk'")
    batch_c, sc = _matrix_strides("c", c, M, N)
    batch_a, sa = _matrix_strides("a", a, M, K)
    batch_b, sb = _matrix_strides("b", b, b_rows, b_cols)
    batch = batch_c or 1
    for name, n in (("a", batch_a), ("b", batch_b)):
        if n is not None and n != batch and n != 1:
            raise ValueError(f"{name} has {n} batch entries, c has {batch}")
    if batch_c is None and (batch_a or 1) * (batch_b or 1) > 1:
        raise ValueError("a batched a or b needs a batched c [batch, M, N]")
    dtype = "bf16" if a.dtype == torch.bfloat16 else "fp16"
    args = GemmArgs()
    args.A, args.B, args.C = a.data_ptr(), b.data_ptr(), c.data_ptr()
    args.M, args.N, args.K = M, N, K
    args.layout = layout_word(b_layout, dtype)
    args.mode = mode_word(mode, atomic, two_pass, tile)
    args.splits = splits
    args.num_cus = num_cus
    if batch > 1:
        args.batch = batch
        args.stride_a, args.stride_b, args.stride_c = sa, sb, (sc if sc else M * N)
    with torch.cuda.device(a.device):
        s = stream if stream is not None else torch.cuda.current_stream(a.device)
        args.stream = s.cuda_stream
        if unit_perm is not None:
            if unit_perm.dtype != torch.int32 or not unit_perm.is_cuda or not unit_perm.is_contiguous():
                raise TypeError("unit_perm must be a contiguous int32 device tensor")
            args.unit_perm = unit_perm.data_ptr()
        if trace is not None:
            if trace.dtype != torch.int32 or not trace.is_cuda or not trace.is_contiguous():
                raise TypeError("trace must be a contiguous int32 device tensor")
            args.trace = trace.data_ptr()
            args.trace_ints = trace.numel()
        if workspace is not None:
            args.workspace = workspace.data_ptr()
            args.workspace_bytes = workspace.numel() * workspace.element_size()
        if timing is not None:
            if timing.dtype != torch.int64 or not timing.is_cuda or not timing.is_contiguous():
                raise TypeError("timing must be a contiguous int64 device tensor")
            args.timing = timing.data_ptr()
        args.spin_limit = spin_limit
        args.debug = debug
        word = ACTIVATIONS[act]
        if alpha is not None or beta is not None:
            word |= GEMM_EPI_ALPHA_BETA
            args.alpha = 1.0 if alpha is None else float(alpha)
            args.beta = 0.0 if beta is None else float(beta)
        if bias is not None:
            if bias.dtype != torch.float32 or not bias.is_cuda or not bias.is_contiguous() or \
                    tuple(bias.shape) != (N,):
                raise TypeError("bias must be a contiguous fp32 [N] device tensor")
            word |= GEMM_EPI_BIAS
            args.bias = bias.data_ptr()
        args.epilogue = word
        _check(gemm_ex_noalloc(args) if noalloc else gemm_ex(args))


def gemm_grouped_tensors(problems, b_layout: str = "kn", mode: str = "heuristic", splits: int = 0,
                         atomic: bool = False, two_pass: bool = False, num_cus: int = 0, trace=None,
                         workspace=None, spin_limit: int = 0, debug: int = 0, timing=None, unit_perm=None,
                         stream=None, tile: str = "128x128") -> None:
    """``c_g = a_g . b_g`` (b [K,N]) or ``a_g . b_g^T`` (b [N,K]) for every (a_g, b_g, c_g)
    in ``problems`` as one grouped call: 2-D contiguous tensors on one device,
    one K and one 16-bit dtype for all, each problem its own M and N."""
    import torch

    if not 1 <= len(problems) <= GEMM_MAX_GROUPS:
        raise ValueError(f"a grouped call takes 1..{GEMM_MAX_GROUPS} problems")
    a0 = problems[0][0]
    K = a0.shape[-1]
    dtype = a0.dtype
    if dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("a and b must be bf16 or fp16")
    groups = []
    for i, (a, b, c) in enumerate(problems):
        if a.dim() != 2 or b.dim() != 2 or c.dim() != 2:
            raise ValueError(f"problem {i}: a, b and c must be 2-D")
        if a.dtype != dtype or b.dtype != dtype or c.dtype != torch.float32:
            raise TypeError(f"problem {i}: a and b of the first problem's dtype, c fp32")
        if not (a.is_cuda and b.is_cuda and c.is_cuda and a.device == b.device == c.device == a0.device):
            raise ValueError(f"problem {i}: tensors must be on the first problem's device")
        if not (a.is_contiguous() and b.is_contiguous() and c.is_contiguous()):
            raise ValueError(f"problem {i}: tensors must be contiguous")
        M = a.shape[0]
        if a.shape[1] != K:
            raise ValueError(f"problem {i}: K = {a.shape[1]}, the call's K is {K}")
        N = b.shape[1] if b_layout == "kn" else b.shape[0]
        if (b_layout == "kn" and b.shape[0] != K) or (b_layout == "nk" and b.shape[1] != K):
            raise ValueError(f"problem {i}: b does not match K = {K}")
        if tuple(c.shape) != (M, N):
            raise ValueError(f"problem {i}: c must be [{M}, {N}]")
        groups.append((a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N))
    args = GemmArgs()
    args.K = K
    args.layout = layout_word(b_layout, "bf16" if dtype == torch.bfloat16 else "fp16")
    args.mode = mode_word(mode, atomic, two_pass, tile)
    args.splits = splits
    args.num_cus = num_cus
    with torch.cuda.device(a0.device):
        s = stream if stream is not None else torch.cuda.current_stream(a0.device)
        args.stream = s.cuda_stream
        if trace is not None:
            args.trace, args.trace_ints = trace.data_ptr(), trace.numel()
        if timing is not None:
            args.timing = timing.data_ptr()
        if unit_perm is not None:
            args.unit_perm = unit_perm.data_ptr()
        if workspace is not None:
            args.workspace = workspace.data_ptr()
            args.workspace_bytes = workspace.numel() * workspace.element_size()
        args.spin_limit = spin_limit
        args.debug = debug
        _check(gemm_grouped(args, groups))


def matmul(a, b, b_layout: str = "kn", out=None, alpha: Optional[float] = None, beta: Optional[float] = None,
           bias=None, act: str = "none", mode: str = "heuristic", splits: int = 0, atomic: bool = False):
    """``a . b`` (or ``a . b^T`` with b_layout "nk") as a new fp32 tensor, or into ``out``.

    2-D operands, or 3-D batches (``a`` or ``b`` may be 2-D and shared); bf16 or
    fp16 in, fp32 out.  ``alpha``, ``beta``, ``bias`` and ``act`` fuse the
    epilogue ``act(alpha a.b + beta out + bias)`` (``beta`` needs ``out``).
    """
    import torch

    M = a.shape[-2]
    N = b.shape[-1] if b_layout == "kn" else b.shape[-2]
    batch = max(a.shape[0] if a.dim() == 3 else 1, b.shape[0] if b.dim() == 3 else 1)
    if out is None:
        if beta:
            raise ValueError("beta != 0 needs out (the prior C)")
        shape = (batch, M, N) if (a.dim() == 3 or b.dim() == 3) else (M, N)
        out = torch.empty(shape, dtype=torch.float32, device=a.device)
    gemm_tensors(a, b, out, b_layout=b_layout, mode=mode, splits=splits, atomic=atomic, alpha=alpha, beta=beta,
                 bias=bias, act=act)
    return out
