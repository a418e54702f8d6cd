"""Host-side tests of the C-ABI library: it loads, exports every entry point that
include/gemm.h declares, rejects bad arguments before touching a GPU, and its
planner agrees with the CPU schedule simulator (oracle/schedule.py)."""
import ctypes
import importlib.util
import itertools
import re
import subprocess
import sys
from pathlib import Path

import pytest

from oracle import schedule as sch

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "gemm.h"


@pytest.fixture(scope="module")
def dg():
    # the build script is loaded from its file: importing the package binds the
    # library, which may predate a symbol the binding asks for
    spec = importlib.util.spec_from_file_location("_dgw_hip_build", ROOT / "dense_gemm_work_amd" / "build.py")
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    if b.is_stale():
        b.build()
    import dense_gemm_work_amd as dg

    return dg


def _declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_core_entry_points():
    names = _declared_functions()
    for n in ("gemm", "gemm_ex", "gemm_plan", "gemm_workspace_size", "gemm_unit_range", "gemm_set_stream",
              "gemm_sync_status", "gemm_release", "gemm_last_error", "gemm_num_cus", "gemm_version"):
        assert n in names


def test_library_exports_every_declared_symbol(dg):
    lib = ctypes.CDLL(str(dg.library_path()))
    for name in _declared_functions():
        assert hasattr(lib, name), f"{name} declared in gemm.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", str(dg.library_path())],
                         capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in _declared_functions():
        assert name in exported


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "gemm.h"\nint main(void){gemm_plan_t p; gemm_args_t a; (void)p; (void)a;'
                   ' return gemm_version() == 2 ? 0 : 1;}\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-c", f"-I{HEADER.parent}", str(src),
                        "-o", str(tmp_path / "t.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_version(dg):
    assert dg.gemm_version() == 2


def test_struct_sizes_match_c(dg, tmp_path):
    src = tmp_path / "s.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "gemm.h"\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(gemm_plan_t), sizeof(gemm_args_t),'
                   ' offsetof(gemm_args_t, stream), offsetof(gemm_plan_t, trace_ints),'
                   ' offsetof(gemm_args_t, epilogue), offsetof(gemm_args_t, bias)); return 0;}\n')
    exe = tmp_path / "s"
    subprocess.run(["gcc", f"-I{HEADER.parent}", str(src), "-o", str(exe)], check=True)
    got = subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()
    assert int(got[0]) == ctypes.sizeof(dg.GemmPlan)
    assert int(got[1]) == ctypes.sizeof(dg.GemmArgs)
    assert int(got[2]) == dg.GemmArgs.stream.offset
    assert int(got[3]) == dg.GemmPlan.trace_ints.offset
    assert int(got[4]) == dg.GemmArgs.epilogue.offset
    assert int(got[5]) == dg.GemmArgs.bias.offset


# -- planner vs simulator -------------------------------------------------------------
def _compare(dg, M, N, K, mode, splits, cus, atomic=False, tile="128x128"):
    mw = dg.mode_word(mode, atomic, tile=tile)
    p = dg.gemm_plan(M, N, K, dg.GEMM_B_KN | dg.GEMM_BF16, mw, splits, cus)
    s = sch.plan_schedule(M, N, K, mode, splits, sms=cus, bm=int(tile.split("x")[0]))
    assert dg.DECISION_NAMES[p.decision] == s.kind
    assert (p.tiles_m, p.tiles_n, p.ipt) == (s.tiles_m, s.tiles_n, s.ipt)
    w = sch.wave_stats(s.tiles, cus)
    assert (p.total_waves, p.tail) == (w.waves, w.tail)
    if s.kind == "StreamK":
        assert (p.sk_units, p.sk_tiles, p.dp_tiles, p.q, p.big) == (s.units, s.sk_tiles, s.dp_tiles, s.q, s.big)
        bounds = sch.unit_ranges(s.sk_tiles * s.ipt, s.units)
        for u in {0, s.units // 2, s.units - 1}:
            assert dg.gemm_unit_range(p, u) == bounds[u]
        segs = [x for x in s.segments if x.unit < s.units]
        per_unit = {}
        for x in segs:
            per_unit[x.unit] = per_unit.get(x.unit, 0) + 1
        assert max(per_unit.values(), default=0) <= p.max_segments
        assert sch.max_units_per_tile(segs) <= p.max_fold
    elif s.kind == "SplitK":
        assert p.splits == s.splits
    return p, s


@pytest.mark.parametrize("name,M,N,K,mode,splits,kind", [
    ("c1", 256, 512, 2048, "streamk", 32, "StreamK"),
    ("c2a", 96, 512, 2048, "splitk", 8, "SplitK"),
    ("c2b", 256, 512, 2048, "splitk", 2, "SplitK"),
    ("c3", 2048, 2176, 4096, "heuristic", 0, "StreamK"),
    ("c4", 8192, 8192, 8192, "heuristic", 0, "DataParallel"),
    ("c5", 1536, 1536, 16384, "streamk", 0, "StreamK"),
])
def test_workload_plans(dg, name, M, N, K, mode, splits, kind):
    p, s = _compare(dg, M, N, K, mode, splits, 256)
    assert s.kind == kind
    if name == "c3":
        assert (p.sk_units, p.sk_tiles, p.q) == (256, 272, 68)
    if name == "c5":
        assert (p.sk_units, p.q) == (256, 144)
    if name == "c1":
        assert p.q == 8


def test_heuristic_sweep_matches_simulator(dg):
    # brute-force sweep: M, N multiples of 32 up to 4096, K up to 4096, several CU counts
    ms = [32, 96, 128, 160, 640, 1024, 1536, 2048, 2176, 3840, 4096]
    ks = [64, 256, 512, 576, 2048, 4096]
    for cus in (4, 108, 132, 148, 256):
        for M, N, K in itertools.product(ms, ms, ks):
            p = dg.gemm_plan(M, N, K, dg.GEMM_B_KN | dg.GEMM_BF16, dg.GEMM_HEURISTIC, 0, cus)
            tm, tn = sch.tile_grid(M, N)
            d = sch.decide(tm * tn, sch.cdiv(K, 64), cus)
            assert dg.DECISION_NAMES[p.decision] == d.kind, (M, N, K, cus)
            if d.kind == "StreamK":
                assert (p.sk_tiles, p.sk_units) == (d.sk_tiles, d.sk_units)
            if d.kind == "SplitK":
                assert p.splits == d.splits


def test_printed_table_decisions(dg):
    # the decisions printed in the book chapter's Case 2 table
    for (M, N, K, cus, kind, skt, units) in [(1536, 1536, 4096, 132, "StreamK", 144, 132),
                                            (128, 4096, 4096, 132, "StreamK", 32, 132),
                                            (3840, 3840, 4096, 148, "StreamK", 160, 148),
                                            (4096, 4096, 4096, 132, "DataParallel", 0, 0)]:
        p = dg.gemm_plan(M, N, K, 0, dg.GEMM_HEURISTIC, 0, cus)
        assert dg.DECISION_NAMES[p.decision] == kind
        if kind == "StreamK":
            assert (p.sk_tiles, p.sk_units) == (skt, units)


def test_streamk_unit_ranges_cover(dg):
    for tiles_m, ipt, units in [(1, 3, 7), (2, 5, 3), (5, 9, 64), (3, 1, 2)]:
        M, K = tiles_m * 128, ipt * 64
        p = dg.gemm_plan(M, 128, K, 0, dg.GEMM_STREAMK, units, 256)
        bounds = [dg.gemm_unit_range(p, u) for u in range(units)]
        assert bounds == sch.unit_ranges(tiles_m * ipt, units)


def test_ragged_shapes_plan(dg):
    p, s = _compare(dg, 300, 200, 200, "streamk", 5, 256)
    assert (p.tiles_m, p.tiles_n, p.ipt) == (3, 2, 4)
    _compare(dg, 1000, 1000, 1000, "heuristic", 0, 256)
    _compare(dg, 130, 136, 72, "splitk", 2, 256)


# -- validation before any GPU work -----------------------------------------------------
def test_plan_rejects_bad_arguments(dg):
    bad = [
        dict(M=-1), dict(layout=0x2), dict(layout=0x20), dict(mode=0x7), dict(mode=0x400),
        dict(mode=dg.GEMM_DP, splits=2), dict(mode=dg.GEMM_SPLITK, splits=0),
        dict(mode=dg.GEMM_SPLITK, splits=3), dict(mode=dg.GEMM_DP | dg.GEMM_ATOMIC),
        dict(mode=dg.GEMM_STREAMK | dg.GEMM_ATOMIC | dg.GEMM_TWO_PASS), dict(mode=dg.GEMM_DP | dg.GEMM_TWO_PASS),
        dict(mode=dg.GEMM_SPLITK | dg.GEMM_ATOMIC | dg.GEMM_TWO_PASS, splits=2),
        dict(cus=0),
    ]
    for b in bad:
        args = dict(M=256, N=256, K=2048, layout=0, mode=dg.GEMM_DP, splits=0, cus=256)
        args.update(b)
        with pytest.raises(dg.GemmError) as ei:
            dg.gemm_plan(args["M"], args["N"], args["K"], args["layout"], args["mode"], args["splits"],
                         args["cus"])
        assert ei.value.status == dg.GEMM_ERR_INVALID, b
    for b in [dict(K=100), dict(N=100), dict(K=(1 << 22) + 8), dict(N=(1 << 22) + 8)]:
        args = dict(M=256, N=256, K=2048)
        args.update(b)
        with pytest.raises(dg.GemmError) as ei:
            dg.gemm_plan(args["M"], args["N"], args["K"], 0, dg.GEMM_DP, 0, 256)
        assert ei.value.status == dg.GEMM_ERR_UNSUPPORTED
    # [N,K] weights only need K % 8 == 0
    dg.gemm_plan(256, 100, 2048, dg.GEMM_B_NK, dg.GEMM_DP, 0, 256)


def test_gemm_rejects_before_launch(dg):
    # host-detectable errors return before any HIP call (no GPU needed)
    assert dg.gemm(0, 0, 0, 256, 256, 256, 0, dg.GEMM_DP, 0) == dg.GEMM_ERR_INVALID
    assert "non-null" in dg.gemm_last_error()
    assert dg.gemm(16, 32, 48, 256, 256, 256, 0, dg.GEMM_SPLITK, 3) == dg.GEMM_ERR_INVALID
    assert dg.gemm(8, 32, 1 << 40, 256, 256, 256, 0, dg.GEMM_DP, 0) == dg.GEMM_ERR_UNSUPPORTED
    # C overlapping A
    assert dg.gemm(1 << 20, 1 << 30, (1 << 20) + 4096, 256, 256, 256, 0, dg.GEMM_DP, 0) == dg.GEMM_ERR_INVALID
    # empty problems are a no-op, even with null pointers
    assert dg.gemm(0, 0, 0, 0, 256, 256, 0, dg.GEMM_DP, 0) == dg.GEMM_OK
    assert dg.gemm(0, 0, 0, 256, 0, 256, 0, dg.GEMM_DP, 0) == dg.GEMM_OK


def _epi_args(dg, epilogue, bias=0, M=256, N=256, K=256, C=1 << 30):
    a = dg.GemmArgs()
    a.A, a.B, a.C = 1 << 20, 1 << 24, C
    a.M, a.N, a.K = M, N, K
    a.mode = dg.GEMM_DP
    a.epilogue = epilogue
    a.bias = bias or None
    return a


def test_epilogue_rejects_before_launch(dg):
    # host-detectable epilogue errors return before any HIP call (no GPU needed)
    bad = [
        (0x4, 0, "unknown bits"),
        (0x100, 0, "unknown bits"),
        (dg.GEMM_EPI_RELU | dg.GEMM_EPI_GELU, 0, "exclude"),
        (dg.GEMM_EPI_BIAS, 0, "exactly when"),
        (dg.GEMM_EPI_ALPHA_BETA, 1 << 28, "exactly when"),
    ]
    for word, bias, text in bad:
        assert dg.gemm_ex(_epi_args(dg, word, bias)) == dg.GEMM_ERR_INVALID, (word, bias)
        assert text in dg.gemm_last_error()
        # checked before the early return of an empty problem
        assert dg.gemm_ex(_epi_args(dg, word, bias, M=0)) == dg.GEMM_ERR_INVALID
    # bias alignment and overlap with C
    assert dg.gemm_ex(_epi_args(dg, dg.GEMM_EPI_BIAS, (1 << 28) + 4)) == dg.GEMM_ERR_UNSUPPORTED
    assert "16-byte" in dg.gemm_last_error()
    assert dg.gemm_ex(_epi_args(dg, dg.GEMM_EPI_BIAS, (1 << 30) + 1024)) == dg.GEMM_ERR_INVALID
    assert "overlap" in dg.gemm_last_error()
    # a valid epilogue on an empty problem is a no-op
    assert dg.gemm_ex(_epi_args(dg, dg.GEMM_EPI_BIAS | dg.GEMM_EPI_GELU, 1 << 28, N=0)) == dg.GEMM_OK


def test_workspace_size_matches_plan(dg):
    for M, N, K, mode, splits in [(2048, 2176, 4096, dg.GEMM_HEURISTIC, 0), (96, 512, 2048, dg.GEMM_SPLITK, 8),
                                  (256, 512, 2048, dg.GEMM_STREAMK, 32), (8192, 8192, 8192, dg.GEMM_DP, 0),
                                  (1536, 1536, 16384, dg.GEMM_STREAMK | dg.GEMM_ATOMIC, 0)]:
        p = dg.gemm_plan(M, N, K, 0, mode, splits, 256)
        assert dg.gemm_workspace_size(M, N, K, 0, mode, splits, 256) == p.workspace_bytes
    # Split-K partials [S, M, N] fp32 plus the control block
    p = dg.gemm_plan(96, 512, 2048, 0, dg.GEMM_SPLITK, 8, 256)
    assert p.workspace_bytes >= 8 * 96 * 512 * 4
    with pytest.raises(dg.GemmError) as ei:
        dg.gemm_workspace_size(96, 512, 2048, 0, dg.GEMM_SPLITK, 3, 256)
    assert ei.value.status == dg.GEMM_ERR_INVALID


def test_batched_plan_and_rejections(dg):
    # the plan sees batch x tiles_m x tiles_n tiles (the simulator's batched plan)
    for M, N, K, batch, mode in [(256, 512, 2048, 6, "heuristic"), (640, 640, 2048, 2, "heuristic"),
                                 (384, 640, 1024, 3, "streamk")]:
        p = dg.gemm_plan_batched(M, N, K, batch, 0, dg.mode_word(mode), 0, 256)
        s = sch.plan_schedule(M, N, K, mode, 0, sms=256, batch=batch)
        assert p.batch == batch and p.tiles == s.tiles
        assert dg.DECISION_NAMES[p.decision] == s.kind
        assert (p.sk_units, p.sk_tiles, p.dp_tiles, p.q, p.big, p.splits) == \
            (s.units, s.sk_tiles, s.dp_tiles, s.q, s.big, s.splits)
    p = dg.gemm_plan_batched(96, 512, 2048, 4, 1, dg.GEMM_SPLITK, 8, 256)
    assert p.workspace_bytes >= 4 * 8 * 96 * 512 * 4     # partials [batch, S, M, N]
    assert dg.gemm_workspace_size(96, 512, 2048, 1, dg.GEMM_SPLITK, 8, 256, batch=4) == p.workspace_bytes
    with pytest.raises(dg.GemmError):
        dg.gemm_plan_batched(96, 512, 2048, 0, 1, dg.GEMM_SPLITK, 8, 256)
    # stride checks happen before any HIP call (fake, aligned, disjoint pointers)
    a = dg.GemmArgs()
    a.A, a.B, a.C = 1 << 20, 1 << 26, 1 << 32
    a.M, a.N, a.K = 128, 128, 64
    a.mode = dg.GEMM_DP
    a.batch = 2
    a.stride_a, a.stride_b, a.stride_c = 128 * 64, 64 * 128, 128 * 128 - 4
    assert dg.gemm_ex(a) == dg.GEMM_ERR_INVALID and "stride_c" in dg.gemm_last_error()
    a.stride_c = 128 * 128 + 2
    assert dg.gemm_ex(a) == dg.GEMM_ERR_UNSUPPORTED
    a.stride_c, a.stride_a = 128 * 128, 12
    assert dg.gemm_ex(a) == dg.GEMM_ERR_UNSUPPORTED
    # C's batch extent reaching into B
    a.stride_a, a.C = 0, (1 << 26) - 2 * 128 * 128 * 4 + 64
    assert dg.gemm_ex(a) == dg.GEMM_ERR_INVALID and "overlap" in dg.gemm_last_error()


def test_splitk_merge_modes_plan(dg):
    # deterministic Split-K adds the partials in split order, by a second kernel
    # when the whole grid fits on the CUs at once (or GEMM_TWO_PASS asks for it),
    # else by the last arriver in the launch; atomics keep no partials
    M, N, K, S = 96, 512, 2048, 8
    lw = dg.layout_word("nk", "bf16")
    auto = dg.gemm_plan(M, N, K, lw, dg.GEMM_SPLITK, S, 256)          # 4 tiles x 8 = 32 <= 256
    fold = dg.gemm_plan(M, N, K, lw, dg.GEMM_SPLITK, S, 16)           # 32 > 16 CUs
    two = dg.gemm_plan(M, N, K, lw, dg.GEMM_SPLITK | dg.GEMM_TWO_PASS, S, 16)
    atom = dg.gemm_plan(M, N, K, lw, dg.GEMM_SPLITK | dg.GEMM_ATOMIC, S, 256)
    # S = 8 on a grid that fits the CUs: in the launch (row bands); on 16 CUs the
    # grid does not fit (last arriver); the second kernel on request
    assert (auto.two_pass, fold.two_pass, two.two_pass, atom.two_pass) == (0, 0, 1, 0)
    # S < 8 on a grid that fits: the second kernel
    assert dg.gemm_plan(M, N, K, lw, dg.GEMM_SPLITK, 4, 256).two_pass == 1
    assert dg.gemm_plan(256, 512, 2048, lw, dg.GEMM_SPLITK, 2, 256).two_pass == 1
    # S >= 8 on a grid of more than half the CUs: the second kernel (32 tiles x 8
    # = 256 workgroups); at most half: in the launch (16 tiles x 8 = 128)
    assert dg.gemm_plan(128, 4096, 4096, lw, dg.GEMM_SPLITK, 8, 256).two_pass == 1
    assert dg.gemm_plan(128, 2048, 4096, lw, dg.GEMM_SPLITK, 8, 256).two_pass == 0
    assert (auto.atomic, fold.atomic, two.atomic, atom.atomic) == (0, 0, 0, 1)
    assert auto.workspace_bytes == fold.workspace_bytes == two.workspace_bytes
    assert fold.workspace_bytes - atom.workspace_bytes == S * M * N * 4
    for p in (auto, fold, two, atom):
        assert (p.decision, p.splits, p.tiles, p.ipt) == (dg.GEMM_SPLITK, S, 4, 32)
    # the large split-K arms of the wave-quantized workload stay in the launch
    big = dg.gemm_plan(2048, 2176, 4096, 0, dg.GEMM_SPLITK, 2, 256)
    assert big.two_pass == 0
    # one split: nothing to merge
    one = dg.gemm_plan(M, N, K, lw, dg.GEMM_SPLITK | dg.GEMM_TWO_PASS, 1, 256)
    assert (one.two_pass, one.atomic) == (0, 0)


def test_streamk_two_pass_plan(dg):
    # the second kernel needs two partial slots per unit (first and last segment);
    # the plan picks it when a tile can have three or more peers (short units)
    c3 = dg.gemm_plan(2048, 2176, 4096, 0, dg.GEMM_HEURISTIC, 0, 256)               # max_fold 2
    c3t = dg.gemm_plan(2048, 2176, 4096, 0, dg.GEMM_HEURISTIC | dg.GEMM_TWO_PASS, 0, 256)
    c5 = dg.gemm_plan(1536, 1536, 16384, dg.GEMM_FP16, dg.GEMM_STREAMK, 0, 256)      # max_fold 3
    c1 = dg.gemm_plan(256, 512, 2048, 0, dg.GEMM_STREAMK, 32, 256)                   # max_fold 5
    c1a = dg.gemm_plan(256, 512, 2048, 0, dg.GEMM_STREAMK | dg.GEMM_ATOMIC, 32, 256)
    assert (c3.max_fold, c5.max_fold, c1.max_fold) == (2, 3, 5)
    assert (c3.two_pass, c3t.two_pass, c5.two_pass, c1.two_pass, c1a.two_pass) == (0, 1, 0, 1, 0)
    assert c3t.workspace_bytes - c3.workspace_bytes == 256 * 128 * 128 * 4
    assert (c3t.q, c3t.big, c3t.sk_units) == (c3.q, c3.big, c3.sk_units)


def test_binding_uses_one_hip_runtime(tmp_path):
    # importing the package first must not load a second HIP runtime next to
    # torch's (torch would then not see the GPU)
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import dense_gemm_work_amd\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read()\n"
            "libs = {l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}\n"
            "print(len(libs))\n") % str(ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_heuristic_splitk_factor_divides_iterations(dg):
    # 64 tiles x 34 iterations on 256 CUs: the rule's units (256) are 4 per tile,
    # but 4 does not divide 34, so the aligned split is impossible and the units
    # run as Stream-K (simulator and planner agree); 32 iterations keep Split-K
    for K, kind, splits in ((34 * 64, "StreamK", 1), (32 * 64, "SplitK", 4)):
        p = dg.gemm_plan(1024, 1024, K, 0, dg.GEMM_HEURISTIC, 0, 256)
        d = sch.decide(64, K // 64, 256)
        assert dg.DECISION_NAMES[p.decision] == d.kind == kind
        assert p.splits == splits
        if kind == "StreamK":
            assert (p.sk_units, p.sk_tiles) == (d.sk_units, d.sk_tiles) == (256, 64)


def test_noalloc_refusals_before_any_hip_call(dg):
    # host-side refusals of gemm_ex_noalloc (no device is touched): a plan whose
    # workspace exceeds the fixed scratch array, and a caller workspace argument.
    # The pointers are never dereferenced (aligned, non-overlapping addresses).
    M = N = K = 2048
    args = dg.GemmArgs()
    args.A, args.B, args.C = 0x100000000, 0x200000000, 0x300000000
    args.M, args.N, args.K = M, N, K
    args.layout = dg.layout_word("kn", "bf16")
    args.mode = dg.GEMM_SPLITK
    args.splits = 4                      # partials [4, 2048, 2048] fp32 = 64 MiB
    args.num_cus = 256
    p = dg.gemm_plan(M, N, K, args.layout, args.mode, 4, 256)
    assert p.workspace_bytes > dg.GEMM_NOALLOC_MAX_BYTES
    assert dg.gemm_ex_noalloc(args) == dg.GEMM_ERR_WORKSPACE
    assert "at most" in dg.gemm_last_error()
    args.splits = 2
    args.workspace, args.workspace_bytes = 0x400000000, 1 << 30
    assert dg.gemm_ex_noalloc(args) == dg.GEMM_ERR_INVALID
    assert "workspace must be NULL" in dg.gemm_last_error()


@pytest.mark.parametrize("M,N,K,units,atomic", [
    (2048, 2176, 4096, 256, False),    # 8 x 17 = 136 tiles of 256 x 128, 256 units of 34 iterations
    (1536, 1536, 16384, 256, False),   # 72 tiles x 256 iterations
    (4096, 4224, 4096, 256, True),     # 528 tiles
    (300, 200, 328, 7, False),         # ragged M, N and K
    (256, 128, 128, 6, False),         # more units than iterations
])
def test_tall_tile_plans_match_simulator(dg, M, N, K, units, atomic):
    p, s = _compare(dg, M, N, K, "streamk", units, 256, atomic=atomic, tile="256x128")
    assert (p.bm, p.bn, p.bk) == (256, 128, 64)
    assert p.tiles_m == -(-M // 256) and p.two_pass == 0
    # one 256 x 128 fp32 slot (128 KiB) per unit for the turnstile, none for atomics
    data = p.workspace_bytes - (256 + -(-max(p.sk_units, 1) * 4 // 256) * 256 + -(-p.tiles * 4 // 256) * 256)
    assert data == (0 if atomic else p.sk_units * 256 * 128 * 4)


def test_tall_tile_refusals(dg):
    lw = dg.GEMM_B_KN | dg.GEMM_BF16
    for mode in ("dp", "splitk", "heuristic"):
        with pytest.raises(dg.GemmError) as ei:
            dg.gemm_plan(2048, 2176, 4096, lw, dg.mode_word(mode, tile="256x128"), 2 if mode == "splitk" else 0, 256)
        assert ei.value.status == dg.GEMM_ERR_UNSUPPORTED
    with pytest.raises(dg.GemmError) as ei:
        dg.gemm_plan(2048, 2176, 4096, lw, dg.mode_word("streamk", two_pass=True, tile="256x128"), 0, 256)
    assert ei.value.status == dg.GEMM_ERR_UNSUPPORTED


@pytest.mark.parametrize("M,N,K,mode,splits,atomic", [
    (96, 512, 2048, "splitk", 8, False),      # 2 x 4 tiles of 64 x 128 (rows 96..127 empty)
    (128, 4096, 4096, "splitk", 4, False),    # a decode-sized batch: 64 tiles, 256 workers
    (64, 4096, 4096, "heuristic", 0, False),  # 32 tiles: Stream-K or Split-K by the rule
    (128, 4096, 4096, "heuristic", 0, False),
    (256, 512, 2048, "streamk", 32, True),
    (300, 200, 328, "streamk", 7, False),     # ragged M, N and K
    (64, 128, 128, "streamk", 6, False),      # more units than iterations
    (1000, 1000, 640, "dp", 0, False),
])
def test_skinny_tile_plans_match_simulator(dg, M, N, K, mode, splits, atomic):
    p, s = _compare(dg, M, N, K, mode, splits, 256, atomic=atomic, tile="64x128")
    assert (p.bm, p.bn, p.bk) == (64, 128, 64)
    assert p.tiles_m == -(-M // 64)
    if s.kind == "StreamK" and not atomic:
        # 64 x 128 fp32 slots (32 KiB): one per unit, two with the second kernel
        data = p.workspace_bytes - (256 + -(-max(p.sk_units, 1) * 4 // 256) * 256 + -(-p.tiles * 4 // 256) * 256)
        assert data == (2 if p.two_pass else 1) * p.sk_units * 64 * 128 * 4


def test_skinny_tile_doubles_tile_rows_of_a_decode_batch(dg):
    # the book chapter's skinny case: M = 128 through a 4096-wide projection has
    # 32 tiles of 128 x 128 and 64 of 64 x 128
    lw = dg.GEMM_B_KN | dg.GEMM_BF16
    p128 = dg.gemm_plan(128, 4096, 4096, lw, dg.mode_word("dp"), 0, 256)
    p64 = dg.gemm_plan(128, 4096, 4096, lw, dg.mode_word("dp", tile="64x128"), 0, 256)
    assert (p128.tiles, p64.tiles) == (32, 64)


def test_tile_bits_beyond_the_four_shapes_are_refused(dg):
    lw = dg.GEMM_B_KN | dg.GEMM_BF16
    for extra in (0x4000, 0x8000, 0x400):
        with pytest.raises(dg.GemmError) as ei:
            dg.gemm_plan(256, 512, 2048, lw, dg.MODES["streamk"] | dg.GEMM_TILE_AUTO | extra, 0, 256)
        assert ei.value.status == dg.GEMM_ERR_INVALID


# (workload, the tile GEMM_TILE_AUTO picks on 256 CUs with the workload's own mode)
AUTO_CASES = [
    ("c1_sk32", "64x128"), ("c2a_m96_s8", "64x128"), ("c2b_m256_s2", "64x128"), ("x3_decode", "64x128"),
    ("c3_wavequant", "128x128"), ("c4_large_dp", "128x128"), ("x2_batched", "128x128"),
    ("c5_longk_fp16", "256x128"), ("x1_hybrid", "256x128"),
]


@pytest.mark.parametrize("name,tile", AUTO_CASES)
def test_auto_tile_is_the_plan_of_the_tile_it_picks(dg, name, tile):
    from workloads import WORKLOADS

    w = WORKLOADS[name]
    lw = dg.layout_word(w.b_layout, w.dtype)
    auto = dg.plan_dict(dg.gemm_plan_batched(w.M, w.N, w.K, w.batch, lw, dg.mode_word(w.mode, tile="auto"),
                                             w.splits, 256))
    # 256 x 128 tiles run as Stream-K, whatever decomposition the caller asked for
    mode = "streamk" if tile == "256x128" else w.mode
    explicit = dg.plan_dict(dg.gemm_plan_batched(w.M, w.N, w.K, w.batch, lw, dg.mode_word(mode, tile=tile),
                                                 w.splits, 256))
    assert auto == explicit
    assert auto["bm"] == int(tile.split("x")[0])


def test_auto_tile_rule_edges(dg):
    lw = dg.GEMM_B_KN | dg.GEMM_BF16
    auto = dg.mode_word("heuristic", tile="auto")

    def bm(M, N, K, mode=auto, splits=0, cus=256):
        return dg.gemm_plan(M, N, K, lw, mode, splits, cus).bm

    # 64 x 128 up to 2 T = C: 128 tiles of 128 x 128 on 256 CUs, 129 not
    assert bm(128 * 16, 128 * 8, 2048) == 64
    assert bm(128 * 129, 128, 2048) == 128
    # the same shapes on fewer CUs
    assert bm(128 * 16, 128 * 8, 2048, cus=255) == 128
    # 256 x 128 needs a Stream-K 128 x 128 plan and >= 64 iterations per unit of the taller tile:
    # 1536^2 x 16384 has 72, 1536^2 x 8192 36
    st = dg.mode_word("streamk", tile="auto")
    assert bm(1536, 1536, 16384, st) == 256
    assert bm(1536, 1536, 8192, st) == 128
    # never with GEMM_TWO_PASS, and not when the 128 x 128 plan is data-parallel or Split-K
    assert bm(1536, 1536, 16384, dg.mode_word("streamk", two_pass=True, tile="auto")) == 128
    assert bm(8192, 8192, 8192) == 128
    assert bm(1536, 1536, 16384, dg.mode_word("dp", tile="auto")) == 128
    assert bm(1536, 1536, 16384, dg.mode_word("splitk", tile="auto"), splits=2) == 128


def test_auto_tile_workspace_is_the_picked_plans(dg):
    lw = dg.GEMM_B_KN | dg.GEMM_FP16
    for M, N, K, mode, splits in [(1536, 1536, 16384, "streamk", 0), (96, 512, 2048, "splitk", 8),
                                  (2048, 2176, 4096, "heuristic", 0)]:
        auto = dg.mode_word(mode, tile="auto")
        p = dg.gemm_plan(M, N, K, lw, auto, splits, 256)
        assert dg.gemm_workspace_size(M, N, K, lw, auto, splits, 256) == p.workspace_bytes


def test_auto_tile_grouped(dg):
    lw = dg.GEMM_B_NK | dg.GEMM_BF16
    small = [(96, 512), (64, 1024), (17, 512)]        # 10 tiles of 128 x 128
    p = dg.gemm_plan_grouped(small, 2048, lw, dg.mode_word("heuristic", tile="auto"), 0, 256)
    q = dg.gemm_plan_grouped(small, 2048, lw, dg.mode_word("heuristic", tile="64x128"), 0, 256)
    assert dg.plan_dict(p) == dg.plan_dict(q) and p.bm == 64
    big = [(2048, 2048)] * 4                          # 1024 tiles
    p = dg.gemm_plan_grouped(big, 2048, lw, dg.mode_word("streamk", tile="auto"), 0, 256)
    assert p.bm == 128


GROUP_SETS = [
    [(96, 512), (0, 512), (300, 1024), (1, 8)],
    [(256, 512)] * 4,
    [(64 * i + 1, 4096) for i in range(8)],       # ragged expert batch sizes through one projection
    [(2048, 2176)] + [(128, 128)] * 3,
]


@pytest.mark.parametrize("shapes", GROUP_SETS, ids=lambda s: f"{len(s)}groups")
@pytest.mark.parametrize("mode,splits,tile", [("heuristic", 0, "128x128"), ("streamk", 0, "128x128"),
                                              ("splitk", 4, "128x128"), ("dp", 0, "64x128"),
                                              ("heuristic", 0, "64x128")])
def test_grouped_plans_match_simulator(dg, shapes, mode, splits, tile):
    K = 2048
    lw = dg.layout_word("nk", "bf16")
    p = dg.gemm_plan_grouped(shapes, K, lw, dg.mode_word(mode, tile=tile), splits, 256)
    bm = int(tile.split("x")[0])
    s = sch.plan_schedule_grouped(shapes, K, mode, splits, 256, bm=bm)
    assert dg.DECISION_NAMES[p.decision] == s.kind
    tiles = sum(-(-M // bm) * -(-N // 128) for M, N in shapes)
    assert (p.tiles, p.tiles_m, p.tiles_n, p.ipt) == (tiles, tiles, 1, K // 64)
    if s.kind == "StreamK":
        assert (p.sk_units, p.sk_tiles, p.dp_tiles, p.q, p.big) == (s.units, s.sk_tiles, s.dp_tiles, s.q, s.big)
    if s.kind == "SplitK":
        assert p.splits == s.splits
    # workspace: control words, the Split-K partials of every problem, the table
    ctrl = 256 + -(-max(p.sk_units, 1) * 4 // 256) * 256 + -(-p.tiles * 4 // 256) * 256
    table = -(-len(shapes) * 48 // 256) * 256
    if s.kind == "SplitK" and p.splits > 1:
        data = p.splits * sum(M * N for M, N in shapes) * 4
    elif s.kind == "StreamK":
        data = (2 if p.two_pass else 1) * p.sk_units * bm * 128 * 4
    else:
        data = 0
    assert p.workspace_bytes == -(-(ctrl + data) // 256) * 256 + table


def test_grouped_plan_refusals(dg):
    lw_kn, lw_nk = dg.layout_word("kn", "bf16"), dg.layout_word("nk", "bf16")
    mw = dg.mode_word("heuristic")
    for shapes, lw, status in (([], lw_nk, dg.GEMM_ERR_INVALID),
                               ([(8, 8)] * (dg.GEMM_MAX_GROUPS + 1), lw_nk, dg.GEMM_ERR_INVALID),
                               ([(8, 8), (-1, 8)], lw_nk, dg.GEMM_ERR_INVALID),
                               ([(8, 12)], lw_kn, dg.GEMM_ERR_UNSUPPORTED)):
        with pytest.raises(dg.GemmError) as ei:
            dg.gemm_plan_grouped(shapes, 2048, lw, mw, 0, 256)
        assert ei.value.status == status
    # the same shapes with B [N,K] are fine
    dg.gemm_plan_grouped([(8, 12)], 2048, lw_nk, mw, 0, 256)
    # grouped calls have no 256-row tile build
    with pytest.raises(dg.GemmError) as ei:
        dg.gemm_plan_grouped([(512, 512)], 2048, lw_nk, dg.mode_word("streamk", tile="256x128"), 0, 256)
    assert ei.value.status == dg.GEMM_ERR_UNSUPPORTED


def test_grouped_call_argument_checks_need_no_gpu(dg):
    # refusals that happen before any HIP call
    common = dg.GemmArgs()
    common.K = 256
    common.layout = dg.layout_word("nk", "bf16")
    common.M = 8   # the common arguments must not carry a problem
    assert dg.gemm_grouped(common, [(0x1000, 0x2000, 0x3000, 8, 8)]) == dg.GEMM_ERR_INVALID
    common.M = 0
    common.epilogue = dg.GEMM_EPI_ALPHA_BETA
    common.alpha = 2.0
    assert dg.gemm_grouped(common, [(0x1000, 0x2000, 0x3000, 8, 8)]) == dg.GEMM_ERR_UNSUPPORTED
    common.epilogue = 0
    assert dg.gemm_grouped(common, [(0x1001, 0x2000, 0x3000, 8, 8)]) == dg.GEMM_ERR_UNSUPPORTED   # misaligned A
    assert dg.gemm_grouped(common, [(0x1000, 0x2000, 0x1000, 8, 8)]) == dg.GEMM_ERR_INVALID       # C overlaps A
