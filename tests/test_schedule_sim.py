"""Pins of the CPU schedule simulator (oracle/schedule.py).

Values come from the pages' printed results (tests/golden/, each file cites its
table), the toy figure of the book chapter's "Mental model" section, the
structural facts printed by its Triton case, and brute force."""
import itertools

import numpy as np
from pathlib import Path

import pytest

from oracle import schedule as sch

GOLDEN = Path(__file__).resolve().parent / "golden"


def _rows(name):
    for line in (GOLDEN / name).read_text().splitlines():
        if line and not line.startswith("#"):
            yield line.split(",")


# -- book chapter, Case 1: the printed wave-quantization table ---------------
@pytest.mark.parametrize("row", list(_rows("wave_quantization.csv")), ids=lambda r: f"{r[0]}x{r[1]}-{r[2]}")
def test_wave_table(row):
    m, n, _gpu, sms, tiles, waves, last, util = row
    tm, tn = sch.tile_grid(int(m), int(n))
    w = sch.wave_stats(tm * tn, int(sms))
    assert (w.tiles, w.waves, w.tail) == (int(tiles), int(waves), int(last))
    assert f"{100 * w.util:.1f}" == util


def test_h100_144_tiles_54_5_percent():
    w = sch.wave_stats(144, 132)
    assert w.waves == 2 and w.tail == 12 and f"{w.util:.1%}" == "54.5%"


# -- book chapter, Case 2: the printed cost-model table --------------------------
@pytest.mark.parametrize("row", list(_rows("cost_model.csv")), ids=lambda r: f"{r[0]}x{r[1]}-{r[7]}")
def test_cost_table(row):
    m, n, k, sms, tiles, iters, ideal, sched, makespan, eff = row
    m, n, k, sms = int(m), int(n), int(k), int(sms)
    tm, tn = sch.tile_grid(m, n)
    T, ipt = tm * tn, sch.cdiv(k, 64)
    assert (T, ipt) == (int(tiles), int(iters))
    assert f"{sch.ideal(T, ipt, sms):.1f}" == ideal
    if sched == "dp":
        v = sch.cost_dp(T, ipt, sms)
    elif sched.startswith("splitk"):
        v = sch.cost_splitk(T, ipt, sms, int(sched[len("splitk"):]))
    elif sched == "streamk":
        v = sch.cost_streamk_shape(T, ipt, sms)
    else:
        _, kind, skt, units = sched.split(":")
        d, v = sch.cost_decided(T, ipt, sms)
        assert (d.kind, d.sk_tiles, d.sk_units) == (kind, int(skt), int(units))
    assert f"{float(v):.1f}" == makespan
    assert f"{100 * sch.ideal(T, ipt, sms) / v:.1f}" == eff


def test_cost_table_needs_big_first_split():
    # the printed Stream-K makespans reproduce only with "big units first":
    # q = ceil gives 26 instead of 29 for 128x4096, floor gives 76 instead of 78 for 1536^2
    assert sch.cost_streamk_shape(32, 64, 132, rule="big_first") == 29.0
    assert sch.cost_streamk_shape(32, 64, 132, rule="cdiv") != 29.0
    assert sch.cost_streamk_shape(144, 64, 132, rule="big_first") == 78.0
    assert sch.cost_streamk_shape(144, 64, 132, rule="floor") != 78.0


# -- book chapter, "Mental model" figure: 4 SMs, 5 tiles of 4 iterations -------
def test_toy_figure():
    tiles, ipt, sms = 5, 4, 4
    assert sch.cost_dp(tiles, ipt, sms, epi=0) == 8
    w = sch.wave_stats(tiles, sms)
    assert w.util == 0.625
    bounds = sch.unit_ranges(tiles * ipt, sms)
    assert all(e - b == 5 for b, e in bounds)               # 5 iterations per SM
    segs = sch.streamk_segments(bounds, ipt)
    assert sch.cost_streamk(segs, sms, ipt, epi=0, part=0) == 5
    first = {}
    for s in segs:
        first.setdefault(s.unit, s)
    # SM1..SM3 start with a partial tile; SM0 starts on a tile's k = 0
    assert first[0].k0 == 0
    assert all(first[u].role == sch.CONTRIB for u in (1, 2, 3))
    # with a fixup cost the makespan is 5 plus fixup
    assert sch.cost_streamk(segs, sms, ipt, epi=0, part=1) > 5


# -- book chapter, Case 3: printed structure of the Triton run -------------------
def test_triton_structure_facts():
    # 256x256x1024 with 64x64 tiles and BK=32: 16 tiles x 32 iterations = 512
    tm, tn = sch.tile_grid(256, 256, 64, 64)
    tiles, ipt = tm * tn, sch.cdiv(1024, 32)
    assert (tiles, ipt, tiles * ipt) == (16, 32, 512)
    assert sch.cdiv(512, 16) == 32 and sch.cdiv(512, 12) == 43 and sch.cdiv(512, 40) == 13
    dp = sch.streamk_segments(sch.unit_ranges(512, 16, "cdiv"), ipt)
    assert all(s.role == sch.FULL for s in dp)               # 16 units: one whole tile each
    s12 = sch.streamk_segments(sch.unit_ranges(512, 12, "cdiv"), ipt)
    assert sch.max_units_per_tile(s12) == 2                  # "up to 2 peers/tile"
    s40 = sch.streamk_segments(sch.unit_ranges(512, 40, "cdiv"), ipt)
    assert sch.max_units_per_tile(s40) == 4                  # "up to 4 peers/tile"


# -- the rule's decisions on the five workloads (256 CUs) --------------------------
def test_workload_decisions():
    d = sch.decide(272, 64, 256)          # 2048x2176x4096
    assert (d.kind, d.sk_tiles, d.sk_units) == ("StreamK", 272, 256)
    assert sch.decide(4096, 128, 256).kind == "DataParallel"   # 8192^3: 16 full waves
    d1 = sch.decide(8, 32, 256)           # 256x512x2048
    assert d1.kind == "SplitK" and d1.splits == 4
    assert sch.decide(144, 256, 256).kind == "DataParallel"    # 2*144 >= 256


@pytest.mark.parametrize("tiles,ipt,units,q,groups", [
    (8, 32, 32, 8, {4: 8}),                 # 256x512x2048, 32 units
    (272, 64, 256, 68, {1: 32, 2: 240}),     # 2048x2176x4096
    (144, 256, 256, 144, {2: 48, 3: 96}),    # 1536x1536x16384
])
def test_workload_tile_groups(tiles, ipt, units, q, groups):
    total = tiles * ipt
    assert total % units == 0 and total // units == q
    segs = sch.streamk_segments(sch.unit_ranges(total, units), ipt)
    count = {}
    for _, (owner, peers) in sch.tile_groups(segs).items():
        count[1 + len(peers)] = count.get(1 + len(peers), 0) + 1
    assert count == groups
    # brute force: units touching a tile, from per-iteration ownership it // q
    brute = {}
    for t in range(tiles):
        us = {it // q for it in range(t * ipt, (t + 1) * ipt)}
        brute[len(us)] = brute.get(len(us), 0) + 1
    assert brute == groups


# -- brute-force structure: coverage, contiguity, roles --------------------------
@pytest.mark.parametrize("rule", ["big_first", "cdiv", "floor"])
def test_coverage_exactly_once(rule):
    for tiles, ipt in itertools.product((1, 2, 3, 5, 8, 13), (1, 2, 3, 4, 7, 9, 16)):
        total = tiles * ipt
        for units in range(1, 65):
            bounds = sch.unit_ranges(total, units, rule)
            assert bounds[0][0] == 0 and bounds[-1][1] == total
            assert all(b <= e for b, e in bounds)
            assert all(bounds[i][1] == bounds[i + 1][0] for i in range(units - 1)) or rule == "cdiv"
            segs = sch.streamk_segments(bounds, ipt)
            cov = sch.coverage(segs, tiles, ipt)
            assert all(c == 1 for row in cov for c in row), (tiles, ipt, units, rule)
            # contributors only ever start a unit's range, owners only ever end one
            by_unit = {}
            for s in segs:
                by_unit.setdefault(s.unit, []).append(s)
            for lst in by_unit.values():
                for i, s in enumerate(lst):
                    if s.role == sch.CONTRIB:
                        assert i == 0
                    if s.role == sch.OWNER:
                        assert i == len(lst) - 1
            # the owner's peers are the next non-empty units, in ascending order
            nonempty = [u for u, (b, e) in enumerate(bounds) if e > b]
            for t, (owner, peers) in sch.tile_groups(segs).items():
                i = nonempty.index(owner)
                assert peers == nonempty[i + 1:i + 1 + len(peers)]
            # roles agree with the tile groups: a tile one unit computes is whole;
            # of a split tile the k = 0 holder is the owner and the rest contribute
            per_tile = {}
            for s in segs:
                per_tile.setdefault(s.tile, []).append(s)
            for t, lst in per_tile.items():
                if len(lst) == 1:
                    assert lst[0].role == sch.FULL and (lst[0].k0, lst[0].k1) == (0, ipt)
                else:
                    lst = sorted(lst, key=lambda s: s.k0)
                    assert lst[0].role == sch.OWNER and lst[0].k0 == 0
                    assert all(s.role == sch.CONTRIB for s in lst[1:])


# -- book chapter, Case 2: "big units first" -------------------------------------
def test_big_units_first():
    # the units that own one iteration more than the others are the first ones:
    # lengths never increase with the unit index and differ by at most one
    for total in range(0, 200, 7):
        for units in range(1, 40):
            lens = [e - b for b, e in sch.unit_ranges(total, units)]
            assert sum(lens) == total
            assert max(lens) - min(lens) <= 1
            assert all(lens[i] >= lens[i + 1] for i in range(units - 1)), (total, units, lens)


# -- brute force: the tile grid covers every output element once ------------------
def test_tile_grid_covers_every_element():
    for bm, bn in ((128, 128), (64, 64), (64, 128), (256, 128)):
        for M in list(range(1, 300, 13)) + [127, 128, 129, 256, 257]:
            for N in (1, 63, 64, 65, 200, 384):
                tm, tn = sch.tile_grid(M, N, bm, bn)
                rows = {i // bm for i in range(M)}
                cols = {j // bn for j in range(N)}
                assert rows == set(range(tm)) and cols == set(range(tn)), (M, N, bm, bn)


def test_rules_agree_when_units_divide():
    for tiles, ipt, units in [(8, 32, 32), (272, 64, 256), (144, 256, 256), (4096, 128, 256)]:
        r = [sch.unit_ranges(tiles * ipt, units, rule) for rule in ("big_first", "cdiv", "floor")]
        assert r[0] == r[1] == r[2]


def test_splitk_segments_cover():
    for tiles, ipt in [(4, 32), (8, 32), (3, 7)]:
        for s in range(1, ipt + 1):
            segs = sch.splitk_segments(tiles, ipt, s)
            cov = sch.coverage(segs, tiles, ipt)
            assert all(c == 1 for row in cov for c in row)
            lens = [x.k1 - x.k0 for x in segs]
            assert max(lens) - min(lens) <= 1
            if ipt % s == 0:
                assert set(lens) == {ipt // s}    # aligned split: constant trip count P/S


def test_plan_schedule_modes():
    s = sch.plan_schedule(2048, 2176, 4096, "heuristic")
    assert (s.kind, s.units, s.sk_tiles, s.dp_tiles, s.q, s.big) == ("StreamK", 256, 272, 0, 68, 0)
    s = sch.plan_schedule(8192, 8192, 8192, "heuristic")
    assert s.kind == "DataParallel" and len(s.segments) == 4096
    s = sch.plan_schedule(96, 512, 2048, "splitk", 8)
    assert s.kind == "SplitK" and s.tiles == 4 and len(s.segments) == 32
    s = sch.plan_schedule(256, 512, 2048, "streamk", 32)
    assert (s.q, s.big) == (8, 0)
    # a hybrid decision: DP waves first, the Stream-K part on the last tiles
    s = sch.plan_schedule(3840, 3840, 4096, "heuristic", sms=148)
    assert (s.sk_tiles, s.dp_tiles, s.units) == (160, 740, 148)
    cov = sch.coverage(s.segments, s.tiles, s.ipt)
    assert all(c == 1 for row in cov for c in row)


@pytest.mark.parametrize("M,N,K,batch,mode,splits", [
    (256, 512, 2048, 4, "heuristic", 0),
    (384, 640, 1024, 3, "streamk", 0),
    (128, 256, 4096, 8, "heuristic", 0),
    (512, 512, 512, 6, "splitk", 2),
    (1024, 1024, 1024, 5, "heuristic", 0),
])
def test_batched_schedule_is_the_stacked_problem(M, N, K, batch, mode, splits):
    # with M a multiple of the tile height, `batch` products of M x N stack into one
    # (batch M) x N problem with the same tile count; the schedules must coincide
    b = sch.plan_schedule(M, N, K, mode, splits, sms=256, batch=batch)
    s = sch.plan_schedule(batch * M, N, K, mode, splits, sms=256)
    assert b.tiles == s.tiles == batch * b.tiles_m * b.tiles_n
    assert (b.kind, b.splits, b.units, b.sk_tiles, b.dp_tiles, b.q, b.big) == \
        (s.kind, s.splits, s.units, s.sk_tiles, s.dp_tiles, s.q, s.big)
    assert [x.as_tuple() for x in b.segments] == [x.as_tuple() for x in s.segments]
    cov = sch.coverage(b.segments, b.tiles, b.ipt)
    assert all(c == 1 for row in cov for c in row)


def test_rule_splitk_needs_aligned_split():
    # units = 4 per tile: Split-K only when 4 divides the tile's iterations
    # (docc StreamK page, aligned split); 34 iterations fall back to Stream-K
    assert sch.decide(64, 32, 256) == sch.Decision("SplitK", 64, 256)
    assert sch.decide(64, 34, 256) == sch.Decision("StreamK", 64, 256)
    assert sch.decide(64, 36, 256).kind == "SplitK"


@pytest.mark.parametrize("shapes,K,mode,splits", [
    ([(256, 512)] * 4, 2048, "heuristic", 0),
    ([(1000, 1000)] * 3, 640, "streamk", 7),
    ([(96, 512)] * 8, 2048, "splitk", 4),
])
def test_grouped_schedule_of_equal_shapes_is_the_batch(shapes, K, mode, splits):
    # problems of one shape, numbered problem after problem, are a batch
    M, N = shapes[0]
    g = sch.plan_schedule_grouped(shapes, K, mode, splits)
    b = sch.plan_schedule(M, N, K, mode, splits, batch=len(shapes))
    assert (g.kind, g.ipt, g.splits, g.units, g.sk_tiles, g.dp_tiles, g.q, g.big) == \
           (b.kind, b.ipt, b.splits, b.units, b.sk_tiles, b.dp_tiles, b.q, b.big)
    assert sorted(x.as_tuple() for x in g.segments) == sorted(x.as_tuple() for x in b.segments)


def test_grouped_schedule_counts_every_problem_tile():
    shapes = [(96, 512), (0, 512), (300, 1024), (1, 8), (64, 0)]
    for bm in (64, 128, 256):
        g = sch.plan_schedule_grouped(shapes, 1024, "streamk", 5, bm=bm)
        tiles = sum(-(-M // bm) * -(-N // 128) for M, N in shapes)
        cov = np.zeros((tiles, 16), dtype=int)
        for x in g.segments:
            cov[x.tile, x.k0:x.k1] += 1
        assert np.all(cov == 1)
