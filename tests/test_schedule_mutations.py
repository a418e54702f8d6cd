"""Teeth of the schedule simulator's pins: each test plants one plausible
mistake in oracle/schedule.py (monkeypatched, on the CPU, for that test only)
and checks that at least one pin of tests/test_schedule_sim.py then fails.

The pins are the pages' printed tables and figures plus brute force; a mistake
none of them notices would mean the simulator is checked against itself only.

One reading has no pin: whether a tail wave of exactly half the SMs counts as
"at least half full" (the decomposition rule keeps data-parallel then).  No
printed case sits on that boundary; the simulator takes the comparison as the
book chapter's Case 2 prints it."""
import itertools

import pytest

import test_schedule_sim as pins
from oracle import schedule as sch

PIN_TESTS = [
    pins.test_wave_table,
    pins.test_h100_144_tiles_54_5_percent,
    pins.test_cost_table,
    pins.test_cost_table_needs_big_first_split,
    pins.test_toy_figure,
    pins.test_triton_structure_facts,
    pins.test_workload_decisions,
    pins.test_workload_tile_groups,
    pins.test_coverage_exactly_once,
    pins.test_big_units_first,
    pins.test_tile_grid_covers_every_element,
    pins.test_rules_agree_when_units_divide,
    pins.test_splitk_segments_cover,
    pins.test_plan_schedule_modes,
]


def _param_sets(fn):
    """Keyword sets of a test's @pytest.mark.parametrize lists (their product)."""
    lists = []
    for m in getattr(fn, "pytestmark", []):
        if m.name != "parametrize":
            continue
        names = m.args[0]
        names = [n.strip() for n in names.split(",")] if isinstance(names, str) else list(names)
        rows = []
        for v in m.args[1]:
            rows.append(dict(zip(names, v if len(names) > 1 else (v,))))
        lists.append(rows)
    out = []
    for combo in itertools.product(*lists):
        kw = {}
        for c in combo:
            kw.update(c)
        out.append(kw)
    return out


def failed_pins():
    failed = []
    for fn in PIN_TESTS:
        for kw in _param_sets(fn):
            try:
                fn(**kw)
            except Exception:   # an assertion, or the mistake breaking the code outright
                failed.append(fn.__name__)
                break
    return failed


def test_pins_pass_on_the_simulator():
    assert failed_pins() == []


_orig_unit_ranges = sch.unit_ranges
_orig_decide = sch.decide


def _small_first(total, units, rule="big_first"):
    # the remainder iterations go to the last units instead of the first
    if rule != "big_first":
        return _orig_unit_ranges(total, units, rule)
    base, extra = divmod(total, units)
    out, start = [], 0
    for u in range(units):
        n = base + (1 if u >= units - extra else 0)
        out.append((start, start + n))
        start += n
    return out


def _role_off_by_one(k0, k1, ipt):
    # a segment one iteration short of the tile end taken for a whole tile
    if k0 > 0:
        return sch.CONTRIB
    return sch.FULL if k1 >= ipt - 1 else sch.OWNER


def _owner_last(segs):
    # the unit holding the highest k taken for the tile's owner
    by_tile = {}
    for s in segs:
        by_tile.setdefault(s.tile, []).append(s)
    out = {}
    for t, lst in by_tile.items():
        lst = sorted(lst, key=lambda s: -s.k0)
        out[t] = (lst[0].unit, [s.unit for s in lst[1:]])
    return out


def _waves_floor(tiles, sms):
    w = max(tiles // sms, 1)
    last = tiles - (w - 1) * sms
    return sch.Waves(tiles, w, last, tiles / (w * sms))


def _grid_floor(M, N, bm=128, bn=128):
    return max(M // bm, 1), max(N // bn, 1)


def _decide_one_wave(tiles, ipt, sms, min_iters=8):
    # Stream-K given only the partial wave instead of the last two waves
    d = _orig_decide(tiles, ipt, sms, min_iters)
    if d.kind == "DataParallel":
        return d
    sk_tiles = tiles - (tiles // sms) * sms
    units = min(sms, (ipt * sk_tiles) // min_iters)
    kind = "SplitK" if units > sk_tiles and units % sk_tiles == 0 else "StreamK"
    return sch.Decision(kind, sk_tiles, units)


def _decide_no_unit_cap(tiles, ipt, sms, min_iters=8):
    # the unit count not capped at the SM count
    d = _orig_decide(tiles, ipt, sms, min_iters)
    if d.kind == "DataParallel":
        return d
    units = (ipt * d.sk_tiles) // min_iters
    kind = "SplitK" if units > d.sk_tiles and units % d.sk_tiles == 0 else "StreamK"
    return sch.Decision(kind, d.sk_tiles, units)


def _cost_dp_floor(tiles, ipt, sms, epi=2):
    return max(tiles // sms, 1) * (ipt + epi)


def _cost_splitk_no_fold(tiles, ipt, sms, s, epi=2, part=2):
    # the k = 0 worker's loads of the other partials left out
    return sch.cdiv(tiles * s, sms) * (sch.cdiv(ipt, s) + part) + epi


_orig_cost_streamk = sch.cost_streamk


def _cost_streamk_half_part(segs, units, ipt, epi=2, part=2):
    # every partial store and load charged half its cost
    return _orig_cost_streamk(segs, units, ipt, epi=epi, part=part / 2)


MUTATIONS = {
    "small-first unit ranges": ("unit_ranges", _small_first),
    "role off by one": ("_role", _role_off_by_one),
    "owner is the last contributor": ("tile_groups", _owner_last),
    "waves floored": ("wave_stats", _waves_floor),
    "tile grid floored": ("tile_grid", _grid_floor),
    "Stream-K takes one wave": ("decide", _decide_one_wave),
    "unit count not capped": ("decide", _decide_no_unit_cap),
    "DP waves floored": ("cost_dp", _cost_dp_floor),
    "Split-K fold not charged": ("cost_splitk", _cost_splitk_no_fold),
    "Stream-K partial cost halved": ("cost_streamk", _cost_streamk_half_part),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_is_caught(monkeypatch, name):
    attr, fake = MUTATIONS[name]
    monkeypatch.setattr(sch, attr, fake)
    assert failed_pins(), f"planted mistake '{name}' slipped through every pin"
