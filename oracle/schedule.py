"""CPU schedule simulator for data-parallel, Split-K and Stream-K GEMM schedules.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Everything here is integer bookkeeping over the flattened (output tile x
k-iteration) space, plus the unit cost model of the Split-K/Stream-K book
chapter.  The simulator is the schedule oracle: the host planner's decisions
and the per-unit ranges, and the segment/role trace that the GPU kernels
record, must equal what this module computes.

Sources, by page and section:

* Wave arithmetic -- book chapter, Case 1: tiles = ceil(M/BM) ceil(N/BN),
  waves = ceil(tiles/SMs), the last wave holds tiles - (waves-1) SMs tiles,
  utilisation = tiles / (waves SMs).
* Flattened space and per-unit ranges -- book chapter, "Mental model" and the
  Stream-K paragraph after the glossary (unit u owns [u q, (u+1) q)); Case 2's
  simulator splits ``total`` so that the first ``total mod units`` units take one
  extra iteration ("big units first"); Case 3's Triton kernel uses
  q = ceil(total/units); the docc StreamK page uses floor(bid total / NB).
* Roles -- book chapter, Stream-K paragraph: the unit holding a tile's k = 0
  iteration owns the fixup; a unit that starts mid-tile stores an fp32 partial
  and raises a flag; the owner waits for its peers, adds their partials and runs
  the epilogue.
* Split-K ranges -- docc StreamK page, "MMA fragment accumulators (aligned
  split)": block (t, s) owns panels [s P / S, (s+1) P / S).
* Decomposition rule -- the toy figure's caption ("Mental model"), Case 2's
  discussion of its table and Case 4's knob table: DP when there is no partial
  wave or a tile has at most 8 k-iterations, DP when the tail wave is at least
  half full, otherwise Stream-K over the last two waves with at least 8
  iterations per unit, and Split-K when the units divide evenly over the split
  tiles -- with the split factor dividing the tile's k-iterations, the aligned
  split of the docc StreamK page ("MMA fragment accumulators").
* Cost model -- book chapter, Case 2: 1 per MAC iteration, EPI per finished tile
  store, PART per fp32 partial store or load; the owner's wait is the later of
  its own progress and the peer's publish time.

Pins: tests/test_schedule_sim.py (printed tables of Cases 1 and 2, the toy
figure of the "Mental model" section, Case 3's structural facts, brute-force
coverage).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Sequence, Tuple

FULL = "full"        # segment covers the whole k range of its tile: plain epilogue
OWNER = "owner"      # starts at k = 0 but stops early: waits for peers, folds, epilogue
CONTRIB = "contrib"  # starts mid-tile: publishes an fp32 partial and a flag

ROLE_CODE = {FULL: 0, OWNER: 1, CONTRIB: 2}


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


# ----------------------------------------------------------------------------
# Wave arithmetic (book chapter, Case 1)
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Waves:
    tiles: int
    waves: int
    tail: int        # tiles in the last wave
    util: float      # tiles / (waves * SMs)


def tile_grid(M: int, N: int, bm: int = 128, bn: int = 128) -> Tuple[int, int]:
    return cdiv(M, bm), cdiv(N, bn)


def wave_stats(tiles: int, sms: int) -> Waves:
    w = cdiv(tiles, sms)
    if w == 0:                        # no tiles: no wave
        return Waves(0, 0, 0, 0.0)
    last = tiles - (w - 1) * sms
    return Waves(tiles, w, last, tiles / (w * sms))


# ----------------------------------------------------------------------------
# Per-unit iteration ranges of the flattened space
# ----------------------------------------------------------------------------
def unit_ranges(total: int, units: int, rule: str = "big_first") -> List[Tuple[int, int]]:
    """Half-open ``[b, e)`` ranges of the flattened space, one per unit.

    Every rule is a start function s(u) with s(0) = 0 and s(units) = total; unit u
    covers [s(u), s(u + 1)).

    rule "big_first": the shares differ by at most one iteration and the longer
                      ones come first (book chapter, Case 2): with
                      q, r = divmod(total, units), s(u) = u q + min(u, r).
    rule "cdiv":      every unit but the last takes ceil(total/units) (Case 3's
                      Triton kernel): s(u) = min(u ceil(total/units), total).
    rule "floor":     s(u) = floor(u total / units) (docc StreamK page).
    """
    if units <= 0:
        raise ValueError("units must be positive")
    if rule == "big_first":
        q, r = divmod(total, units)
        start = lambda u: u * q + min(u, r)
    elif rule == "cdiv":
        step = cdiv(total, units)
        start = lambda u: min(u * step, total)
    elif rule == "floor":
        start = lambda u: u * total // units
    else:
        raise ValueError(f"unknown split rule {rule!r}")
    return [(start(u), start(u + 1)) for u in range(units)]


# ----------------------------------------------------------------------------
# Segments and roles
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Segment:
    unit: int
    tile: int
    k0: int          # first k-iteration of the tile covered
    k1: int          # one past the last
    role: str

    def as_tuple(self):
        return (self.unit, self.tile, self.k0, self.k1, ROLE_CODE[self.role])


def _role(k0: int, k1: int, ipt: int) -> str:
    if k0 > 0:
        return CONTRIB
    return FULL if k1 == ipt else OWNER


def streamk_segments(bounds: Sequence[Tuple[int, int]], ipt: int) -> List[Segment]:
    """Cut every unit's range at tile edges and label each piece."""
    segs = []
    for u, (b, e) in enumerate(bounds):
        pos = b
        while pos < e:
            tile = pos // ipt
            k0 = pos - tile * ipt
            k1 = min(e - tile * ipt, ipt)
            segs.append(Segment(u, tile, k0, k1, _role(k0, k1, ipt)))
            pos = tile * ipt + k1
    return segs


def splitk_ranges(ipt: int, splits: int) -> List[Tuple[int, int]]:
    """k-iteration range of split s of one tile: [s P / S, (s+1) P / S)."""
    return [(s * ipt // splits, (s + 1) * ipt // splits) for s in range(splits)]


def splitk_segments(tiles: int, ipt: int, splits: int) -> List[Segment]:
    """Worker ``tile*S + s`` covers split s of its tile; every piece is a partial when S > 1."""
    segs = []
    for t in range(tiles):
        for s, (k0, k1) in enumerate(splitk_ranges(ipt, splits)):
            role = FULL if splits == 1 else (OWNER if s == 0 else CONTRIB)
            segs.append(Segment(t * splits + s, t, k0, k1, role))
    return segs


def dp_segments(tiles: int, ipt: int) -> List[Segment]:
    return [Segment(t, t, 0, ipt, FULL) for t in range(tiles)]


def tile_groups(segs: Sequence[Segment]) -> Dict[int, Tuple[int, List[int]]]:
    """Per tile: (unit holding k = 0, [other units in ascending k order])."""
    by_tile: Dict[int, List[Segment]] = {}
    for s in segs:
        by_tile.setdefault(s.tile, []).append(s)
    out = {}
    for t, lst in by_tile.items():
        lst = sorted(lst, key=lambda s: s.k0)
        out[t] = (lst[0].unit, [s.unit for s in lst[1:]])
    return out


def coverage(segs: Sequence[Segment], tiles: int, ipt: int) -> List[List[int]]:
    """How many times each (tile, k) pair is executed; must be all ones."""
    cov = [[0] * ipt for _ in range(tiles)]
    for s in segs:
        for k in range(s.k0, s.k1):
            cov[s.tile][k] += 1
    return cov


def max_units_per_tile(segs: Sequence[Segment]) -> int:
    g = tile_groups(segs)
    return max((1 + len(c) for _, c in g.values()), default=0)


# ----------------------------------------------------------------------------
# Decomposition rule (book chapter, Case 2 and Case 4)
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Decision:
    kind: str         # "DataParallel" | "SplitK" | "StreamK"
    sk_tiles: int     # tiles handled by the split/stream part (0 for DP)
    sk_units: int     # workers for that part (0 for DP)

    @property
    def splits(self) -> int:
        return self.sk_units // self.sk_tiles if self.kind == "SplitK" else 1


def decide(tiles: int, ipt: int, sms: int, min_iters: int = 8) -> Decision:
    """The decomposition rule, stated in terms of the data-parallel waves.

    * Nothing to balance -- the tiles fill whole waves, or a tile's K loop has
      at most ``min_iters`` iterations -- or a last wave at least half full:
      data-parallel.
    * Otherwise the partial last wave and the full wave before it (if there is
      one) become the Stream-K part; earlier waves stay data-parallel.
    * Its units: one per SM, but never so many that a unit averages fewer than
      ``min_iters`` iterations.
    * If the units come out as a whole number S > 1 per Stream-K tile and S
      divides the tile's iterations, every tile is simply split S ways: Split-K.
    """
    w = wave_stats(tiles, sms)
    partial_last_wave = 0 < w.tail < sms
    if not partial_last_wave or ipt <= min_iters or 2 * w.tail >= sms:
        return Decision("DataParallel", 0, 0)
    stream_waves = min(w.waves, 2)
    sk_tiles = tiles - (w.waves - stream_waves) * sms
    units = min(sms, sk_tiles * ipt // min_iters)
    per_tile, left = divmod(units, sk_tiles)
    if left == 0 and per_tile > 1 and ipt % per_tile == 0:
        return Decision("SplitK", sk_tiles, units)
    return Decision("StreamK", sk_tiles, units)


# ----------------------------------------------------------------------------
# Unit cost model (book chapter, Case 2).  Times are in MAC-iteration units.
# ----------------------------------------------------------------------------
def cost_dp(tiles: int, ipt: int, sms: int, epi: float = 2) -> float:
    """Every data-parallel wave costs one whole tile: its K loop and its epilogue."""
    return wave_stats(tiles, sms).waves * (ipt + epi)


def cost_splitk(tiles: int, ipt: int, sms: int, s: int, epi: float = 2, part: float = 2) -> float:
    """Split-K in the chapter's model: the tiles x s workers run in waves of one
    per SM; a wave lasts as long as its longest worker, which runs ceil(ipt / s)
    iterations and moves one fp32 partial (stores it, or loads one); after the
    last wave the tile's k = 0 worker adds the other s - 1 partials (a load
    each) and writes the tile."""
    worker = cdiv(ipt, s) + part
    fold = (s - 1) * part + epi
    return wave_stats(tiles * s, sms).waves * worker + fold


def cost_streamk(segs: Sequence[Segment], units: int, ipt: int,
                 epi: float = 2, part: float = 2) -> float:
    """Makespan of a Stream-K schedule given its segments (one unit per SM)."""
    by_unit: Dict[int, List[Segment]] = {}
    for s in segs:
        by_unit.setdefault(s.unit, []).append(s)
    groups = tile_groups(segs)
    # A contributor segment is always its unit's first, so it is published at
    # (its length + one partial store) after the unit starts.
    publish: Dict[Tuple[int, int], float] = {}
    for u, lst in by_unit.items():
        first = lst[0]
        if first.role == CONTRIB:
            publish[(u, first.tile)] = (first.k1 - first.k0) + part
    finish = 0.0
    for u, lst in by_unit.items():
        clock = 0.0
        for s in lst:
            clock += s.k1 - s.k0
            if s.role == CONTRIB:
                clock += part
                continue
            if s.role == OWNER:
                for peer in groups[s.tile][1]:
                    clock = max(clock, publish[(peer, s.tile)]) + part
            clock += epi
        finish = max(finish, clock)
    return finish


def cost_streamk_shape(tiles: int, ipt: int, units: int, epi: float = 2, part: float = 2,
                       rule: str = "big_first") -> float:
    segs = streamk_segments(unit_ranges(tiles * ipt, units, rule), ipt)
    return cost_streamk(segs, units, ipt, epi, part)


def cost_decided(tiles: int, ipt: int, sms: int, epi: float = 2, part: float = 2):
    """(decision, makespan) of the rule's choice: its split part costed as
    Stream-K units over the split tiles (Split-K is the special case whose
    segments are whole splits), followed by the data-parallel waves it keeps."""
    d = decide(tiles, ipt, sms)
    kept = cost_dp(tiles - d.sk_tiles, ipt, sms, epi)
    if d.kind == "DataParallel":
        return d, kept
    return d, cost_streamk_shape(d.sk_tiles, ipt, d.sk_units, epi, part) + kept


def ideal(tiles: int, ipt: int, sms: int, epi: float = 2) -> float:
    return tiles * (ipt + epi) / sms


# ----------------------------------------------------------------------------
# Whole-schedule view used to compare against the host planner and GPU traces
# ----------------------------------------------------------------------------
@dataclass
class Schedule:
    kind: str                     # "DataParallel" | "SplitK" | "StreamK"
    tiles_m: int
    tiles_n: int
    ipt: int
    splits: int                   # Split-K factor (1 otherwise)
    units: int                    # Stream-K units (0 otherwise)
    sk_tiles: int                 # tiles in the Stream-K part (Stream-K only)
    dp_tiles: int                 # tiles left to DP waves (hybrid), 0 otherwise
    q: int                        # floor(total / units) for Stream-K
    big: int                      # total mod units
    segments: List[Segment]
    batch: int = 1                # matrices in a batched call (tile grids numbered batch after batch)

    @property
    def tiles(self):
        return self.batch * self.tiles_m * self.tiles_n


def plan_schedule(M: int, N: int, K: int, mode: str, splits: int = 0, sms: int = 256,
                  bm: int = 128, bn: int = 128, bk: int = 64, batch: int = 1) -> Schedule:
    """What a GEMM call does, per mode ("heuristic", "dp", "splitk", "streamk").

    For "splitk", ``splits`` is S; for "streamk" it is the unit count (0 = one per SM).
    In a hybrid Stream-K decision the Stream-K part takes the *last* sk_tiles tiles
    and the first dp_tiles tiles run as plain data-parallel tiles.

    A batched call (``batch`` independent products of one shape) is one problem
    of batch x tiles_m x tiles_n output tiles, numbered batch after batch: the
    decomposition rule, the Stream-K flattening and every unit range apply to
    that tile count unchanged (book chapter, Case 1 arithmetic on the total
    tile count; docc StreamK page, generality: batched GEMM).
    """
    tm, tn = tile_grid(M, N, bm, bn)
    tiles = batch * tm * tn
    ipt = cdiv(K, bk)
    if mode == "heuristic":
        d = decide(tiles, ipt, sms)
        if d.kind == "DataParallel":
            mode, splits = "dp", 0
        elif d.kind == "SplitK":
            mode, splits = "splitk", d.splits
        else:
            units = d.sk_units
            dp_tiles = tiles - d.sk_tiles
            total = d.sk_tiles * ipt
            segs = [Segment(s.unit, s.tile + dp_tiles, s.k0, s.k1, s.role)
                    for s in streamk_segments(unit_ranges(total, units), ipt)]
            segs += [Segment(units + t, t, 0, ipt, FULL) for t in range(dp_tiles)]
            return Schedule("StreamK", tm, tn, ipt, 1, units, d.sk_tiles, dp_tiles,
                            total // units, total % units, segs, batch)
    if mode == "dp":
        return Schedule("DataParallel", tm, tn, ipt, 1, 0, 0, 0, 0, 0, dp_segments(tiles, ipt), batch)
    if mode == "splitk":
        return Schedule("SplitK", tm, tn, ipt, splits, 0, 0, 0, 0, 0,
                        splitk_segments(tiles, ipt, splits), batch)
    if mode == "streamk":
        units = splits if splits > 0 else sms
        total = tiles * ipt
        return Schedule("StreamK", tm, tn, ipt, 1, units, tiles, 0, total // units, total % units,
                        streamk_segments(unit_ranges(total, units), ipt), batch)
    raise ValueError(f"unknown mode {mode!r}")
def plan_schedule_grouped(shapes, K: int, mode: str, splits: int = 0, sms: int = 256,
                          bm: int = 128, bn: int = 128, bk: int = 64) -> Schedule:
    """What a grouped call does: problems of the given (M, N) shapes with one K.

    Reading (the docc StreamK page lists grouped GEMM among what the rewrite
    covers but gives no schedule): the problems' tiles are numbered problem after
    problem, like a batch's entries, so the rule, the Stream-K flattening and the
    unit ranges see one tile count; the schedule is that of a single problem
    with that many tiles (one column of them).  Problems with no tile add none.
    """
    tiles = sum(cdiv(M, bm) * cdiv(N, bn) for M, N in shapes)
    return plan_schedule(tiles * bm, bn, K, mode, splits, sms, bm, bn, bk)


