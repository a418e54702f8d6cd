#!/usr/bin/env python3
"""Benchmark of the MI355X DP / Split-K / Stream-K GEMM.

One step = one GEMM call on the wave-quantized workload (2048 x 2176 x 4096,
bf16 operands, fp32 accumulate and output, B stored [K,N]; 16 x 17 = 272 tiles
of 128x128 on 256 CUs = one full wave plus a 16-tile tail).  The call runs the
whole hot path: host plan and decomposition rule (it chooses Stream-K over 256
units), the persistent Stream-K kernel (mainloop, partial publish, k-ordered
turnstile fixup, epilogue).  Operands are resident in HBM before timing starts.

Prints ONE JSON line: throughput in TFLOP/s (2 M N K per step), the fraction of
the BF16 dense MFMA peak, the Stream-K speedup over the data-parallel tile grid
(and over Split-K s=2, 4) on the same shape, per-shape results for the other
workloads, the roofline of the dominant kernel (timed with HIP events on the
launch stream over the timed region) and the fp64 CPU oracle's throughput on
the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense BF16/FP16 MFMA peak (published)
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E (published)
METRIC = "GEMM TFLOP/s and % of BF16 MFMA peak per shape; Stream-K speedup vs DP"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="c3_wavequant")
    ap.add_argument("--no-shapes", action="store_true", help="skip the per-shape arms")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--rounds", type=int, default=9, help="rounds of the per-shape comparison protocol")
    ap.add_argument("--vendor", action="store_true",
                    help="also time the vendor BLAS alternately with the library (context only)")
    ap.add_argument("--mode", default=None, choices=["heuristic", "dp", "splitk", "streamk"],
                    help="override the workload's decomposition (for profiling one arm)")
    ap.add_argument("--splits", type=int, default=None, help="Split-K factor or Stream-K units")
    ap.add_argument("--atomic", action="store_true", help="Stream-K atomic fixup")
    ap.add_argument("--tile", default="128x128", choices=["128x128", "256x128", "64x128"],
                    help="output tile of the timed call (256x128: Stream-K only)")
    ap.add_argument("--shape", default=None,
                    help="MxNxK: time the workload's recipe at another shape (profiling one launch)")
    ap.add_argument("--no-timeline", action="store_true",
                    help="skip the per-CU busy-time measurement (instrumented launches)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a known-size "
                         "reference dispatch for HBM byte counters)")
    return ap.parse_args()


class Call:
    """A prepared gemm_ex call (argument struct built once; each call is one ctypes call)."""

    def __init__(self, dg, a, b, c, b_layout, mode, splits=0, atomic=False, stream=None, epilogue=None,
                 tile="128x128"):
        import torch

        self.dg = dg
        args = dg.GemmArgs()
        M, K = a.shape[-2], a.shape[-1]
        N = c.shape[-1]
        args.A, args.B, args.C = a.data_ptr(), b.data_ptr(), c.data_ptr()
        args.M, args.N, args.K = M, N, K
        batch = c.shape[0] if c.dim() == 3 else 1
        if batch > 1:   # contiguous [batch, ...] operands
            args.batch = batch
            args.stride_a, args.stride_b, args.stride_c = a.stride(0), b.stride(0), c.stride(0)
        args.layout = dg.layout_word(b_layout, "bf16" if a.dtype == torch.bfloat16 else "fp16")
        # `atomic`: False, True, "two_pass" (partials of split tiles added by a
        # second kernel), "in_launch" (added in the launch: Split-K last arriver,
        # Stream-K turnstile) or "bands" (Split-K: every split adds up its row
        # bands in the launch)
        args.mode = dg.mode_word(mode, atomic is True, atomic == "two_pass", tile)
        if atomic == "in_launch":
            args.debug = dg.GEMM_DEBUG_IN_LAUNCH
        if atomic == "bands":
            args.debug = dg.GEMM_DEBUG_SPLITK_BANDS
        args.splits = splits
        if epilogue is not None:
            # fused epilogue c = act(alpha a.b + beta c + bias): (alpha, beta, bias tensor, act)
            alpha, beta, bias, act = epilogue
            args.epilogue = dg.GEMM_EPI_ALPHA_BETA | dg.GEMM_EPI_BIAS | dg.ACTIVATIONS[act]
            args.alpha, args.beta, args.bias = alpha, beta, bias.data_ptr()
            self.bias = bias
        self.stream = stream or torch.cuda.current_stream()
        args.stream = self.stream.cuda_stream
        self.args = args
        self.plan = dg.gemm_plan_batched(M, N, K, batch, args.layout, args.mode, splits, dg.gemm_num_cus())

    def __call__(self):
        st = self.dg.gemm_ex(self.args)
        if st != 0:
            raise self.dg.GemmError(st, self.dg.gemm_last_error())


class GroupedCall:
    """A prepared gemm_grouped call over (a_g, b_g, c_g) device tensors (one K,
    one dtype; argument struct and problem table built once)."""

    def __init__(self, dg, problems, b_layout, mode="heuristic", splits=0, stream=None, tile="128x128"):
        import torch

        self.dg = dg
        common = dg.GemmArgs()
        K = problems[0][0].shape[-1]
        common.K = K
        common.layout = dg.layout_word(b_layout, "bf16" if problems[0][0].dtype == torch.bfloat16 else "fp16")
        common.mode = dg.mode_word(mode, tile=tile)
        common.splits = splits
        self.stream = stream or torch.cuda.current_stream()
        common.stream = self.stream.cuda_stream
        self.common = common
        shapes = [(a.shape[0], c.shape[1]) for a, _, c in problems]
        self.groups = dg.group_array([(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N)
                                      for (a, b, c), (M, N) in zip(problems, shapes)])
        self.plan = dg.gemm_plan_grouped(shapes, K, common.layout, common.mode, splits, dg.gemm_num_cus())

    def __call__(self):
        st = self.dg.gemm_grouped(self.common, self.groups)
        if st != 0:
            raise self.dg.GemmError(st, self.dg.gemm_last_error())


class SeparateCalls:
    """The same problems as one gemm_ex call each, back to back on one stream."""

    def __init__(self, calls):
        self.calls = calls
        self.stream = calls[0].stream

    def __call__(self):
        for c in self.calls:
            c()


def time_call(call: Call, steps: int, warmup: int):
    """Warm up, then time exactly `steps` back-to-back calls: the wall clock of
    the timed region (synchronised on both sides) and one HIP event pair on the
    launch stream around it.  Returns (wall seconds, event milliseconds); the
    event time / steps is the average launch duration (a per-call event pair
    would add its own marker packets between the launches)."""
    import torch

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(call.stream)
    for _ in range(steps):
        call()
    e1.record(call.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1)


def time_arms(calls, rounds, samples, pack, warmup=20):
    """The Metal split-K note's comparison protocol ("Comparison and independent
    confirmation"): every arm warmed up, then `rounds` rounds of `samples`
    samples; within a round the arm order is rotated by one at every sample and
    every other round runs the rotated order in reverse, so no arm keeps a fixed
    place in the clock and power history of a power-capped chip.  A sample is
    one HIP event pair on the launch stream around `pack` back-to-back calls
    (its mean per call).  Returns {arm: [[samples of round 0], [round 1], ...]}
    in microseconds."""
    import torch

    names = list(calls)
    for n in names:
        for _ in range(warmup):
            calls[n]()
    torch.cuda.synchronize()
    out = {n: [] for n in names}
    for r in range(rounds):
        recs = []
        for i in range(samples):
            k = i % len(names)
            order = names[k:] + names[:k]
            if r % 2 == 1:
                order = order[::-1]
            for n in order:
                c = calls[n]
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(c.stream)
                for _ in range(pack):
                    c()
                e1.record(c.stream)
                recs.append((n, e0, e1))
        torch.cuda.synchronize()
        per = {n: [] for n in names}
        for n, e0, e1 in recs:
            per[n].append(e0.elapsed_time(e1) * 1e3 / pack)
        for n in names:
            out[n].append(per[n])
    return out


def _q(xs, f):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(f * (len(xs) - 1)))))]


def arm_result(w, call, rounds_us):
    """Median and spread of an arm's samples (all rounds pooled)."""
    flat = [x for r in rounds_us for x in r]
    med = statistics.median(flat)
    return {
        "decision": call.dg.DECISION_NAMES[call.plan.decision],
        "units_or_splits": int(call.plan.sk_units or call.plan.splits),
        "median_us": round(med, 3),
        "p10_us": round(_q(flat, 0.1), 3),
        "p90_us": round(_q(flat, 0.9), 3),
        "min_us": round(min(flat), 3),
        "round_medians_us": [round(statistics.median(r), 3) for r in rounds_us],
        "tflops": round(w.flops / (med * 1e-6) / 1e12, 2),
        "pct_peak": round(100 * w.flops / (med * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 2),
        # the bytes every method must move (A and B read once, C written once) per
        # the median time: the HBM view of the skinny, memory-side shapes
        "compulsory_gbps": round(compulsory_bytes(w) / (med * 1e-6) / 1e9, 1),
        "pct_hbm_peak": round(100 * compulsory_bytes(w) / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
    }


def compulsory_bytes(w) -> int:
    """A [M,K] and B read once (16-bit), C [M,N] fp32 written once, per batch entry."""
    return w.batch * (w.M * w.K * 2 + w.K * w.N * 2 + w.M * w.N * 4)


def paired_speedup(base_rounds, arm_rounds):
    """Speedup of an arm over the base from paired rounds: per round the ratio of
    the two arms' median samples (both timed interleaved in that round); the
    median ratio and the smallest and largest round's."""
    ratios = [statistics.median(b) / statistics.median(a) for b, a in zip(base_rounds, arm_rounds)]
    return {"median": round(statistics.median(ratios), 3), "min": round(min(ratios), 3),
            "max": round(max(ratios), 3)}


# samples per round and calls per sample: a few seconds of GPU time per workload
PROTOCOL = {"c1": (40, 8), "c2": (40, 8), "c3": (40, 8), "c4": (6, 2), "c5": (20, 8), "x1": (12, 4), "x2": (20, 8),
            "x3": (40, 8), "x4": (20, 4)}


def shape_arms(dg, name, rounds):
    import torch
    from workloads import WORKLOADS, make_operands

    w = WORKLOADS[name]
    A, B = make_operands(w)
    a, b = A.cuda(), B.cuda()
    c = torch.zeros(((w.batch,) if w.batch > 1 else ()) + (w.M, w.N), dtype=torch.float32, device="cuda")
    bias = torch.linspace(-1.0, 1.0, w.N, dtype=torch.float32, device="cuda")
    epi = (0.75, -0.5, bias, "gelu")   # alpha, beta, bias, activation of the "_epilogue" arms
    arms = {"dp": ("dp", 0, False)}
    if name.startswith("c2"):
        arms["splitk%d" % w.splits] = ("splitk", w.splits, False)
        arms["splitk%d_in_launch" % w.splits] = ("splitk", w.splits, "in_launch")
        arms["splitk%d_atomic" % w.splits] = ("splitk", w.splits, True)
        arms["splitk%d_64x128" % w.splits] = ("splitk", w.splits, False)
    if name.startswith("c1"):
        arms["streamk32"] = ("streamk", 32, False)
        arms["streamk32_in_launch"] = ("streamk", 32, "in_launch")
        arms["splitk4"] = ("splitk", 4, False)
        arms["splitk4_in_launch"] = ("splitk", 4, "in_launch")
        arms["heuristic"] = ("heuristic", 0, False)
        arms["streamk32_64x128"] = ("streamk", 32, False)
        arms["heuristic_64x128"] = ("heuristic", 0, False)
    if name.startswith("c3"):
        arms["heuristic"] = ("heuristic", 0, False)
        arms["heuristic_epilogue"] = ("heuristic", 0, False, epi)
        arms["heuristic_two_pass"] = ("heuristic", 0, "two_pass")
        arms["splitk2"] = ("splitk", 2, False)
        arms["splitk4"] = ("splitk", 4, False)
        arms["splitk2_two_pass"] = ("splitk", 2, "two_pass")
        arms["splitk4_two_pass"] = ("splitk", 4, "two_pass")
        arms["streamk_256x128"] = ("streamk", 0, False)
    if name.startswith("c4"):
        arms = {"heuristic": ("heuristic", 0, False), "heuristic_epilogue": ("heuristic", 0, False, epi)}
    if name.startswith("c5"):
        arms["streamk_det"] = ("streamk", 0, False)
        arms["streamk_det_two_pass"] = ("streamk", 0, "two_pass")
        arms["streamk_atomic"] = ("streamk", 0, True)
        arms["streamk_256x128"] = ("streamk", 0, False)
    if name.startswith("x1"):
        arms["heuristic"] = ("heuristic", 0, False)
        arms["streamk"] = ("streamk", 0, False)
        arms["streamk_256x128"] = ("streamk", 0, False)
    if name.startswith("x3"):
        arms["heuristic"] = ("heuristic", 0, False)
        arms["dp_64x128"] = ("dp", 0, False)
        arms["heuristic_64x128"] = ("heuristic", 0, False)
        arms["splitk8_64x128"] = ("splitk", 8, False)
    if name.startswith("x2"):
        arms["heuristic"] = ("heuristic", 0, False)
        arms["streamk"] = ("streamk", 0, False)
        arms["heuristic_epilogue"] = ("heuristic", 0, False, epi)
    out = {"M": w.M, "N": w.N, "K": w.K, "dtype": w.dtype, "b_layout": w.b_layout}
    if w.batch > 1:
        out["batch"] = w.batch
    calls = {}
    for arm, (mode, splits, atomic, *ep) in arms.items():
        tile = next((t for t in ("256x128", "64x128") if arm.endswith("_" + t)), "128x128")
        calls[arm] = Call(dg, a, b, c, w.b_layout, mode, splits, atomic, epilogue=ep[0] if ep else None, tile=tile)
    samples, pack = PROTOCOL[name[:2]]
    timed = time_arms(calls, rounds, samples, pack)
    out["protocol"] = {"rounds": rounds, "samples_per_round": samples, "calls_per_sample": pack,
                       "order": "rotated every sample, reversed every other round"}
    for arm, call in calls.items():
        out[arm] = arm_result(w, call, timed[arm])
        if "dp" in timed and arm != "dp":
            out[arm]["speedup_vs_dp"] = paired_speedup(timed["dp"], timed[arm])
        log(f"  {name:14s} {arm:20s} {out[arm]['median_us']:9.3f} us  {out[arm]['tflops']:8.2f} TFLOP/s"
            f"  {out[arm]['compulsory_gbps']:7.1f} GB/s"
            + (f"  x{out[arm]['speedup_vs_dp']['median']} vs dp" if "speedup_vs_dp" in out[arm] else ""))
    if pack > 1 and name[:2] in ("c1", "c2", "x3"):
        # the small shapes also at pack 1 (one call per event pair, the Metal
        # note's other pack size): each call then also carries the event markers'
        # and the launch's own latency
        timed1 = time_arms(calls, rounds, samples, 1)
        out["protocol"]["also_pack_1"] = True
        for arm, call in calls.items():
            r = arm_result(w, call, timed1[arm])
            out[arm]["pack1"] = {k: r[k] for k in ("median_us", "p10_us", "p90_us", "min_us")}
            if "dp" in timed1 and arm != "dp":
                out[arm]["pack1"]["speedup_vs_dp"] = paired_speedup(timed1["dp"], timed1[arm])
            log(f"  {name:14s} {arm:20s} {r['median_us']:9.3f} us  (pack 1)"
                + (f"  x{out[arm]['pack1']['speedup_vs_dp']['median']} vs dp" if arm != "dp" and "dp" in timed1 else ""))
    return out


def grouped_operands(gw):
    """Device operands of a grouped workload: the problems' A_g, their weights
    as one [G, ...] tensor, and fp32 outputs."""
    import torch
    from workloads import make_group_operands

    As, B = make_group_operands(gw)
    a = [x.cuda() for x in As]
    b = B.cuda()
    c = [torch.zeros((M, gw.N), dtype=torch.float32, device="cuda") for M in gw.Ms]
    return a, b, c


def grouped_arms(dg, name, rounds):
    """A grouped workload three ways: one grouped call (the rule over all the
    problems' tiles), one call per problem (the rule per problem), and a batched
    call over the problems padded to the largest row count; speedups paired
    against the per-problem calls."""
    import torch
    from workloads import GROUPED

    gw = GROUPED[name]
    a, b, c = grouped_operands(gw)
    G, Mmax = len(gw.Ms), max(gw.Ms)
    a_pad = torch.zeros((G, Mmax, gw.K), dtype=a[0].dtype, device="cuda")
    for g, x in enumerate(a):
        a_pad[g, : x.shape[0]] = x
    c_pad = torch.zeros((G, Mmax, gw.N), dtype=torch.float32, device="cuda")
    calls = {
        "separate": SeparateCalls([Call(dg, a[g], b[g], c[g], gw.b_layout, "heuristic") for g in range(G)]),
        "grouped": GroupedCall(dg, list(zip(a, b, c)), gw.b_layout),
        "grouped_64x128": GroupedCall(dg, list(zip(a, b, c)), gw.b_layout, tile="64x128"),
        "batched_padded": Call(dg, a_pad, b, c_pad, gw.b_layout, "heuristic"),
    }
    samples, pack = PROTOCOL[name[:2]]
    timed = time_arms(calls, rounds, samples, pack)
    out = {"Ms": list(gw.Ms), "N": gw.N, "K": gw.K, "dtype": gw.dtype, "b_layout": gw.b_layout,
           "protocol": {"rounds": rounds, "samples_per_round": samples, "calls_per_sample": pack,
                        "order": "rotated every sample, reversed every other round"}}
    # A and the outputs once, every problem's weights once
    compulsory = sum(M * gw.K * 2 + M * gw.N * 4 for M in gw.Ms) + G * gw.N * gw.K * 2
    for arm, call in calls.items():
        flat = [x for r in timed[arm] for x in r]
        med = statistics.median(flat)
        r = {"median_us": round(med, 3), "p10_us": round(_q(flat, 0.1), 3), "p90_us": round(_q(flat, 0.9), 3),
             "min_us": round(min(flat), 3),
             "tflops": round(gw.flops / (med * 1e-6) / 1e12, 2),   # useful flops (padding rows not counted)
             "pct_peak": round(100 * gw.flops / (med * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 2),
             "compulsory_gbps": round(compulsory / (med * 1e-6) / 1e9, 1)}
        plan = getattr(call, "plan", None)
        if plan is not None:
            r["decision"] = dg.DECISION_NAMES[plan.decision]
            r["tiles"] = int(plan.tiles)
            r["units_or_splits"] = int(plan.sk_units or plan.splits)
        if arm != "separate":
            r["speedup_vs_separate"] = paired_speedup(timed["separate"], timed[arm])
        out[arm] = r
        log(f"  {name:14s} {arm:20s} {r['median_us']:9.3f} us  {r['tflops']:8.2f} TFLOP/s"
            + (f"  x{r['speedup_vs_separate']['median']} vs separate" if "speedup_vs_separate" in r else ""))
    return out


def vendor_blas(dg, name, calls, rounds=6):
    """Context, not a baseline: the vendor BLAS (torch.mm with fp32 output) and
    this library's call on the workload's operands, timed alternately in this
    process (median over `rounds` of the mean of `calls` back-to-back calls)."""
    import torch
    from workloads import WORKLOADS, make_operands

    w = WORKLOADS[name]
    A, B = make_operands(w)
    a, b = A.cuda(), B.cuda()
    c = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    ours = Call(dg, a, b, c, w.b_layout, w.mode, w.splits, w.atomic)
    stream = ours.stream

    def vendor():
        torch.mm(a, b, out_dtype=torch.float32)

    res = {"ours": [], "vendor": []}
    with torch.cuda.stream(stream):
        for f in (ours, vendor):
            for _ in range(calls):
                f()
        torch.cuda.synchronize()
        for r in range(rounds):
            for tag, f in ((("ours", ours), ("vendor", vendor)) if r % 2 == 0 else
                           (("vendor", vendor), ("ours", ours))):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(calls):
                    f()
                e1.record(stream)
                torch.cuda.synchronize()
                res[tag].append(e0.elapsed_time(e1) * 1e3 / calls)
    o, v = statistics.median(res["ours"]), statistics.median(res["vendor"])
    return {"mode": w.mode, "ours_us": round(o, 3), "vendor_us": round(v, 3), "vendor_over_ours": round(v / o, 3)}


def kernel_kind(dg, plan):
    kind = {dg.GEMM_DP: "gemm_dp", dg.GEMM_SPLITK: "gemm_splitk", dg.GEMM_STREAMK: "gemm_streamk"}[plan.decision]
    # the library runs 2x2 tile groups when their waves finish sooner (its rule, restated)
    cus = dg.gemm_num_cus()
    groups = ((plan.tiles_m + 1) // 2) * ((plan.tiles_n + 1) // 2)
    if plan.decision == dg.GEMM_DP and -(-groups // cus) * 40 < -(-plan.tiles // cus) * 14:
        kind = "gemm_dp_group"
    return kind


def kernel_name(dg, plan, w):
    lay = "B[K,N]" if w.b_layout == "kn" else "B[N,K]"
    fix = (", atomic" if plan.atomic else ", deterministic") if plan.decision == dg.GEMM_STREAMK else ""
    tile = f", {plan.bm}x{plan.bn} tiles" if plan.bm != 128 else ""
    return f"{kernel_kind(dg, plan)}<{w.dtype}, {lay}{fix}{tile}>"


def profile_key(dg, plan, w):
    """Name of the committed profile summary of this launch (profiles/<key>.md)."""
    tile = f"_{plan.bm}x{plan.bn}" if plan.bm != 128 else ""
    return f"{kernel_kind(dg, plan)}_{w.dtype}_{w.b_layout}_{w.M}x{w.N}x{w.K}{tile}"


def kernel_code_digest(path=None) -> str:
    """sha256 of the kernel source with comments removed and whitespace runs
    collapsed: it changes with the code, not with its comments."""
    import hashlib
    import re

    path = path or ROOT / "dense_gemm_work_amd" / "csrc" / "gemm_kernels.hip"
    text = Path(path).read_text()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()


def measured_traffic(profile: str):
    """HBM bytes per launch of the profiled kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary `profile` (scaled by a plain copy of known
    size), or None when there is none or the kernel code has changed since it
    was taken."""
    path = ROOT / "profiles" / "traffic.json"
    if not path.exists():
        return None
    entry = json.loads(path.read_text()).get(profile)
    if not entry:
        return None
    if kernel_code_digest() != entry.get("code_sha256"):
        return None
    return int(entry["bytes"])


def _power_sensor():
    """The board power file (microwatts) and cap of the first GPU hwmon, or None."""
    import glob

    for d in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*")):
        p = os.path.join(d, "power1_input")
        if os.access(p, os.R_OK):
            cap = os.path.join(d, "power1_cap")
            cap_w = int(open(cap).read()) / 1e6 if os.access(cap, os.R_OK) else None
            return p, cap_w
    return None, None


def power_snapshot(dg, name, mode, splits=0, atomic=False, seconds=1.5):
    """Board power while `name` runs back to back for about `seconds` (sampled
    every 10 ms from the GPU's hwmon power1_input), next to the power cap."""
    import threading

    import torch
    from workloads import WORKLOADS, make_operands

    path, cap_w = _power_sensor()
    if path is None:
        return None
    w = WORKLOADS[name]
    A, B = make_operands(w)
    a, b = A.cuda(), B.cuda()
    c = torch.empty(((w.batch,) if w.batch > 1 else ()) + (w.M, w.N), dtype=torch.float32, device="cuda")
    call = Call(dg, a, b, c, w.b_layout, mode, splits, atomic)
    for _ in range(20):
        call()
    torch.cuda.synchronize()
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                samples.append(int(open(path).read()) / 1e6)
            except (OSError, ValueError):
                pass
            stop.wait(0.01)

    th = threading.Thread(target=sample, daemon=True)
    t0 = time.perf_counter()
    calls = 0
    th.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            call()
        calls += 20
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return None
    steady = sorted(samples[len(samples) // 4:]) or sorted(samples)   # past the ramp-up
    return {"watts_median": round(steady[len(steady) // 2], 1), "watts_max": round(max(samples), 1),
            "cap_watts": cap_w, "samples": len(samples), "calls": calls}


def cu_timeline(dg, name, mode, splits=0, atomic=False):
    """Per-CU busy time of one launch with the kernels' timing records (every
    workgroup stores its start and end on the 100 MHz clock plus the CU it ran
    on).  Returns the launch span, the busy fraction of the 256 CUs over the
    span (1 - idle fraction), and how the CUs' last end times spread."""
    import collections

    import numpy as np
    import torch
    from workloads import WORKLOADS, make_operands

    w = WORKLOADS[name]
    A, B = make_operands(w)
    a, b = A.cuda(), B.cuda()
    c = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    p = dg.gemm_plan(w.M, w.N, w.K, dg.layout_word(w.b_layout, w.dtype), dg.mode_word(mode, atomic), splits,
                     dg.gemm_num_cus())
    tim = torch.full((8 * int(p.workers),), -1, dtype=torch.int64, device="cuda")
    for _ in range(3):
        dg.gemm_tensors(a, b, c, b_layout=w.b_layout, mode=mode, splits=splits, atomic=atomic)
    dg.gemm_tensors(a, b, c, b_layout=w.b_layout, mode=mode, splits=splits, atomic=atomic, timing=tim)
    torch.cuda.synchronize()
    t = tim.cpu().numpy().reshape(-1, 8).astype(np.float64)
    t = t[t[:, 0] >= 0]
    t0 = t[:, 0].min()
    start, end = (t[:, 0] - t0) / 100.0, (t[:, 1] - t0) / 100.0      # microseconds
    span = float(end.max())
    # HW_ID: CU id in bits 8..11, shader array bit 12, shader engine bits 13..15; XCC_ID separately
    hwx = t[:, 2].astype(np.int64)
    hw, xcc = hwx & 0xFFFFFFFF, hwx >> 32
    # mean shader clock of each workgroup: s_memtime cycles over its real-time span
    mhz = t[:, 3] / np.maximum(t[:, 1] - t[:, 0], 1) * 100.0
    cu_key = xcc * 4096 + ((hw >> 13) & 7) * 256 + ((hw >> 12) & 1) * 16 + ((hw >> 8) & 15)
    busy, last = collections.defaultdict(float), collections.defaultdict(float)
    for k, s_, e_ in zip(cu_key, start, end):
        busy[k] += e_ - s_
        last[k] = max(last[k], e_)
    ncu = dg.gemm_num_cus()
    frac = sum(busy.values()) / (ncu * span)
    ends = np.array(sorted(last.values()))
    return {
        "decision": dg.DECISION_NAMES[p.decision], "workgroups": int(p.workers), "cus_used": len(busy),
        "span_us": round(span, 2), "busy_fraction": round(float(frac), 4), "idle_fraction": round(float(1 - frac), 4),
        "cu_last_end_us": {"min": round(float(ends.min()), 2), "median": round(float(np.median(ends)), 2),
                           "max": round(float(ends.max()), 2)},
        "shader_clock_mhz": {"median": round(float(np.median(mhz))), "min": round(float(mhz.min())),
                             "max": round(float(mhz.max()))},
    }


def cpu_baseline(w, A, B, min_seconds=10.0, max_runs=30):
    """The fp64 oracle timed on the host's cores over the whole workload, the
    product repeated until about `min_seconds` of CPU work are timed; also
    returns the first product's (C, S), which check the GPU's output."""
    from oracle import gemm as og

    t0 = time.perf_counter()
    C, S = og.ref_gemm(A, B, w.M, w.N, w.K, w.b_layout, w.dtype)
    secs, runs = time.perf_counter() - t0, 1
    while secs < min_seconds and runs < max_runs:
        t1 = time.perf_counter()
        og.ref_gemm(A, B, w.M, w.N, w.K, w.b_layout, w.dtype)
        secs += time.perf_counter() - t1
        runs += 1
    flops = 2.0 * w.M * w.N * w.K * runs
    return {
        "value": round(flops / secs / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": og.num_threads(),
        "kind": "oracle",
        "sample": f"all {w.M} rows of {w.M}x{w.N}x{w.K} ({w.dtype}), the whole product {runs} times: fp64 C and "
                  f"sum|a||b| in {secs:.1f} s; flops counted as 2*M*N*K of C only",
    }, (C, S)


def output_check(c_before, c_after, ref):
    """Every element of the timed call's output, as it stood before and after the
    timed region, against the fp64 oracle: |C - C_ref| <= 1e-4 sum|a||b| (Metal
    split-K note, "Comparison and independent confirmation": complete-output
    fp64 checks around the timing)."""
    import numpy as np

    from oracle import gemm as og

    C, S = ref
    res = {"elements": int(C.size), "tolerance": "1e-4 * sum_k |a_ik||b_kj|"}
    ok_all = True
    for tag, c in (("before", c_before), ("after", c_after)):
        ok, worst, idx = og.within_tolerance(c.numpy().astype(np.float64), C, S)
        res[f"worst_err_over_bound_{tag}"] = round(worst, 6)
        ok_all = ok_all and ok
    res["bit_identical_before_after"] = bool(np.array_equal(c_before.numpy().view(np.int32),
                                                            c_after.numpy().view(np.int32)))
    res["pass"] = bool(ok_all)
    return res


def copy_probe(mib: int) -> None:
    """One plain device copy of `mib` MiB: a dispatch of known size for scaling
    the HBM byte counters."""
    import torch

    if mib <= 0:
        return
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"bench: copy probe {mib} MiB read + {mib} MiB written")


def grouped_profile_key(dg, plan, gw) -> str:
    """Name of the committed profile summary of a grouped launch (profiles/<key>.md)."""
    kind = {dg.GEMM_DP: "gemm_dp", dg.GEMM_SPLITK: "gemm_splitk", dg.GEMM_STREAMK: "gemm_streamk"}[plan.decision]
    return (f"{kind}_grouped_{gw.dtype}_{gw.b_layout}_{len(gw.Ms)}_problems_{sum(gw.Ms)}x{gw.N}x{gw.K}"
            + (f"_{plan.bm}x{plan.bn}" if plan.bm != 128 else ""))


def grouped_main(args, dg) -> int:
    """--workload of a grouped workload: time exactly `steps` grouped calls (for
    profiling that launch), one JSON line; the headline workload is single."""
    import torch
    from workloads import GROUPED

    gw = GROUPED[args.workload]
    a, b, c = grouped_operands(gw)
    mode = args.mode or "heuristic"
    call = GroupedCall(dg, list(zip(a, b, c)), gw.b_layout, mode, args.splits or 0, tile=args.tile)
    p = call.plan
    log(f"bench: {gw.name} {len(gw.Ms)} problems, {p.tiles} tiles, plan={dg.DECISION_NAMES[p.decision]} "
        f"units={p.sk_units} steps={args.steps} warmup={args.warmup}")
    wall, ev_ms = time_call(call, args.steps, args.warmup)
    st = dg.gemm_sync_status()
    if st != 0:
        raise RuntimeError(f"device status {st}: {dg.gemm_last_error()}")
    kern_ms = ev_ms / args.steps
    achieved = gw.flops / (kern_ms * 1e-3) / 1e12
    log(f"bench: kernel mean {kern_ms * 1e3:.2f} us ({achieved:.1f} TFLOP/s)")
    copy_probe(args.copy_probe_mb)
    profile = grouped_profile_key(dg, p, gw)
    line = {
        "metric": "grouped GEMM TFLOP/s (useful flops)", "value": round(gw.flops * args.steps / wall / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5), "higher_is_better": True, "scaling": "strong",
        "vs_baseline": None, "dtype": gw.dtype, "data": f"synthetic (seeded uniform[{gw.low},{gw.high}))",
        "config": {"workload": f"{gw.name}: {len(gw.Ms)} problems M={list(gw.Ms)}, N={gw.N}, K={gw.K}, "
                               f"{p.bm}x{p.bn}x64 tiles, {mode} -> {dg.DECISION_NAMES[p.decision]}",
                   "tiles": int(p.tiles), "cus": dg.gemm_num_cus()},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(profile),
                     "kernel_mean_us": round(kern_ms * 1e3, 3)},
    }
    print(json.dumps(line), flush=True)
    return 0


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding over several GPUs is designed, not implemented).", file=sys.stderr)
        return 2
    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    import dense_gemm_work_amd as dg
    from workloads import GROUPED, WORKLOADS, make_operands

    if args.workload in GROUPED:
        return grouped_main(args, dg)
    w = WORKLOADS[args.workload]
    if args.mode is not None:
        w = w.with_(mode=args.mode, splits=args.splits if args.splits is not None else 0,
                    atomic=args.atomic)
    if args.shape is not None:
        M, N, K = (int(x) for x in args.shape.lower().split("x"))
        w = w.with_(name=f"{w.name}@{M}x{N}x{K}", M=M, N=N, K=K)
    A, B = make_operands(w)
    a, b = A.cuda(), B.cuda()
    c = torch.empty(((w.batch,) if w.batch > 1 else ()) + (w.M, w.N), dtype=torch.float32, device="cuda")
    call = Call(dg, a, b, c, w.b_layout, w.mode, w.splits, w.atomic, tile=args.tile)
    log(f"bench: {w.name} {w.M}x{w.N}x{w.K} {w.dtype} plan={dg.plan_dict(call.plan)['decision_name']} "
        f"units={call.plan.sk_units} steps={args.steps} warmup={args.warmup}")

    # ---- headline: whole-job throughput over exactly `steps` steps ----------------
    call()
    torch.cuda.synchronize()
    c_before = c.cpu()   # the output of an untimed call, checked against the oracle below
    wall, ev_ms = time_call(call, args.steps, args.warmup)
    c_after = c.cpu()    # ... and the output of the last timed call
    ms_per_step = wall * 1e3 / args.steps
    value = w.flops * args.steps / wall / 1e12
    kern_ms = ev_ms / args.steps
    achieved = w.flops / (kern_ms * 1e-3) / 1e12
    st = dg.gemm_sync_status()
    if st != 0:
        raise RuntimeError(f"device status {st}: {dg.gemm_last_error()}")
    log(f"bench: {value:.1f} TFLOP/s whole-job, kernel mean {kern_ms * 1e3:.2f} us "
        f"({achieved:.1f} TFLOP/s, {100 * achieved / PEAK_BF16_TFLOPS:.1f}% of peak)")

    # ---- arms on the same shape and the other shapes -------------------------------
    copy_probe(args.copy_probe_mb)

    shapes = {}
    if not args.no_shapes:
        for name in ("c3_wavequant", "c1_sk32", "c2a_m96_s8", "c2b_m256_s2", "c5_longk_fp16", "c4_large_dp",
                     "x1_hybrid", "x2_batched", "x3_decode"):
            shapes[name] = shape_arms(dg, name, args.rounds)
        shapes["x4_grouped"] = grouped_arms(dg, "x4_grouped", args.rounds)
    vendor = {}
    if args.vendor and not args.no_shapes:
        # operands with B [K,N] only (torch.mm is then given contiguous operands)
        for name, calls in (("c3_wavequant", 100), ("c5_longk_fp16", 50), ("c4_large_dp", 5), ("x1_hybrid", 30)):
            vendor[name] = vendor_blas(dg, name, calls)
            log(f"  vendor {name:14s} {vendor[name]}")
    c3 = shapes.get("c3_wavequant", {})
    speedups = {}
    if c3:
        speedups["streamk_vs_dp"] = c3["heuristic"]["speedup_vs_dp"]
        for arm in ("splitk2", "splitk4"):
            # Stream-K over Split-K: quotient of the two arms' paired speedups over DP
            speedups[f"streamk_vs_{arm}"] = round(c3["heuristic"]["speedup_vs_dp"]["median"] /
                                                  c3[arm]["speedup_vs_dp"]["median"], 3)

    timeline = {}
    if not args.no_timeline:
        for key, (name, mode, splits, atomic) in {
            "c3_dp": ("c3_wavequant", "dp", 0, False), "c3_streamk": ("c3_wavequant", "heuristic", 0, False),
            "c5_dp": ("c5_longk_fp16", "dp", 0, False), "c5_streamk": ("c5_longk_fp16", "streamk", 0, False),
        }.items():
            timeline[key] = cu_timeline(dg, name, mode, splits, atomic)
            log(f"  timeline {key:11s} {timeline[key]}")

    power = {}
    if not args.no_timeline:
        for key, (name, mode) in {"c3_streamk": ("c3_wavequant", "heuristic"),
                                  "c4_dp": ("c4_large_dp", "heuristic")}.items():
            power[key] = power_snapshot(dg, name, mode)
            log(f"  power {key:11s} {power[key]}")

    cpu, check = None, None
    if not args.no_cpu and w.batch == 1:
        log("bench: timing the fp64 CPU oracle on the same workload")
        cpu, ref = cpu_baseline(w, A, B)
        log(f"bench: cpu oracle {cpu['value']} TFLOP/s on {cpu['cores']} threads")
        check = output_check(c_before, c_after, ref)
        del ref
        log(f"bench: output check {check}")

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded " + (f"normal(0,1)*{w.scale}" if w.dist == "normal" else
                                        f"uniform[{w.low},{w.high})") + f" rounded to {w.dtype})",
        "config": {
            "workload": f"{w.name}: {w.dtype.upper()} GEMM {w.M}x{w.N}x{w.K}, "
                        f"B {'[K,N]' if w.b_layout == 'kn' else '[N,K]'}, fp32 out, "
                        f"{call.plan.bm}x{call.plan.bn}x64 tiles, {w.mode} -> "
                        f"{dg.DECISION_NAMES[call.plan.decision]}"
                        + (f" ({call.plan.sk_units} units x {call.plan.q} iterations)"
                           if call.plan.decision == dg.GEMM_STREAMK else
                           f" (S = {call.plan.splits})" if call.plan.decision == dg.GEMM_SPLITK else ""),
            "M": w.M, "N": w.N, "K": w.K, "tiles": int(call.plan.tiles), "cus": dg.gemm_num_cus(),
        },
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "speedups": speedups,
        "roofline": {
            "bound": "mfma",
            "kernel": kernel_name(dg, call.plan, w),
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(profile_key(dg, call.plan, w)),
            "kernel_mean_us": round(kern_ms * 1e3, 3),
        },
        "cpu_baseline": cpu,
        "output_check": check,
        "cu_timeline": timeline,
        "power": power,
        "shapes": shapes,
        "vendor_blas": vendor,
    }
    print(json.dumps(line), flush=True)
    if check is not None and not check["pass"]:
        log("bench: the timed call's output is outside the oracle's tolerance")
        return 3
    return 0


if __name__ == "__main__":
    sys.exit(main())
