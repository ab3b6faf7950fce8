#!/usr/bin/env python3
"""Bench: staged halo exchange on one MI355X (coordinates Z->Y->X with relay,
forces X->Y->Z with scatter-add), all domains virtual ranks in one GPU's HBM.

A step is one coordinate pass plus one force pass over the workload's
synthetic atoms (the whole hot path; the map build runs once before the
timed region and is reported separately, as a neighbour-search step would
be). Inputs are resident in HBM when timing starts. Default workload: 12,000,000
atoms, 8x8x8 domains, rc 1.2 nm (the largest one-GPU configuration, the one
the bandwidth target is stated for); the other four workloads follow under
`also`. Variant "auto" (default) runs what the library's automatic mode
picks: "step" (both passes in one launch, all pulses chained on device
counters) for a small pass, "pulse" (one launch per pulse) for a large one.

Prints one JSON line. `value` is halo atoms moved per second (sum of every
(domain, pulse) map size, counted once per pass). The timed region replays a
graph of G captured steps (G at most --graph-steps, and small enough that
--steps gives at least five replays), so the host never starves the GPU;
HIP events on the launch stream bracket every replay, and the median, p10
and p90 are taken over the replays. `cold` times the same workload with the
caches evicted before every (eager) step by reading a 1 GiB buffer (so they
hold only clean lines), and once more with the buffer written instead (the
step then also writes back the eviction's dirty lines). `roofline` compares the
step's algorithmic bytes (28 B per halo atom for the coordinate pass, 40 B
for the force pass) with the 8 TB/s HBM peak over the measured GPU time per
launch; `cpu_baseline` times the CPU oracle on a bounded sample of the same
workload. The 96k and 1M entries under `also` carry `overlap`: the step
beside a bf16 matrix-product load on a second stream (per-pulse launches,
and the fused launch at one work-group per compute unit, at half and at a
quarter of them).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1..5]
       [--variant auto|step|split|pulse|staged] [--cold] [--eager]
Counter traffic: profiles/traffic_<variant>_<workload>.md, written by
`python bench.py --summarize-pmc FETCH_CSV WRITE_CSV ...` from two rocprofv3
--pmc runs of this script with --copy-probe; it is reported only while the
exchange kernel source is unchanged since those runs.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import shlex
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "halo exchange µs/step + halo atoms/s & HBM GB/s fraction (1 MI355X)"
HBM_PEAK_GBS = 8000.0
BYTES_X, BYTES_F = 28, 40
# calls behind each side figure (each pass alone, flags off, the single
# fused launch), in graphs of --graph-steps calls
AUX_CALLS = 200
# workloads whose entry under `also` carries the overlap figures (96k, 1M)
OVERLAP_WORKLOADS = (2, 3)
# the sources that decide what the exchange launches read and write
KERNEL_SRCS = [os.path.join(ROOT, "domain_decomposition_halo_amd", "csrc", f)
               for f in ("ddh_exchange.hip", "ddh_build.hip", "ddh_internal.h")]
PROFILES = os.path.join(ROOT, "profiles")
VARIANTS = ("auto", "step", "split", "pulse", "staged")


def graph_size(steps: int, graph_steps: int, min_replays: int = 5) -> int:
    """Steps per captured graph in the timed region: the largest divisor of
    `steps` that is at most `graph_steps` and still leaves `min_replays`
    replays (one step per graph when `steps` is below that), so exactly
    `steps` steps are timed and the replays give a spread."""
    cap = max(1, min(graph_steps, steps // min_replays))
    return max(d for d in range(1, cap + 1) if steps % d == 0)


def code_text(src: str) -> str:
    """C++ source without its comments and with whitespace runs collapsed:
    what the compiler sees, so that an edit of the comments alone keeps the
    stored counters current. String literals are kept as written."""
    out, i, n = [], 0, len(src)
    while i < n:
        ch = src[i]
        if ch == '"' or ch == "'":
            j = i + 1
            while j < n and src[j] != ch:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(ch)
            i += 1
    return " ".join("".join(out).split())


def kernel_hash() -> str:
    """Hash of the code (comments aside) of the sources that decide what the
    exchange launches read and write."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_file(variant: str, wname: str, pass_: str = "step") -> str:
    tag = variant if pass_ == "step" else f"{variant}_{pass_}"
    return os.path.join(PROFILES, f"traffic_{tag}_{wname}.md")


def read_traffic(variant: str, wname: str, pass_: str = "step"):
    """Counter bytes per launch from a stored summary, if still current."""
    path = traffic_file(variant, wname, pass_)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != kernel_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ GPU run

def run_gpu(args, w):
    import numpy as np
    import torch

    import domain_decomposition_halo_amd as ddh
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    x = W.positions(w)
    xg = torch.from_numpy(x).to(dev)
    plan = ddh.Plan(**w.params())
    # the timed region replays captured graphs itself, so the library's own
    # graph mode stays off here
    mode = {"auto": ddh.DDH_MODE_AUTO, "step": ddh.DDH_MODE_FUSED, "split": ddh.DDH_MODE_FUSED,
            "pulse": ddh.DDH_MODE_PULSE, "staged": ddh.DDH_MODE_STAGED}[args.variant]
    if args.lib_graph:
        if not args.eager:
            sys.exit("--lib-graph replays the library's own graphs: use it with --eager")
        mode |= ddh.DDH_MODE_GRAPH
    plan.set_mode(mode)
    if args.chunk:
        plan.tune(ddh.DDH_TUNE_CHUNK, args.chunk)
    if args.grid:
        plan.tune(ddh.DDH_TUNE_GRID, args.grid)
    if args.block:
        plan.tune(ddh.DDH_TUNE_BLOCK, args.block)
    if args.static_first:
        plan.tune(ddh.DDH_TUNE_STATIC_FIRST, 1)
    if args.no_flags:
        plan.tune(ddh.DDH_TUNE_FLAGS, 0)
    if args.wide_maps:
        plan.tune(ddh.DDH_TUNE_NARROW_MAPS, 0)
    if args.wave_chunks:
        plan.tune(ddh.DDH_TUNE_WAVE_CHUNKS, 1)
    if args.exit_publish:
        plan.tune(ddh.DDH_TUNE_EXIT_PUBLISH, args.exit_publish)
    if args.pad_maps:
        plan.tune(ddh.DDH_TUNE_PAD_MAPS, args.pad_maps)
    if args.heads_first:
        plan.tune(ddh.DDH_TUNE_HEADS_FIRST, 1)
    if args.home_sort:
        plan.tune(ddh.DDH_TUNE_HOME_SORT, args.home_sort)
    if args.lds_stage:
        plan.tune(ddh.DDH_TUNE_LDS_STAGE, args.lds_stage)

    torch.cuda.synchronize()
    lay = plan.build_maps(xg)
    torch.cuda.synchronize()
    # the reported build time: the median of nine warm rebuilds
    builds = []
    for _ in range(9):
        t0 = time.perf_counter()
        lay = plan.build_maps(xg)
        torch.cuda.synchronize()
        builds.append((time.perf_counter() - t0) * 1e3)
    build_ms = sorted(builds)[len(builds) // 2]

    n_slots, n_halo = lay["n_slots"], lay["n_halo"]
    # "auto" runs what the library's automatic mode picks: per-pulse launches
    # when the calls are replayed from a graph, and for eager calls unless the
    # pass is tiny
    variant = args.variant
    if variant == "auto":
        eager = (args.eager or args.cold) and not args.lib_graph
        variant = "step" if (eager and n_halo <= ddh.DDH_AUTO_FUSED_MAX) else "pulse"
    xl = torch.zeros((n_slots, 3), dtype=torch.float32, device=dev)
    plan.gather_home(xg, xl)
    fl = torch.from_numpy(W.forces(w, n_slots)).to(dev)
    flush = None
    if args.cold:
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

    if args.pass_ == "coords":
        calls = [("coords", lambda: plan.exchange_coords(xl), BYTES_X * n_halo)]
    elif args.pass_ == "forces":
        calls = [("forces", lambda: plan.exchange_forces(fl), BYTES_F * n_halo)]
    elif variant == "split":
        calls = [("coords", lambda: plan.exchange_coords(xl), BYTES_X * n_halo),
                 ("forces", lambda: plan.exchange_forces(fl), BYTES_F * n_halo)]
    else:
        calls = [("step", lambda: plan.exchange_step(xl, fl), (BYTES_X + BYTES_F) * n_halo)]

    # pulse mode: a step pairs coordinate pulse q with force pulse P-1-q in
    # one launch, then one flag launch
    # (a call whose last launch publishes its own flags needs no flag launch)
    exit_pub = args.exit_publish == 1
    launches_per_step = {"step": 1, "split": 2,
                         "staged": 2 * lay["n_pulses"] + 1}.get(
        variant, lay["n_pulses"] + (0 if (args.no_flags or exit_pub) else 1))
    for _ in range(args.warmup):
        for _, fn, _ in calls:
            fn()
    assert plan.check() == ddh.DDH_OK

    torch.cuda.synchronize()
    if args.cold:
        # eager, one step at a time: caches evicted before every step; the
        # eviction keeps the GPU busy while the host enqueues the step.
        # Reading 1 GiB leaves only clean lines behind; writing it leaves
        # dirty lines that the step's own traffic then writes back.
        durs = []
        for _ in range(args.steps):
            if args.cold_flush == "write":
                flush.fill_(1.0)
            else:
                flush.sum()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _, fn, _ in calls:
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            durs.append(e0.elapsed_time(e1) * 1e-3)
        wall = sum(durs)
        steps_done = args.steps
    elif args.eager:
        # eager: the host enqueues every call of every step itself (no graph),
        # as an MD code without graph capture would
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            for _, fn, _ in calls:
                fn()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        steps_done = args.steps
        durs = [e0.elapsed_time(e1) * 1e-3 / args.steps]
    else:
        # G steps captured in one graph and replayed: the host enqueues one
        # graph per G steps, so the GPU never waits for the host. G divides
        # the step count, so exactly --steps steps are timed.
        G = graph_size(args.steps, args.graph_steps, args.min_replays)
        n_rep = args.steps // G
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(G):
                for _, fn, _ in calls:
                    fn()
        graph.replay()
        torch.cuda.synchronize()
        assert plan.check() == ddh.DDH_OK
        evs = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n_rep):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        steps_done = n_rep * G
        durs = [a.elapsed_time(b) * 1e-3 / G for a, b in evs]
        del graph
    assert plan.check() == ddh.DDH_OK

    # each pass alone (pack = coordinate pass, unpack = force pass), the same
    # way: graphs of G calls, replayed. These side figures take AUX_CALLS
    # calls whatever --steps is, so a short headline run does not leave them
    # to one replay of a small graph.
    passes = None
    if not args.cold and not args.eager and not args.only_step:
        passes = {}
        G = max(1, args.graph_steps)
        n_rep = max(1, AUX_CALLS // G)
        for name, fn, nb in (("coords", lambda: plan.exchange_coords(xl), BYTES_X * n_halo),
                             ("forces", lambda: plan.exchange_forces(fl), BYTES_F * n_halo)):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(G):
                    fn()
            graph.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n_rep):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (n_rep * G)
            passes[name + "_us"] = round(us, 3)
            passes[name + "_frac"] = round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
            del graph
        assert plan.check() == ddh.DDH_OK

    def time_steps(fn, reps):
        """GPU us per call of fn, from graphs of G calls replayed reps times."""
        G = max(1, args.graph_steps)
        fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(G):
                fn()
        graph.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        del graph
        return e0.elapsed_time(e1) * 1e3 / (reps * G)

    # the same step with the completion flags off (callers that rely on
    # stream order alone): one launch fewer per call in per-pulse mode
    without_flags = None
    if not args.cold and not args.eager and not args.only_step and not args.no_flags:
        plan.tune(ddh.DDH_TUNE_FLAGS, 0)
        us = time_steps(calls[0][1] if len(calls) == 1 else
                        (lambda: [fn() for _, fn, _ in calls]),
                        max(1, AUX_CALLS // max(1, args.graph_steps)))
        plan.tune(ddh.DDH_TUNE_FLAGS, 1)
        without_flags = {"us_per_step": round(us, 3),
                         "frac": round((BYTES_X + BYTES_F) * n_halo / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        assert plan.check() == ddh.DDH_OK

    # the single persistent launch (both passes, all pulses, one kernel), the
    # same way, when it is not already the variant timed above
    single = None
    if not args.cold and not args.eager and not args.only_step and variant != "step":
        plan.set_mode(ddh.DDH_MODE_FUSED)
        G = max(1, args.graph_steps)
        n_rep = max(1, AUX_CALLS // G)
        fn = lambda: plan.exchange_step(xl, fl)
        fn()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(G):
                fn()
        graph.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_rep):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (n_rep * G)
        single = {"kernel": "wave_kernel" if args.wave_chunks else "exchange_kernel",
                  "us_per_step": round(us, 3),
                  "frac": round((BYTES_X + BYTES_F) * n_halo / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del graph
        assert plan.check() == ddh.DDH_OK

    # the latency floor of the same number of dependent launches: tiny
    # one-block kernels (a one-element add) replayed from a graph
    launch_floor = None
    if not args.cold and not args.eager and variant != "staged":
        tiny = torch.zeros(1, dtype=torch.float32, device=dev)
        G = 50
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(G * launches_per_step):
                tiny.add_(1.0)
        graph.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(4):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        launch_floor = e0.elapsed_time(e1) * 1e3 / (4 * G)
        del graph

    durs = sorted(durs)
    avg_step_gpu = sum(durs) / len(durs)
    step_bytes = sum(nb for _, _, nb in calls)
    avg_launch = avg_step_gpu / launches_per_step
    achieved = step_bytes / avg_step_gpu / 1e9
    # the stored counters were taken with the default settings
    tuned = (args.chunk or args.grid or args.block or args.static_first or args.no_flags
             or args.wide_maps or args.wave_chunks or args.cold or args.exit_publish
             or args.pad_maps or args.heads_first or args.lds_stage or args.pass_ != "step")
    traffic = None if tuned else read_traffic(variant, w.name)
    if passes is not None:
        # each pass's counter traffic, from its own stored summary
        for nm in ("coords", "forces"):
            t = None if tuned else read_traffic(variant, w.name, nm)
            passes[nm + "_traffic"] = t
    fused_name = "wave_kernel" if args.wave_chunks else "exchange_kernel"
    kernel = {"step": f"{fused_name} (fused step, one launch)",
              "split": f"{fused_name} (coordinate launch + force launch)",
              "staged": "pulse_kernel pack/unpack + one hipMemcpyAsync per sender and pulse, "
                        "two host waits per pulse"}.get(
                  variant, "pulse_kernel (coordinate pulse q + force pulse P-1-q per launch) + signal_kernel")

    if args.copy_probe:
        # a plain copy of known size, for scaling the HBM byte counters
        nb = args.copy_probe << 20
        a = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()

    # the kernels read 16-bit map entries when every domain has at most
    # 65536 slots: the bytes a step must move are then 2 B per entry and
    # pass below the 28 + 40 B of the index-map accounting
    max_total = max(plan.domain_info(d)[2] for d in range(lay["n_domains"]))
    map_bytes = 2 if (max_total <= 65536 and not args.wide_maps) else 4
    min_bytes = step_bytes - 2 * (4 - map_bytes) * n_halo

    step_s = wall / steps_done
    res = dict(
        n_slots=n_slots, n_halo=n_halo, n_pulses=lay["n_pulses"], build_ms=build_ms,
        variant=variant, passes=passes, single=single, without_flags=without_flags,
        step_s=step_s, steps=steps_done, gpu_step_us=round(avg_step_gpu * 1e6, 3),
        roofline=dict(bound="hbm", achieved=round(achieved, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic, kernel=kernel,
                      launches_per_step=launches_per_step,
                      per="launch" if launches_per_step == 1 else
                          f"step ({launches_per_step} launches; achieved and traffic are per step)",
                      algorithmic_bytes_per_step=step_bytes,
                      map_entry_bytes=map_bytes,
                      min_bytes_per_step=min_bytes,
                      frac_at_min_bytes=round(min_bytes / avg_step_gpu / 1e9 / HBM_PEAK_GBS, 4),
                      avg_launch_us=round(avg_launch * 1e6, 3),
                      traffic_GBps=(round(traffic / avg_step_gpu / 1e9, 2) if traffic else None),
                      latency=dict(
                          hop_count=2 * lay["n_pulses"],
                          dependent_stages=lay["n_pulses"] if variant in ("pulse", "step")
                          else 2 * lay["n_pulses"],
                          launches_per_step=launches_per_step,
                          launch_floor_us=(round(launch_floor, 3) if launch_floor else None),
                          hbm_floor_us=round(step_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 3)),
                      median_step_us=round(durs[len(durs) // 2] * 1e6, 3),
                      p10_step_us=round(durs[len(durs) // 10] * 1e6, 3),
                      p90_step_us=round(durs[(9 * len(durs)) // 10] * 1e6, 3)),
    )
    plan.close()
    return res


# ------------------------------------------------------------- map builds

def run_builds(args, w):
    """The map build alone, as at every neighbour-search step: one plan
    rebuilt --steps times from the same positions (after one warm-up build);
    host wall time per build, the device work included."""
    import torch

    import domain_decomposition_halo_amd as ddh
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    xg = torch.from_numpy(W.positions(w)).to(dev)
    plan = ddh.Plan(**w.params())
    if args.home_sort:
        plan.tune(ddh.DDH_TUNE_HOME_SORT, args.home_sort)
    plan.build_maps(xg)
    torch.cuda.synchronize()
    times = []
    for _ in range(args.steps):
        t0 = time.perf_counter()
        plan.build_maps(xg)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    plan.close()
    times.sort()
    return {"workload": w.name, "builds": len(times),
            "median_ms": round(times[len(times) // 2] * 1e3, 3),
            "mean_ms": round(sum(times) / len(times) * 1e3, 3),
            "min_ms": round(times[0] * 1e3, 3)}


# ------------------------------------------------------ overlap with compute

def overlap_once(w, mode_name, grid=0, static_first=False, no_flags=False, wide_maps=False,
                 wave_chunks=False, dim=2048, reps=4):
    """Exchange step beside a CU-filling compute load on a second stream.

    The load stands in for the local non-bonded work that runs while the
    halo exchange is in flight: a chain of `reps` bf16 matrix products of
    size dim. Every stream keeps the default priority. Each of (load alone,
    exchange alone, both) is captured as G iterations in one graph (the two
    streams forked and joined inside it) and replayed; exposed = both - load
    alone, hidden = 1 - exposed / exchange alone. grid > 0 caps the fused
    launch's work-groups (DDH_TUNE_GRID), leaving compute units to the
    load."""
    import torch

    import domain_decomposition_halo_amd as ddh
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    main_s = torch.cuda.current_stream()
    x = W.positions(w)
    xg = torch.from_numpy(x).to(dev)
    plan = ddh.Plan(**w.params())
    mode = {"auto": ddh.DDH_MODE_AUTO, "step": ddh.DDH_MODE_FUSED,
            "pulse": ddh.DDH_MODE_PULSE}.get(mode_name, ddh.DDH_MODE_AUTO)
    plan.set_mode(mode)
    if grid:
        plan.tune(ddh.DDH_TUNE_GRID, grid)
    if static_first:
        plan.tune(ddh.DDH_TUNE_STATIC_FIRST, 1)
    if no_flags:
        plan.tune(ddh.DDH_TUNE_FLAGS, 0)
    if wide_maps:
        plan.tune(ddh.DDH_TUNE_NARROW_MAPS, 0)
    if wave_chunks:
        plan.tune(ddh.DDH_TUNE_WAVE_CHUNKS, 1)
    lay = plan.build_maps(xg)
    n_slots = lay["n_slots"]
    xl = torch.zeros((n_slots, 3), dtype=torch.float32, device=dev)
    plan.gather_home(xg, xl)
    fl = torch.from_numpy(W.forces(w, n_slots)).to(dev)
    g = torch.Generator(device="cpu").manual_seed(7)
    a = torch.randn((dim, dim), generator=g).to(dev, torch.bfloat16)
    b = torch.randn((dim, dim), generator=g).to(dev, torch.bfloat16)
    c = torch.empty((dim, dim), dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream()

    def load():
        for _ in range(reps):
            torch.mm(a, b, out=c)

    def exchange():
        plan.exchange_step(xl, fl)

    def both():
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            load()
        exchange()
        torch.cuda.current_stream().wait_stream(side)

    G = 20
    out = {}
    for name, fn in (("load", load), ("exchange", exchange), ("both", both)):
        fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(G):
                fn()
        graph.replay()
        torch.cuda.synchronize()
        best = None
        for _ in range(5):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(main_s)
            graph.replay()
            e1.record(main_s)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / G
            best = us if best is None else min(best, us)
        out[name + "_us"] = round(best, 3)
        del graph
    assert plan.check() == ddh.DDH_OK
    plan.close()
    exposed = out["both_us"] - out["load_us"]
    out["exposed_exchange_us"] = round(exposed, 3)
    out["hidden_frac"] = round(1.0 - exposed / out["exchange_us"], 4) if out["exchange_us"] else None
    return out


def overlap_set(w, dim=2048, reps=4):
    """The overlap of the per-pulse launches and of the fused launch, the
    latter at its automatic grid (one work-group per compute unit) and
    capped at half and a quarter of the compute units."""
    import torch

    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    res = {"load": f"{reps} x bf16 mm {dim}x{dim}x{dim} on a second stream (default priority)",
           "how": "graphs of 20 iterations, best of 5 replays; exposed = both - load alone, "
                  "hidden = 1 - exposed / exchange alone"}
    for key, mode, grid in (("per_pulse", "pulse", 0), ("fused", "step", 0),
                            ("fused_grid_half", "step", n_cu // 2),
                            ("fused_grid_quarter", "step", n_cu // 4)):
        o = overlap_once(w, mode, grid=grid, dim=dim, reps=reps)
        if grid:
            o["grid"] = grid
        res[key] = o
    return res


def run_overlap(args, w):
    """--overlap: one exchange mode beside the compute load (its own JSON)."""
    out = overlap_once(w, args.variant, grid=args.grid, static_first=args.static_first,
                       no_flags=args.no_flags, wide_maps=args.wide_maps,
                       wave_chunks=args.wave_chunks, dim=args.overlap_dim, reps=args.overlap_reps)
    out["load"] = (f"{args.overlap_reps} x bf16 mm {args.overlap_dim}x{args.overlap_dim}x"
                   f"{args.overlap_dim} on a second stream (default priority)")
    out["workload"] = w.name
    out["mode"] = args.variant
    if args.grid:
        out["grid"] = args.grid
    return out


# ------------------------------------------------------ fused launch events

def run_event_trace(args, w, out_path):
    """One fused step with the library's device event log (DDH_TUNE_TRACE):
    per work-group, the ticket claims, independent part done, wait done,
    chunk done, release and exit, on the 100 MHz wall clock. Writes a summary
    per stage (pass and pulse): when its chunks start and end, and the
    medians of their work, wait and release times."""
    import collections

    import numpy as np
    import torch

    import domain_decomposition_halo_amd as ddh
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    xg = torch.from_numpy(W.positions(w)).to(dev)
    plan = ddh.Plan(**w.params())
    plan.set_mode(ddh.DDH_MODE_FUSED)
    grid = args.grid or torch.cuda.get_device_properties(dev).multi_processor_count
    if args.grid:
        plan.tune(ddh.DDH_TUNE_GRID, args.grid)
    if args.heads_first:
        plan.tune(ddh.DDH_TUNE_HEADS_FIRST, 1)
    lay = plan.build_maps(xg)
    n = lay["n_slots"]
    xl = torch.zeros((n, 3), dtype=torch.float32, device=dev)
    plan.gather_home(xg, xl)
    fl = torch.from_numpy(W.forces(w, n)).to(dev)
    for _ in range(max(args.warmup, 3)):
        plan.exchange_step(xl, fl)
    torch.cuda.synchronize()
    buf = torch.zeros(2 * 64 * grid, dtype=torch.int64, device=dev)
    plan.tune(ddh.DDH_TUNE_TRACE, buf.data_ptr())
    plan.exchange_step(xl, fl)
    torch.cuda.synchronize()
    plan.tune(ddh.DDH_TUNE_TRACE, 0)
    assert plan.check() == ddh.DDH_OK
    D, P = lay["n_domains"], lay["n_pulses"]
    # tickets: coordinate chunks pulse by pulse (with --heads-first: every
    # pulse's heads, then every pulse's tails), then force chunks in
    # decreasing pulse order. At the fused launch's default chunk size of
    # 8192 entries a map of n entries has max(1, ceil(n / 8192)) chunks, or
    # ceil(head / 8192) + ceil(tail / 8192) (at least one) heads first.
    CH = 8192
    info = [[plan.pulse_info(S, q) for q in range(P)] for S in range(D)]
    def n_head(S, q):
        n, h = info[S][q][0], info[S][q][1]
        nh, nt = -(-h // CH), -(-(n - h) // CH)
        return nh if nh + nt else 1
    def n_tail(S, q):
        n, h = info[S][q][0], info[S][q][1]
        return -(-(n - h) // CH)
    def n_all(S, q):
        return n_head(S, q) + n_tail(S, q) if args.heads_first else max(1, -(-info[S][q][0] // CH))
    bounds = []
    acc = 0
    if args.heads_first:
        for q in range(P):
            m = sum(n_head(S, q) for S in range(D))
            bounds.append((acc, acc + m, f"coords heads pulse {q}"))
            acc += m
        for q in range(P):
            m = sum(n_tail(S, q) for S in range(D))
            bounds.append((acc, acc + m, f"coords tails pulse {q}"))
            acc += m
    else:
        for q in range(P):
            m = sum(n_all(S, q) for S in range(D))
            bounds.append((acc, acc + m, f"coords pulse {q}"))
            acc += m
    for q in range(P - 1, -1, -1):
        m = sum(n_all(S, q) for S in range(D))
        bounds.append((acc, acc + m, f"forces pulse {q}"))
        acc += m
    rec = buf.cpu().numpy().view(np.uint64).reshape(grid, 64, 2)
    starts = [int(rec[b, 0, 1]) for b in range(grid) if int(rec[b, 0, 0]) >> 32 == 1]
    t0 = min(starts)
    chunks, exits = [], []
    for b in range(grid):
        cur = None
        for r in rec[b]:
            code, info, t = int(r[0]) >> 32, int(r[0]) & 0xFFFFFFFF, (int(r[1]) - t0) * 10
            if code == 2:
                if cur:
                    chunks.append(cur)
                cur = dict(wg=b, ticket=info, claim=t)
            elif code in (3, 4, 5, 6) and cur is not None:
                cur[{3: "head", 4: "waited", 5: "done", 6: "released"}[code]] = t
                if code == 5:
                    cur["n"] = info
            elif code == 7:
                if cur:
                    chunks.append(cur)
                cur = None
                exits.append(t)
    plan.close()
    if not exits:
        # a work-group that logged more than 64 events stops logging: its
        # exit is then the last event it logged
        exits = [max(c.get("released", c.get("done", c["claim"])) for c in chunks)]

    def stage(t):
        return next((name for lo, hi, name in bounds if lo <= t < hi), "other")
    by = collections.defaultdict(list)
    for c in chunks:
        by[stage(c["ticket"])].append(c)
    span = max(exits) / 1e3

    def q3(vals):
        a = np.asarray(vals, dtype=np.float64) / 1e3
        return "%.2f / %.2f / %.2f" % (np.percentile(a, 10), np.median(a), np.percentile(a, 90))
    order = [name for _, _, name in bounds]
    busy = collections.defaultdict(float)
    for c in chunks:
        busy[c["wg"]] += c.get("released", c.get("done", c["claim"])) - c["claim"]
    with open(out_path, "w") as fh:
        fh.write(f"# Fused launch event log, workload {w.name}\n\n")
        fh.write("One fused step (`exchange_kernel`, both passes, all pulses) with the "
                 "library's device event log (`DDH_TUNE_TRACE`), after warm-up steps. "
                 "Times in us from the first work-group's start (100 MHz wall clock). "
                 "Command (repository root, one MI355X):\n\n")
        cmd = args.pmc_command or " ".join(["python3"] + [shlex.quote(a) for a in sys.argv])
        fh.write(f"```\n{cmd}\n```\n\n")
        fh.write(f"- work-groups: {grid} (1024 lanes); chunks: {len(chunks)}; "
                 f"span to the last exit: {span:.1f} us\n")
        fh.write(f"- median work-group busy fraction (claim to release, summed): "
                 f"{np.median([busy[b] * 1e-3 / span for b in busy]):.2f}\n\n")
        fh.write("| stage | chunks | entries (median) | chunk start (p10 / median / p90) | "
                 "chunk end | work: claim to done | wait | release |\n"
                 "|---|---|---|---|---|---|---|---|\n")
        for k in order:
            v = by.get(k, [])
            if not v:
                continue
            fh.write(f"| {k} | {len(v)} | {int(np.median([c.get('n', 0) for c in v]))} | "
                     f"{q3([c['claim'] for c in v])} | "
                     f"{q3([c.get('released', c.get('done', c['claim'])) for c in v])} | "
                     f"{q3([c.get('done', c['claim']) - c['claim'] for c in v])} | "
                     f"{q3([(c['waited'] - c.get('head', c['claim'])) if 'waited' in c else 0 for c in v])} | "
                     f"{q3([c.get('released', c.get('done', 0)) - c.get('done', 0) for c in v])} |\n")
    print(out_path)


# ------------------------------------------------------------- CPU baseline

def host_cpu():
    """The host's processor model and core counts: os.cpu_count() (what nproc
    reports without an affinity mask), the cores this process may run on, and
    the thread count the process is held to by OMP_NUM_THREADS (unset: none)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    omp = int(env) if env.strip().isdigit() and int(env) > 0 else None
    return dict(model=model, cpu_count=os.cpu_count() or 1, affinity=affinity, omp_num_threads=omp)


def run_cpu_baseline(w, seconds: float):
    import numpy as np

    import oracle
    import workloads as W

    x = W.positions(w)
    ref = oracle.OraclePlan(x, **w.params())
    # every core the process may use, unless OMP_NUM_THREADS holds it to fewer
    # (the share of the host's cores a job is given)
    cpu = host_cpu()
    threads = cpu["affinity"] if cpu["omp_num_threads"] is None else min(cpu["affinity"],
                                                                          cpu["omp_num_threads"])
    threads = max(1, threads)
    xl = ref.x_local.copy()
    f = W.forces(w, ref.n_slots)
    steps = 0
    t0 = time.perf_counter()
    while True:
        ref.exchange_coords(xl, nthreads=threads)
        ref.exchange_forces(f, nthreads=threads)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds or steps >= 100000:
            break
    per_step = el / steps
    # the same loops on one thread, for a quarter of the time
    steps1 = 0
    t0 = time.perf_counter()
    while True:
        ref.exchange_coords(xl, nthreads=1)
        ref.exchange_forces(f, nthreads=1)
        steps1 += 1
        el1 = time.perf_counter() - t0
        if el1 >= seconds / 4 or steps1 >= 100000:
            break
    per_step1 = el1 / steps1
    return dict(value=round(ref.halo_atoms / per_step, 1), unit="halo atoms/s", cores=threads,
                kind="oracle",
                sample=(f"{steps} steps (coordinate + force pass) of workload {w.name} "
                        f"in {el:.1f} s, OpenMP over the domains of each pulse on {threads} "
                        f"threads, maps prebuilt (oracle map build "
                        f"{ref.build_seconds * 1e3:.0f} ms, not timed)"),
                us_per_step=round(per_step * 1e6, 2),
                host_cores=cpu["cpu_count"], affinity_cores=cpu["affinity"],
                omp_num_threads=cpu["omp_num_threads"], cpu_model=cpu["model"],
                threads_note=("threads = the cores this process may use"
                              + ("" if cpu["omp_num_threads"] is None else
                                 ", held to OMP_NUM_THREADS")),
                single_thread={"value": round(ref.halo_atoms / per_step1, 1),
                               "us_per_step": round(per_step1 * 1e6, 2),
                               "sample": f"{steps1} steps in {el1:.1f} s"})


# --------------------------------------------------------- counter summary

def summarize_pmc(fetch_csv, write_csv, variant, wname, copy_mb, command, pass_="step"):
    """Turn two rocprofv3 --pmc runs into profiles/traffic_<variant>[_<pass>]_<wname>.md."""
    def rows(path):
        with open(path) as fh:
            return list(csv.DictReader(fh))

    def per_kernel(rows_, counter):
        out = {}
        for r in rows_:
            name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
            if r.get("Counter_Name", counter) != counter:
                continue
            v = float(r.get("Counter_Value") or r.get(counter) or 0.0)
            out.setdefault(name, []).append(v)
        return out

    fk = per_kernel(rows(fetch_csv), "FETCH_SIZE")
    wk = per_kernel(rows(write_csv), "WRITE_SIZE")
    cp = [k for k in fk if "copy" in k.lower() or "elementwise" in k.lower()]
    if variant == "pulse":
        # per step: every per-pulse launch of the step; each step ends with
        # exactly one signal_kernel launch
        ex = sorted(k for k in fk if "pulse_kernel" in k)
        sig = [k for k in fk if "signal_kernel" in k]
        if not ex or not sig or not cp:
            raise SystemExit(f"kernels not found: pulse={ex} signal={sig} copy={cp}")
        n_steps = len(fk[sig[0]])
        f_ex = sum(sum(fk[k]) for k in ex) / n_steps
        w_ex = sum(sum(wk.get(k, [])) for k in ex) / n_steps
        n_disp = sum(len(fk[k]) for k in ex)
        unit = ("step (all per-pulse launches of one step)" if pass_ == "step" else
                f"call (all per-pulse launches of one {pass_} call)")
    else:
        ex = [k for k in fk if "exchange_kernel" in k]
        if not ex or not cp:
            raise SystemExit(f"kernels not found: exchange={ex} copy={cp}")
        import statistics
        f_ex = statistics.median(fk[ex[0]])
        w_ex = statistics.median(wk[ex[0]])
        n_disp = len(fk[ex[0]])
        unit = "dispatch"
    # the copy probe: the largest copy-like dispatch
    cbest = max(cp, key=lambda k: max(fk[k]))
    f_cp = max(fk[cbest])
    w_cp = max(wk.get(cbest, [0.0]))
    expect_kib = copy_mb * 1024.0
    sf = expect_kib / f_cp if f_cp else 1.0
    sw = expect_kib / w_cp if w_cp else 1.0
    traffic = (f_ex * sf + w_ex * sw) * 1024.0
    path = traffic_file(variant, wname, pass_)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    what = {"step": "coordinate + force pass", "coords": "coordinate pass alone",
            "forces": "force pass alone"}[pass_]
    with open(path, "w") as fh:
        fh.write(f"# HBM traffic of the exchange, variant {variant}, {what}, workload {wname}\n\n")
        fh.write("Two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch),\n"
                 "scaled by what the same counters read for a plain copy of known size.\n\n")
        fh.write(f"Command (each counter in its own run):\n\n```\n{command}\n```\n\n")
        fh.write(f"- kernel_source_sha256: `{kernel_hash()}`\n")
        fh.write(f"- kernels: {', '.join('`' + k[:90] + '`' for k in ex)}\n")
        fh.write(f"- dispatches: {n_disp}\n")
        fh.write(f"- unit: {unit}\n")
        fh.write(f"- FETCH_SIZE_KiB_per_unit: {f_ex:.1f}\n")
        fh.write(f"- WRITE_SIZE_KiB_per_unit: {w_ex:.1f}\n")
        fh.write(f"- copy_probe_kernel: `{cbest[:90]}`\n")
        fh.write(f"- copy_probe_MiB: {copy_mb}\n")
        fh.write(f"- copy_probe_FETCH_KiB: {f_cp:.1f}\n")
        fh.write(f"- copy_probe_WRITE_KiB: {w_cp:.1f}\n")
        fh.write(f"- scale_fetch: {sf:.4f}\n")
        fh.write(f"- scale_write: {sw:.4f}\n")
        fh.write(f"- traffic_bytes_per_launch: {traffic:.0f}\n")
        fh.write(f"- scaled_FETCH_bytes_per_unit: {f_ex * sf * 1024.0:.0f}\n")
        fh.write(f"- scaled_WRITE_bytes_per_unit: {w_ex * sw * 1024.0:.0f}\n")
    print(path)


def summarize_markers(trace_dir, title, command):
    """A markdown section from a rocprofv3 --marker-trace --stats run: the
    host ranges (entry points and the map build's phases) with their calls
    and average, minimum and maximum durations."""
    import glob

    hits = sorted(glob.glob(os.path.join(trace_dir, "**", "*marker_api_stats.csv"), recursive=True))
    if not hits:
        raise SystemExit(f"no marker statistics under {trace_dir}")
    rows = list(csv.DictReader(open(hits[-1])))
    lines = [f"## {title}", "", "```", command, "```", "",
             "| range | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    return "\n".join(lines) + "\n"


def summarize_trace(trace_dir, wname, label, command, bench_line, out_path):
    """Turn a rocprofv3 --kernel-trace --stats run into a profiles/ summary:
    the statistics table and, for the exchange's launches, the median
    duration of each launch position in one step over the last 200 steps."""
    import glob
    import statistics

    def find(pattern):
        hits = sorted(glob.glob(os.path.join(trace_dir, "**", pattern), recursive=True))
        if not hits:
            raise SystemExit(f"no {pattern} under {trace_dir}")
        return hits[-1]

    with open(find("*kernel_stats.csv")) as fh:
        stats = list(csv.DictReader(fh))
    with open(find("*kernel_trace.csv")) as fh:
        trace = list(csv.DictReader(fh))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))

    def short(name, n=70):
        name = name.replace("ddh::(anonymous namespace)::", "")
        return name if len(name) <= n else name[:n]

    # one step: the exchange launches (pulse or fused kernels) from one
    # signal_kernel (or fused launch) to the next
    ex = [r for r in trace if any(k in r["Kernel_Name"] for k in
                                  ("pulse_kernel", "signal_kernel", "exchange_kernel", "wave_kernel"))]
    steps, cur = [], []
    for r in ex:
        cur.append(r)
        if "signal_kernel" in r["Kernel_Name"] or "exchange_kernel" in r["Kernel_Name"] \
                or "wave_kernel" in r["Kernel_Name"]:
            steps.append(cur)
            cur = []
    # the timed steps all have the launch count of the last step
    n_l = len(steps[-1]) if steps else 0
    steps = [st for st in steps if len(st) == n_l][-200:]
    rows = []
    for k in range(n_l):
        durs = [(int(st[k]["End_Timestamp"]) - int(st[k]["Start_Timestamp"])) / 1e3 for st in steps]
        gaps = [(int(st[k]["Start_Timestamp"]) - int(st[k - 1]["End_Timestamp"])) / 1e3
                for st in steps] if k > 0 else [0.0]
        r = steps[-1][k]
        grid = r.get("Grid_Size_X") or r.get("Grid_Size") or ""
        vgpr = r.get("VGPR_Count") or r.get("Arch_VGPR_Count") or ""
        rows.append((short(r["Kernel_Name"], 60), grid, vgpr, statistics.median(durs),
                     statistics.median(gaps)))
    with open(out_path, "w") as fh:
        fh.write(f"# Kernel trace: {label}, workload {wname}\n\n")
        fh.write("Command (run from the repository root on one MI355X):\n\n")
        fh.write(f"```\n{command}\n```\n\n")
        if bench_line:
            fh.write(f"bench line of the same run: {bench_line}\n\n")
        fh.write("## Kernel statistics (rocprofv3 `--stats`, all dispatches of the run)\n\n")
        fh.write("| kernel | calls | avg us | min us | max us | share % |\n|---|---|---|---|---|---|\n")
        for r in stats[:10]:
            fh.write(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |\n")
        fh.write(f"\n## Launches of one step (kernel trace, median over the last {len(steps)} steps)\n\n")
        fh.write("| # | kernel | grid (threads) | VGPRs | median us | median gap before (us) |\n"
                 "|---|---|---|---|---|---|\n")
        for k, (name, grid, vgpr, d, g) in enumerate(rows):
            fh.write(f"| {k} | `{name}` | {grid} | {vgpr} | {d:.2f} | {g:.2f} |\n")
        fh.write(f"| | sum of durations | | | {sum(r[3] for r in rows):.2f} | |\n")
    print(out_path)


# ------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--variant", default="auto", choices=VARIANTS)
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--grid", type=int, default=0)
    ap.add_argument("--block", type=int, default=0, choices=[0, 256, 512, 1024])
    ap.add_argument("--static-first", action="store_true",
                    help="fused launch: first tickets unclaimed (DDH_TUNE_STATIC_FIRST)")
    ap.add_argument("--no-flags", action="store_true",
                    help="calls skip the per-pulse completion flags (DDH_TUNE_FLAGS = 0)")
    ap.add_argument("--wave-chunks", action="store_true",
                    help="fused launch with wavefront workers (DDH_TUNE_WAVE_CHUNKS = 1)")
    ap.add_argument("--wide-maps", action="store_true",
                    help="kernels read the 32-bit maps (DDH_TUNE_NARROW_MAPS = 0)")
    ap.add_argument("--exit-publish", type=int, default=0, choices=[0, 1, 2],
                    help="DDH_TUNE_EXIT_PUBLISH (0 automatic)")
    ap.add_argument("--pad-maps", type=int, default=0, choices=[0, 1, 2],
                    help="DDH_TUNE_PAD_MAPS (0 automatic)")
    ap.add_argument("--heads-first", action="store_true",
                    help="fused launch: heads-first ticket order (DDH_TUNE_HEADS_FIRST = 1)")
    ap.add_argument("--lds-stage", type=int, default=0, choices=[0, 1, 2],
                    help="per-pulse coordinate stores staged through LDS (DDH_TUNE_LDS_STAGE: "
                         "1 gathered in registers, 2 by LDS loads)")
    ap.add_argument("--home-sort", type=int, default=0, choices=[0, 1, 2],
                    help="DDH_TUNE_HOME_SORT (0 automatic, 1 counting, 2 partition)")
    ap.add_argument("--pass", dest="pass_", default="step", choices=["step", "coords", "forces"],
                    help="time one pass alone (coordinate or force pass) instead of the step; "
                         "with --only-step, for per-pass profiler runs")
    ap.add_argument("--cold", action="store_true", help="evict caches before every step")
    ap.add_argument("--cold-flush", choices=("read", "write"), default="read",
                    help="how --cold evicts the caches: read a 1 GiB buffer (clean lines "
                         "left behind) or write it (dirty lines left behind)")
    ap.add_argument("--eager", action="store_true",
                    help="enqueue every step from the host (no graph replay)")
    ap.add_argument("--build-only", action="store_true",
                    help="time the map build alone (--steps builds of one plan)")
    ap.add_argument("--overlap", action="store_true",
                    help="time the step beside a compute load on a second stream "
                         "(prints one JSON object of its own)")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the overlap figures of the 96k and 1M entries under 'also'")
    ap.add_argument("--overlap-dim", type=int, default=2048)
    ap.add_argument("--overlap-reps", type=int, default=4)
    ap.add_argument("--only-step", action="store_true",
                    help="time the step only (no per-pass or single-launch lines); "
                         "for profiler runs")
    ap.add_argument("--lib-graph", action="store_true",
                    help="with --eager: each call replays the library's cached hipGraph")
    ap.add_argument("--also", default="1,2,3,4,5",
                    help="comma-separated workload keys timed after the main one (which "
                         "is skipped there) and "
                         "summarized under 'also', each with its own default step count "
                         "(empty: none; skipped with --only-step)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache figure of the main workload")
    ap.add_argument("--graph-steps", type=int, default=50,
                    help="steps captured per graph replay in the timed region")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MiB",
                    help="after timing, copy a buffer of this size (counter scaling)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--pmc-command", default="",
                    help="the profiler command, recorded in a --summarize-* output")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("TRACE_DIR", "OUT_MD", "LABEL"),
                    help="write a kernel-trace summary from a rocprofv3 --kernel-trace --stats "
                         "output directory")
    ap.add_argument("--event-log", metavar="OUT_MD", default="",
                    help="run one fused step with the device event log and write its "
                         "per-stage summary (give the command line with --pmc-command)")
    ap.add_argument("--summarize-markers", nargs=2, metavar=("TRACE_DIR", "TITLE"),
                    help="print a markdown section of the host ranges of a rocprofv3 "
                         "--marker-trace --stats run (give the command with --pmc-command)")
    ap.add_argument("--bench-line", default="",
                    help="with --summarize-trace: the bench result of the profiled run")
    ap.add_argument("--min-replays", type=int, default=5,
                    help="timed graphs hold at most --steps / this many steps")
    args = ap.parse_args()
    if args.variant == "staged":
        # the host-orchestrated baseline waits on the host inside every call:
        # it cannot be captured, so it is timed eagerly
        args.eager = True

    import workloads as W

    w = W.WORKLOADS[args.workload]
    if args.summarize_pmc:
        if args.variant == "auto":
            sys.exit("--summarize-pmc names the variant the counters were taken on: "
                     "pass --variant step|split|pulse")
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.variant, w.name,
                      args.copy_probe, args.pmc_command, args.pass_)
        return
    if args.summarize_markers:
        print(summarize_markers(args.summarize_markers[0], args.summarize_markers[1],
                                args.pmc_command), end="")
        return
    if args.summarize_trace:
        tdir, out_path, label = args.summarize_trace
        summarize_trace(tdir, w.name, label, args.pmc_command, args.bench_line, out_path)
        return
    if args.event_log:
        run_event_trace(args, w, args.event_log)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: every domain is a virtual rank inside one "
              f"GPU's HBM (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.steps is None:
        args.steps = 1000 if w.n_atoms <= 100_000 else 200

    if args.overlap:
        print(json.dumps({"overlap": run_overlap(args, w)}), flush=True)
        return
    if args.build_only:
        print(json.dumps({"map_build": run_builds(args, w)}), flush=True)
        return
    gpu = run_gpu(args, w)
    # the same workload with caches evicted before every step (eager steps)
    cold = None
    if not args.cold and not args.eager and not args.only_step and not args.copy_probe \
            and not args.no_cold:
        sub = argparse.Namespace(**vars(args))
        sub.cold = True
        sub.steps = max(5, min(args.steps, 50))
        sub.warmup = 2
        sub.cold_flush = "read"
        gc = run_gpu(sub, w)
        sub.cold_flush = "write"
        gw = run_gpu(sub, w)
        bytes_step = (BYTES_X + BYTES_F) * gc["n_halo"]
        cold = {"us_per_step": gc["roofline"]["median_step_us"],
                "p10_step_us": gc["roofline"]["p10_step_us"],
                "p90_step_us": gc["roofline"]["p90_step_us"],
                "frac": round(bytes_step / (gc["roofline"]["median_step_us"] * 1e-6) / 1e9
                              / HBM_PEAK_GBS, 4),
                "variant": gc["variant"], "steps": gc["steps"],
                "how": "eager steps, each after a 1 GiB buffer is read (caches evicted, "
                       "only clean lines left in them); median over the steps",
                "after_write_flush": {
                    "us_per_step": gw["roofline"]["median_step_us"],
                    "frac": round(bytes_step / (gw["roofline"]["median_step_us"] * 1e-6) / 1e9
                                  / HBM_PEAK_GBS, 4),
                    "how": "the same, with the 1 GiB buffer written instead: the step also "
                           "writes back the dirty lines the eviction left in the caches"}}
    also = {}
    keys = [int(k) for k in args.also.split(",") if k.strip()] if args.also else []
    if not args.only_step and not args.copy_probe:
        for k in keys:
            if k == args.workload:
                continue
            wk = W.WORKLOADS[k]
            sub = argparse.Namespace(**vars(args))
            sub.steps = 1000 if wk.n_atoms <= 100_000 else 200
            g2 = run_gpu(sub, wk)
            also[wk.name] = {
                "variant": g2["variant"], "halo_atoms_per_pass": g2["n_halo"],
                "gpu_us_per_step": g2["gpu_step_us"],
                "halo_atoms_per_s": round(g2["n_halo"] / g2["step_s"], 1),
                "roofline_frac": g2["roofline"]["frac"], "achieved_GBps": g2["roofline"]["achieved"],
                "map_entry_bytes": g2["roofline"]["map_entry_bytes"],
                "frac_at_min_bytes": g2["roofline"]["frac_at_min_bytes"],
                "latency": g2["roofline"]["latency"],
                "steps": g2["steps"],
                "median_step_us": g2["roofline"]["median_step_us"],
                "p10_step_us": g2["roofline"]["p10_step_us"],
                "p90_step_us": g2["roofline"]["p90_step_us"],
                "passes": g2["passes"], "single_launch": g2["single"],
                "without_flags": g2["without_flags"]}
            if k in OVERLAP_WORKLOADS and not args.no_overlap:
                also[wk.name]["overlap"] = overlap_set(wk, args.overlap_dim, args.overlap_reps)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(w, args.cpu_seconds)
    step_s = gpu["step_s"]
    value = gpu["n_halo"] / step_s
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "halo atoms/s",
        "n_gpus": 1,
        "steps": gpu["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 6),
        "gpu_us_per_step": gpu["gpu_step_us"],
        "us_per_step": round(step_s * 1e6, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "atoms": w.n_atoms, "box_nm": w.box32[0], "grid": list(w.grid),
            "rc_nm": w.rc, "cell_nm": w.cell, "pulses": gpu["n_pulses"],
            "halo_atoms_per_pass": gpu["n_halo"], "slots": gpu["n_slots"],
            "variant": gpu["variant"], "cache": "cold" if args.cold else "warm",
            "launch": "eager" if (args.eager or args.cold) else "graph replay",
            "completion_flags": not args.no_flags,
            "step": "coordinate pass + force pass",
        },
        "step_hbm_frac": round((BYTES_X + BYTES_F) * gpu["n_halo"] / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "map_build_ms": round(gpu["build_ms"], 3),
        "passes": gpu["passes"],
        "single_launch": gpu["single"],
        "without_flags": gpu["without_flags"],
        "cold": cold,
        "roofline": gpu["roofline"],
        "cpu_baseline": cpu,
        "also": also or None,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
