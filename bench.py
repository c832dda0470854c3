#!/usr/bin/env python3
"""Decode-attention benchmark: achieved unique-KV HBM GB/s and decode-attention µs per step.

One step is one pass of the whole path over one batch: for every layer of the workload, the
split (streaming) kernel and the merge kernel through the C ABI. Inputs are seeded, synthetic
and already resident in HBM when timing starts. The default workload is C2 (LLaMA-7B-shaped
decode attention: B=8, h_q=h_kv=32, d=128, T=4096, bf16, 32 layers with their own caches,
i.e. 32 launches of each kernel per step, 16 GiB of KV per step, far above the 256 MB
last-level cache so every step streams from HBM).

Measurement (Ch. 10 "System Model of Throughput and Latency" §8: warm up, time on the device
with events, never time host submission):
  * pass A: W warm-up steps (default: >= 0.25 s of GPU work), then K steps launched from the
    host as a serving loop would (``--step-graph`` replays a captured HIP graph of one step
    instead), bracketed by device events on the launch stream, with torch.cuda.synchronize()
    on both sides -> ms_per_step, value = unique KV bytes / step time;
  * pass B: K rounds of split-kernel launches only (at least 8 per round), captured once in a
    HIP graph and replayed (``--eager`` launches them from the host), back to back between two
    device events -> that kernel's average duration, free of host-submission gaps even for
    launches of a few microseconds, and roofline.achieved = its unique KV bytes per launch /
    that duration (the merge launches follow outside the events);
  * with --window W, only the attended positions (the first sinks and the last W) count as
    bytes, both in value and in roofline.achieved;
  * with --scores every layer also exports the per-position attention weights (the split
    kernel's score-export instantiation, then the weighting kernel) in pass A; pass B still
    times the regular split kernel;
  * with --gamma G (speculative-decoding verification) every sequence has G query tokens, the
    last G cached positions, each attending to its own prefix; bytes count the union of the
    positions they attend (each KV element once) and tokens_per_s counts B * G tokens;
  * a workload whose bytes fit near the 256 MB last-level cache is also timed cold: each step,
    and each split launch, alone after writing 512 MiB (``cache.cold_us_per_step`` and
    ``roofline.cold``; ``roofline.cache`` then says that pass B ran warm);
  * cpu_baseline: the fp64 oracle (oracle/) timed on the host on a bounded sample of the same
    workload (whole (layer, sequence, KV head) units in order, about 15 s of CPU work).

The plain default run (C2) also measures C3, C4 and C5 the same way, one after the other, and
reports each in the line's ``configs`` object (its step time and rate, the split kernel's
roofline fraction and counter traffic, and a CPU baseline of about 3 s); ``--also`` chooses
other workloads or none. Prints one JSON line. Only one GPU is used; --gpus above 1 exits with
a message.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (unique KV bytes/time) + decode-attn µs/step"
HBM_PEAK_GBPS = 8000.0
LLC_BYTES = 256 << 20  # MI355X last-level cache (MALL, "Infinity Cache")
KERNEL_SOURCES = [os.path.join(ROOT, "kv_cache_decode_split_amd", "csrc", f)
                  for f in ("kv_attn_split.h", "kv_attn_split_mfma64.hip", "kv_attn_split_mfma128.hip",
                            "kv_attn_split_vector64.hip", "kv_attn_split_vector128.hip",
                            "kv_attn_split_rows.hip", "kv_attn_kernels.hip", "kv_attn_internal.h",
                            "kv_attn_plan.cpp")]
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash() -> str:
    """Hash of the sources that decide what the split kernel reads and writes."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload: str):
    """HBM bytes per split launch from the committed counter summary, if it is current."""
    path = os.path.join(PROFILES, f"traffic_split_kernel_{workload}.json")
    if not os.path.exists(path):
        return None, "no counter summary"
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    return float(rec["hbm_bytes_per_launch"]), path


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="warm-up steps (default: enough for >= 0.25 s of GPU work, at least 5)")
    ap.add_argument("--config", default="C2", choices=["C1", "C2", "C3", "C4", "C5"])
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads measured after the main one and reported in "
                         "the line's 'configs' object (default: C3,C4,C5 for the plain C2 run, "
                         "none otherwise; '' for none)")
    ap.add_argument("--also-cpu-seconds", type=float, default=3.0,
                    help="CPU-baseline time budget of each --also workload")
    ap.add_argument("--num-splits", type=int, default=0, help="0 = the library's automatic plan")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip timing the library's read probe (the practical read ceiling)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-baseline time budget")
    ap.add_argument("--append", action="store_true",
                    help="each layer first appends the current token's K/V (kv_attn_append_decode)")
    ap.add_argument("--window", type=int, default=None,
                    help="sliding window: attend only the last W positions (plus the sinks)")
    ap.add_argument("--attn-sinks", type=int, default=None,
                    help="with --window: leading positions always attended (default: the "
                         "workload's sink count)")
    ap.add_argument("--gamma", type=int, default=1,
                    help="query tokens per sequence (speculative-decoding verification: the last "
                         "gamma cached positions, causal among themselves)")
    ap.add_argument("--block-order", choices=["random", "sequential"], default=None,
                    help="paged workloads: deal the physical blocks to the sequences in a random "
                         "order (the workload's default) or in physical order")
    ap.add_argument("--layout", choices=["head_major", "token_major"], default=None,
                    help="cache layout: [.., KV head, position, d] (the workloads' default) or "
                         "[.., position, KV head, d]")
    ap.add_argument("--scores", action="store_true",
                    help="each layer also exports the attention weight of every cached position "
                         "(kv_attn_decode_scores)")
    ap.add_argument("--evict", choices=["E1", "E2"], default=None,
                    help="time the budgeted eviction selection on this score workload instead of "
                         "decode attention")
    ap.add_argument("--eager", action="store_true",
                    help="pass B: launch the split kernels from the host instead of replaying a "
                         "captured HIP graph")
    ap.add_argument("--step-graph", action="store_true",
                    help="pass A: replay each step from a captured HIP graph instead of launching "
                         "it from the host (a graph launch costs a few microseconds of its own)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run plain device copies of this size (counter calibration runs)")
    return ap.parse_args()


VARIANT_FLAGS = ("window", "attn_sinks", "block_order", "layout", "scores", "append", "evict")


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode-attention path has no multi-GPU component here).", file=sys.stderr)
        sys.exit(2)

    import torch

    from kv_cache_decode_split_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.evict is not None:
        bench_evict(args, W)
        return
    spec, tag = resolve_spec(args, args.config, W)
    if args.scores and (args.append or args.gamma > 1):
        print("bench.py: --scores takes one query token and no --append", file=sys.stderr)
        sys.exit(2)
    also = args.also
    if also is None:  # the long-context workloads ride along with the plain headline run
        plain = args.config == "C2" and args.gamma == 1 and args.num_splits == 0 and not any(
            getattr(args, f) not in (None, False) for f in VARIANT_FLAGS)
        also = "C3,C4,C5" if plain else ""
    also = [c.strip() for c in also.split(",") if c.strip()]
    for c in also:
        if c not in W.PRESETS:
            print(f"bench.py: --also names an unknown workload {c!r}", file=sys.stderr)
            sys.exit(2)

    # Every GPU timing runs back to back (the device slows down for a while after sitting idle,
    # e.g. during a CPU-baseline leg), and the CPU baselines follow once they are all done.
    # The read probe runs after every workload: timed right after it frees its 4 GiB buffer, C3's
    # split kernel ran 318 instead of 307 us per launch.
    line, main_inputs = measure_decode(args, spec, tag)
    extras, extra_inputs = {}, {}
    for c in also:
        extra_spec, extra_tag = resolve_spec(args, c, W)
        extras[c], extra_inputs[c] = measure_decode(args, extra_spec, extra_tag)
    ceiling = None if args.no_read_probe else read_ceiling()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(*main_inputs, args.cpu_seconds, single_thread=True)
        for c in also:
            extras[c]["cpu_baseline"] = cpu_baseline(*extra_inputs[c], args.also_cpu_seconds,
                                                     single_thread=False)
    del main_inputs, extra_inputs
    for ln in [line, *extras.values()]:
        roof = ln["roofline"]
        roof["stream_ceiling"] = ceiling
        roof["frac_of_stream_ceiling"] = (round(roof["achieved"] / ceiling["achieved"], 4)
                                          if ceiling else None)
    if extras:
        line["configs"] = {c: config_summary(ln) for c, ln in extras.items()}
    print(json.dumps(line), flush=True)


def resolve_spec(args, config, W):
    """The workload spec of ``config`` with the command line's variant options, and its tag (the
    name of its counter summary in profiles/)."""
    spec = W.PRESETS[config]
    tag = config
    if args.window is not None:
        if args.window < 1:
            print("bench.py: --window must be >= 1", file=sys.stderr)
            sys.exit(2)
        sinks = spec.num_sinks if args.attn_sinks is None else args.attn_sinks
        spec = W.preset(config, window=args.window, num_sinks=sinks)
        tag = f"{config}_w{args.window}_s{sinks}"
    elif args.attn_sinks is not None:
        print("bench.py: --attn-sinks needs --window", file=sys.stderr)
        sys.exit(2)
    if args.block_order is not None:
        if not spec.paged:
            print("bench.py: --block-order needs a paged workload (C4, C5)", file=sys.stderr)
            sys.exit(2)
        spec = dataclasses.replace(spec, block_order=args.block_order)
        if args.block_order != "random":
            tag = f"{tag}_{args.block_order}"
    if args.layout is not None and args.layout != spec.layout:
        spec = dataclasses.replace(spec, layout=args.layout)
        tag = f"{tag}_{args.layout}"
    if args.gamma < 1:
        print("bench.py: --gamma must be >= 1", file=sys.stderr)
        sys.exit(2)
    if args.gamma > 1:
        spec = dataclasses.replace(spec, num_queries=args.gamma)
        tag = f"{tag}_g{args.gamma}"
    return spec, tag


def config_summary(line):
    """The fields of a full bench line that the 'configs' object reports per workload."""
    roof = line["roofline"]
    return {
        "workload": line["config"]["workload"],
        "value": line["value"], "unit": line["unit"],
        "ms_per_step": line["ms_per_step"], "us_per_step": line["us_per_step"],
        "tokens_per_s": line["tokens_per_s"],
        "step_frac_of_hbm_peak": line["step_frac_of_hbm_peak"],
        "step_us_spread": line["step_us_spread"],
        "unique_kv_bytes_per_step": line["config"]["unique_kv_bytes_per_step"],
        "sum_ctx_len": line["config"]["sum_ctx_len"],
        "plan": line["config"]["plan"],
        "roofline": {k: roof[k] for k in ("bound", "kernel", "achieved", "peak", "unit", "frac",
                                          "traffic", "traffic_over_algorithmic",
                                          "algorithmic_bytes_per_launch", "avg_launch_us",
                                          "launches_timed", "timed_by", "cache",
                                          "frac_of_stream_ceiling") if k in roof},
        "cache": line["cache"],
        "outputs_finite": line["outputs_finite"],
        "cpu_baseline": line["cpu_baseline"],
    }


def read_ceiling():
    """The library's read probe timed on a 4 GiB buffer: the practical read ceiling."""
    import torch

    from kv_cache_decode_split_amd import kv_attn as K

    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda").fill_(3)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        K.kv_attn_read_probe(buf, sink)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    n_probe = 10
    a.record()
    for _ in range(n_probe):
        K.kv_attn_read_probe(buf, sink)
    b.record()
    torch.cuda.synchronize()
    probe_us = 1e3 * a.elapsed_time(b) / n_probe
    out = {"achieved": round(buf.numel() / (probe_us * 1e-6) / 1e9, 1), "unit": "GB/s",
           "bytes_per_launch": buf.numel(), "avg_launch_us": round(probe_us, 2),
           "kernel": "kv_attn_read_probe (16-byte nontemporal loads, 1 MiB contiguous "
                     "per workgroup, no compute)"}
    del buf, sink
    torch.cuda.empty_cache()
    return out


def measure_decode(args, spec, tag):
    """Passes A and B (and the append and cold-cache timings) on one workload: its bench line
    (cpu_baseline still None) and the inputs the CPU baseline needs (the workload, kept on the
    device)."""
    import torch

    from kv_cache_decode_split_amd import accounting as A
    from kv_cache_decode_split_amd import kv_attn as K
    from kv_cache_decode_split_amd import workloads as W

    layers = spec.layers
    print(f"[bench] building {spec.name} ({layers} layer(s)) on the GPU", file=sys.stderr, flush=True)
    wls = [W.make_workload(spec, device="cuda", layer=l) for l in range(layers)]
    outs = [torch.empty(w.q.shape, dtype=torch.float32, device="cuda") for w in wls]
    # One call (and workspace) per layer, so that pass B can run all split launches before the
    # merges without one layer's split states overwriting another's.
    calls = [K.decode_call_for(w, o, num_splits=args.num_splits, with_scores=args.scores)
             for w, o in zip(wls, outs)]
    score_bufs = ([torch.empty((spec.batch, spec.num_kv_heads, w.max_ctx_len), dtype=torch.float32,
                               device="cuda") for w in wls] if args.scores else [])
    plan = calls[0].plan()
    elem = 2 if spec.kv_dtype == "bf16" else 4
    lens = [int(x) for x in wls[0].ctx_lens.cpu().tolist()]
    # Algorithmic bytes: the KV of the positions attended (all of them without a window).
    gamma = max(spec.num_queries, 1)
    att = [A.attended_length(t, spec.window, spec.num_sinks, gamma) for t in lens]
    kv_bytes_layer = A.unique_kv_read_bytes(att, spec.num_kv_heads, spec.head_dim, elem)
    kv_bytes_step = kv_bytes_layer * layers
    flops_step = layers * sum(A.verify_attention_flops(t, spec.num_q_heads, spec.head_dim, gamma,
                                                       spec.window, spec.num_sinks) for t in lens)

    calib = None
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        calib = (torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1),
                 torch.empty(n, dtype=torch.uint8, device="cuda"))

    news = []
    if args.append:  # the current token's K/V rows for every layer (at ctx_lens[b] - gamma ..)
        g = torch.Generator(device="cuda").manual_seed(4242)
        for w in wls:
            shape = ((spec.batch, spec.num_kv_heads, spec.head_dim) if gamma == 1
                     else (spec.batch, gamma, spec.num_kv_heads, spec.head_dim))
            news.append(tuple(torch.randn(shape, generator=g, device="cuda").to(w.k_cache.dtype)
                              for _ in range(2)))

    def step():
        if args.scores:
            for c, buf in zip(calls, score_bufs):
                c.decode_scores(buf)
            return
        if args.append:
            for c, (kn, vn) in zip(calls, news):
                c.append_decode(kn, vn)
        else:
            for c in calls:
                c.decode()

    def capture(fn):
        """``fn``'s launches captured once in a HIP graph (torch's capture stream is the current
        stream the library launches on). Replaying it issues them back to back with no host work
        in between, so small launches are not timed at the host's submission rate."""
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        torch.cuda.synchronize()
        return graph.replay

    # ---- pass A: whole steps -------------------------------------------------------------------
    # The first tens of milliseconds of sustained load on a fresh device run measurably slower
    # (kernel durations drift for ~50-100 launches, then settle), so the default warm-up covers
    # at least 0.25 s of GPU work.
    run_step = capture(step) if args.step_graph else step
    warmup = args.warmup
    if warmup is None:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_step()
        torch.cuda.synchronize()
        warmup = max(5, int(0.25 / max(time.perf_counter() - t0, 1e-6)) + 1)
    for _ in range(warmup):
        run_step()
    torch.cuda.synchronize()
    # An event at every step boundary: the first and last bracket the K steps (ms_per_step), the
    # ones between give each step's duration for the spread.
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for i in range(args.steps):
        run_step()
        marks[i + 1].record()
    torch.cuda.synchronize()
    ms_per_step = marks[0].elapsed_time(marks[-1]) / args.steps
    step_us = [1e3 * marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    print(f"[bench] {spec.name} pass A done: {ms_per_step * 1e3:.1f} us/step", file=sys.stderr,
          flush=True)

    # ---- cache state ------------------------------------------------------------------------------
    # Steps run back to back, so a step whose inputs fit the 256 MB last-level cache (MALL) could
    # find them there. When the bytes a step touches are under 4x that, the steps are timed once
    # more one at a time, each after writing a 512 MiB scratch buffer (outside the timed region),
    # so that they start cold; pass B below is then timed cold the same way as well.
    touched = kv_bytes_step + sum(int(w.q.numel()) * w.q.element_size() * 2 for w in wls)
    fits_cache = touched < 4 * LLC_BYTES
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if fits_cache else None

    def time_cold(fn, n):
        """Durations (µs) of ``n`` calls of ``fn``, each alone after 512 MiB of writes."""
        out = []
        for _ in range(n):
            scratch.fill_(7)
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            a0.record()
            fn()
            a1.record()
            torch.cuda.synchronize()
            out.append(1e3 * a0.elapsed_time(a1))
        return out

    cold_us = time_cold(run_step, args.steps) if fits_cache else None

    # ---- pass B: the split kernel alone, launched back to back ------------------------------------
    # Two events bracket K rounds of split launches (each round: every layer's launch, repeated so
    # that a round holds at least 8 launches; same stream, nothing in between), so the average
    # launch duration carries neither event nor host-submission overhead.
    reps = max(1, -(-8 // len(calls)))

    def split_round():
        for _ in range(reps):
            for c in calls:
                c.split()

    run_round = split_round if args.eager else capture(split_round)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        run_round()
    b.record()
    for c in calls:  # keep the outputs complete (merge pass), outside the bracket
        c.merge()
    torch.cuda.synchronize()
    launches_timed = args.steps * reps * len(calls)
    split_us_avg = 1e3 * a.elapsed_time(b) / launches_timed
    print(f"[bench] {spec.name} pass B done: split kernel {split_us_avg:.1f} us/launch",
          file=sys.stderr, flush=True)
    split_cold_us = None
    if fits_cache:  # each layer's split launch alone, after a flush (the data is then in HBM)
        split_cold_us = time_cold(lambda: calls[0].split(), args.steps)
        for c in calls:
            c.merge()
        torch.cuda.synchronize()
    del scratch

    append_info = None
    if args.append:  # the append kernel alone, launched back to back
        positions = [(w.ctx_lens - gamma).to(torch.int32) for w in wls]
        ks_vs = [w.kv_strides() for w in wls]

        def append_all():
            for w, (kn, vn), pos, (ks, vs) in zip(wls, news, positions, ks_vs):
                K.kv_attn_append(kn, vn, w.k_cache, w.v_cache, w.block_table, pos,
                                 num_kv_heads=spec.num_kv_heads, k_strides=ks, v_strides=vs,
                                 block_size=w.block_size, num_blocks=w.num_blocks)
        # One launch per layer is a few microseconds of GPU work, less than a Python call takes
        # to issue, so the launches are captured once in a HIP graph and the graph is replayed.
        append_all()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            append_all()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for _ in range(reps):
                append_all()
        graph.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        n = reps * args.steps * len(wls)
        row_bytes = spec.batch * gamma * spec.num_kv_heads * spec.head_dim * elem
        append_info = {"avg_launch_us": round(a.elapsed_time(b) * 1e3 / n, 3), "timed_by": "HIP graph replay",
                       "bytes_written_per_launch": 2 * row_bytes,
                       "bytes_read_per_launch": 2 * row_bytes, "launches_timed": n}

    if calib is not None:  # plain copies of known size, for the counter-calibration runs
        for _ in range(4):
            calib[1].copy_(calib[0])
        torch.cuda.synchronize()
        del calib

    finite = all(bool(torch.isfinite(o).all()) for o in outs)

    achieved = kv_bytes_layer / (split_us_avg * 1e-6) / 1e9
    traffic, traffic_src = load_traffic(tag)
    value = kv_bytes_step / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "tokens_per_s": round(A.aggregate_tokens_per_s(spec.batch * gamma, ms_per_step * 1e-3), 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{spec.name}: {spec.description}" + (
                f"; sliding window of {spec.window} positions plus the first {spec.num_sinks} "
                "(attention sinks), the rest NaN-poisoned and never read" if spec.window else "")
                + ("; blocks dealt to the sequences in physical order"
                   if spec.paged and spec.block_order == "sequential" else "")
                + ("; token-major cache layout" if spec.layout == "token_major" else "")
                + (f"; {gamma} query tokens per sequence (speculative-decoding verification: the "
                   "last gamma cached positions, causal among themselves)" if gamma > 1 else ""),
            "num_queries": gamma,
            "batch": spec.batch, "num_q_heads": spec.num_q_heads, "num_kv_heads": spec.num_kv_heads,
            "head_dim": spec.head_dim, "max_ctx_len": max(lens), "sum_ctx_len": sum(lens),
            "window": spec.window, "attn_sinks": spec.num_sinks if spec.window else None,
            "sum_attended_len": sum(att),
            "layers": layers, "kv_dtype": spec.kv_dtype, "q_dtype": spec.q_dtype,
            "paged": spec.paged, "layout": spec.layout,
            "block_order": spec.block_order if spec.paged else None,
            "unique_kv_bytes_per_step": kv_bytes_step, "flops_per_step": flops_step,
            "plan": {k: plan[k] for k in ("num_splits", "split_len", "grid_split", "grid_merge",
                                          "kernel_variant", "wave_heads", "unit_order", "num_cus")},
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "split_kernel",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_over_algorithmic": round(traffic / kv_bytes_layer, 4) if traffic else None,
            "algorithmic_bytes_per_launch": kv_bytes_layer,
            "avg_launch_us": round(split_us_avg, 2),
            "launches_timed": launches_timed,
            "timed_by": "host launches" if args.eager else "HIP graph replay",
            "cache": ("streamed: the launches read far more than the 256 MB last-level cache"
                      if split_cold_us is None else
                      "warm: back-to-back launches re-read data that fits the 256 MB last-level "
                      "cache; 'cold' times each launch alone after writing 512 MiB"),
            "stream_ceiling": None,
            "frac_of_stream_ceiling": None,
        },
        "step_frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "step_us_spread": _spread(step_us),
        "cache": {
            "bytes_touched_per_step": touched,
            "state": ("streamed: a step touches more than 4x the 256 MB last-level cache; steps run "
                      "back to back with no flush" if cold_us is None else
                      "a step's bytes fit near the 256 MB last-level cache: ms_per_step is back to "
                      "back (warm); cold_us_per_step times each step after writing 512 MiB"),
            "cold_us_per_step": _spread(cold_us) if cold_us else None,
        },
        "outputs_finite": finite,
        "cpu_baseline": None,
        "context": page_context(A, kv_bytes_step, ms_per_step),
    }
    if split_cold_us is not None:
        cold_avg = sum(split_cold_us) / len(split_cold_us)
        cold_rate = kv_bytes_layer / (cold_avg * 1e-6) / 1e9
        line["roofline"]["cold"] = {"avg_launch_us": round(cold_avg, 2),
                                    "achieved": round(cold_rate, 1),
                                    "frac": round(cold_rate / HBM_PEAK_GBPS, 4),
                                    "launches_timed": len(split_cold_us),
                                    "timed_by": "device events around each launch"}
    if args.scores:
        line["config"]["scores"] = ("each layer also writes every attended position's attention "
                                    "weight summed over its KV head's query heads")
    if args.append:
        fused = plan["kernel_variant"] in (1, 2)
        how = ("in the split kernel (the tile holding the new rows takes them from the new-row "
               "buffers and writes them to the cache)" if fused else "by the append kernel first")
        line["config"]["append"] = (("each layer appends the current token's K/V, " if gamma == 1 else
                                     f"each layer appends the {gamma} draft tokens' K/V, ") + how)
        # The standalone append kernel, for reference (kv_attn_append_decode launches it only on
        # the fp32 vector path).
        line["append"] = dict(append_info, kernel="kv_attn_append alone", fused_in_step=fused)
    if traffic is None:
        line["roofline"]["traffic_note"] = traffic_src
    del calls, outs, score_bufs, news
    torch.cuda.empty_cache()
    return line, (wls, spec, elem)


def _spread(xs):
    """p10 / median / p90 of per-step durations (µs)."""
    ys = sorted(xs)

    def q(f):
        pos = f * (len(ys) - 1)
        lo = int(pos)
        hi = min(lo + 1, len(ys) - 1)
        return round(ys[lo] + (ys[hi] - ys[lo]) * (pos - lo), 2)
    return {"p10": q(0.1), "p50": q(0.5), "p90": q(0.9), "n": len(ys)}


def page_context(A, kv_bytes_step, ms_per_step):
    """The pages' analytic A100 figures (Ch. 19 §19.2.1 and §19.3.2), quoted as context for the
    measured step, not as targets: the same unique-KV bytes at A100's bandwidth, and the 7B decode
    step bound the page derives (weights plus the KV of 1024 tokens, read once per step)."""
    a100_bw = 1.55e12
    return {
        "kind": "the pages' analytic estimates for A100 (context, not targets)",
        "a100_hbm_tb_s": 1.55,
        "a100_fp16_tflop_s": 312,
        "a100_ridge_flop_per_byte": round(A.ridge_point(312e12, a100_bw), 1),
        "a100_floor_us_for_this_step": round(kv_bytes_step / a100_bw * 1e6, 1),
        "measured_us_per_step": round(ms_per_step * 1e3, 2),
        "llama7b_decode_step_bound_ms_a100": round(
            A.decode_step_bandwidth_bound(7e9, 32, 4096, 1024, a100_bw) * 1e3, 2),
    }


def bench_evict(args, W):
    """Budgeted eviction selection (kv_evict_select) on a seeded score workload.

    One call is the whole selection (all its launches). Algorithmic bytes per call: every score
    read once (4 bytes) and every mask byte written once; the calls are captured in a HIP graph
    and replayed back to back between device events."""
    import numpy as np
    import torch

    from kv_cache_decode_split_amd import kv_evict as E

    cfg = W.EVICT_PRESETS[args.evict]
    L, H, N = cfg["num_layers"], cfg["num_heads"], cfg["num_tokens"]
    n = L * H * N
    budget = int(cfg["budget_frac"] * n)
    print(f"[bench] building {args.evict} scores ({L}x{H}x{N}) on the GPU", file=sys.stderr, flush=True)
    scores = W.make_scores(L, H, N, cfg["kind"], seed=cfg["seed"], device="cuda", sigma=cfg["sigma"])
    keep = torch.empty((L, H, N), dtype=torch.uint8, device="cuda")
    p = E.make_evict_params(L, H, N, budget)
    ws = torch.empty(max(E.kv_evict_workspace_size(p), 1), dtype=torch.uint8, device="cuda")

    def call():
        E.kv_evict_select(scores, budget, keep=keep, workspace=ws)

    call()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    warmup = args.warmup if args.warmup is not None else 20
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / args.steps
    if args.calib_copy_mib:  # plain copies of known size, for the counter-calibration runs
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    kept = int(keep.sum().item())
    alg_bytes = 5 * n
    achieved = alg_bytes / (us * 1e-6) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import evict_select
        host = scores.cpu().numpy()
        layers, spent = L, 0.0
        while True:  # the oracle on the first `layers` layers, shrunk until it fits the budget
            t0 = time.perf_counter()
            evict_select(host[:layers], int(cfg["budget_frac"] * layers * H * N))
            spent = time.perf_counter() - t0
            if spent <= args.cpu_seconds or layers == 1:
                break
            layers = max(1, int(layers * args.cpu_seconds / spent / 2))
        cpu = {"value": round(5 * layers * H * N / spent / 1e9, 4), "unit": "GB/s",
               "cores": _blas_threads(), "kind": "oracle",
               "sample": f"the first {layers} of {L} layers ({layers * H * N} entries, budget "
                         f"fraction {cfg['budget_frac']}), {spent:.1f} s of oracle time"}
    line = {
        "metric": "eviction selection: achieved HBM GB/s (score bytes read + mask bytes written "
                  "/ time) + µs/call",
        "value": round(achieved, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": round(us * 1e-3, 5),
        "us_per_step": round(us, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.evict}: budgeted KV eviction selection over L={L} layers x H={H} "
                        f"KV heads x N={N} positions ({n} entries), scores {cfg['kind']} "
                        f"(sigma {cfg['sigma']}), budget M = {budget} ({cfg['budget_frac']:.0%}), "
                        "current position N-1",
            "num_layers": L, "num_heads": H, "num_tokens": N, "budget": budget,
            "entries_kept": kept,
            "algorithmic_bytes_per_call": alg_bytes,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "kv_evict_select (whole call: init sample, one streaming pass, list pass, final)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": alg_bytes,
            "avg_launch_us": round(us, 2),
            "launches_timed": args.steps,
            "timed_by": "HIP graph replay",
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:  # pragma: no cover - threadpoolctl missing
        return os.cpu_count() or 1


def cpu_baseline(wls, spec, elem, budget_s, single_thread=True):
    """The oracle, as it stands, on whole (layer, sequence, KV head) units of the workload, in
    order, until the time budget is spent (at least one unit). Host copies of each unit are made
    outside the timed region. Returns the oracle's unique-KV GB/s on the host's BLAS threads and,
    for C1-C3, also on one thread (a third of the budget)."""
    from kv_cache_decode_split_amd import accounting as A
    from kv_cache_decode_split_amd import workloads as W
    from oracle import decode_attention, verify_attention

    gamma = max(spec.num_queries, 1)
    units = [(l, b, h) for l in range(len(wls)) for b in range(spec.batch)
             for h in range(spec.num_kv_heads)]
    lens = [w.ctx_lens.cpu().tolist() for w in wls]

    def run(budget):
        done_bytes, spent, n = 0, 0.0, 0
        for l, b, h in units:
            v = W.oracle_sample(wls[l], [b], [h])
            t0 = time.perf_counter()
            fn = decode_attention if gamma == 1 else verify_attention
            fn(v["q"], v["k_cache"], v["v_cache"], v["ctx_lens"], v["block_table"],
               block_size=v["block_size"] if v["block_table"] is not None else None,
               window=spec.window, num_sinks=spec.num_sinks)
            spent += time.perf_counter() - t0
            done_bytes += 2 * A.attended_length(lens[l][b], spec.window, spec.num_sinks,
                                                gamma) * spec.head_dim * elem
            n += 1
            if spent >= budget:
                break
        sample = (f"{n} of {len(units)} (layer, sequence, KV head) units of {spec.name}, in order "
                  f"({done_bytes} unique KV bytes, {spent:.1f} s of oracle time)")
        return round(done_bytes / spent / 1e9, 4), sample

    value, sample = run(budget_s)
    out = {"value": value, "unit": "GB/s", "cores": _blas_threads(), "kind": "oracle", "sample": sample}
    if single_thread and spec.name in ("C1", "C2", "C3"):
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:
            threadpool_limits = None
        if threadpool_limits is not None:
            with threadpool_limits(limits=1):
                v1, s1 = run(budget_s / 3)
            out["single_thread"] = {"value": v1, "unit": "GB/s", "cores": 1, "sample": s1}
    return out


if __name__ == "__main__":
    main()
