"""Benchmark of the MoE finalize + residual + RMSNorm path on one MI355X.

Default workload (one "step" = one call of the whole path over one decode batch): 128 tokens,
hidden 7168, top-8 routes with a quarter of them marked -1, float32 softmax expert scales, RSF
2.5, shared-expert add, residual add and RMSNorm (eps 1e-6), bf16 activations, seeded synthetic
inputs resident in HBM. Each timed call reads a different copy of the inputs, rotating over 2.1 GB
(8x the 256 MiB Infinity Cache), so every input comes from HBM (cold). Every call is a HIP graph
node: a warm-up graph over all copies is replayed first, then a graph of exactly K calls is
replayed once between two HIP events on the launch stream (timing_plan); nothing is launched
eagerly in the timed region, whatever K is.

Output: one JSON line (metric, value = achieved algorithmic GB/s, us/call, roofline of the
finalize kernel, the FP64 CPU oracle's throughput on the host as a baseline). Beside the HBM
peak it reports the streaming ceiling: the library's plain stream kernel moving exactly the same
bytes in one launch (every load issued up front, nothing else to do).
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--sweep [--no-large]] [--no-cpu-baseline]
--sweep adds, for every workload of the pages' configurations (decode shapes at hidden 1024, 6144
and 7168, top-22/16/6/10 with fp32 and bf16 scales, NVFP4 / FP8 outputs) and the large-batch
regime (T = 256..2048), warm µs/call against the launch floor, and from T = 32 on cold µs/call
against the streaming ceiling of the same bytes; for the hidden 1024/6144/7168 shapes also the
unfused alternative (moe_finalize_run, then moe_residual_rmsnorm_run) beside the fused call.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

METRIC = "µs/call and achieved HBM GB/s (% of peak) for MoE finalize+RMSNorm, T=1..128"
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["moe_expert_output_amd/csrc/finalize_kernels.hip",
                  "moe_expert_output_amd/csrc/device_utils.h"]
# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (two runs), scaled
# by the same counters' reading for a plain copy of known size; valid only for the kernel code
# it was taken with.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_finalize_rmsnorm_T128_H7168_K8.json")


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace collapsed: what the compiler sees (the
    sources hold no string literal with a comment marker in it)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    """Hash of the kernel sources' code (comments and whitespace excluded, so editing a comment
    keeps a traffic measurement valid)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, or None if the kernel changed."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")
PEAK_GBS = 8000.0
ACT_BYTES = 2
# Cold timings rotate over at least this much memory (8x the 256 MiB Infinity Cache): with only
# ~2-3x, part of the data still hits in it (measured: 6.50 us at 705 MB vs 7.42 us at 2.1 GB for
# the headline call).
ROTATE_BYTES = 2 << 30
MAX_SETS = 384


def _read_bytes(T, H, K, n_valid, scale_bytes=4, shared=True, entry="rmsnorm"):
    """Bytes the path must read: valid rows, route metadata, shared; + residual and gamma for the
    RMSNorm entry points. The rank sum reads K = world_size partial rows per token and no route
    metadata."""
    e = ACT_BYTES
    if entry == "rank_sum":
        return K * T * H * e + T * H * e + H * e
    rd = n_valid * H * e + T * K * (4 + scale_bytes) + (T * H * e if shared else 0)
    if entry != "finalize":
        rd += T * H * e + H * e
    return rd


def algorithmic_bytes(T, H, K, n_valid, scale_bytes=4, shared=True, entry="rmsnorm",
                      quant=None, norm_out=True):
    """Bytes the path must move: valid rows, route metadata, shared, residual, gamma reads;
    residual_out + norm_out writes (finalize-only: one output; quant: residual_out + codes + block
    scales, + norm_out when it is stored)."""
    e = ACT_BYTES
    rd = _read_bytes(T, H, K, n_valid, scale_bytes, shared, entry)
    if entry == "finalize":
        return rd + T * H * e
    if quant in ("nvfp4", "nvfp4_linear"):
        nb = H // 16
        sf = ((T + 127) // 128 * 128) * ((nb + 3) // 4 * 4) if quant == "nvfp4" else T * nb
        return rd + T * H * e + T * H // 2 + sf + (T * H * e if norm_out else 0)
    if quant == "fp8":
        return rd + T * H * e + T * H + (T * H * e if norm_out else 0)
    return rd + 2 * T * H * e


def timing_plan(steps: int, warmup: int, n_sets: int) -> dict:
    """How the headline run spends its calls; every call is a graph-node launch, none is eager.

    Timed: a graph of exactly `steps` calls on copies 0, 1, ..., n_sets - 1, 0, 1, ... replayed
    ONCE between the two events. Before that, untimed: that graph is replayed once (its first
    replay also uploads it to the device, a one-time cost of ~10 us that would otherwise land in
    the timed region), then a graph that makes one call on each of the n_sets copies in order is
    replayed ceil(warmup / n_sets) times (at least once), so at least `warmup` calls run untimed.
    The last warm-up replay is enqueued after the host synchronizes, right before the first
    event, so the GPU is running when the timed graph is queued behind it: the timed calls see
    the steady state of back-to-back calls (clocks up, launch latency overlapped) rather than a
    start from idle, which at 20 calls added ~0.3-0.7 us per call.
    Copy i was last read n_sets - i calls before the timed graph reads it (the warm-up ends on
    copy n_sets - 1), and n_sets copies are 8x the Infinity Cache, so every timed call reads its
    inputs from HBM."""
    if steps < 1 or n_sets < 1 or warmup < 0:
        raise ValueError("steps >= 1, warmup >= 0 and n_sets >= 1 are required")
    replays = max(1, -(-warmup // n_sets))
    timed = [i % n_sets for i in range(steps)]
    return {"upload_replay_sets": timed, "warmup_sets": list(range(n_sets)),
            "warmup_replays": replays, "warmup_calls": steps + replays * n_sets,
            "timed_sets": timed, "timed_replays": 1, "timed_calls": steps, "eager_calls": 0}


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=960)
    p.add_argument("--warmup", type=int, default=192)
    p.add_argument("--sets", type=int, default=96,
                   help="input copies rotated per graph (96 x 22 MB = 2.1 GB, 8x the Infinity Cache)")
    p.add_argument("--sweep", action="store_true")
    p.add_argument("--no-large", action="store_true", help="sweep without the T >= 256 cases")
    p.add_argument("--scan", action="store_true",
                   help="warm timings over a grid of uncommon shapes (performance-cliff check)")
    p.add_argument("--groups", default="", help="comma-separated sweep groups to run (default all)")
    p.add_argument("--stream-sweep", action="store_true",
                   help="only sweep the stream kernel's launch shape (loads per round, workgroup "
                        "lanes, workgroups, nontemporal) cold at the T=64 and T=128 byte counts")
    p.add_argument("--stream-shapes", default="",
                   help="with --stream-sweep: only these shapes, 'loads:lanes:workgroups:nt,...' "
                        "(workgroups 0 = one round)")
    p.add_argument("--stream-tokens", default="64,128",
                   help="with --stream-sweep: which byte counts (T = 64 and / or 128)")
    p.add_argument("--stream-repeats", type=int, default=1,
                   help="with --stream-sweep: time every shape this many times")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    return p.parse_args()


def main():
    a = _parse()
    if a.gpus != 1:
        print(json.dumps({"error": "the finalize path runs on one GPU; --gpus must be 1",
                          "n_gpus": a.gpus}), flush=True)
        sys.exit(2)

    import torch
    import moe_expert_output_amd as M
    from synth import make_inputs, workload_seed

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if a.stream_sweep:
        print(json.dumps({"stream_sweep": _stream_sweep(
            torch, M, dev, a.stream_shapes, [int(t) for t in a.stream_tokens.split(",")],
            a.stream_repeats)}), flush=True)
        return
    T, H, K = 128, 7168, 8
    inp = make_inputs(T, H, K, seed=workload_seed("larger", T))
    n_valid = int((inp.idx >= 0).sum())
    nbytes = algorithmic_bytes(T, H, K, n_valid)

    def dev_set():
        d = {k: getattr(inp, k).to(dev).contiguous() for k in
             ("rows", "idx", "scales", "shared", "residual", "gamma")}
        d["res_out"] = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        d["norm_out"] = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        return d

    sets = [dev_set() for _ in range(a.sets)]
    set_bytes = sum(v.numel() * v.element_size() for v in sets[0].values())
    # one zero-filled workspace serves every call (the calls are serialized on one stream)
    ws = torch.zeros(M.moe_finalize_workspace_size(T, H, K), dtype=torch.uint8, device=dev)

    def call(d):
        M.moe_finalize_rmsnorm_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                                   d["residual"], d["gamma"], inp.eps, d["res_out"],
                                   d["norm_out"], ws)

    # Warm-up: one graph that calls the path once on every input copy, replayed. Timed: a second
    # graph of exactly K calls over the copies in the same order (see timing_plan), replayed once.
    stream = torch.cuda.Stream(device=dev)
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for d in sets[:3]:
            call(d)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    n_sets = len(sets)
    K_steps, W = int(a.steps), int(a.warmup)
    plan = timing_plan(K_steps, W, n_sets)
    warm_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(warm_graph, stream=stream):
        for i in plan["warmup_sets"]:
            call(sets[i])
    timed_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(timed_graph, stream=stream):
        for i in plan["timed_sets"]:
            call(sets[i])
    with torch.cuda.stream(stream):
        timed_graph.replay()                       # untimed: uploads the timed graph
        for _ in range(plan["warmup_replays"] - 1):
            warm_graph.replay()
        torch.cuda.synchronize()
        t_host0 = time.perf_counter()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        # the last warm-up replay keeps the GPU busy while the timed graph is enqueued behind it
        warm_graph.replay()
        ev0.record(stream)
        timed_graph.replay()
        ev1.record(stream)
        ev1.synchronize()
        t_host1 = time.perf_counter()
    torch.cuda.synchronize()
    del warm_graph, timed_graph
    us_per_call = ev0.elapsed_time(ev1) * 1e3 / K_steps
    gbs = nbytes / (us_per_call * 1e-6) / 1e9

    # The pages' protocol (warm): one graph of 20 calls on the same inputs, median of 50 replays.
    warm = _warm_us(torch, stream, lambda: call(sets[0]))
    # The same protocol with every access cacheable (MOE_FIN_CACHE_KEEP), so the replayed input
    # set stays in the caches: the warm figure a pipeline sees when its inputs are cached.
    prev = M.moe_finalize_set_cache_policy(M.MOE_FIN_CACHE_KEEP)
    try:
        warm_cached = _warm_us(torch, stream, lambda: call(sets[0]))
    finally:
        M.moe_finalize_set_cache_policy(prev)
    # Context: a plain device copy moving the same number of bytes (half read, half written),
    # rotated over the same amount of memory; also the known-size kernel that calibrates the
    # FETCH_SIZE / WRITE_SIZE counters.
    copy_us = _copy_reference(torch, stream, dev, nbytes, n_sets)
    floor = _warm_us(torch, stream, lambda: M.moe_finalize_launch_floor_run(1, T, H, K,
                                                                           device=dev))
    # The streaming ceiling: the library's plain stream kernel moving the same bytes in one
    # launch, rotated over the same amount of memory.
    rd = _read_bytes(T, H, K, n_valid)
    ceil_us = _stream_ceiling(torch, M, stream, dev, rd, nbytes - rd,
                              min_rotate=n_sets * set_bytes)
    out = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": W,
        "ms_per_step": round(us_per_call / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) rows / shared / residual, softmax fp32 scales, 25% -1 "
                "routes); inputs resident in HBM, rotated over 2.1 GB of copies (8x the MALL)",
        "config": {"workload": "moe_finalize_rmsnorm decode batch: T=128 tokens, hidden 7168, "
                               "top_k 8 (25% absent), bf16, fp32 scales, shared expert, "
                               "residual + RMSNorm", "tokens": T, "hidden": H, "top_k": K,
                   "parallelism": "none (1 GPU)", "input_copies": n_sets,
                   "rotated_bytes": n_sets * set_bytes},
        "us_per_call": round(us_per_call, 3),
        "us_per_call_warm_median": round(warm, 3),
        "us_per_call_warm_cached_policy": round(warm_cached, 3),
        "launch_floor_us": round(floor, 3),
        "algorithmic_bytes_per_call": nbytes,
        "host_wall_s": round(t_host1 - t_host0, 4),
        "timing": {"warmup_calls": plan["warmup_calls"], "timed_graph_calls": plan["timed_calls"],
                   "timed_graph_replays": plan["timed_replays"], "eager_calls": plan["eager_calls"]},
        "plain_copy_same_bytes_us": round(copy_us, 3),
        "stream_ceiling_same_bytes_us": round(ceil_us, 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": _headline_kernel(M, T, H, K),
                     "per_launch_bytes": nbytes, "kernel_source_hash": kernel_source_hash(),
                     "stream_ceiling_GBs": round(nbytes / (ceil_us * 1e-6) / 1e9, 1),
                     "frac_of_stream_ceiling": round(ceil_us / us_per_call, 4)},
    }
    # The other configurations of the metric in brief: decode T = 1 / 4 / 16 (hidden 6144) warm,
    # against the launch floor; T = 64 (hidden 7168) cold; the same generators and protocols as
    # --sweep, which covers every configuration in full.
    del sets
    torch.cuda.empty_cache()
    out["other_configs"] = _brief(torch, M, stream, dev)
    if a.sweep:
        out["cases"] = _sweep(torch, M, stream, dev, large=not a.no_large,
                              groups=[g for g in a.groups.split(",") if g],
                              cpu=not a.no_cpu_baseline)
    if a.scan:
        out["scan"] = _scan(torch, M, stream, dev)
    out["workspace_flag"] = int(ws[:4].view(torch.int32).item())
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(inp, nbytes, a.cpu_seconds)
    print(json.dumps(out), flush=True)


def _brief(torch, M, stream, dev):
    """Decode T = 1 / 4 / 16 at hidden 6144 (warm µs/call, launch floor, excess) and T = 64 at
    hidden 7168 (cold µs/call, GB/s, fraction of 8 TB/s and of the stream ceiling)."""
    from synth import make_inputs, workload_seed
    ws = torch.zeros(M.moe_finalize_workspace_size(64, 0, 0), dtype=torch.uint8, device=dev)
    res = []
    for T, H, grp in ((1, 6144, "decode"), (4, 6144, "decode"), (16, 6144, "decode"),
                      (64, 7168, "larger")):
        inp = make_inputs(T, H, 8, seed=workload_seed(grp, T))
        n_valid = int((inp.idx >= 0).sum())
        nb = algorithmic_bytes(T, H, 8, n_valid)
        cold = T >= 32
        n = max(2, min(MAX_SETS, -(-ROTATE_BYTES // _set_bytes(inp)))) if cold else 1
        sets = [_dev_set(torch, inp, dev) for _ in range(n)]

        def fn(d):
            return lambda: M.moe_finalize_rmsnorm_run(
                d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf, d["residual"],
                d["gamma"], inp.eps, d["ro"], d["no"], ws, stream=stream)
        r = {"workload": f"moe_finalize_rmsnorm T={T} hidden {H} top_k 8 bf16", "T": T, "H": H,
             "bytes": nb}
        if cold:
            us = _graph_us(torch, stream, [fn(d) for d in sets], 20)
            rd = _read_bytes(T, H, 8, n_valid)
            del sets
            ceil_us = _stream_ceiling(torch, M, stream, dev, rd, nb - rd)
            r.update({"protocol": "cold", "us_per_call": round(us, 3),
                      "gbs": round(nb / (us * 1e-6) / 1e9, 1),
                      "frac_peak": round(nb / (us * 1e-6) / 1e9 / PEAK_GBS, 4),
                      "stream_ceiling_us": round(ceil_us, 3),
                      "frac_of_stream_ceiling": round(ceil_us / us, 4)})
        else:
            us = _warm_us(torch, stream, fn(sets[0]))
            floor = _warm_us(torch, stream, lambda T=T, H=H: M.moe_finalize_launch_floor_run(
                1, T, H, 8, device=dev, stream=stream))
            del sets
            r.update({"protocol": "warm (20 calls on one input set, median of 50 replays)",
                      "us_per_call": round(us, 3), "launch_floor_us": round(floor, 3),
                      "excess_over_floor_us": round(us - floor, 3)})
        res.append(r)
        torch.cuda.empty_cache()
    assert int(ws[:4].view(torch.int32).item()) == 0, "a split row timed out"
    return res


def _headline_kernel(M, T, H, K):
    """Names the headline call's kernel and the launch configuration the library picks for it."""
    c = M.moe_finalize_launch_config(1, T, H, K, True)
    return (f"mfin::finalize_kernel<0, 1, {c['route_groups']}, {c['slots_per_lane']}, 8, "
            f"{2 if c['nontemporal'] else 0}> (bf16, RMSNorm): {c['slices']} workgroup(s) per token "
            f"x {c['lanes']} lanes, {c['route_groups']} route group(s)"
            f"{', nontemporal streams' if c['nontemporal'] else ''}")


def _copy_reference(torch, stream, dev, nbytes, n_sets, replays=20):
    half = nbytes // 2 // 2 * 2
    srcs = [torch.empty(half // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
            for _ in range(n_sets)]
    dsts = [torch.empty_like(x) for x in srcs]
    return _graph_us(torch, stream, [(lambda s_=s_, d_=d_: d_.copy_(s_))
                                     for s_, d_ in zip(srcs, dsts)], replays)


def _stream_ceiling(torch, M, stream, dev, read_bytes, write_bytes, min_rotate=ROTATE_BYTES,
                    replays=20):
    """µs per launch of the library's streaming-ceiling kernel moving the same bytes (cold:
    source and destination rotate over at least ROTATE_BYTES)."""
    rb, wb = read_bytes // 16 * 16, (write_bytes + 15) // 16 * 16
    n = max(2, min(MAX_SETS, -(-min_rotate // max(rb + wb, 1))))
    srcs = [torch.ones(max(rb, 16), dtype=torch.uint8, device=dev) for _ in range(n)]
    dsts = [torch.empty(max(wb, 16), dtype=torch.uint8, device=dev) for _ in range(n)]
    us = _graph_us(torch, stream, [(lambda s_=s_, d_=d_: M.moe_finalize_stream_floor_run(
        s_, rb, d_, wb, stream=stream)) for s_, d_ in zip(srcs, dsts)], replays)
    del srcs, dsts
    return us


def _stream_sweep(torch, M, dev, shapes="", tokens=(64, 128), repeats=1):
    """Cold µs per launch of the stream probe over launch shapes, at the byte counts of the
    larger-decode workloads (T = 64 and 128, hidden 7168, top_k 8: reads / writes of the fused
    RMSNorm call). Each shape is timed like the finalize: a graph of one launch per copy,
    rotating over >= 2 GiB of copies, median of replays."""
    T_cases = [c for c in [(64, 7_358_464, 1_835_008), (128, 14_702_592, 3_670_016)]
               if c[0] in tokens]
    if shapes:
        todo = [tuple(int(v) for v in x.split(":")) for x in shapes.split(",")]
    else:
        todo = [(l, w, g, nt) for l in (1, 2, 4, 8, 16) for w in (256, 512, 1024)
                for g in (0, 256, 512, 1024) for nt in (1, 0)]
    stream = torch.cuda.Stream(device=dev)
    out = []
    for T, rb, wb in T_cases:
        n = max(2, min(MAX_SETS, -(-ROTATE_BYTES // (rb + wb))))
        srcs = [torch.ones(rb, dtype=torch.uint8, device=dev) for _ in range(n)]
        dsts = [torch.empty(wb, dtype=torch.uint8, device=dev) for _ in range(n)]
        for (loads, lanes, grid, nt) in [x for _ in range(repeats) for x in todo]:
            g = grid or -(-(rb // 16) // (lanes * loads))
            print(f"stream T={T} loads={loads} lanes={lanes} workgroups={g} nt={nt}",
                  file=sys.stderr, flush=True)
            us = _graph_us(torch, stream, [
                (lambda s_=s_, d_=d_, g=g, loads=loads, lanes=lanes, nt=nt:
                 M.moe_finalize_stream_probe_run(s_, rb, d_, wb, loads, lanes, g, bool(nt),
                                                 stream=stream))
                for s_, d_ in zip(srcs, dsts)], 10)
            out.append({"T": T, "read_bytes": rb, "write_bytes": wb, "loads": loads,
                        "lanes": lanes, "workgroups": g, "one_round": grid == 0,
                        "nontemporal": nt, "us": round(us, 3),
                        "frac_peak": round((rb + wb) / (us * 1e-6) / 1e9 / PEAK_GBS, 4)})
        del srcs, dsts
        torch.cuda.empty_cache()
    return out


def _graph_us(torch, stream, fns, replays):
    """One HIP graph that makes each call of `fns` once, replayed; median µs per call."""
    with torch.cuda.stream(stream):
        for f in fns:
            f()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for f in fns:
                f()
        times = []
        for _ in range(replays):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / len(fns))
    return statistics.median(times)


def _warm_us(torch, stream, fn, launches=20, replays=50):
    """The pages' protocol: one graph of `launches` calls on the same inputs, median of
    `replays` replays, µs per call."""
    return _graph_us(torch, stream, [fn] * launches, replays)


def _scan(torch, M, stream, dev):
    """Warm µs per call (the pages' protocol, 15 replays) over a grid of shapes outside the
    measured workloads: tokens 1..250, hidden 1024..16384, top_k 1..64, for the finalize, RMSNorm,
    NVFP4 (swizzled scales, norm_out not stored) and FP8 entry points, with the RMSNorm launch
    floor. A check for performance cliffs; inputs are drawn on the device (bf16, fp32 scales,
    shared expert, a quarter of the routes absent) and the per-tensor scale is fixed at 100."""
    from synth import make_inputs_on_device
    ws = torch.zeros(M.moe_finalize_workspace_size(256, 0, 0), dtype=torch.uint8, device=dev)
    qs = torch.tensor([100.0], dtype=torch.float32, device=dev)
    swz = M.MOE_SF_SWIZZLED_128x4
    recs = []
    for T in (1, 3, 16, 100, 250):
        for H in (1024, 4096, 7168, 16384):
            for K in (1, 4, 8, 22, 64):
                print(f"scan T={T} H={H} K={K}", file=sys.stderr, flush=True)
                i = make_inputs_on_device(T, H, K, seed=9000 + T, device=dev)
                ro = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
                no = torch.empty_like(ro)
                q4 = torch.empty(T, H // 2, dtype=torch.uint8, device=dev)
                q8 = torch.empty(T, H, dtype=torch.uint8, device=dev)
                sf = torch.empty(M.moe_finalize_sf_size(T, H, swz), dtype=torch.uint8, device=dev)
                calls = {
                    "finalize": lambda: M.moe_finalize_run(i.rows, i.idx, i.scales, i.shared, i.rsf,
                                                           no, stream=stream),
                    "rmsnorm": lambda: M.moe_finalize_rmsnorm_run(
                        i.rows, i.idx, i.scales, i.shared, i.rsf, i.residual, i.gamma, i.eps, ro,
                        no, ws, stream=stream),
                    "nvfp4": lambda: M.moe_finalize_quant_run(
                        i.rows, i.idx, i.scales, i.shared, i.rsf, i.residual, i.gamma, i.eps,
                        M.MOE_QUANT_NVFP4, qs, q4, sf, swz, ro, None, ws, stream=stream),
                    "fp8": lambda: M.moe_finalize_quant_run(
                        i.rows, i.idx, i.scales, i.shared, i.rsf, i.residual, i.gamma, i.eps,
                        M.MOE_QUANT_FP8_E4M3, qs, q8, None, 0, ro, None, ws, stream=stream),
                    "floor": lambda: M.moe_finalize_launch_floor_run(1, T, H, K, device=dev,
                                                                     stream=stream),
                }
                r = {"T": T, "H": H, "K": K,
                     "bytes_rmsnorm": algorithmic_bytes(T, H, K, int((i.idx >= 0).sum()), 4, True,
                                                        "rmsnorm")}
                for name, fn in calls.items():
                    r[name] = round(_warm_us(torch, stream, fn, replays=15), 3)
                recs.append(r)
                del i, ro, no, q4, q8, sf
    assert int(ws[:4].view(torch.int32).item()) == 0, "a split row timed out in the scan"
    return recs


# Sweep cases: (group, entry, T, H, K, act, scales, shared, quant). entry: "rmsnorm" (fused
# finalize + residual + RMSNorm), "finalize" (finalize only), "two_kernel" (finalize, then
# moe_residual_rmsnorm_run), "quant" (moe_finalize_quant_run; quant = nvfp4 / nvfp4_linear /
# fp8, "+norm" when norm_out is also stored), "quant_two_kernel" (moe_finalize_rmsnorm_run, then
# moe_quantize_run of norm_out), "rank_sum" (moe_rank_sum_rmsnorm_run of K = world_size partials).
def _sweep_cases(large):
    c = [("tiny", e, 4, 1024, 8, "bf16", "fp32", True, None) for e in ("rmsnorm", "two_kernel")]
    c += [("decode", e, t, 6144, 8, "bf16", "fp32", True, None) for t in (1, 4, 16)
          for e in ("rmsnorm", "two_kernel")]
    c += [("larger", e, t, 7168, 8, act, "fp32", True, None) for act in ("bf16", "fp16")
          for t in (32, 64, 128) for e in ("rmsnorm", "two_kernel")]
    c += [("highk", e, t, h, k, "bf16", sdt, False, None)
          for (h, k) in ((2048, 22), (3584, 16), (2048, 6), (2048, 10))
          for sdt in ("fp32", "bf16") for t in (1, 8, 16, 32) for e in ("finalize", "rmsnorm")]
    c += [("quant", "quant", t, 6144, 8, "bf16", "fp32", True, q)
          for t in (1, 16) for q in ("nvfp4", "nvfp4_linear", "fp8")]
    c += [("quant", "quant", 64, 6144, 8, "bf16", "fp32", True, q)
          for q in ("nvfp4", "nvfp4+norm", "nvfp4_linear", "fp8", "fp8+norm")]
    c += [("quant", "quant_two_kernel", 64, 6144, 8, "bf16", "fp32", True, q)
          for q in ("nvfp4+norm", "fp8+norm")]
    c += [("quant", "rmsnorm", 64, 6144, 8, "bf16", "fp32", True, None)]
    # one GPU's share of the cross-rank reduction at the pages' TP4 shapes (world size 4)
    c += [("ranksum", "rank_sum", t, h, 4, "bf16", None, False, None)
          for (h, ts) in ((6144, (1, 16)), (7168, (1, 16, 64, 128))) for t in ts]
    c += [("ranksum", "rank_sum_quant", t, h, 4, "bf16", None, False, q)
          for h in (6144, 7168) for t in (1, 16) for q in ("nvfp4", "fp8")]
    if large:
        c += [("batch", e, t, 7168, 8, "bf16", "fp32", True, None) for t in (256, 512, 1024, 2048)
              for e in ("rmsnorm", "finalize")]
    return c


def _sweep(torch, M, stream, dev, large=True, groups=(), cpu=False):
    """Every case: warm µs/call (the pages' protocol) and the launch floor; from T = 32 on also
    cold µs/call (inputs rotated over ROTATE_BYTES, up to MAX_SETS copies) and the streaming
    ceiling for the same bytes. GB/s use the fused path's algorithmic bytes (the two-kernel path's extra write and
    re-read of the finalize output is the cost the fusion removes)."""
    from synth import make_inputs, workload_seed
    cases = []
    todo = [c for c in _sweep_cases(large) if not groups or c[0] in groups]
    # one zero-filled workspace for every case (calls are serialized on one stream)
    ws_big = torch.zeros(M.moe_finalize_workspace_size(max(c[2] for c in todo), 0, 0),
                         dtype=torch.uint8, device=dev)
    for (grp, entry, T, H, K, act, sdt, sh, quant) in todo:
        # the clock readings let a profiler's dispatch timestamps be assigned to the case
        print(f"sweep {grp} {entry} T={T} H={H} K={K} {act} {sdt} {quant or ''} "
              f"mono_ns={time.monotonic_ns()} boot_ns={time.clock_gettime_ns(time.CLOCK_BOOTTIME)}",
              file=sys.stderr, flush=True)
        kvar = K if grp == "highk" else None
        inp = make_inputs(T, H, K, act_dtype=act, scale_dtype=sdt, with_shared=sh,
                          seed=workload_seed(grp, T, act, sdt, kvar),
                          mask_frac=0.0 if entry.startswith("rank_sum") else 0.25)
        n_valid = int((inp.idx >= 0).sum())
        dt = inp.rows.dtype
        qkind = (quant or "").split("+")[0]
        keep_norm = quant is None or quant.endswith("+norm")
        q_scale = None
        if entry.startswith("quant") or entry == "rank_sum_quant":
            # the caller's per-tensor scale from the tensor's amax (448*6/amax or 448/amax)
            probe = _dev_set(torch, inp, dev)
            if entry == "rank_sum_quant":
                M.moe_rank_sum_rmsnorm_run(probe["rows"].view(inp.K, inp.T, inp.H),
                                           probe["residual"], probe["gamma"], inp.eps,
                                           probe["ro"], probe["no"], ws_big)
            else:
                M.moe_finalize_rmsnorm_run(probe["rows"], probe["idx"], probe["scales"],
                                           probe["shared"], inp.rsf, probe["residual"],
                                           probe["gamma"], inp.eps, probe["ro"], probe["no"],
                                           ws_big)
            amax = float(probe["no"].float().abs().max())
            q_scale = torch.tensor([(2688.0 if qkind.startswith("nvfp4") else 448.0) / amax],
                                   dtype=torch.float32, device=dev)
            del probe
        set_bytes = _set_bytes(inp, qkind)
        cold = T >= 32
        n_sets = max(2, min(MAX_SETS, -(-ROTATE_BYTES // set_bytes))) if cold else 1
        sets = [_dev_set(torch, inp, dev, qkind) for _ in range(n_sets)]

        def fn_for(d, inp=inp, entry=entry, qkind=qkind, keep_norm=keep_norm, q_scale=q_scale):
            if entry == "rmsnorm":
                return lambda: M.moe_finalize_rmsnorm_run(
                    d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf, d["residual"],
                    d["gamma"], inp.eps, d["ro"], d["no"], ws_big, stream=stream)
            if entry == "finalize":
                return lambda: M.moe_finalize_run(d["rows"], d["idx"], d["scales"], d["shared"],
                                                  inp.rsf, d["no"], stream=stream)
            if entry == "rank_sum":
                parts = d["rows"].view(inp.K, inp.T, inp.H)
                return lambda: M.moe_rank_sum_rmsnorm_run(parts, d["residual"], d["gamma"],
                                                          inp.eps, d["ro"], d["no"], ws_big,
                                                          stream=stream)
            if entry == "two_kernel":
                def f():
                    M.moe_finalize_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                                       d["s"], stream=stream)
                    M.moe_residual_rmsnorm_run(d["s"], d["residual"], d["gamma"], inp.eps,
                                               d["ro"], d["no"], ws_big, stream=stream)
                return f
            qt = M.MOE_QUANT_FP8_E4M3 if qkind == "fp8" else M.MOE_QUANT_NVFP4
            lay = M.MOE_SF_LINEAR if qkind == "nvfp4_linear" else M.MOE_SF_SWIZZLED_128x4
            if entry == "rank_sum_quant":
                parts = d["rows"].view(inp.K, inp.T, inp.H)
                return lambda: M.moe_rank_sum_quant_run(parts, d["residual"], d["gamma"], inp.eps,
                                                        qt, q_scale, d["q"], d.get("sf"), lay,
                                                        d["ro"], None, ws_big, stream=stream)
            if entry == "quant_two_kernel":
                # the unfused alternative: finalize + residual + RMSNorm, then quantize norm_out
                def f2():
                    M.moe_finalize_rmsnorm_run(d["rows"], d["idx"], d["scales"], d["shared"],
                                               inp.rsf, d["residual"], d["gamma"], inp.eps,
                                               d["ro"], d["no"], ws_big, stream=stream)
                    M.moe_quantize_run(d["no"], qt, q_scale, d["q"], d.get("sf"), lay,
                                       stream=stream)
                return f2
            return lambda: M.moe_finalize_quant_run(
                d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf, d["residual"],
                d["gamma"], inp.eps, qt, q_scale, d["q"], d.get("sf"), lay, d["ro"],
                d["no"] if keep_norm else None, ws_big, stream=stream)

        floor_entry = {"finalize": 0, "rmsnorm": 1, "quant": 2, "rank_sum": 1,
                       "rank_sum_quant": 2}.get(entry, 1)
        if entry in ("two_kernel", "quant_two_kernel"):
            def floor_fn(T=T, H=H, K=K):                 # two empty launches
                M.moe_finalize_launch_floor_run(0, T, H, K, device=dev, stream=stream)
                M.moe_finalize_launch_floor_run(1, T, H, 1, device=dev, stream=stream)
        else:
            def floor_fn(T=T, H=H, K=K, e=floor_entry):
                M.moe_finalize_launch_floor_run(e, T, H, K, device=dev, stream=stream)
        warm = _warm_us(torch, stream, fn_for(sets[0]))
        floor = _warm_us(torch, stream, floor_fn)
        base_entry = {"two_kernel": "rmsnorm", "quant_two_kernel": "quant"}.get(entry, entry)
        if entry == "rank_sum":
            nb = _read_bytes(T, H, K, n_valid, entry="rank_sum") + 2 * T * H * ACT_BYTES
        elif entry == "rank_sum_quant":
            # the rank sum's reads, the quantized entry's writes (residual_out, codes, scales)
            wr = (algorithmic_bytes(T, H, K, n_valid, 4, False, "quant", quant=qkind,
                                    norm_out=False) - _read_bytes(T, H, K, n_valid, 4, False, "quant"))
            nb = _read_bytes(T, H, K, n_valid, entry="rank_sum") + wr
        else:
            nb = algorithmic_bytes(T, H, K, n_valid, 4 if sdt == "fp32" else 2, sh, base_entry,
                                   quant=qkind or None, norm_out=keep_norm)
        rec = {"group": grp, "entry": entry, "T": T, "H": H, "K": K, "act": act, "scales": sdt,
               "quant": quant, "us_warm": round(warm, 3), "floor_us": round(floor, 3),
               "excess_us": round(warm - floor, 3), "bytes": nb,
               "gbs_warm": round(nb / (warm * 1e-6) / 1e9, 1)}
        if cold:
            us = _graph_us(torch, stream, [fn_for(d) for d in sets],
                           max(5, min(40, 2000 // n_sets)))
            rd = _read_bytes(T, H, K, n_valid, 4 if sdt == "fp32" else 2, sh, base_entry)
            del sets
            ceil_us = _stream_ceiling(torch, M, stream, dev, rd, nb - rd)
            rec.update({"sets": n_sets, "us_cold": round(us, 3),
                        "gbs_cold": round(nb / (us * 1e-6) / 1e9, 1),
                        "frac_peak_cold": round(nb / (us * 1e-6) / 1e9 / PEAK_GBS, 4),
                        "stream_ceiling_us": round(ceil_us, 3),
                        "frac_of_stream_ceiling": round(ceil_us / us, 3)})
        else:
            del sets
        torch.cuda.empty_cache()
        rec["workspace_flag"] = int(ws_big[:4].view(torch.int32).item())
        if cpu and entry in ("rmsnorm", "finalize", "rank_sum", "quant"):
            qv = None if q_scale is None else float(q_scale.item())
            o_us, o_runs = _oracle_case_us(inp, entry, qkind, qv)
            rec.update({"oracle_us": round(o_us, 1), "oracle_runs": o_runs,
                        "oracle_gbs": round(nb / (o_us * 1e-6) / 1e9, 4)})
        cases.append(rec)
    return cases


def _oracle_case_us(inp, entry, qkind, q_scale):
    """The FP64 oracle (unmodified) on this host, one thread, on the case's own inputs: one
    warm-up call, then the median of 5 calls (2 when one call takes over a second)."""
    import statistics

    import oracle as O
    f = lambda t: None if t is None else t.double().numpy()  # noqa: E731
    rows, idx, sc, sh = f(inp.rows), inp.idx.numpy(), f(inp.scales), f(inp.shared)
    res, gam = f(inp.residual), f(inp.gamma)

    def call():
        if entry == "finalize":
            return O.finalize(rows, idx, sc, sh, inp.rsf, inp.act_dtype)
        if entry == "rank_sum":
            s = O.rank_sum_rounded(rows.reshape(inp.K, inp.T, inp.H), inp.act_dtype)
            return O.residual_rmsnorm(s, res, gam, inp.eps, inp.act_dtype)
        out = O.finalize_rmsnorm(rows, idx, sc, sh, inp.rsf, res, gam, inp.eps, inp.act_dtype)
        if entry == "quant":
            N = out[2]
            if qkind == "fp8":
                return O.quant_fp8(N, q_scale)
            layout = O.SF_LINEAR if qkind == "nvfp4_linear" else O.SF_SWIZZLED_128x4
            return O.quant_nvfp4(N, q_scale, layout)
        return out

    t0 = time.perf_counter()
    call()
    n = 2 if time.perf_counter() - t0 > 1.0 else 5
    ts = []
    for _ in range(n):
        t0 = time.perf_counter()
        call()
        ts.append(time.perf_counter() - t0)
    return statistics.median(ts) * 1e6, n


def _dev_set(torch, inp, dev, qkind=""):
    T, H, dt = inp.T, inp.H, inp.rows.dtype
    d = {k: (None if getattr(inp, k) is None else getattr(inp, k).to(dev).contiguous())
         for k in ("rows", "idx", "scales", "shared", "residual", "gamma")}
    d["ro"] = torch.empty(T, H, dtype=dt, device=dev)
    d["no"] = torch.empty(T, H, dtype=dt, device=dev)
    d["s"] = torch.empty(T, H, dtype=dt, device=dev)
    if qkind:
        import moe_expert_output_amd as M
        fp8 = qkind == "fp8"
        d["q"] = torch.empty(T, H if fp8 else H // 2, dtype=torch.uint8, device=dev)
        if not fp8:
            lay = M.MOE_SF_LINEAR if qkind == "nvfp4_linear" else M.MOE_SF_SWIZZLED_128x4
            d["sf"] = torch.empty(M.moe_finalize_sf_size(T, H, lay), dtype=torch.uint8,
                                  device=dev)
    return d


def _set_bytes(inp, qkind=""):
    b = sum(getattr(inp, k).numel() * getattr(inp, k).element_size()
            for k in ("rows", "idx", "scales", "shared", "residual", "gamma")
            if getattr(inp, k) is not None)
    return b + 3 * inp.T * inp.H * 2 + (inp.T * inp.H if qkind else 0)


def _cpu_baseline(inp, nbytes, seconds):
    """The FP64 oracle (unmodified) on this host: whole headline calls, single thread."""
    import oracle as O
    rows = inp.rows.double().numpy()
    idx = inp.idx.numpy()
    sc = inp.scales.double().numpy()
    sh = inp.shared.double().numpy()
    res = inp.residual.double().numpy()
    gam = inp.gamma.double().numpy()
    # pinned to one core for the duration, so the reported core count is a fact of the run
    prev = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else None
    core = min(prev) if prev else None
    if prev:
        os.sched_setaffinity(0, {core})
    try:
        n, t0 = 0, time.perf_counter()
        while True:
            O.finalize_rmsnorm(rows, idx, sc, sh, inp.rsf, res, gam, inp.eps, inp.act_dtype)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    finally:
        if prev:
            os.sched_setaffinity(0, prev)
    per = el / n
    return {"value": round(nbytes / per / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} whole calls of the T=128 H=7168 K=8 workload ({el:.1f} s), "
                      f"{per * 1e3:.1f} ms/call, FP64 numpy, one thread pinned to core {core}",
            "us_per_call": round(per * 1e6, 1), "cpu": _cpu_model(), "nproc": os.cpu_count()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
