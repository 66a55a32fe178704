"""Benchmark of the MoE finalize + residual + RMSNorm path on one MI355X.

Default workload (one "step" = one call of the whole path over one decode batch): 128 tokens,
hidden 7168, top-8 routes with a quarter of them marked -1, float32 softmax expert scales, RSF
2.5, shared-expert add, residual add and RMSNorm (eps 1e-6), bf16 activations, seeded synthetic
inputs resident in HBM. Each timed call reads a different copy of the inputs, rotating over more
than twice the 256 MiB Infinity Cache, so rows come from HBM (cold). The calls are captured in a
HIP graph and replayed; HIP events on the launch stream bracket exactly K calls.

Output: one JSON line (metric, value = achieved algorithmic GB/s, us/call, roofline of the
finalize kernel, the FP64 CPU oracle's throughput on the host as a baseline).
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--sweep] [--no-cpu-baseline]
--sweep adds warm µs/call and the launch floor for every decode shape of the pages' workloads,
and, for the hidden 1024/6144/7168 shapes, the unfused alternative (moe_finalize_run, then
moe_residual_rmsnorm_run) beside the fused call.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

METRIC = "µs/call and achieved HBM GB/s (% of peak) for MoE finalize+RMSNorm, T=1..128"
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["moe_expert_output_amd/csrc/finalize_kernels.hip",
                  "moe_expert_output_amd/csrc/device_utils.h"]
# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (two runs), scaled
# by the same counters' reading for a plain copy of known size; valid only for the kernel
# sources it was taken with.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_finalize_rmsnorm_T128_H7168_K8.json")


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
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


def algorithmic_bytes(T, H, K, n_valid, scale_bytes=4, shared=True, entry="rmsnorm",
                      quant=None):
    """Bytes the path must move: valid rows, route metadata, shared, residual, gamma reads;
    residual_out + norm_out writes (finalize-only: one output; quant: residual_out + codes + SF)."""
    e = ACT_BYTES
    rd = n_valid * H * e + T * K * (4 + scale_bytes) + (T * H * e if shared else 0)
    if entry == "finalize":
        return rd + T * H * e
    rd += T * H * e + H * e
    if quant == "nvfp4":
        sf = ((T + 127) // 128 * 128) * ((H // 16 + 3) // 4 * 4)
        return rd + T * H * e + T * H // 2 + sf
    if quant == "fp8":
        return rd + T * H * e + T * H
    return rd + 2 * T * H * e


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3200)
    p.add_argument("--warmup", type=int, default=320)
    p.add_argument("--sets", type=int, default=32, help="input copies rotated per graph")
    p.add_argument("--sweep", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    return p.parse_args()


def main():
    a = _parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "n_gpus": a.gpus}), flush=True)
        sys.exit(2)

    import torch
    import moe_expert_output_amd as M
    from synth import make_inputs, workload_seed

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
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

    # Capture one graph that calls the path once on every input copy.
    stream = torch.cuda.Stream(device=dev)
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for d in sets[:3]:
            call(d)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for d in sets:
            call(d)

    n_sets = len(sets)
    K_steps, W = int(a.steps), int(a.warmup)
    with torch.cuda.stream(stream):
        for _ in range(max(1, W // n_sets)):
            graph.replay()
        torch.cuda.synchronize()
        t_host0 = time.perf_counter()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(K_steps // n_sets):
            graph.replay()
        for i in range(K_steps % n_sets):          # remainder, launched directly
            call(sets[i])
        ev1.record(stream)
        ev1.synchronize()
        t_host1 = time.perf_counter()
    torch.cuda.synchronize()
    us_per_call = ev0.elapsed_time(ev1) * 1e3 / K_steps
    gbs = nbytes / (us_per_call * 1e-6) / 1e9

    # The pages' protocol (warm): one graph of 20 calls on the same inputs, median of 50 replays.
    warm = _warm_us(torch, stream, lambda: call(sets[0]))
    # Context: a plain device copy moving the same number of bytes (half read, half written),
    # rotated over the same amount of memory; also the known-size kernel that calibrates the
    # FETCH_SIZE / WRITE_SIZE counters.
    copy_us = _copy_reference(torch, stream, dev, nbytes, n_sets)
    floor = _warm_us(torch, stream, lambda: M.moe_finalize_launch_floor_run(1, T, H, K,
                                                                           device=dev))
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
                "routes); inputs resident in HBM, rotated over copies larger than the MALL",
        "config": {"workload": "moe_finalize_rmsnorm decode batch: T=128 tokens, hidden 7168, "
                               "top_k 8 (25% absent), bf16, fp32 scales, shared expert, "
                               "residual + RMSNorm", "tokens": T, "hidden": H, "top_k": K,
                   "parallelism": "none (1 GPU)", "input_copies": n_sets,
                   "rotated_bytes": n_sets * set_bytes},
        "us_per_call": round(us_per_call, 3),
        "us_per_call_warm_median": round(warm, 3),
        "launch_floor_us": round(floor, 3),
        "algorithmic_bytes_per_call": nbytes,
        "host_wall_s": round(t_host1 - t_host0, 4),
        "plain_copy_same_bytes_us": round(copy_us, 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "mfin::finalize_kernel<0, 1, 1, 1, 8> (bf16, RMSNorm, whole rows)",
                     "per_launch_bytes": nbytes, "kernel_source_hash": kernel_source_hash()},
    }
    if a.sweep:
        out["cases"] = _sweep(torch, M, stream, dev, ws)
    out["workspace_flag"] = int(ws[:4].view(torch.int32).item())
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = _cpu_baseline(inp, nbytes, a.cpu_seconds)
    print(json.dumps(out), flush=True)


def _copy_reference(torch, stream, dev, nbytes, n_sets, replays=20):
    half = nbytes // 2 // 2 * 2
    srcs = [torch.empty(half // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
            for _ in range(n_sets)]
    dsts = [torch.empty_like(x) for x in srcs]
    with torch.cuda.stream(stream):
        for s_, d_ in zip(srcs, dsts):
            d_.copy_(s_)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for s_, d_ in zip(srcs, dsts):
                d_.copy_(s_)
        times = []
        for _ in range(replays):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / n_sets)
    return statistics.median(times)


def _warm_us(torch, stream, fn, launches=20, replays=50):
    with torch.cuda.stream(stream):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(launches):
                fn()
        times = []
        for _ in range(replays):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / launches)
    return statistics.median(times)


def _sweep(torch, M, stream, dev, ws_big):
    """µs/call for the pages' decode shapes: warm (same inputs) and cold (rotated copies)."""
    from synth import make_inputs, workload_seed
    cases = []
    shapes = [("tiny", 4, 1024, 8, "bf16", "fp32", True)]
    shapes += [("decode", t, 6144, 8, "bf16", "fp32", True) for t in (1, 4, 16)]
    shapes += [("larger", t, 7168, 8, act, "fp32", True) for act in ("bf16", "fp16")
               for t in (32, 64, 128)]
    shapes += [("highk", t, h, k, "bf16", sdt, False) for (h, k) in ((2048, 22), (3584, 16))
               for sdt in ("fp32",) for t in (1, 8, 16, 32)]
    for (grp, T, H, K, act, sdt, sh) in shapes:
        inp = make_inputs(T, H, K, act_dtype=act, scale_dtype=sdt, with_shared=sh,
                          seed=workload_seed(grp, T, act, sdt, K if grp == "highk" else None))
        n_valid = int((inp.idx >= 0).sum())
        dt = inp.rows.dtype
        d = {k: (None if getattr(inp, k) is None else getattr(inp, k).to(dev)) for k in
             ("rows", "idx", "scales", "shared", "residual", "gamma")}
        ro = torch.empty(T, H, dtype=dt, device=dev)
        no = torch.empty(T, H, dtype=dt, device=dev)
        ws = ws_big
        s_buf = torch.empty(T, H, dtype=dt, device=dev)
        for entry in ("rmsnorm", "finalize", "two_kernel"):
            if entry == "finalize" and grp not in ("highk",):
                continue
            if entry == "two_kernel" and grp not in ("tiny", "decode", "larger"):
                continue
            if entry == "two_kernel":
                # the unfused alternative: finalize, then residual + RMSNorm as its own kernel
                def fn(d=d, ro=ro, no=no, inp=inp, ws=ws, s_buf=s_buf):
                    M.moe_finalize_run(d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf,
                                       s_buf)
                    M.moe_residual_rmsnorm_run(s_buf, d["residual"], d["gamma"], inp.eps, ro, no,
                                               ws)

                def floor_fn(T=T, H=H, K=K):               # two empty launches
                    M.moe_finalize_launch_floor_run(0, T, H, K, device=dev)
                    M.moe_finalize_launch_floor_run(1, T, H, 1, device=dev)
            elif entry == "rmsnorm":
                fn = (lambda d=d, ro=ro, no=no, inp=inp, ws=ws: M.moe_finalize_rmsnorm_run(
                    d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf, d["residual"],
                    d["gamma"], inp.eps, ro, no, ws))
                floor_fn = (lambda T=T, H=H, K=K:
                            M.moe_finalize_launch_floor_run(1, T, H, K, device=dev))
            else:
                fn = (lambda d=d, no=no, inp=inp: M.moe_finalize_run(
                    d["rows"], d["idx"], d["scales"], d["shared"], inp.rsf, no))
                floor_fn = (lambda T=T, H=H, K=K:
                            M.moe_finalize_launch_floor_run(0, T, H, K, device=dev))
            us = _warm_us(torch, stream, fn)
            floor = _warm_us(torch, stream, floor_fn)
            # the fused path's algorithmic bytes for both rmsnorm entries: the two-kernel
            # path's extra write and re-read of s is the cost the fusion removes
            nb = algorithmic_bytes(T, H, K, n_valid, 4 if sdt == "fp32" else 2, sh,
                                   "rmsnorm" if entry == "two_kernel" else entry)
            cases.append({"group": grp, "entry": entry, "T": T, "H": H, "K": K, "act": act,
                          "scales": sdt, "us_warm": round(us, 3), "floor_us": round(floor, 3),
                          "excess_us": round(us - floor, 3), "bytes": nb,
                          "gbs_warm": round(nb / (us * 1e-6) / 1e9, 1)})
    return cases


def _cpu_baseline(inp, nbytes, seconds):
    """The FP64 oracle (unmodified) on this host: whole headline calls, single thread."""
    import oracle as O
    rows = inp.rows.double().numpy()
    idx = inp.idx.numpy()
    sc = inp.scales.double().numpy()
    sh = inp.shared.double().numpy()
    res = inp.residual.double().numpy()
    gam = inp.gamma.double().numpy()
    n, t0 = 0, time.perf_counter()
    while True:
        O.finalize_rmsnorm(rows, idx, sc, sh, inp.rsf, res, gam, inp.eps, inp.act_dtype)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / n
    return {"value": round(nbytes / per / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} whole calls of the T=128 H=7168 K=8 workload ({el:.1f} s), "
                      f"{per * 1e3:.1f} ms/call, FP64 numpy, one thread",
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
