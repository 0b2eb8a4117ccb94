#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE FFN layer on one MI355X.

Workload: Mixtral-8x7B expert shape (hidden 4096, intermediate 14336, 8
experts, top-2), BF16 row-major weights ~ N(0, 0.02), routing forced so that
every expert gets exactly m tokens (T = 4m), m in {1, 2, 4, 8, 16}; router
logits ~ N(0,1) (HiNa-MoE §7.3 and Table 3 shapes, 1-16 tokens per expert).
One step = one layer call at each m (five layers).  Inputs are resident in
HBM before timing; the router runs once per batch before the timed region.

Printed (one JSON line): weight-stream throughput in GB/s (algorithmic bytes:
active experts' weights + x + out + routing ids/weights, per layer) over the
timed steps, microseconds per layer for each m, the roofline of the dominant
kernel (gate/up) from per-kernel HIP events, and the CPU oracle timed on a
bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per MoE FFN layer + weight-stream GB/s (% HBM peak), BF16, 1–16 tok/expert"
HBM_PEAK_GBS = 8000.0
MS = (1, 2, 4, 8, 16)


def layer_bytes(wl) -> int:
    """Algorithmic HBM bytes of one layer: every active expert's three weight
    matrices once, x read, out written, routing ids and weights read."""
    import workloads
    active = min(wl.E, wl.T * wl.k)    # forced routing: all experts active
    return (active * workloads.weight_bytes_per_expert(wl) + 2 * wl.T * wl.H * 2
            + wl.T * wl.k * 8)


def gateup_bytes(wl) -> int:
    """Algorithmic bytes of one gate/up launch: W_gate and W_up of every active
    expert plus the token rows (h is scratch and not credited)."""
    active = min(wl.E, wl.T * wl.k)
    return active * 2 * wl.I * wl.H * 2 + wl.T * wl.H * 2


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "expert_gemm_mixtral8x7b_m1-16_hbm_traffic.md")
KERNEL_SOURCES = ("routed_expert_ffn_topk_amd/csrc/expert_gemm.hip",
                  "routed_expert_ffn_topk_amd/csrc/common.hpp")


def recorded_traffic():
    """HBM bytes per gate/up launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record (scaled by a plain copy of known size), or None when the
    kernel sources have changed since the counters were taken."""
    try:
        text = open(TRAFFIC_PROFILE).read()
        digests = "".join(hashlib.sha256(open(os.path.join(ROOT, f), "rb").read()).hexdigest()
                          for f in KERNEL_SOURCES)
    except OSError:
        return None
    rec = dict(re.findall(r"^(kernel_source_sha256_16|gateup_traffic_bytes_per_launch): (\S+)$",
                          text, re.M))
    if rec.get("kernel_source_sha256_16") != hashlib.sha256(digests.encode()).hexdigest()[:16]:
        return None
    return int(rec["gateup_traffic_bytes_per_launch"])


def cpu_baseline(wl, Wg, Wu, Wd, logits_cpu, x_cpu, reps=3):
    """The CPU oracle on one m=1 layer (T=4: every expert streamed once)."""
    import numpy as np

    import oracle
    import workloads
    ids, w = oracle.route_topk(logits_cpu.numpy(), wl.k)
    need = sorted(set(ids.reshape(-1).tolist()))
    host = [{e: workloads.bf16_bits(W[e]) for e in need} for W in (Wg, Wu, Wd)]
    xb = workloads.bf16_bits(x_cpu)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.moe_ffn_bf16(xb, ids, w, host[0].get, host[1].get, host[2].get, E=wl.E)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    del host
    return {"value": round(layer_bytes(wl) / t / 1e9, 3), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "us_per_layer": round(t * 1e6, 1),
            "sample": f"one Mixtral-8x7B layer at m=1 (T=4, all 8 experts), median of {reps} "
                      f"runs, plain C oracle (FP32 accumulation, per-token loops)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB, 5 times "
                         "(calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE), then exit")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 5}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this build runs the MoE FFN "
              "layer on one GPU only (see the sharding notes in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch

    import routed_expert_ffn_topk_amd as moe
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wls = [workloads.WORKLOADS[f"mixtral8x7b_m{m}"] for m in MS]
    wl0 = wls[0]
    Wg, Wu, Wd = workloads.gen_weights(wl0, "cuda")
    batches = []
    for wl in wls:
        x = workloads.gen_x(wl)
        lg = workloads.gen_logits(wl)
        ids, w = moe.moe_route_topk(lg.to(dev), wl.k)
        batches.append(dict(wl=wl, x_cpu=x, lg_cpu=lg, x=x.to(dev), ids=ids, w=w,
                            out=torch.empty(wl.T, wl.H, dtype=torch.bfloat16, device=dev),
                            ws=moe.alloc_workspace(wl.T, wl.H, wl.I, wl.E, wl.k, dev)))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def layer(b):
        moe.moe_ffn_forward(b["x"], b["ids"], b["w"], Wg, Wu, Wd, out=b["out"],
                            workspace=b["ws"], stream=stream)

    def step():
        for b in batches:
            layer(b)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    step_bytes = sum(layer_bytes(b["wl"]) for b in batches)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # microseconds per layer at each m (same calls, timed per batch)
    per_m = {}
    reps = max(5, args.steps // 2)
    for b in batches:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            layer(b)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        per_m[str(b["wl"].T // 4)] = {
            "us": round(us, 1),
            "GBps": round(layer_bytes(b["wl"]) / (us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100 * layer_bytes(b["wl"]) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
        }

    # per-kernel durations from HIP events recorded between the kernels of
    # each call (stage 0 permute, 1 gate/up, 2 down, 3 combine)
    names = ("permute", "gateup", "down", "combine")
    dur = {n: [] for n in names}
    dur_m = {str(b["wl"].T // 4): {n: [] for n in names} for b in batches}
    gu_bytes = []
    for _ in range(max(3, args.steps // 5)):
        for b in batches:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            for e in ev:
                e.record(stream)          # materialise the HIP events
            ev[0].record(stream)
            moe.moe_ffn_set_stage_events(ev[1:])
            layer(b)
            torch.cuda.synchronize()
            for i, n in enumerate(names):
                d = ev[i].elapsed_time(ev[i + 1]) * 1e3
                dur[n].append(d)
                dur_m[str(b["wl"].T // 4)][n].append(d)
            gu_bytes.append(gateup_bytes(b["wl"]))
    for m, d in dur_m.items():
        per_m[m]["stage_us"] = {n: round(statistics.mean(v), 1) for n, v in d.items()}
    gu_us = statistics.mean(dur["gateup"])
    achieved = statistics.mean(gu_bytes) / (gu_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": "expert_gemm_kernel (gate/up)",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
                "algorithmic_bytes": int(statistics.mean(gu_bytes)), "avg_us": round(gu_us, 2),
                "stage_us": {n: round(statistics.mean(v), 2) for n, v in dur.items()}}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mixtral8x7b_forced_m1-16", "hidden": 4096,
                   "intermediate": 14336, "experts": 8, "top_k": 2,
                   "tokens_per_expert": list(MS), "layers_per_step": len(MS),
                   "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
                   "per_m": per_m, "device": torch.cuda.get_device_name(dev)},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        b = batches[0]
        result["cpu_baseline"] = cpu_baseline(b["wl"], Wg, Wu, Wd, b["lg_cpu"], b["x_cpu"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
