#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE FFN layer on one MI355X.

Default workload (``--workload mixtral8x7b_forced_m1-16``): Mixtral-8x7B expert
shape (hidden 4096, intermediate 14336, 8 experts, top-2), BF16 row-major
weights ~ N(0, 0.02), routing forced so that every expert gets exactly m
tokens (T = 4m), m in {1, 2, 4, 8, 16}; router logits ~ N(0,1) (HiNa-MoE §7.3
and Table 3 shapes, 1-16 tokens per expert).  One step = one layer call at
each m (five layers).

Other workloads: ``mixtral8x7b_int8_forced_m1-16`` and
``mixtral8x7b_int4_forced_m1-16`` (the same with INT8 / INT4 group-quantised
weights), and any single layer of the workload registry
(``deepseekv3_t16``, ``deepseekv3_zipf_t16``, ``mixtral8x22b_t{1,4,16}``,
``qwen3_235b_t{1,4,16}``, and the prefill-sized ``mixtral8x7b_t{512,2048}``,
``qwen3_235b_t2048``, ``deepseekv3_t4096``): one step = one call of that
layer.  When the active experts' weights of a layer are small enough to stay
in the 256 MB last-level cache between calls, the step cycles through several
distinct weight sets (as consecutive layers of a model would), so that every
call streams its weights from HBM.  Prefill-sized layers (more than 64 tokens,
BF16) run the tiled product, which the matrix unit bounds: their roofline is
reported in TFLOP/s against the dense BF16 peak.

Decode attention (HiNa-MoE §6.1; ``--workload attn_*``: Qwen3-30B-A3B,
Mixtral-8x7B and Qwen2-57B-A14B head layouts, batches of 1-32 sequences of up
to 32768 positions): one step = one ``moe_attn_decode`` call over the batch;
value = K and V bytes of the valid positions (+ q and out) per second, the
roofline that of the split kernel, which streams every K and V byte.

Inputs are resident in HBM before timing; the router runs once per batch
before the timed region.  Printed (one JSON line): weight-stream throughput in
GB/s (algorithmic bytes: active experts' weights + x + out + routing ids and
weights, per layer) over the timed steps, microseconds per layer, the roofline
of the dominant kernel (gate/up) from per-kernel HIP events, and the CPU
oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per MoE FFN layer + weight-stream GB/s (% HBM peak), BF16, 1–16 tok/expert"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense BF16 matrix-unit peak of MI355X
TILED_MIN_BATCH = 64             # batches above this take the tiled product (BF16)
MS = (1, 2, 4, 8, 16)
DEFAULT_WORKLOAD = "mixtral8x7b_forced_m1-16"
ROTATE_BELOW = 2 << 30         # a step streams >= 2 GiB (8x the 256 MB last-level cache)
CPU_SAMPLE_MACS = 2.0e10       # oracle sample: multiply-adds per run ...
CPU_SAMPLE_BYTES = 3 << 30     # ... and expert bytes copied to the host


def suite_layers(name: str):
    """Layers (workload registry entries) of one benchmark step."""
    import workloads
    if name == DEFAULT_WORKLOAD:
        return [workloads.WORKLOADS[f"mixtral8x7b_m{m}"] for m in MS]
    if name == "mixtral8x7b_int8_forced_m1-16":
        return [workloads.WORKLOADS[f"mixtral8x7b_int8_m{m}"] for m in MS]
    if name == "mixtral8x7b_int4_forced_m1-16":
        return [workloads.WORKLOADS[f"mixtral8x7b_int4_m{m}"] for m in MS]
    if name == "mixtral8x7b_resplit_forced_m1-16":
        return [workloads.WORKLOADS[f"mixtral8x7b_resplit_m{m}"] for m in MS]
    if name in workloads.WORKLOADS:
        return [workloads.WORKLOADS[name]]
    raise SystemExit(f"bench.py: unknown workload {name!r}")


def expert_bytes(wl) -> int:
    import workloads
    return workloads.weight_bytes_per_expert(wl)


def layer_bytes(wl, active: int, weight_bytes=None) -> int:
    """Algorithmic HBM bytes of one layer: every active expert's three weight
    matrices (and scales) once, x read, out written, routing ids and weights
    read.  ``weight_bytes`` overrides active * expert_bytes (residual split,
    where an expert's bytes depend on its precision)."""
    wb = active * expert_bytes(wl) if weight_bytes is None else weight_bytes
    return wb + 2 * wl.T * wl.H * 2 + wl.T * wl.k * 8


def layer_flops(wl) -> float:
    """Multiply-add FLOPs of one layer: 3 products of H x I per routed slot."""
    return 6.0 * wl.T * wl.k * wl.H * wl.I


def uses_tiled(wl) -> bool:
    return not wl.int8 and not wl.int4 and not wl.resplit and wl.T > TILED_MIN_BATCH


def gateup_bytes(wl, active: int, n_critical: int = 0) -> int:
    """Algorithmic bytes of one gate/up launch: W_gate and W_up (and their
    scales) of every active expert plus the token rows (h is scratch and not
    credited).  Residual split: n_critical of the active experts also read
    W^R and its scales."""
    if wl.resplit:
        per = wl.I * wl.H * (0.5 + 4 / wl.group)
        return int((active + n_critical) * 2 * per) + wl.T * wl.H * 2
    if wl.int8:
        per = wl.I * wl.H * (1 + 4 / wl.group)
    elif wl.int4:
        per = wl.I * wl.H * (0.5 + 4 / wl.group)
    else:
        per = wl.I * wl.H * 2
    return int(active * 2 * per) + wl.T * wl.H * 2


PROFILES = os.path.join(ROOT, "profiles")


def source_hash(files) -> str:
    """First 16 hex digits of SHA-256 over the SHA-256 hex digests of the
    given source files (paths relative to the repository root)."""
    digests = "".join(hashlib.sha256(open(os.path.join(ROOT, f), "rb").read()).hexdigest()
                      for f in files)
    return hashlib.sha256(digests.encode()).hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per launch of the workload's dominant kernel from a committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE record (profiles/*_hbm_traffic.md,
    scaled by a plain copy of known size), or None when there is none or the
    kernel sources it names have changed since the counters were taken."""
    import glob
    for path in sorted(glob.glob(os.path.join(PROFILES, "*_hbm_traffic.md"))):
        try:
            text = open(path).read()
        except OSError:
            continue
        rec = dict(re.findall(r"^(kernel_sources|kernel_source_sha256_16|workload|"
                              r"gateup_traffic_bytes_per_launch|traffic_bytes_per_launch): "
                              r"(\S+)$", text, re.M))
        if rec.get("workload") != workload or "kernel_sources" not in rec:
            continue
        try:
            digest = source_hash(rec["kernel_sources"].split(","))
        except OSError:
            return None
        if rec.get("kernel_source_sha256_16") != digest:
            return None
        return int(rec.get("traffic_bytes_per_launch") or rec["gateup_traffic_bytes_per_launch"])
    return None


def read_ceiling(stream, nbytes=4 << 30, reps=10) -> float:
    """Measured HBM streaming-read ceiling (GB/s): the library's read probe
    over a 4 GiB buffer, best of `reps` timed passes after two warm-ups."""
    import torch

    import routed_expert_ffn_topk_amd as moe
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        moe.moe_ffn_read_probe(buf, sink, stream)
    best = None
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        moe.moe_ffn_read_probe(buf, sink, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3
        best = us if best is None else min(best, us)
    del buf
    torch.cuda.empty_cache()
    return nbytes / (best * 1e-6) / 1e9


def cpu_baseline(wl, host_weights, logits_cpu, x_cpu, reps=5, critical=None):
    """The CPU oracle on a bounded token sample of one layer of the workload:
    the leading tokens, as many as fit CPU_SAMPLE_MACS multiply-adds and
    CPU_SAMPLE_BYTES of expert weights copied to the host."""
    import torch

    import oracle
    import workloads
    ids, w = oracle.route_topk(logits_cpu.numpy(), wl.k)
    n, need = 0, set()
    per_slot = 3 * wl.H * wl.I
    while n < wl.T:
        cand = need | set(ids[n].tolist())
        if n > 0 and ((n + 1) * wl.k * per_slot > CPU_SAMPLE_MACS
                      or len(cand) * expert_bytes(wl) > CPU_SAMPLE_BYTES):
            break
        need, n = cand, n + 1
    need = sorted(need)
    to_host = lambda t: (workloads.bf16_bits(t) if t.dtype == torch.bfloat16  # noqa: E731
                         else t.cpu().numpy())
    tables = [{e: to_host(W[e]) for e in need} for W in host_weights]
    xb = workloads.bf16_bits(x_cpu[:n])
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        if wl.resplit:
            oracle.moe_ffn_resplit(xb, ids[:n], w[:n], *(t.get for t in tables), critical,
                                   E=wl.E)
        elif wl.int8 or wl.int4:
            # INT4 is the INT8 definition on values in [-7, 7] (unpacked here)
            oracle.moe_ffn_int8(xb, ids[:n], w[:n], *(t.get for t in tables), E=wl.E)
        else:
            oracle.moe_ffn_bf16(xb, ids[:n], w[:n], *(t.get for t in tables), E=wl.E)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    wbytes = (sum(workloads.weight_bytes_per_expert(wl, bool(critical[e])) for e in need)
              if wl.resplit else len(need) * expert_bytes(wl))
    sample_bytes = wbytes + 2 * n * wl.H * 2 + n * wl.k * 8
    return {"value": round(sample_bytes / t / 1e9, 3), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
            "us_per_layer": round(t * 1e6, 1), "runs": reps,
            "tiny_single_thread": tiny_single_thread(),
            "sample": f"{wl.name}: the first {n} of {wl.T} tokens ({len(need)} experts), "
                      f"median of {reps} runs, plain C oracle (FP32 accumulation, per-token "
                      f"loops, {'residual-split INT4/INT8' if wl.resplit else 'INT8' if wl.int8 else 'INT4' if wl.int4 else 'BF16'} weights)"}


def per_call_us(call, n, stream):
    """GPU microseconds of each of n back-to-back calls: an event is recorded
    on the launch stream before the first call and after every call, with one
    synchronisation at the end (the host enqueues ahead of the GPU)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record(stream)
    for i in range(n):
        call(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n)]


def call_stats(us):
    """Median and geometric mean (the pages' summary statistic) of per-call
    times, with the spread."""
    return {"calls": len(us), "median": round(statistics.median(us), 2),
            "geomean": round(math.exp(statistics.mean(math.log(u) for u in us)), 2),
            "min": round(min(us), 2), "max": round(max(us), 2)}


def launch_gap_us(stream, n=2000):
    """Dispatch gap between back-to-back kernels on the stream: GPU time of a
    chain of n empty kernels (the library's launch probe) divided by n."""
    import torch

    import routed_expert_ffn_topk_amd as moe
    moe.moe_ffn_launch_probe(100, stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    moe.moe_ffn_launch_probe(n, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) * 1e3 / n, 3)


def cpu_model() -> str:
    """The host CPU's model name (lscpu), or the platform's processor string."""
    import platform
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for ln in out.splitlines():
            if ln.strip().startswith("Model name:"):
                return ln.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    return platform.processor() or "unknown"


def tiny_single_thread(reps=100):
    """The oracle on the Tiny layer (hidden 256, intermediate 512, 8 experts,
    top-2, 16 tokens) on one thread, median of reps runs."""
    import oracle
    import workloads
    wl = workloads.WORKLOADS["tiny"]
    xb = workloads.bf16_bits(workloads.gen_x(wl))
    ids, w = oracle.route_topk(workloads.gen_logits(wl).numpy(), wl.k)
    W = [workloads.bf16_bits(t) for t in workloads.gen_weights(wl, "cpu")]
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        used = oracle.num_threads()
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.moe_ffn_bf16(xb, ids, w, W[0], W[1], W[2], E=wl.E)
            times.append(time.perf_counter() - t0)
    finally:
        oracle.set_num_threads(threads)
    return {"us": round(statistics.median(times) * 1e6, 1), "threads": used, "runs": reps}


ATTN_METRIC = "decode GQA attention: KV-stream GB/s (% HBM peak) and µs per call, BF16"


def cpu_baseline_attn(wl, q, k_host, v_host, lens, reps=5):
    """The CPU oracle on a bounded sample of the same attention batch: the
    leading sequences whose KV positions total at most 2^23 (a few seconds of
    CPU work), median of `reps` runs, in the same GB/s unit."""
    import oracle
    import workloads
    n, pos = 0, 0
    while n < wl.B and (n == 0 or pos + int(lens[n]) <= (1 << 23)):
        pos += int(lens[n])
        n += 1
    qb = workloads.bf16_bits(q[:n])
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.attn_decode(qb, k_host[:n], v_host[:n], lens[:n].numpy())
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    nbytes = pos * wl.h_kv * wl.d * 4 + 2 * n * wl.h_q * wl.d * 2
    return {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(), "us_per_call": round(t * 1e6, 1),
            "runs": reps,
            "sample": f"{wl.name}: the first {n} of {wl.B} sequences ({pos} KV positions), "
                      f"median of {reps} runs, plain C oracle (FP32 scores, softmax and "
                      f"value sums, BF16 inputs)"}


def run_attn(args):
    """Decode attention: one step = one moe_attn_decode call over the batch
    (several distinct KV caches in turn when one is small enough to stay in
    the last-level cache)."""
    import torch

    import routed_expert_ffn_topk_amd as moe
    import workloads
    wl = workloads.ATTN_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    q = workloads.gen_attn_q(wl)
    lens = workloads.gen_attn_lens(wl)
    kv_bytes = workloads.attn_kv_bytes(wl, lens)
    n_sets = max(1, math.ceil(ROTATE_BELOW / kv_bytes)) if kv_bytes < ROTATE_BELOW else 1
    sets = [workloads.gen_attn_kv(workloads.AttnWorkload(**{**wl.__dict__, "seed": wl.seed + r}),
                                  dev) for r in range(n_sets)]
    qd, ld = q.to(dev), lens.to(dev)
    out = torch.empty_like(qd)
    ws = torch.empty(moe.moe_attn_decode_workspace_bytes(wl.B, wl.h_q, wl.h_kv, wl.d, wl.max_len),
                     dtype=torch.uint8, device=dev)

    def call(i):
        k, v = sets[i % n_sets]
        moe.moe_attn_decode(qd, k, v, ld, out=out, workspace=ws, stream=stream)

    def step():
        for i in range(n_sets):
            call(i)

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
    call_bytes = kv_bytes + 2 * wl.B * wl.h_q * wl.d * 2
    per_call = call_stats(per_call_us(call, max(100, args.calls), stream))
    value = n_sets * call_bytes / (ms_per_step * 1e-3) / 1e9
    # per-kernel durations from HIP events on the launch stream: split kernel
    # (the dominant one: every K and V byte), then the merge of the splits
    split_us, merge_us = [], []
    for i in range(max(5, args.steps)):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for e in ev:
            e.record(stream)
        ev[0].record(stream)
        moe.moe_ffn_set_stage_events(ev[1:])
        call(i)
        torch.cuda.synchronize()
        split_us.append(ev[0].elapsed_time(ev[1]) * 1e3)
        merge_us.append(ev[1].elapsed_time(ev[2]) * 1e3)
    s_us = statistics.mean(split_us)
    algo = kv_bytes + wl.B * wl.h_q * wl.d * 2
    achieved = algo / (s_us * 1e-6) / 1e9
    ceiling = read_ceiling(stream)
    result = {
        "metric": ATTN_METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "q_heads": wl.h_q, "kv_heads": wl.h_kv,
                   "head_dim": wl.d, "max_len": wl.max_len, "lengths": wl.lens,
                   "kv_positions": int(lens.sum()), "kv_sets": n_sets,
                   "us_per_call": round(ms_per_step * 1e3 / n_sets, 1),
                   "per_call_us": per_call, "launch_gap_us": launch_gap_us(stream),
                   "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
                   "pct_measured_read_ceiling": round(100 * value / ceiling, 1),
                   "device": torch.cuda.get_device_name(dev)},
        "roofline": {"bound": "hbm", "kernel": "attn_split_kernel (scores, softmax, values)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(args.workload),
                     "measured_read_ceiling": round(ceiling, 1),
                     "frac_of_measured_ceiling": round(achieved / ceiling, 4),
                     "algorithmic_bytes": algo, "avg_us": round(s_us, 2),
                     "stage_us": {"split": round(s_us, 2),
                                  "merge": round(statistics.mean(merge_us), 2)}},
    }
    if not args.no_cpu_baseline:
        k, v = sets[0]
        n_host = min(wl.B, 64)
        kh = workloads.bf16_bits(k[:n_host])
        vh = workloads.bf16_bits(v[:n_host])
        result["cpu_baseline"] = cpu_baseline_attn(wl, q, kh, vh, lens)
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calls", type=int, default=100,
                    help="calls per layer timed one by one for the median / geometric mean")
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
        print(f"bench.py: --gpus {args.gpus} is not supported: the MoE FFN layer is measured "
              "on one GPU only", file=sys.stderr)
        sys.exit(2)

    import workloads
    if args.workload in workloads.ATTN_WORKLOADS:
        run_attn(args)
        return

    import torch

    import routed_expert_ffn_topk_amd as moe

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = suite_layers(args.workload)
    int8 = layers[0].int8
    int4 = layers[0].int4
    resplit = layers[0].resplit
    quant = int8 or int4 or resplit
    # residual split: one set of per-expert precision flags for the suite
    crit = workloads.gen_critical(layers[0]) if resplit else None
    stream = torch.cuda.current_stream()

    batches = []
    for wl in layers:
        x = workloads.gen_x(wl)
        lg = workloads.gen_logits(wl)
        ids, w = moe.moe_route_topk(lg.to(dev), wl.k)
        act = sorted(set(ids.cpu().reshape(-1).tolist()))
        active = len(act)
        wbytes = (sum(workloads.weight_bytes_per_expert(wl, bool(crit[e])) for e in act)
                  if resplit else active * expert_bytes(wl))
        n_crit = int(sum(int(crit[e]) for e in act)) if resplit else 0
        batches.append(dict(wl=wl, x_cpu=x, lg_cpu=lg, lg=lg.to(dev), x=x.to(dev), ids=ids, w=w,
                            active=active, wbytes=wbytes, n_crit=n_crit,
                            out=torch.empty(wl.T, wl.H, dtype=torch.bfloat16, device=dev),
                            ws=moe.alloc_workspace(wl.T, wl.H, wl.I, wl.E, wl.k, dev)))
    # distinct weight sets so that one step streams at least ROTATE_BELOW bytes
    step_weight_bytes = sum(b["wbytes"] for b in batches)
    n_sets = max(1, math.ceil(ROTATE_BELOW / step_weight_bytes)) \
        if step_weight_bytes < ROTATE_BELOW else 1
    wl0 = layers[0]
    sets = []
    for r in range(n_sets):
        wlr = workloads.Workload(**{**wl0.__dict__, "seed": wl0.seed + r})
        if resplit:
            tens = workloads.gen_weights_resplit(wlr, dev)
            p4 = workloads.pack_int4
            Qg, Sg, Rg, SRg, Qu, Su, Ru, SRu, Qdl, Sdl, Qdh, Sdh = tens
            sets.append((p4(Qg), Sg, p4(Rg), SRg, p4(Qu), Su, p4(Ru), SRu,
                         p4(Qdl), Sdl, Qdh, Sdh, torch.from_numpy(crit).to(dev)))
            if r == 0:
                host_rowmajor = tens
            else:
                del tens, Qg, Sg, Rg, SRg, Qu, Su, Ru, SRu, Qdl, Sdl, Qdh, Sdh
        elif quant:
            gen = workloads.gen_weights_int8 if int8 else workloads.gen_weights_int4
            Qg, Sg, Qu, Su, Qd, Sd = gen(wlr, dev)
            store = (lambda q: q) if int8 else workloads.pack_int4  # noqa: E731
            sets.append((store(Qg), Sg, store(Qu), Su, store(Qd), Sd))
            if r == 0:
                host_rowmajor = (Qg, Sg, Qu, Su, Qd, Sd)
            else:
                del Qg, Qu, Qd, Sg, Su, Sd
        else:
            sets.append(workloads.gen_weights(wlr, dev))
    torch.cuda.synchronize()
    fwd = (moe.moe_ffn_forward_int8 if int8 else moe.moe_ffn_forward_int4 if int4
           else moe.moe_ffn_forward_resplit if resplit else moe.moe_ffn_forward)

    def layer(b, s):
        fwd(b["x"], b["ids"], b["w"], *sets[s], out=b["out"], workspace=b["ws"], stream=stream)

    def step():
        for b in batches:
            for s in range(n_sets):
                layer(b, s)

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
    step_bytes = n_sets * sum(layer_bytes(b["wl"], b["active"], b["wbytes"]) for b in batches)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # microseconds per layer (same calls, timed per batch)
    per_layer = {}
    reps = max(5, args.steps // 2)
    for b in batches:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            layer(b, i % n_sets)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        lb = layer_bytes(b["wl"], b["active"], b["wbytes"])
        per_layer[b["wl"].name] = {
            "T": b["wl"].T, "active_experts": b["active"], "us": round(us, 1),
            "GBps": round(lb / (us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100 * lb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
            "TFLOPs": round(layer_flops(b["wl"]) / (us * 1e-6) / 1e12, 1),
        }
        if not quant:
            # the same layer from router logits (router fused with the gather
            # index); its ids / weights go to scratch tensors
            rid = torch.empty_like(b["ids"])
            rw = torch.empty_like(b["w"])
            e0.record(stream)
            for i in range(reps):
                moe.moe_ffn_forward_logits(b["x"], b["lg"], b["wl"].k, *sets[i % n_sets],
                                           out=b["out"], topk_ids=rid, topk_w=rw,
                                           workspace=b["ws"], stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            per_layer[b["wl"].name]["us_from_logits"] = round(e0.elapsed_time(e1) * 1e3 / reps, 1)
            # the same from two calls: the router, then the layer on its ids
            e0.record(stream)
            for i in range(reps):
                moe.moe_route_topk(b["lg"], b["wl"].k, topk_ids=rid, topk_w=rw, stream=stream)
                layer_ids = dict(b, ids=rid, w=rw)
                layer(layer_ids, i % n_sets)
            e1.record(stream)
            torch.cuda.synchronize()
            per_layer[b["wl"].name]["us_route_then_layer"] = round(
                e0.elapsed_time(e1) * 1e3 / reps, 1)
            # the routers alone: the softmax gate, and (256 experts: DeepSeek-V3's
            # grouping, 8 groups, 4 kept, scale 2.5) the grouped sigmoid gate
            for key, route in (("us_route_topk", lambda: moe.moe_route_topk(
                    b["lg"], b["wl"].k, topk_ids=rid, topk_w=rw, stream=stream)),
                    ("us_route_grouped", lambda: moe.moe_route_grouped(
                        b["lg"], b["wl"].k, 8, 4, scale=2.5, topk_ids=rid, topk_w=rw,
                        stream=stream))):
                if key == "us_route_grouped" and b["wl"].E != 256:
                    continue
                e0.record(stream)
                for i in range(reps):
                    route()
                e1.record(stream)
                torch.cuda.synchronize()
                per_layer[b["wl"].name][key] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)

    # per-call statistics: every layer timed call by call, at least 100 calls
    ncalls = max(100, args.calls)
    for b in batches:
        us = per_call_us(lambda i, b=b: layer(b, i % n_sets), ncalls, stream)
        per_layer[b["wl"].name]["per_call_us"] = call_stats(us)
    names_l = [b["wl"].name for b in batches]
    m1 = next((n for n in names_l if n.endswith("_m1")), None)
    m16 = next((n for n in names_l if n.endswith("_m16")), None)
    m16_over_m1 = (round(per_layer[m16]["per_call_us"]["median"] /
                         per_layer[m1]["per_call_us"]["median"], 3) if m1 and m16 else None)
    gap = launch_gap_us(stream)

    # per-kernel durations from HIP events recorded on the launch stream
    # between the kernels of each call (stage 0 the gather-index kernel, 1
    # gate/up, 2 down, 3 combine).  Batches of up to 256 slots from given ids
    # have no index kernel (gate/up builds the index in its prologue): their
    # stage 0 is two events back to back, which measures the events' own
    # overhead, and is reported as "index" all the same.
    names = ("index", "gateup", "down", "combine")
    dur = {n: [] for n in names}
    dur_l = {b["wl"].name: {n: [] for n in names} for b in batches}
    gu_bytes = []
    for i in range(max(3, args.steps // 5)):
        for b in batches:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            for e in ev:
                e.record(stream)          # materialise the HIP events
            ev[0].record(stream)
            moe.moe_ffn_set_stage_events(ev[1:])
            layer(b, i % n_sets)
            torch.cuda.synchronize()
            for j, n in enumerate(names):
                d = ev[j].elapsed_time(ev[j + 1]) * 1e3
                dur[n].append(d)
                dur_l[b["wl"].name][n].append(d)
            gu_bytes.append(gateup_bytes(b["wl"], b["active"], b["n_crit"]))
    for name, d in dur_l.items():
        per_layer[name]["stage_us"] = {n: round(statistics.mean(v), 1) for n, v in d.items()}
    gu_us = statistics.mean(dur["gateup"])
    ceiling = read_ceiling(stream)
    if all(uses_tiled(b["wl"]) for b in batches):
        # many tokens per expert: the tiled product is bound by the matrix
        # unit; achieved = gate/up FLOPs per launch over the gate/up stage
        # (the small-m launch before it finds no expert and exits)
        gu_flops = statistics.mean(4.0 * b["wl"].T * b["wl"].k * b["wl"].H * b["wl"].I
                                   for b in batches)
        achieved = gu_flops / (gu_us * 1e-6) / 1e12
        roofline = {"bound": "mfma",
                    "kernel": "expert_tile_kernel<0> (gate/up, 256-row tiles, register-staged, "
                              "SiLU*up epilogue)",
                    "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": recorded_traffic(args.workload),
                    "algorithmic_flops": gu_flops, "avg_us": round(gu_us, 2),
                    "measured_read_ceiling": round(ceiling, 1),
                    "stage_us": {n: round(statistics.mean(v), 2) for n, v in dur.items()}}
    else:
        achieved = statistics.mean(gu_bytes) / (gu_us * 1e-6) / 1e9
        kern = ("expert_gemm_kernel<Int8Weights, 2, ...>" if int8 else
                "expert_gemm_kernel<Int4Weights, 2, ...>" if int4 else
                "expert_gemm_kernel<MixedWeights<Int4Weights, Int4ResidualWeights>, 2, ...>"
                if resplit else "expert_gemm_kernel<Bf16Weights, 2, ...>")
        roofline = {"bound": "hbm", "kernel": f"{kern} (gate/up, SiLU*up epilogue)",
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": recorded_traffic(args.workload),
                    "measured_read_ceiling": round(ceiling, 1),
                    "frac_of_measured_ceiling": round(achieved / ceiling, 4),
                    "algorithmic_bytes": int(statistics.mean(gu_bytes)),
                    "avg_us": round(gu_us, 2),
                    "stage_us": {n: round(statistics.mean(v), 2) for n, v in dur.items()}}

    wl = layers[0]
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("int8-weights/bf16" if int8 else "int4-weights/bf16" if int4 else
                  "int4+int4-residual/int8-weights/bf16" if resplit else "bf16"),
        "data": "synthetic",
        "config": {"workload": args.workload, "hidden": wl.H, "intermediate": wl.I,
                   "experts": wl.E, "top_k": wl.k, "tokens": [b["wl"].T for b in batches],
                   "layers_per_step": len(batches) * n_sets, "weight_sets": n_sets,
                   "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
                   "TFLOPs": round(sum(layer_flops(b["wl"]) for b in batches) * n_sets /
                                   (ms_per_step * 1e-3) / 1e12, 1),
                   "pct_measured_read_ceiling": round(100 * value / ceiling, 1),
                   "us_m16_over_m1": m16_over_m1, "launch_gap_us": gap,
                   "per_layer": per_layer, "device": torch.cuda.get_device_name(dev)},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        b = batches[0]
        host = host_rowmajor if quant else sets[0]
        result["cpu_baseline"] = cpu_baseline(b["wl"], host, b["lg_cpu"], b["x_cpu"],
                                              critical=crit)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
