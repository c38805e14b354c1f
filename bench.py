"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one pass of the whole hot path over the LLM-prefill workload
(B=4, H=32, N=4096, d=128, causal, bf16 inputs): the bf16 fused forward, then
the 8-bit preparation and the 8-bit fused forward on the same inputs.  Inputs
are resident in device memory before the timed region.  ``value`` is the
attention FLOPs the step computes (4*B*H*N^2*d/2 per forward, two forwards)
divided by the step time.  Per-kernel times come from HIP events recorded on
the stream the kernels run on.  Other workloads are timed after the main
loop and reported under ``workloads`` (they are not part of ``value``).

Prints ONE JSON line.  Only one GPU is supported: --gpus above 1 exits.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOPS and % of MFMA peak at 1 MI355X (bf16 and int8/fp8)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA, datasheet
PEAK_8BIT_TFLOPS = 5000.0   # MI355X dense fp8 / int8 MFMA, datasheet
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--workload", type=int, default=0,
                    help="profiling mode: run only this workload (1-5) --steps times and print its timing")
    ap.add_argument("--path", default="bf16", choices=["bf16", "sage8"],
                    help="profiling mode: which path to run")
    return ap.parse_args()


def _time_launches(fn, iters, stream):
    """Average ms of fn() over iters launches, timed by event pairs on stream."""
    import torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    for i in range(iters):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms.sort()
    return sum(ms) / len(ms), ms[len(ms) // 2], ms[0]


def cpu_baseline(inp, cfg, seconds):
    """The fp64 oracle on the host cores, on a bounded row sample of the same
    workload; returns TFLOPS counted like the GPU metric (4*d flops per
    visible score)."""
    import numpy as np
    import oracle
    q, k, v = (inp[n].float().numpy() for n in ("q", "k", "v"))
    B, H, N, d = q.shape
    rng = np.random.default_rng(12345)
    done_rows, flops, elapsed = 0, 0.0, 0.0
    batch = 64
    while elapsed < seconds and done_rows < 10_000_000:
        rows = np.stack([rng.integers(0, B, batch), rng.integers(0, H, batch),
                         rng.integers(0, N, batch)], axis=1)
        vis = rows[:, 2] + 1 if cfg["causal"] else np.full(batch, N)
        t0 = time.perf_counter()
        oracle.attn_rows(q, k, v, rows, causal=cfg["causal"], scale=1 / math.sqrt(d))
        elapsed += time.perf_counter() - t0
        flops += float((4.0 * d * vis).sum())
        done_rows += batch
        batch = min(batch * 2, 4096)
    return dict(value=flops / elapsed / 1e12, unit="TFLOPS", cores=oracle.max_threads(), kind="oracle",
                sample=f"{done_rows} random query rows of the {cfg['name']} workload "
                       f"(fp64 three-loop oracle, {elapsed:.1f} s; flops counted as 4*d per visible key)")


def profile_one(args):
    """Run one workload's kernel --steps times (for rocprofv3 runs)."""
    import torch
    import bit_attention_attn_amd as attn
    import workloads
    dev = torch.device("cuda:0")
    cfg, inp = workloads.config_inputs(args.workload)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    bias = inp["bias"].to(dev) if inp["bias"] is not None else None
    F = workloads.flops(cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"])
    out_dtype = torch.float32 if cfg["out"] == "f32" else None
    if args.path == "bf16":
        fn = lambda: attn.fwd(q, k, v, causal=cfg["causal"], bias=bias, out_dtype=out_dtype)  # noqa: E731
    else:
        def fn():
            prep = attn.sage8_prep(q, k, v)
            return attn.fwd_sage8(prep, causal=cfg["causal"], bias=bias, out_dtype=out_dtype)
    for _ in range(args.warmup):
        fn()
    avg, med, mn = _time_launches(fn, args.steps, torch.cuda.current_stream(dev))
    print(json.dumps({"workload": cfg["name"], "path": args.path, "ms_avg": round(avg, 4),
                      "ms_min": round(mn, 4), "tflops": round(F / (avg * 1e-3) / 1e12, 2)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(attention heads shard across GPUs with no communication; see the design notes).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import __graft_entry__
    __graft_entry__._ensure_built()
    if args.workload:
        return profile_one(args)
    import bit_attention_attn_amd as attn
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    cfg, inp = workloads.config_inputs(2)
    B, H, N, d, causal = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"]
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    F = workloads.flops(B, H, N, d, causal)
    torch.cuda.synchronize()

    def bf16_fwd():
        return attn.fwd(q, k, v, causal=causal)

    for _ in range(args.warmup):
        bf16_fwd()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(K):
        ev[s][0].record(stream)
        bf16_fwd()
        ev[s][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    bf16_ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    bf16_avg = sum(bf16_ms) / K
    ms_per_step = total_ms / K
    flops_per_step = F
    value = flops_per_step / (ms_per_step * 1e-3) / 1e12
    bf16_tflops = F / (bf16_avg * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg['name']}: B={B} H={H} N={N} d={d} causal bf16 in/out",
                   "batch": B, "heads": H, "seq_len": N, "head_dim": d, "causal": causal},
        "roofline": {"bound": "mfma", "achieved": round(bf16_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(bf16_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "fwd16_kernel<128,bf16,causal>",
                     "ms_avg": round(bf16_avg, 4), "ms_median": round(bf16_ms[K // 2], 4)},
        "paths": {"bf16": {"ms": round(bf16_avg, 4), "tflops": round(bf16_tflops, 2),
                           "frac_of_peak": round(bf16_tflops / PEAK_BF16_TFLOPS, 4)}},
    }

    if not args.no_extra:
        extra = {}
        for cid in (3, 5):
            c2, i2 = workloads.config_inputs(cid)
            q2, k2, v2 = (i2[n].to(dev) for n in ("q", "k", "v"))
            b2 = i2["bias"].to(dev) if i2["bias"] is not None else None
            F2 = workloads.flops(c2["B"], c2["H"], c2["N"], c2["d"], c2["causal"])
            fn = lambda: attn.fwd(q2, k2, v2, causal=c2["causal"], bias=b2)  # noqa: E731
            for _ in range(2):
                fn()
            avg, med, mn = _time_launches(fn, 10, stream)
            extra[f"{c2['name']} bf16"] = {"ms_avg": round(avg, 4), "ms_min": round(mn, 4),
                                           "tflops": round(F2 / (avg * 1e-3) / 1e12, 2),
                                           "frac_of_peak": round(F2 / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
            del q2, k2, v2, b2
            torch.cuda.empty_cache()
        out["workloads"] = extra

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
