"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]

A step is one launch of the bf16 fused forward on the long-context workload
(B=1, H=32, N=32768, d=128, causal, bf16 Q/K/V ~ N(0,1), scale 1/sqrt(128),
bf16 output).  Inputs are resident in device memory before the timed region
and no cache is flushed between steps.  ``value`` is the step's attention
FLOPs (4*B*H*N^2*d/2) divided by the step time: the bf16 forward's TFLOPS,
with ``roofline`` its fraction of the bf16 dense matrix peak.  Each launch is
bracketed by HIP events on the stream the kernels run on (torch's current
stream, which the binding passes to the library).

On the same inputs the 8-bit path is then timed (its preparation and its
forward, 20 launches each after warm-up; INT8 scores with FP8 P and V, the
FP8-QK variant, and INT8 scores with the 16-bit P V) and reported under ``paths``
with its speedup over the bf16 forward, attention alone and with the
preparation.  Other workloads follow under ``workloads`` and ``backward``;
none of them is part of ``value``.  With the CPU baseline (the oracle timed
on the host cores) comes ``accuracy``: every path's output on sampled rows
of the same workload against the oracle's exact attention, with the bars.

Prints ONE JSON line.  Only one GPU is supported: --gpus above 1 exits.

Extra modes (for profiler runs):
    --workload W --path bf16|sage8|sage8pv16|bwd  run one workload's path --steps times
    --copy-bytes NBYTES                 run a plain device copy --steps times
    --trace-summary CSV [--skip S]      per (kernel, grid) durations of a rocprofv3
                                        kernel-trace CSV, the first S dispatches of
                                        each (kernel, grid) left out (warm-up)
"""
from __future__ import annotations

import argparse
import hashlib
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
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, datasheet

# HBM traffic per launch (bytes) of a kernel on a workload, from rocprofv3
# --pmc FETCH_SIZE / WRITE_SIZE runs, scaled by the same counters on a plain
# 1 GiB device copy (FETCH_SIZE reads half the copied bytes: factor 2;
# WRITE_SIZE reads them exactly: factor 1); profiles/fwd16_long-context_hbm-traffic.txt.
# Valid only for the kernel sources it was taken on: the sha256 of the listed
# sources must match, else traffic is reported as null.
TRAFFIC = {
    # 1053830 KiB fetched (x2) + 262144 KiB written, mean of 7 dispatches (sources
    # hashed after host-only edits, a comment and the lock of the occupancy
    # cache: the device code compiles identically)
    ("fwd16", 3): {"sources": ["attn_fwd.hip", "attn_common.hpp"], "bytes": 2426679387,
                   "sha256": "2e0a2c7d923faf0ce6cd731cd0bd7e3b10da202c6e8725f02667ee45cad3e5ab"},
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU reaches its sustained clock after ~50 back-to-back launches of
    # the attention forward (~30 ms); fewer warm-up steps time the ramp
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--workload", type=int, default=0,
                    help="profiling mode: run only this workload (1-5) --steps times and print its timing")
    ap.add_argument("--path", default="bf16", choices=["bf16", "sage8", "sage8pv16", "bwd"],
                    help="profiling mode: which path to run")
    ap.add_argument("--trace-summary", default="",
                    help="print per (kernel, grid) durations of a rocprofv3 kernel-trace CSV and exit")
    ap.add_argument("--skip", type=int, default=0,
                    help="with --trace-summary: leave out the first SKIP dispatches of each (kernel, grid)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="calibration mode: time a plain device copy of this many bytes")
    return ap.parse_args()


def log(msg):
    """Progress on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def sources_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "bit_attention_attn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_for(kernel, workload):
    t = TRAFFIC.get((kernel, workload))
    if t is None or t["bytes"] is None or t["sha256"] != sources_sha(t["sources"]):
        return None
    return t["bytes"]


def _time_launches(fn, iters, stream):
    """Per-launch ms of fn() over iters launches, from event pairs on stream."""
    import torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    for i in range(iters):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    return sorted(s.elapsed_time(e) for s, e in zip(starts, ends))


def _warm(fn, seconds=0.1):
    """Run fn back to back for about `seconds` (at least 3 launches), so the
    timed launches that follow run at the sustained clock."""
    import torch
    t0, n = time.time(), 0
    while n < 3 or time.time() - t0 < seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
        n += 4


def _stats(ms):
    ms = sorted(ms)
    return dict(ms_avg=round(sum(ms) / len(ms), 4), ms_median=round(ms[len(ms) // 2], 4), ms_min=round(ms[0], 4))


def prep_bytes(B, H, N, d, with_v=True):
    """Algorithmic bytes of the 8-bit preparation: Q, K, V (2 bytes) read
    once, Qq, Kq, Vq (1 byte) written once (without V: Q, K read, Qq, Kq
    written); scales and means are < 0.1%."""
    return B * H * N * d * ((3 * 2 + 3 * 1) if with_v else (2 * 2 + 2 * 1))


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
    return dict(value=round(flops / elapsed / 1e12, 6), unit="TFLOPS", cores=oracle.max_threads(), kind="oracle",
                cpu_model=cpu_model(),
                sample=f"{done_rows} random query rows of the {cfg['name']} workload, fp64 three-loop oracle "
                       f"(OpenMP over rows) for {elapsed:.1f} s; flops counted as 4*d per visible key, as on the GPU")


def path_rows(attn, workloads, q, k, v, causal, rows):
    """Every path's output on the given (b,h,i) rows of one call on the
    workload (device outputs gathered to the host as fp64)."""
    out = {"bf16": workloads.gather_rows(attn.fwd(q, k, v, causal=causal), rows)}
    for name, qk in (("int8_qk_fp8_pv", "int8"), ("fp8_qk_fp8_pv", "fp8"), ("int8_qk_16bit_pv", "int8_no_v")):
        prep = attn.sage8_prep(q, k, v, qk=qk)
        o = attn.fwd_sage8_pv16(prep, v, causal=causal) if qk == "int8_no_v" else attn.fwd_sage8(prep, causal=causal)
        out[name] = workloads.gather_rows(o, rows)
        del prep, o
    return out


def accuracy(inp, cfg, rows, got):
    """The paths' outputs on the sampled rows against the fp64 oracle's exact
    attention of the same rounded inputs (the oracle runs here, in the CPU
    baseline leg, untimed)."""
    import numpy as np
    import oracle
    import workloads
    q, k, v = (inp[n].float().numpy() for n in ("q", "k", "v"))
    ref, _ = oracle.attn_rows(q, k, v, rows, causal=cfg["causal"], scale=1 / math.sqrt(cfg["d"]))
    res = {"rows": f"{len(rows)} rows (fixed block-edge rows and seeded random rows of heads 0, H/2, H-1)",
           "bars": {"bf16": "max_abs <= 1e-2 and mean_abs <= 1e-3", "8-bit": "cos >= 0.999 and rel_l1 <= 2e-2"}}
    for name, g in got.items():
        m = workloads.error_metrics(g, ref)
        res[name] = {key: float(f"{val:.4g}") for key, val in m.items()}
        if name == "bf16":
            res[name]["meets_bar"] = bool(m["max_abs"] <= 1e-2 and m["mean_abs"] <= 1e-3)
        else:
            res[name]["meets_bar"] = bool(m["cos"] >= 0.999 and m["rel_l1"] <= 2e-2)
    return res


def profile_one(args):
    """Run one workload's path --steps times (for rocprofv3 runs)."""
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
    elif args.path == "bwd":
        # the backward (five products: 2.5x the forward's flops) from the
        # forward's O and LSE, with a seeded dO
        o, lse = attn.fwd(q, k, v, causal=cfg["causal"], bias=bias, return_lse=True)
        dout = torch.randn(q.shape, generator=torch.Generator(device=dev).manual_seed(args.workload),
                           device=dev, dtype=q.dtype)
        F *= 2.5

        def fn():
            return attn.bwd(q, k, v, o, dout, lse, causal=cfg["causal"], bias=bias, return_dbias=bias is not None)
    elif args.path == "sage8pv16":
        ws = attn.sage8_prep(q, k, v, qk="int8_no_v").workspace

        def fn():
            prep = attn.sage8_prep(q, k, v, workspace=ws, qk="int8_no_v")
            return attn.fwd_sage8_pv16(prep, v, causal=cfg["causal"], bias=bias, out_dtype=out_dtype)
    else:
        ws = attn.sage8_prep(q, k, v).workspace

        def fn():
            prep = attn.sage8_prep(q, k, v, workspace=ws)
            return attn.fwd_sage8(prep, causal=cfg["causal"], bias=bias, out_dtype=out_dtype)
    for _ in range(args.warmup):
        fn()
    ms = _time_launches(fn, args.steps, torch.cuda.current_stream(dev))
    st = _stats(ms)
    print(json.dumps({"workload": cfg["name"], "path": args.path, **st,
                      "tflops": round(F / (st["ms_avg"] * 1e-3) / 1e12, 2)}), flush=True)


def copy_calibration(args):
    """A plain device-to-device copy of --copy-bytes bytes, --steps times:
    the reference for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    dev = torch.device("cuda:0")
    n = args.copy_bytes // 4
    x = torch.ones(n, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    for _ in range(args.warmup):
        y.copy_(x)
    ms = _time_launches(lambda: y.copy_(x), args.steps, torch.cuda.current_stream(dev))
    st = _stats(ms)
    print(json.dumps({"copy_bytes": n * 4, **st,
                      "GBs_read_plus_write": round(2 * n * 4 / (st["ms_avg"] * 1e-3) / 1e9, 1)}), flush=True)


def cpu_model():
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# INT8 scores with the 16-bit P V product: half the FLOPs at the int8 rate,
# half at the bf16 rate, so the time at peak is F/2/5000 + F/2/2500 = F/3333.
PEAK_MIXED_TFLOPS = 1.0 / (0.5 / PEAK_8BIT_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)


def sage8_paths(attn, q, k, v, causal, bias, F, t16_ms, stream):
    """The 8-bit path on the given inputs: preparation and forward timed
    separately (20 launches each after 0.1 s of warm-up) for each recipe, with
    the speedup over the bf16 forward time t16_ms (when given), attention
    alone and with the preparation (page 1, "SageAttention": the conversion
    overhead counts).  Recipes: INT8 scores with FP8 P and V (the pages'
    recipe), FP8 scores with FP8 P and V, INT8 scores with the 16-bit P V."""
    res = {}
    shape = tuple(q.shape)
    for name, qk in (("int8_qk_fp8_pv", "int8"), ("fp8_qk_fp8_pv", "fp8"), ("int8_qk_16bit_pv", "int8_no_v")):
        ws = attn.sage8_prep(q, k, v, qk=qk).workspace
        prep = attn.Sage8Prepared(ws, shape, q.dtype, qk=qk)
        fp = lambda: attn.sage8_prep(q, k, v, workspace=ws, qk=qk)  # noqa: E731
        if name == "int8_qk_16bit_pv":
            f8 = lambda: attn.fwd_sage8_pv16(prep, v, causal=causal, bias=bias)  # noqa: E731
            peak = PEAK_MIXED_TFLOPS
        else:
            f8 = lambda: attn.fwd_sage8(prep, causal=causal, bias=bias)  # noqa: E731
            peak = PEAK_8BIT_TFLOPS
        _warm(fp)
        sp = _stats(_time_launches(fp, 20, stream))
        _warm(f8)
        s8 = _stats(_time_launches(f8, 20, stream))
        tf8 = F / (s8["ms_avg"] * 1e-3) / 1e12
        tfe = F / ((s8["ms_avg"] + sp["ms_avg"]) * 1e-3) / 1e12
        res[name] = {"attention": {**s8, "tflops": round(tf8, 2), "peak": round(peak, 1),
                                   "frac_of_peak": round(tf8 / peak, 4)},
                     "prep": {**sp, "GBs": round(prep_bytes(*shape, with_v=qk != "int8_no_v") / (sp["ms_avg"] * 1e-3)
                                                 / 1e9, 1)},
                     "tflops_prep_plus_attention": round(tfe, 2)}
        if t16_ms is not None:
            res[name]["speedup_vs_bf16_attention"] = round(t16_ms / s8["ms_avg"], 3)
            res[name]["speedup_vs_bf16_end_to_end"] = round(t16_ms / (s8["ms_avg"] + sp["ms_avg"]), 3)
        del ws, prep
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(attention heads shard across GPUs with no communication).", file=sys.stderr)
        sys.exit(2)
    if args.trace_summary:
        return trace_summary(args.trace_summary, args.skip)
    import torch
    import __graft_entry__
    __graft_entry__._ensure_built()
    if args.copy_bytes:
        return copy_calibration(args)
    if args.workload:
        return profile_one(args)
    import bit_attention_attn_amd as attn
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    cfg, inp = workloads.config_inputs(3)
    log(f"inputs ready: {cfg['name']}")
    B, H, N, d, causal = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"]
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    F = workloads.flops(B, H, N, d, causal)
    torch.cuda.synchronize()

    def step():
        attn.fwd(q, k, v, causal=causal)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(K):
        ev[s][0].record(stream)
        step()
        ev[s][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / K
    log(f"timed {K} steps: {ms_per_step:.4f} ms per step")
    k16 = _stats([e[0].elapsed_time(e[1]) for e in ev])
    value = F / (ms_per_step * 1e-3) / 1e12
    tf16 = F / (k16["ms_avg"] * 1e-3) / 1e12
    roof = dict(bound="mfma", achieved=round(tf16, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                frac=round(tf16 / PEAK_BF16_TFLOPS, 4), traffic=traffic_for("fwd16", 3),
                kernel="fwd16_kernel<128, bf16, causal, 1, 8, dense> (bf16 fused forward)",
                ms_avg=k16["ms_avg"], units_per_launch=f"{F:.4e} flop (4*B*H*N^2*d/2)")

    log("8-bit path on the same inputs")
    paths = {"bf16": {**k16, "tflops": round(tf16, 2), "frac_of_peak": round(tf16 / PEAK_BF16_TFLOPS, 4)}}
    paths.update(sage8_paths(attn, q, k, v, causal, None, F, k16["ms_avg"], stream))

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
        "data": "synthetic (seeded N(0,1) Q/K/V, no dataset)",
        "config": {"workload": f"{cfg['name']}: B={B} H={H} N={N} d={d} causal, bf16 in/out; "
                               "step = one bf16 fused forward",
                   "batch": B, "heads": H, "seq_len": N, "head_dim": d, "causal": causal,
                   "cache_flush": False},
        "roofline": roof,
        "paths": paths,
    }
    if not args.no_extra:
        out["workloads"] = extra_workloads(attn, workloads, stream, dev)
        out["backward"] = backward_workloads(attn, workloads, stream, dev)

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on host cores)")
        out["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_seconds)
        log("accuracy of every path on sampled rows against the oracle")
        rows = workloads.parity_rows(B, H, N, seed=3)
        out["accuracy"] = accuracy(inp, cfg, rows, path_rows(attn, workloads, q, k, v, causal, rows))
    print(json.dumps(out), flush=True)


def trace_summary(path, skip):
    """Per (kernel, grid) dispatch durations of a rocprofv3 kernel-trace CSV,
    leaving out the first `skip` dispatches of each (kernel, grid)."""
    import csv
    groups = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            key = (name, r.get("Grid_Size_X", r.get("Grid_Size", "")), r.get("Workgroup_Size_X",
                                                                                r.get("Workgroup_Size", "")))
            groups.setdefault(key, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows = []
    for (name, grid, wg), ts in groups.items():
        ts.sort()
        durs = [(e - s) / 1e6 for s, e in ts]
        kept = durs[skip:] if len(durs) > skip else durs
        rows.append((sum(durs), name, grid, wg, len(durs), sum(durs) / len(durs), len(kept), sum(kept) / len(kept)))
    rows.sort(reverse=True)
    print(f"{'n':>6} {'avg ms':>9} {'kept':>5} {'kept avg':>9}  kernel [grid x; workgroup]")
    for _, name, grid, wg, n, avg, nk, avgk in rows:
        short = name if len(name) < 110 else name[:107] + "..."
        print(f"{n:>6} {avg:9.4f} {nk:>5} {avgk:9.4f}  {short} [{grid}; {wg}]")


def extra_workloads(attn, workloads, stream, dev):
    """The llm-prefill, 8-bit-outlier, DiT-gated and block-sparse DiT
    workloads at full size: 20 timed launches per path after 0.1 s of
    warm-up launches."""
    import torch
    extra = {}
    for cid in (2, 4, 5, 6):
        c2, i2 = workloads.config_inputs(cid)
        log(f"workload {c2['name']}")
        q2, k2, v2 = (i2[n].to(dev) for n in ("q", "k", "v"))
        b2 = i2["bias"].to(dev) if i2["bias"] is not None else None
        # block-sparse gates: count the FLOPs of the (query block, key block)
        # pairs that are not gated off (the ones the kernels compute)
        sparse = c2.get("gate_keep") is not None
        F2 = (workloads.active_flops(i2["bias"], c2["N"], c2["d"], c2["causal"]) if sparse
              else workloads.flops(c2["B"], c2["H"], c2["N"], c2["d"], c2["causal"]))
        del i2
        res = {}
        t16 = None
        if cid != 4:
            fn = lambda: attn.fwd(q2, k2, v2, causal=c2["causal"], bias=b2)  # noqa: E731
            _warm(fn)
            st = _stats(_time_launches(fn, 20, stream))
            tf = F2 / (st["ms_avg"] * 1e-3) / 1e12
            res["bf16"] = {**st, "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
            t16 = st["ms_avg"]
        res.update(sage8_paths(attn, q2, k2, v2, c2["causal"], b2, F2, t16, stream))
        if cid == 2:
            # the whole hot path once: bf16 forward, then 8-bit preparation and forward
            r8 = res["int8_qk_fp8_pv"]
            res["hot_path_step_ms"] = round(t16 + r8["prep"]["ms_avg"] + r8["attention"]["ms_avg"], 4)
        if sparse:
            res["flops_counted"] = f"{F2:.4e} (gated-on block pairs only, {c2['gate_keep']} of the off-diagonal kept)"
        extra[f"{c2['name']}: B={c2['B']} H={c2['H']} N={c2['N']} d={c2['d']} "
              f"{'causal' if c2['causal'] else 'non-causal'}{' +gate bias' if b2 is not None else ''}"
              f"{' (block-sparse)' if sparse else ''}"] = res
        del q2, k2, v2, b2
        torch.cuda.empty_cache()
    return extra


def backward_workloads(attn, workloads, stream, dev):
    """The backward (D, dQ, dK, dV, and the bias gradient where a bias is
    given) on llm-prefill, long-context and DiT-gated: whole-call times of 10
    launches after 0.1 s of warm-up.  FLOPs: the five products of the
    algorithm (S, dP, dV, dQ, dK), 2.5 times the forward's; the kernels
    compute S and dP twice (once per side), seven products in all."""
    import torch
    res = {}
    for cid in (2, 3, 5):
        c2 = workloads.CONFIGS[cid]
        B, H, N, d = c2["B"], c2["H"], c2["N"], c2["d"]
        log(f"backward {c2['name']}")
        g = torch.Generator(device=dev).manual_seed(cid)
        q, k, v, dout = (torch.randn((B, H, N, d), device=dev, dtype=torch.bfloat16, generator=g) for _ in range(4))
        nb = (N + 63) // 64
        b = torch.zeros((B, H, nb, nb), device=dev) if c2.get("gate_bias") else None
        o, lse = attn.fwd(q, k, v, causal=c2["causal"], bias=b, return_lse=True)
        fn = lambda: attn.bwd(q, k, v, o, dout, lse, causal=c2["causal"], bias=b,  # noqa: E731
                              return_dbias=b is not None)
        _warm(fn)
        st = _stats(_time_launches(fn, 10, stream))
        F = 2.5 * workloads.flops(B, H, N, d, c2["causal"])
        tf = F / (st["ms_avg"] * 1e-3) / 1e12
        res[f"{c2['name']}: B={B} H={H} N={N} d={d} {'causal' if c2['causal'] else 'non-causal'}"
            f"{' +bias grad' if b is not None else ''}"] = {
            **st, "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "flops_counted": f"{F:.4e} (5 products, 2.5 x forward)"}
        del q, k, v, dout, o, lse, b
        torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
