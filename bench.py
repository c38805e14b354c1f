"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]

A step is one pass of the whole hot path over the LLM-prefill workload
(B=4, H=32, N=4096, d=128, causal, bf16 Q/K/V ~ N(0,1), scale 1/sqrt(128),
bf16 output): the bf16 fused forward, then the 8-bit preparation (K mean,
INT8 Q/K, e4m3 V into a preallocated workspace) and the 8-bit fused forward
on the same inputs.  Inputs are resident in device memory before the timed
region and no cache is flushed between steps.  ``value`` is the attention
FLOPs the step computes (two forwards, 4*B*H*N^2*d/2 each) divided by the
step time.  Each kernel launch is bracketed by HIP events on the stream the
kernels run on (torch's current stream, which the binding passes to the
library), giving per-kernel averages; ``roofline`` describes the kernel with
the largest share of the step.  Other workloads are timed after the main loop
and reported under ``workloads`` (not part of ``value``).

Prints ONE JSON line.  Only one GPU is supported: --gpus above 1 exits.

Extra modes (for profiler runs):
    --workload W --path bf16|sage8   run one workload's path --steps times
    --copy-bytes NBYTES              run a plain device copy --steps times
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

# HBM traffic per launch (bytes) from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
# runs on the LLM-prefill workload, scaled by the same counters on a plain
# 1 GiB device copy (FETCH_SIZE reads half the copied bytes: factor 2;
# WRITE_SIZE reads them exactly: factor 1); profiles/llm-prefill_hbm-traffic.txt.
# Valid only for the kernel sources it was taken on: the sha256 of the listed
# sources must match, else traffic is reported as null.
TRAFFIC = {
    "fwd16": {"sources": ["attn_fwd.hip", "attn_common.hpp"], "bytes": 710497717,
              "sha256": "e042dba7eed10de822d1cbfbddea59740ff952b6cdb5023d713116396fce9014"},
    "fwd8": {"sources": ["attn_sage8.hip", "attn_common.hpp"], "bytes": 580376390,
             "sha256": "671fc2311657d9cac2fce501171ac72388ff21e21af1fe4767749100fe510e67"},
    "prep8": {"sources": ["attn_sage8.hip", "attn_common.hpp"], "bytes": 880751721,
              "sha256": "671fc2311657d9cac2fce501171ac72388ff21e21af1fe4767749100fe510e67"},
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
    ap.add_argument("--path", default="bf16", choices=["bf16", "sage8", "bwd"],
                    help="profiling mode: which path to run")
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


def traffic_for(key):
    t = TRAFFIC[key]
    if t["bytes"] is None or t["sha256"] != sources_sha(t["sources"]):
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


def prep_bytes(B, H, N, d):
    """Algorithmic bytes of the 8-bit preparation: Q, K, V (2 bytes) read
    once, Qq, Kq, Vq (1 byte) written once; scales and means are < 0.1%."""
    return B * H * N * d * (3 * 2 + 3 * 1)


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
                sample=f"{done_rows} random query rows of the {cfg['name']} workload, fp64 three-loop oracle "
                       f"(OpenMP over rows) for {elapsed:.1f} s; flops counted as 4*d per visible key, as on the GPU")


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


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(attention heads shard across GPUs with no communication).", file=sys.stderr)
        sys.exit(2)
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

    cfg, inp = workloads.config_inputs(2)
    log(f"inputs ready: {cfg['name']}")
    B, H, N, d, causal = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"]
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    F = workloads.flops(B, H, N, d, causal)
    ws = attn.sage8_prep(q, k, v).workspace
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        attn.fwd(q, k, v, causal=causal)
        if ev is not None:
            ev[1].record(stream)
        prep = attn.sage8_prep(q, k, v, workspace=ws)
        if ev is not None:
            ev[2].record(stream)
        attn.fwd_sage8(prep, causal=causal)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(K):
        step(ev[s])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / K
    log(f"timed {K} steps: {ms_per_step:.4f} ms per step")
    k16 = _stats([e[0].elapsed_time(e[1]) for e in ev])
    kprep = _stats([e[1].elapsed_time(e[2]) for e in ev])
    k8 = _stats([e[2].elapsed_time(e[3]) for e in ev])
    value = 2 * F / (ms_per_step * 1e-3) / 1e12

    tf16 = F / (k16["ms_avg"] * 1e-3) / 1e12
    tf8 = F / (k8["ms_avg"] * 1e-3) / 1e12
    tf8_e2e = F / ((k8["ms_avg"] + kprep["ms_avg"]) * 1e-3) / 1e12
    pbytes = prep_bytes(B, H, N, d)
    prep_gbs = pbytes / (kprep["ms_avg"] * 1e-3) / 1e9
    kernels = {
        "fwd16": dict(bound="mfma", achieved=round(tf16, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                      frac=round(tf16 / PEAK_BF16_TFLOPS, 4), traffic=traffic_for("fwd16"),
                      kernel="fwd16_kernel<128, bf16, causal> (bf16 fused forward)", ms=k16["ms_avg"],
                      units_per_launch=f"{F:.4e} flop (4*B*H*N^2*d/2)"),
        "fwd8": dict(bound="mfma", achieved=round(tf8, 2), peak=PEAK_8BIT_TFLOPS, unit="TFLOP/s",
                     frac=round(tf8 / PEAK_8BIT_TFLOPS, 4), traffic=traffic_for("fwd8"),
                     kernel="fwd8_kernel<128, causal> (INT8 QK^T, FP8 PV fused forward)", ms=k8["ms_avg"],
                     units_per_launch=f"{F:.4e} flop (4*B*H*N^2*d/2)"),
        "prep8": dict(bound="hbm", achieved=round(prep_gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                      frac=round(prep_gbs / PEAK_HBM_GBS, 4), traffic=traffic_for("prep8"),
                      kernel="sage8 colstats + finalize + quant (three launches)", ms=kprep["ms_avg"],
                      units_per_launch=f"{pbytes} bytes (9 per element of Q/K/V)"),
    }
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    roof = {kk: kernels[dom][kk] for kk in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel")}
    roof["ms_avg"] = kernels[dom]["ms"]

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
        "dtype": "bf16 + int8/fp8(e4m3)",
        "data": "synthetic (seeded N(0,1) Q/K/V, no dataset)",
        "config": {"workload": f"{cfg['name']}: B={B} H={H} N={N} d={d} causal, bf16 in/out; "
                               "step = bf16 forward + 8-bit prep + 8-bit forward",
                   "batch": B, "heads": H, "seq_len": N, "head_dim": d, "causal": causal,
                   "cache_flush": False},
        "roofline": roof,
        "kernels": {n: {kk: vv for kk, vv in kv.items()} for n, kv in kernels.items()},
        "per_kernel_ms": {"fwd16": k16, "prep8": kprep, "fwd8": k8},
        "paths": {
            "bf16": {"tflops": round(tf16, 2), "frac_of_peak": round(tf16 / PEAK_BF16_TFLOPS, 4)},
            "sage8": {"tflops_attention": round(tf8, 2), "frac_of_8bit_peak": round(tf8 / PEAK_8BIT_TFLOPS, 4),
                      "tflops_prep_plus_attention": round(tf8_e2e, 2),
                      "speedup_vs_bf16_attention": round(tf8 / tf16, 3),
                      "speedup_vs_bf16_end_to_end": round(tf8_e2e / tf16, 3)},
        },
    }

    if not args.no_extra:
        out["workloads"] = extra_workloads(attn, workloads, stream, dev)
        out["backward"] = backward_workloads(attn, workloads, stream, dev)

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on host cores)")
        out["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def extra_workloads(attn, workloads, stream, dev):
    """The long-context, 8-bit-outlier, DiT-gated and block-sparse DiT
    workloads at full size: 20 timed launches per path after 0.1 s of
    warm-up launches."""
    import torch
    extra = {}
    for cid in (3, 4, 5, 6):
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
        if cid != 4:
            fn = lambda: attn.fwd(q2, k2, v2, causal=c2["causal"], bias=b2)  # noqa: E731
            _warm(fn)
            st = _stats(_time_launches(fn, 20, stream))
            tf = F2 / (st["ms_avg"] * 1e-3) / 1e12
            res["bf16"] = {**st, "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        ws = attn.sage8_prep(q2, k2, v2).workspace
        prep = attn.Sage8Prepared(ws, tuple(q2.shape), q2.dtype)
        fp = lambda: attn.sage8_prep(q2, k2, v2, workspace=ws)  # noqa: E731
        f8 = lambda: attn.fwd_sage8(prep, causal=c2["causal"], bias=b2)  # noqa: E731
        _warm(fp)
        sp = _stats(_time_launches(fp, 20, stream))
        _warm(f8)
        s8 = _stats(_time_launches(f8, 20, stream))
        tf8 = F2 / (s8["ms_avg"] * 1e-3) / 1e12
        tfe = F2 / ((s8["ms_avg"] + sp["ms_avg"]) * 1e-3) / 1e12
        res["sage8"] = {"attention": {**s8, "tflops": round(tf8, 2), "frac_of_8bit_peak": round(tf8 / PEAK_8BIT_TFLOPS, 4)},
                        "prep": {**sp, "GBs": round(prep_bytes(*q2.shape) / (sp["ms_avg"] * 1e-3) / 1e9, 1)},
                        "tflops_prep_plus_attention": round(tfe, 2)}
        if "bf16" in res:
            res["sage8"]["speedup_vs_bf16_attention"] = round(tf8 / res["bf16"]["tflops"], 3)
            res["sage8"]["speedup_vs_bf16_end_to_end"] = round(tfe / res["bf16"]["tflops"], 3)
        # the FP8-QK variant (Q and centred K in e4m3 blocks) on the same data
        wsf = attn.sage8_prep(q2, k2, v2, qk="fp8").workspace
        prepf = attn.Sage8Prepared(wsf, tuple(q2.shape), q2.dtype, qk="fp8")
        fpf = lambda: attn.sage8_prep(q2, k2, v2, workspace=wsf, qk="fp8")  # noqa: E731
        f8f = lambda: attn.fwd_sage8(prepf, causal=c2["causal"], bias=b2)  # noqa: E731
        _warm(fpf)
        spf = _stats(_time_launches(fpf, 20, stream))
        _warm(f8f)
        s8f = _stats(_time_launches(f8f, 20, stream))
        tff = F2 / (s8f["ms_avg"] * 1e-3) / 1e12
        tffe = F2 / ((s8f["ms_avg"] + spf["ms_avg"]) * 1e-3) / 1e12
        res["sage8_fp8qk"] = {"attention": {**s8f, "tflops": round(tff, 2),
                                            "frac_of_8bit_peak": round(tff / PEAK_8BIT_TFLOPS, 4)},
                              "prep": {**spf, "GBs": round(prep_bytes(*q2.shape) / (spf["ms_avg"] * 1e-3) / 1e9, 1)},
                              "tflops_prep_plus_attention": round(tffe, 2),
                              "speedup_vs_int8_qk_attention": round(tff / tf8, 3)}
        del wsf, prepf
        if sparse:
            res["flops_counted"] = f"{F2:.4e} (gated-on block pairs only, {c2['gate_keep']} of the off-diagonal kept)"
        extra[f"{c2['name']}: B={c2['B']} H={c2['H']} N={c2['N']} d={c2['d']} "
              f"{'causal' if c2['causal'] else 'non-causal'}{' +gate bias' if b2 is not None else ''}"
              f"{' (block-sparse)' if sparse else ''}"] = res
        del q2, k2, v2, b2, ws, prep
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
