"""Seeded synthetic inputs for the attention forward workloads.

This module is the only thing the CPU oracle side and the GPU side share: it
draws inputs and holds none of the method's arithmetic (no scores, softmax,
quantisation or products).  Every input is synthetic and seeded.

Workloads (shapes and distributions as the benchmark configuration names
them; N(mu, v) is read with v the variance):

  1 tiny-exact    B=1  H=2  N=256   d=64   non-causal  fp16 in, fp32 out
  2 llm-prefill   B=4  H=32 N=4096  d=128  causal      bf16
  3 long-context  B=1  H=32 N=32768 d=128  causal      bf16
  4 sage8-outlier B=2  H=32 N=8192  d=128  causal      bf16 -> 8-bit path;
                  Q and K get a per-channel offset shared by all tokens of a
                  (b,h): N(0,4) on 8 seeded channels (the same 8 for Q and K),
                  N(0,0.1) elsewhere, drawn independently for Q and K
  5 dit-gated     B=2  H=24 N=16384 d=64   non-causal  bf16, both paths;
                  additive log-gate bias per (b,h,64-query block,64-key
                  block): for each query block the gates of the other key
                  blocks are the softmax of g ~ N(0,2); the block's own gate
                  is 1, so its bias is log 1 = 0 (page 5, "SAS": log-form
                  gate inside the softmax, normalised softmax gates, the
                  current block always kept)

Draw order for workload s (generator ``torch.Generator('cpu')`` seeded with
s): Q, K, V as fp32 standard normals [B,H,N,d]; then workload 4's channel
permutations and offsets; then workload 5's gates.  Tensors are then rounded
to the workload dtype (round-to-nearest-even).
"""
from __future__ import annotations

import math

import numpy as np
import torch

BIAS_BLOCK = 64

CONFIGS = {
    1: dict(name="tiny-exact", B=1, H=2, N=256, d=64, causal=False, dtype="f16",
            out="f32", paths=("f16",)),
    2: dict(name="llm-prefill", B=4, H=32, N=4096, d=128, causal=True, dtype="bf16",
            out="same", paths=("bf16",)),
    3: dict(name="long-context", B=1, H=32, N=32768, d=128, causal=True, dtype="bf16",
            out="same", paths=("bf16",)),
    4: dict(name="sage8-outlier", B=2, H=32, N=8192, d=128, causal=True, dtype="bf16",
            out="same", paths=("sage8",), outliers=True),
    5: dict(name="dit-gated", B=2, H=24, N=16384, d=64, causal=False, dtype="bf16",
            out="same", paths=("bf16", "sage8"), gate_bias=True),
    # block-sparse variant of the DiT shape: each query block keeps its own
    # key block and the top quarter of the others by gate logit
    6: dict(name="dit-sparse", B=2, H=24, N=16384, d=64, causal=False, dtype="bf16",
            out="same", paths=("bf16", "sage8"), gate_bias=True, gate_keep=0.25),
}

_TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Algorithmic forward FLOPs: 4*B*H*N^2*d, halved when causal."""
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def gate_bias(g: torch.Tensor, keep=None) -> torch.Tensor:
    """Log-gate bias from raw gate logits g [B,H,nb,nb]: off-diagonal entries
    of each row are log(softmax(g over the other key blocks)), the diagonal is
    log(1) = 0.  With keep (a fraction in (0, 1]) only the top
    ceil(keep*(nb-1)) off-diagonal blocks of each row by g keep their gate
    (softmax over the kept ones); the others are gated off, bias -inf
    (block-sparse selection).  Computed in fp64, returned in fp32."""
    g = g.to(torch.float64)
    nb = g.shape[-1]
    eye = torch.eye(nb, dtype=torch.bool)
    masked = g.masked_fill(eye, float("-inf"))
    if keep is not None and nb > 1:
        kcount = max(1, math.ceil(keep * (nb - 1)))
        thresh = torch.topk(masked, kcount, dim=-1).values[..., -1:]
        masked = masked.masked_fill(masked < thresh, float("-inf"))
    if nb > 1:
        out = masked - torch.logsumexp(masked, dim=-1, keepdim=True)
    else:
        out = torch.zeros_like(g)
    out = out.masked_fill(eye, 0.0)
    return out.to(torch.float32)


def make_inputs(B, H, N, d, dtype="bf16", seed=0, outliers=False, gate=False,
                randn_scale=1.0, gate_keep=None):
    """Draw Q, K, V (and optional bias) on the CPU.  Returns a dict with torch
    CPU tensors q, k, v in ``dtype`` and bias (fp32 or None)."""
    gen = torch.Generator("cpu").manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=gen, dtype=torch.float32)
    k = torch.randn(shape, generator=gen, dtype=torch.float32)
    v = torch.randn(shape, generator=gen, dtype=torch.float32)
    if randn_scale != 1.0:
        q.mul_(randn_scale)
        k.mul_(randn_scale)
        v.mul_(randn_scale)
    if outliers:
        n_out = max(1, d // 16)  # 8 of 128 channels
        off_q = torch.randn((B, H, d), generator=gen, dtype=torch.float32) * math.sqrt(0.1)
        off_k = torch.randn((B, H, d), generator=gen, dtype=torch.float32) * math.sqrt(0.1)
        for b in range(B):
            for h in range(H):
                ch = torch.randperm(d, generator=gen)[:n_out]
                off_q[b, h, ch] = torch.randn((n_out,), generator=gen) * 2.0
                off_k[b, h, ch] = torch.randn((n_out,), generator=gen) * 2.0
        q.add_(off_q[:, :, None, :])
        k.add_(off_k[:, :, None, :])
    bias = None
    if gate:
        nb = (N + BIAS_BLOCK - 1) // BIAS_BLOCK
        g = torch.randn((B, H, nb, nb), generator=gen, dtype=torch.float32) * math.sqrt(2.0)
        bias = gate_bias(g, gate_keep)
    tdt = torch_dtype(dtype)
    return dict(q=q.to(tdt), k=k.to(tdt), v=v.to(tdt), bias=bias)


def config_inputs(cfg_id: int):
    """Inputs of workload cfg_id (1..6) with its seed; returns (cfg, inputs)."""
    cfg = CONFIGS[cfg_id]
    inp = make_inputs(cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["dtype"], seed=cfg_id,
                      outliers=cfg.get("outliers", False), gate=cfg.get("gate_bias", False),
                      gate_keep=cfg.get("gate_keep"))
    return cfg, inp


def parity_rows(B, H, N, seed=0, n_random=48, heads=None):
    """Rows (b,h,i) checked at full size: for each b and h in {0, H/2, H-1},
    fixed rows at block edges plus n_random seeded random rows."""
    rng = np.random.default_rng(1000 + int(seed))
    if heads is None:
        heads = sorted({0, H // 2, H - 1})
    fixed = [0, 1, 2, 63, 64, 65, 127, 128, 129, N // 2 - 1, N // 2,
             N - 129, N - 128, N - 65, N - 64, N - 1]
    fixed = sorted({i for i in fixed if 0 <= i < N})
    rows = []
    for b in range(B):
        for h in heads:
            extra = rng.choice(N, size=min(n_random, N), replace=False)
            for i in sorted(set(fixed) | set(int(x) for x in extra)):
                rows.append((b, h, i))
    return np.asarray(rows, dtype=np.int64)


def chunk_gate_inputs(d, seed, dtype="bf16"):
    """B=2, H=2, N=64*150 (150 key blocks) with random gates (keep 0.3) plus
    two gate patterns across runs of 64 key blocks: (0,0) key blocks 60..130
    off for every query block (64 consecutive blocks and their edges), (0,1)
    only key blocks 0, 63, 64, 127, 128, 149 on.  Returns the inputs and the
    rows (b,h,i) to check: block edges, random rows and rows next to those
    runs."""
    N = 64 * 150
    inp = make_inputs(2, 2, N, d, dtype, seed=seed, gate=True, gate_keep=0.3)
    bias = inp["bias"]
    bias[0, 0, :, 60:131] = float("-inf")
    on = torch.zeros(150, dtype=torch.bool)
    on[[0, 63, 64, 127, 128, 149]] = True
    bias[0, 1] = bias[0, 1].masked_fill(~on, float("-inf"))
    bias[0, 1, :, 0] = 0.0
    rows = parity_rows(2, 2, N, seed=seed, n_random=16, heads=[0, 1])
    extra = [(b, h, i) for b in range(2) for h in range(2)
             for i in (63 * 64 + 5, 64 * 64, 127 * 64 + 63, 128 * 64, 131 * 64 + 1, N - 1)]
    return inp, np.unique(np.concatenate([rows, np.asarray(extra, dtype=np.int64)]), axis=0)


def gather_rows(t: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    """Pick rows (b,h,i) of a [B,H,N,d] tensor (any device) as fp64 numpy."""
    idx = torch.as_tensor(rows, dtype=torch.long, device=t.device)
    sel = t[idx[:, 0], idx[:, 1], idx[:, 2]]
    return sel.detach().to("cpu", torch.float64).numpy()


def error_metrics(got: np.ndarray, ref: np.ndarray) -> dict:
    """max/mean abs error, cosine similarity and relative L1 (sum|got-ref| /
    sum|ref|), all in fp64."""
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    diff = np.abs(got - ref)
    denom = np.linalg.norm(got) * np.linalg.norm(ref)
    return dict(
        max_abs=float(diff.max()) if diff.size else 0.0,
        mean_abs=float(diff.mean()) if diff.size else 0.0,
        cos=float(np.dot(got, ref) / denom) if denom > 0 else 1.0,
        rel_l1=float(diff.sum() / max(np.abs(ref).sum(), 1e-300)),
    )


def active_flops(bias: torch.Tensor, N: int, d: int, causal: bool) -> float:
    """FLOPs of the (query block, key block) pairs whose gate is not 0 (bias
    finite): 4*d per visible score, the causal diagonal counted by its
    visible half-plus-diagonal."""
    nb = bias.shape[-1]
    sizes = torch.tensor([min(64, N - 64 * i) for i in range(nb)], dtype=torch.float64)
    pair = sizes[:, None] * sizes[None, :]
    if causal:
        tri = torch.tril(torch.ones(nb, nb, dtype=torch.float64), diagonal=-1)
        diag = torch.diag(sizes * (sizes + 1) / 2)
        pair = pair * tri + diag
    live = torch.isfinite(bias).to(torch.float64)
    return float(4.0 * d * (live * pair).sum())
