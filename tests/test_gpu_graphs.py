"""GPU tests of the entry points under HIP graph capture.

The library allocates nothing and issues no memset (the bias gradient is
cleared by a kernel), so every path can be recorded into a graph by a
caller that replays it, e.g. a serving loop.  Each test records one call
with torch.cuda.graph, then replays it several times with eager calls of
the same path and synchronisations between the replays; before each replay
the recorded outputs are overwritten, and after it every output must equal
the eager result bit for bit.
"""
import itertools

import pytest
import torch

import bit_attention_attn_amd as attn
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 3


def _as_tuple(x):
    return tuple(t for t in (x if isinstance(x, tuple) else (x,)) if t is not None)


def _check_graph(fn, label):
    print(f"[gpu] graph {label}", flush=True)
    eager = _as_tuple(fn())
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # first use on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = _as_tuple(fn())
    for i in range(REPLAYS):
        for t in out:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(out, eager)):
            assert torch.equal(a, b), (label, i, k)
        again = _as_tuple(fn())  # eager work between the replays
        torch.cuda.synchronize()
        for a, b in zip(again, eager):
            assert torch.equal(a, b), (label, i, "eager")


def _inputs(B, H, N, d, seed, gate=False):
    inp = workloads.make_inputs(B, H, N, d, "bf16", seed=seed, gate=gate)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    bias = inp["bias"].to(DEV) if inp["bias"] is not None else None
    return q, k, v, bias


def test_graph_fwd16_with_bias():
    q, k, v, bias = _inputs(2, 3, 700, 128, seed=1, gate=True)
    _check_graph(lambda: attn.fwd(q, k, v, causal=True, bias=bias, return_lse=True), "fwd16 causal+bias")


@pytest.mark.parametrize("qk", ["int8", "fp8"])
def test_graph_sage8(qk):
    q, k, v, bias = _inputs(1, 4, 1000, 64, seed=2, gate=True)
    _check_graph(lambda: attn.sageattn(q, k, v, causal=False, bias=bias, return_lse=True, qk=qk), f"sage8 {qk}")


def test_graph_backward_with_bias_gradient():
    q, k, v, bias = _inputs(1, 2, 500, 64, seed=3, gate=True)
    o, lse = attn.fwd(q, k, v, causal=True, bias=bias, return_lse=True)
    dout = torch.randn(q.shape, generator=torch.Generator(device=DEV).manual_seed(4), device=DEV, dtype=q.dtype)
    _check_graph(lambda: attn.bwd(q, k, v, o, dout, lse, causal=True, bias=bias, return_dbias=True),
                 "backward + dbias")


def test_graph_packed_sequences():
    lens = [300, 1, 129, 64]
    H, d = 2, 128
    g = torch.Generator(device=DEV).manual_seed(5)
    total = sum(lens)
    q, k, v = (torch.randn((total, H, d), device=DEV, dtype=torch.bfloat16, generator=g) for _ in range(3))
    cu = torch.tensor([0] + list(itertools.accumulate(lens)), dtype=torch.int32, device=DEV)
    N = max(lens)
    # (no LSE here: its rows past a sequence's length are never written)
    _check_graph(lambda: attn.fwd_varlen(q, k, v, cu, N, causal=True), "fwd16 packed")
    _check_graph(lambda: attn.sageattn_varlen(q, k, v, cu, N, causal=True), "sage8 packed")
    nb = (N + 63) // 64
    bias = workloads.gate_bias(torch.randn((len(lens), H, nb, nb), generator=torch.Generator("cpu").manual_seed(6)),
                               keep=0.5).to(DEV)
    _check_graph(lambda: attn.fwd_varlen(q, k, v, cu, N, causal=True, bias=bias), "fwd16 packed + bias")
    _check_graph(lambda: attn.sageattn_varlen(q, k, v, cu, N, causal=True, bias=bias), "sage8 packed + bias")
