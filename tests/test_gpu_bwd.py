"""GPU parity of the backward (dQ, dK, dV and the block-bias gradient)
against the fp64 oracle backward, which recomputes everything from the same
rounded inputs.

Bar (max |err| / max |ref|, ||err|| / ||ref||).  The kernels round P and dS
to the input dtype for the products that use them and round the gradients to
the output dtype.  A CPU model of exactly those roundings against the fp64
gradients gives, for bf16 inputs on these shapes, at most 5.9e-3 and 2.7e-3
with bf16 gradients and 3.8e-3 and 2.1e-3 with fp32 gradients.  The GPU adds
what the model leaves out: P = exp(s - LSE) takes the forward's LSE, which
deviates by up to ln(1 + 2^-8) = 3.9e-3 on rows with few keys (the forward's
row sum adds P rounded to bf16), so single elements of dQ on such rows carry
up to that much more: 3.9e-3 + 2^-9 (dS) + 2^-9 (output) = 7.8e-3.  The bars
are max 1e-2 and norm 5e-3 (bf16 gradients) or 4e-3 (fp32).  fp16 keeps 3
more bits throughout.

The block-bias gradient sums dS in fp32 over 64 x 64 blocks.  Its rows need
D = rowsum(dO * O) to equal sum_j P_ij dP_ij, which holds only up to
dD_i = dO_i . (O_used - O_exact) for the O the backward is given (the
forward's rounded output); each row of dS then sums to about -dD_i instead of
0.  The bar for an entry of block row qb is 2e-3 of the largest entry plus
sum over the rows i of qb of |dD_i|, computed from the two O's, plus the
rounding of the two fp32 sums D and dP themselves (4 sqrt(d) 2^-24 times the
root-sum-square of their products): with one visible key dS is exactly 0 and
only that rounding is left.
"""
import math

import numpy as np
import pytest
import torch

import bit_attention_attn_amd as attn
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BAR = {(torch.bfloat16, torch.bfloat16): (1e-2, 5e-3), (torch.bfloat16, torch.float32): (1e-2, 4e-3),
       (torch.float16, torch.float16): (3e-3, 1.5e-3), (torch.float16, torch.float32): (2e-3, 1e-3)}
DBIAS_BAR = 2e-3


def _dout(shape, dtype, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype)


def _compare(label, got, ref, bar, floor=0.0):
    got = got.double().cpu().numpy()
    m = float(np.abs(ref).max())
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), label
    assert err.max() <= bar[0] * m + floor + 1e-6, (label, float(err.max()), m, floor)
    if m > 0:  # an all-zero reference (e.g. dq at scale 0) is held by the line above
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        assert rel <= bar[1], (label, rel)


def _run(inp, causal, scale, label, grad_dtype=None, with_dbias=True, seed=0, o_f32=False):
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    bias = inp["bias"].to(DEV) if inp["bias"] is not None else None
    dout_cpu = _dout(q.shape, q.dtype, seed)
    print(f"[gpu] bwd {label} shape={tuple(q.shape)} {q.dtype} causal={causal} bias={bias is not None} "
          f"o_f32={o_f32}", flush=True)
    o, lse = attn.fwd(q, k, v, causal=causal, scale=scale, bias=bias, return_lse=True,
                      out_dtype=torch.float32 if o_f32 else None)
    g = attn.bwd(q, k, v, o, dout_cpu.to(DEV), lse, causal=causal, scale=scale, bias=bias,
                 grad_dtype=grad_dtype, return_dbias=with_dbias)
    torch.cuda.synchronize()
    qn, kn, vn = (inp[n].float().numpy() for n in ("q", "k", "v"))
    dn = dout_cpu.float().numpy()
    bn = inp["bias"].numpy() if inp["bias"] is not None else None
    ref = oracle.attn_bwd(qn, kn, vn, dn, causal=causal, scale=scale, bias=bn)
    bar = BAR[(q.dtype, grad_dtype or q.dtype)]
    # D and dP are fp32 sums of d products, taken in different orders, so
    # dS = P (dP - D) carries per row up to `noise` (4 sqrt(d) 2^-24 times the
    # root-sum-square of the products of each sum: the usual size of a rounded
    # sum, with a 4-sigma margin).  Where the exact dS is 0 (one visible key)
    # that is all of dQ = scale dS K and dK = scale dS^T Q: the floors below
    # carry it through (P <= 1; over the rows of dK the errors have random
    # signs and add as a root-sum-square).
    d = q.shape[-1]
    vmax = np.abs(vn).max(axis=2, keepdims=True)  # [B,H,1,d]
    od = o.double().cpu().numpy()
    prods = np.sqrt(np.sum((dn * od) ** 2, axis=-1) + np.sum((dn * vmax) ** 2, axis=-1))  # [B,H,N]
    noise = 4.0 * math.sqrt(d) * 2.0 ** -24 * prods
    sc = abs(scale if scale is not None else 1.0 / math.sqrt(d))
    floors = {"dq": sc * float(noise.max()) * float(np.abs(kn).max()),
              "dk": sc * float(np.sqrt((noise ** 2).sum(axis=-1)).max()) * float(np.abs(qn).max()), "dv": 0.0}
    for name, i in (("dq", 0), ("dk", 1), ("dv", 2)):
        _compare(f"{label} {name}", g[i], ref[i], bar, floors[name])
    if with_dbias:
        db_ref = ref[3] if ref[3] is not None else oracle.attn_bwd(
            qn, kn, vn, dn, causal=causal, scale=scale, bias=np.zeros(g[3].shape, dtype=np.float32))[3]
        o_ex, _ = oracle.attn_full(qn, kn, vn, causal=causal, scale=scale, bias=bn)
        dD = np.abs(np.sum(dn.astype(np.float64) * (od - o_ex), axis=-1)) + noise  # [B,H,N]
        B, H, N, _ = q.shape
        nb = (N + 63) // 64
        row_bound = np.zeros((B, H, nb))
        for qb in range(nb):
            row_bound[:, :, qb] = dD[:, :, 64 * qb:64 * qb + 64].sum(axis=-1)
        got = g[3].double().cpu().numpy()
        tol = DBIAS_BAR * np.abs(db_ref).max() + row_bound[..., None]
        excess = np.abs(got - db_ref) - tol
        assert excess.max() <= 0, (label, float(excess.max()), float(np.abs(got - db_ref).max()))
    return g


@pytest.mark.parametrize("N", [1, 17, 64, 65, 130, 300])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("with_bias", [False, True])
def test_sweep_bf16(N, d, causal, with_bias):
    inp = workloads.make_inputs(1, 2, N, d, "bf16", seed=7 * N + d + causal, gate=with_bias)
    _run(inp, causal, 1 / math.sqrt(d), f"sweep N={N} d={d}", seed=N + d)


@pytest.mark.parametrize("N", [65, 300])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_f16_and_f32_gradients(N, d, causal):
    inp = workloads.make_inputs(2, 1, N, d, "f16", seed=N + d, gate=causal)
    _run(inp, causal, 1 / math.sqrt(d), f"f16 N={N} d={d}", seed=3)
    inp = workloads.make_inputs(1, 2, N, d, "bf16", seed=N + d + 1, gate=not causal)
    _run(inp, causal, 1 / math.sqrt(d), f"bf16->f32 N={N} d={d}", grad_dtype=torch.float32, seed=4)


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_forward_output(d, causal):
    """O handed over in fp32 (out_dtype float32 in the forward)."""
    inp = workloads.make_inputs(1, 2, 300, d, "bf16", seed=200 + d + causal, gate=True)
    _run(inp, causal, 1 / math.sqrt(d), f"o f32 d={d}", seed=11, o_f32=True)


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_several_tiles_and_heads(d, causal):
    """N = 1000: four 256-query tiles of the dQ kernel (ragged last), eight
    128-key tiles of the key-side kernel, 16 bias blocks per side."""
    inp = workloads.make_inputs(2, 3, 1000, d, "bf16", seed=100 + d + causal, gate=True)
    _run(inp, causal, 1 / math.sqrt(d), f"N=1000 d={d}", seed=5)


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_gates(causal):
    """Gated-off blocks (bias -inf) pass no gradient, and a query block gated
    off everywhere (no visible key, LSE = -inf) passes none at all."""
    inp = workloads.make_inputs(1, 2, 700, 64, "bf16", seed=21 + causal, gate=True, gate_keep=0.3)
    inp["bias"][0, 1, 3, :] = -math.inf
    g = _run(inp, causal, 0.125, "sparse gates", seed=6)
    assert (g[0][0, 1, 192:256] == 0).all()


def test_scale_edges_and_masked_rows():
    inp = workloads.make_inputs(1, 2, 200, 128, "bf16", seed=31, gate=True)
    for scale in (-0.3, 0.0):
        _run(inp, True, scale, f"scale={scale}", seed=7)


def test_deterministic():
    """Identical calls give bit-identical gradients (the block-bias gradient
    takes at most two atomic additions per entry, onto zero)."""
    inp = workloads.make_inputs(2, 2, 600, 128, "bf16", seed=41, gate=True)
    q, k, v, b = (inp[n].to(DEV) for n in ("q", "k", "v", "bias"))
    o, lse = attn.fwd(q, k, v, causal=True, bias=b, return_lse=True)
    dout = _dout(q.shape, q.dtype, 8).to(DEV)
    g1 = attn.bwd(q, k, v, o, dout, lse, causal=True, bias=b, return_dbias=True)
    g2 = attn.bwd(q, k, v, o, dout, lse, causal=True, bias=b, return_dbias=True)
    torch.cuda.synchronize()
    for a, c in zip(g1, g2):
        assert torch.equal(a, c)


def test_autograd_wrapper_matches_bwd():
    """attention() under torch.autograd returns the forward kernel's output
    and the backward kernels' gradients, including the bias's."""
    inp = workloads.make_inputs(1, 2, 300, 64, "bf16", seed=51, gate=True)
    q, k, v = (inp[n].to(DEV).requires_grad_() for n in ("q", "k", "v"))
    b = inp["bias"].to(DEV).requires_grad_()
    o = attn.attention(q, k, v, causal=True, bias=b)
    dout = _dout(q.shape, q.dtype, 9).to(DEV)
    o.backward(dout)
    o2, lse = attn.fwd(q.detach(), k.detach(), v.detach(), causal=True, bias=b.detach(), return_lse=True)
    g = attn.bwd(q.detach(), k.detach(), v.detach(), o2, dout, lse, causal=True, bias=b.detach(),
                 return_dbias=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    for t, ref in zip((q, k, v, b), g):
        assert torch.equal(t.grad, ref)


@pytest.mark.parametrize("cfg_id", [2, 5])
def test_workload_sampled(cfg_id):
    """Full-size workloads (llm-prefill; DiT with gates, d = 64) in the launch
    configuration the benchmark times: gradients of a loss that weighs only a
    few sampled query rows (dout zero elsewhere), so the oracle backward stays
    small: dQ is compared on those rows, dK and dV on all keys of the heads
    that hold them."""
    cfg, inp = workloads.config_inputs(cfg_id)
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    bias = inp["bias"].to(DEV) if inp["bias"] is not None else None
    scale = 1 / math.sqrt(d)
    o, lse = attn.fwd(q, k, v, causal=cfg["causal"], scale=scale, bias=bias, return_lse=True)
    heads = [(0, 0), (B - 1, H - 1)]
    rows = [0, 1, 63, 64, 1000, N // 2, N - 65, N - 1]
    dout = torch.zeros_like(q)
    g = torch.Generator("cpu").manual_seed(cfg_id)
    for b_, h_ in heads:
        dout[b_, h_, rows] = torch.randn((len(rows), d), generator=g).to(q.dtype).to(DEV)
    print(f"[gpu] bwd workload {cfg['name']}", flush=True)
    dq, dk, dv = attn.bwd(q, k, v, o, dout, lse, causal=cfg["causal"], scale=scale, bias=bias)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    for b_, h_ in heads:
        sl = lambda t: t[b_:b_ + 1, h_:h_ + 1].float().cpu().numpy()  # noqa: E731
        bn = inp["bias"][b_:b_ + 1, h_:h_ + 1].numpy() if inp["bias"] is not None else None
        ref = oracle.attn_bwd(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(dout), causal=cfg["causal"],
                              scale=scale, bias=bn)
        _compare(f"{cfg['name']} dq rows", dq[b_, h_, rows], ref[0][0, 0, rows], BAR[(q.dtype, q.dtype)])
        _compare(f"{cfg['name']} dk", dk[b_:b_ + 1, h_:h_ + 1], ref[1], BAR[(q.dtype, q.dtype)])
        _compare(f"{cfg['name']} dv", dv[b_:b_ + 1, h_:h_ + 1], ref[2], BAR[(q.dtype, q.dtype)])
    # heads with dout = 0 get exactly zero gradients
    assert not dq[0, 1].any() and not dk[0, 1].any() and not dv[0, 1].any()
