"""GPU tests of the 8-bit path on strided inputs and outputs (token-major
[B,N,H,d] tensors, views into a fused QKV projection, a token-major O).

Bar: bit-for-bit equality with the contiguous entry points on the same
logical [B,H,N,d] data.  The preparation must write the same workspace bytes
(codes, scales, K mean), and the forward the same output and LSE; the
contiguous pair is held to the oracle by test_gpu_sage8.py and
test_gpu_fp8qk.py.
"""
import pytest
import torch

import bit_attention_attn_amd as attn
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REGIONS = ("qq", "kq", "vq", "sq", "sk", "sv", "kmean")


def _same_workspace(a, b, label):
    va, vb = attn.sage8_workspace_views(a), attn.sage8_workspace_views(b)
    for name in REGIONS:
        x, y = va[name], vb[name]
        if x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), (label, name)


def _inputs(B, H, N, d, dtype, seed, outliers=False):
    inp = workloads.make_inputs(B, H, N, d, dtype, seed=seed, outliers=outliers)
    return [inp[n].to(DEV) for n in ("q", "k", "v")]


@pytest.mark.parametrize("N", [1, 65, 200, 300])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("qk", ["int8", "fp8"])
def test_token_major_prep_and_forward(N, d, qk):
    print(f"[gpu] sage8 strided token-major N={N} d={d} qk={qk}", flush=True)
    q, k, v = _inputs(2, 3, N, d, "bf16", seed=N + d, outliers=True)
    # token-major storage, viewed as [B,H,N,d]
    qt, kt, vt = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    assert qt.is_contiguous() == (N == 1)  # a single token is in contiguous order anyway
    ref = attn.sage8_prep(q, k, v, qk=qk)
    got = attn.sage8_prep(qt, kt, vt, qk=qk)
    _same_workspace(ref, got, f"N={N} d={d} {qk}")
    for causal in (False, True):
        o_ref, l_ref = attn.fwd_sage8(ref, causal=causal, return_lse=True)
        o_got, l_got = attn.fwd_sage8(got, causal=causal, return_lse=True, layout_like=qt)
        torch.cuda.synchronize()
        assert N == 1 or (not o_got.is_contiguous() and o_got.stride() == qt.stride())
        assert torch.equal(o_got, o_ref) and torch.equal(l_got, l_ref), (N, d, qk, causal)


@pytest.mark.parametrize("qk", ["int8", "fp8"])
def test_fused_qkv_views_and_fp32_output(qk):
    """q, k, v as slices of one [B,N,3,H,d] projection output (token stride
    3*H*d), the output in fp32 into a token-major tensor, with a gate bias."""
    B, H, N, d = 1, 4, 333, 128
    print(f"[gpu] sage8 strided fused-qkv qk={qk}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(11)
    qkv = torch.randn((B, N, 3, H, d), device=DEV, dtype=torch.float16, generator=g)
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    ref = attn.sage8_prep(q.contiguous(), k.contiguous(), v.contiguous(), qk=qk)
    got = attn.sage8_prep(q, k, v, qk=qk)
    _same_workspace(ref, got, f"fused {qk}")
    nb = (N + 63) // 64
    bias = workloads.gate_bias(torch.randn((B, H, nb, nb), generator=torch.Generator().manual_seed(3)) * 1.4,
                               0.5).to(DEV)
    like = torch.empty((B, N, H, d), device=DEV, dtype=torch.float16).transpose(1, 2)
    o_ref = attn.fwd_sage8(ref, causal=True, bias=bias, out_dtype=torch.float32)
    o_got = attn.fwd_sage8(got, causal=True, bias=bias, out_dtype=torch.float32, layout_like=like)
    torch.cuda.synchronize()
    assert o_got.dtype == torch.float32 and o_got.stride() == like.stride()
    assert torch.equal(o_got, o_ref)


def test_sageattn_nhd_layout():
    B, H, N, d = 2, 2, 190, 64
    print("[gpu] sageattn tensor_layout=NHD", flush=True)
    q, k, v = _inputs(B, H, N, d, "f16", seed=5)
    o_hnd = attn.sageattn(q, k, v, causal=True)
    qn, kn, vn = (x.transpose(1, 2).contiguous() for x in (q, k, v))  # [B,N,H,d]
    o_nhd = attn.sageattn(qn, kn, vn, causal=True, tensor_layout="NHD")
    torch.cuda.synchronize()
    assert o_nhd.shape == (B, N, H, d) and o_nhd.is_contiguous()
    assert torch.equal(o_nhd.transpose(1, 2), o_hnd)


def test_workload_token_major():
    """The DiT-gated workload's shape (2 x 24 x 16384, d = 64) with token-major
    inputs: prep bytes equal, output equal on every row."""
    cfg, inp = workloads.config_inputs(5)
    print(f"[gpu] sage8 strided workload {cfg['name']}", flush=True)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    bias = inp["bias"].to(DEV)
    del inp
    ref = attn.sage8_prep(q, k, v)
    qt, kt, vt = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    del q, k, v
    got = attn.sage8_prep(qt, kt, vt)
    _same_workspace(ref, got, "dit-gated")
    o_ref = attn.fwd_sage8(ref, bias=bias)
    o_got = attn.fwd_sage8(got, bias=bias, layout_like=qt)
    torch.cuda.synchronize()
    assert torch.equal(o_got, o_ref)


def test_token_major_against_oracle():
    """One strided case held to the oracle directly (not only to the
    contiguous entry): token-major Q, K, V and O, against the kernel-precision
    model of the recipe fed the oracle's own quantisation of the logical
    [B,H,N,d] data (max abs 1e-3, the contiguous path's bar) and against the
    exact fp64 attention (cosine >= 0.999)."""
    import numpy as np
    import oracle
    B, H, N, d = 2, 2, 300, 128
    inp = workloads.make_inputs(B, H, N, d, "bf16", seed=17, outliers=True)
    q, k, v = (inp[n].to(DEV).transpose(1, 2).contiguous().transpose(1, 2) for n in ("q", "k", "v"))
    prep = attn.sage8_prep(q, k, v)
    o = attn.fwd_sage8(prep, causal=True, out_dtype=torch.float32, layout_like=q)
    torch.cuda.synchronize()
    assert not o.is_contiguous()
    rows = np.array([(b, h, i) for b in range(B) for h in range(H) for i in range(N)], dtype=np.int64)
    got = workloads.gather_rows(o, rows)
    qn, kn, vn = (inp[n].float().numpy() for n in ("q", "k", "v"))
    ref = oracle.sage8_prepare(qn, kn, vn)
    o_emu, _ = oracle.sage8_emulate_rows_fp32(ref, rows, causal=True, scale=1 / d ** 0.5)
    m_emu = workloads.error_metrics(got, o_emu)
    o_ref, _ = oracle.attn_rows(qn, kn, vn, rows, causal=True, scale=1 / d ** 0.5)
    m_ref = workloads.error_metrics(got, o_ref)
    print(f"    token-major vs fp32 model: {m_emu}; vs fp64 attention: {m_ref}", flush=True)
    assert m_emu["max_abs"] <= 1e-3 and m_emu["mean_abs"] <= 2e-5, m_emu
    assert m_ref["cos"] >= 0.999, m_ref
