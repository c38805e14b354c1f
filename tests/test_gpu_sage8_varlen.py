"""GPU tests of the 8-bit path on packed sequences (q, k, v [total,H,d] with
int32 offsets cu_seqlens [B+1]).

Reading: a packed batch is a batch of independent sequences, so every
statistic of the recipe (K mean over tokens, V channel scales, 64-row Q/K
blocks) is taken over one sequence alone.  Bars:
  * preparation: slot b of the workspace holds bit for bit what the
    contiguous preparation writes for sequence b on its own, with zero codes
    (scale 1) past the sequence's blocks; in one case also bit for bit the
    oracle's quantisers applied to each sequence;
  * forward: the rows of sequence b in O, and its LSE, are bit for bit those
    of the contiguous forward on sequence b alone (held to the oracle by
    test_gpu_sage8.py and test_gpu_fp8qk.py).
"""
import numpy as np
import pytest
import torch

import bit_attention_attn_amd as attn
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REGIONS = ("qq", "kq", "sq", "sk", "sv", "kmean", "vq_logical")


def _packed(lens, H, d, dtype, seed):
    """Sequence b drawn on its own (its own channel offsets, so the K means
    differ between sequences), then packed token-major."""
    parts = {n: [] for n in ("q", "k", "v")}
    for b, n in enumerate(lens):
        if n == 0:
            continue
        inp = workloads.make_inputs(1, H, n, d, dtype, seed=seed + 101 * b, outliers=True)
        for name in parts:
            parts[name].append(inp[name][0].transpose(0, 1))  # [n,H,d]
    packed = {name: torch.cat(parts[name]).contiguous().to(DEV) for name in parts}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    return packed["q"], packed["k"], packed["v"], cu


def _seq(x, cu, b):
    """Sequence b of a packed [total,H,d] tensor as a contiguous [1,H,n,d]."""
    t0, t1 = int(cu[b]), int(cu[b + 1])
    return x[t0:t1].transpose(0, 1).unsqueeze(0).contiguous()


def _check_slot(views, b, ref_views, n):
    nb = (n + 63) // 64
    for name in REGIONS:
        got, want = views[name][b], ref_views[name][0] if ref_views is not None else None
        if got.dtype == torch.float32:
            got = got.view(torch.int32)
            want = want.view(torch.int32) if want is not None else None
        if name in ("qq", "kq", "vq_logical"):
            if want is not None:
                assert torch.equal(got[:, :n], want[:, :n]), (b, name)
            assert not got[:, n:].any(), (b, name, "padding")
        elif name in ("sq", "sk"):
            if want is not None:
                assert torch.equal(got[:, :nb], want[:, :nb]), (b, name)
            one = torch.tensor(1.0, device=DEV).view(torch.int32)
            assert (got[:, nb:] == one).all(), (b, name, "padding scale")
        elif want is not None:
            assert torch.equal(got, want), (b, name)


def _run(lens, H, d, dtype, qk, seed, out_dtype=None):
    q, k, v, cu = _packed(lens, H, d, dtype, seed)
    N = max(lens)
    prep = attn.sage8_prep_varlen(q, k, v, cu, N, qk=qk)
    views = attn.sage8_workspace_views(prep)
    outs = {}
    for causal in (False, True):
        outs[causal] = attn.fwd_sage8(prep, causal=causal, out_dtype=out_dtype, return_lse=True)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        if n == 0:
            _check_slot(views, b, None, 0)
            zero = torch.tensor(0.0, device=DEV)
            assert torch.equal(views["kmean"][b], zero.expand_as(views["kmean"][b]))
            continue
        ref = attn.sage8_prep(_seq(q, cu, b), _seq(k, cu, b), _seq(v, cu, b), qk=qk)
        _check_slot(views, b, attn.sage8_workspace_views(ref), n)
        t0 = int(cu[b])
        for causal in (False, True):
            o_ref, l_ref = attn.fwd_sage8(ref, causal=causal, out_dtype=out_dtype, return_lse=True)
            o, lse = outs[causal]
            assert torch.equal(o[t0:t0 + n], o_ref[0].transpose(0, 1)), (lens, b, causal)
            assert torch.equal(lse[b, :, :n], l_ref[0]), (lens, b, causal)
    return q, k, v, cu, prep


@pytest.mark.parametrize("lens", [[1, 65, 200, 300], [130, 0, 64, 257, 1], [128, 128]])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("qk", ["int8", "fp8"])
def test_packed_equals_separate(lens, d, qk):
    print(f"[gpu] sage8 varlen lens={lens} d={d} qk={qk}", flush=True)
    _run(lens, 3, d, "bf16", qk, seed=sum(lens) + d)


def test_packed_fp16_fp32_output():
    print("[gpu] sage8 varlen f16 -> fp32 output", flush=True)
    _run([77, 190, 5], 2, 128, "f16", "int8", seed=3, out_dtype=torch.float32)


def test_packed_prep_matches_oracle():
    """The workspace of a packed call against the oracle's quantisers run on
    each sequence on its own."""
    lens, H, d = [70, 1, 193], 2, 64
    print(f"[gpu] sage8 varlen prep vs oracle lens={lens}", flush=True)
    q, k, v, cu = _packed(lens, H, d, "bf16", seed=9)
    prep = attn.sage8_prep_varlen(q, k, v, cu, max(lens))
    torch.cuda.synchronize()
    cpu = {name: t.cpu() for name, t in attn.sage8_workspace_views(prep).items()}
    for b, n in enumerate(lens):
        ref = oracle.sage8_prepare(*(_seq(x, cu, b).float().cpu().numpy() for x in (q, k, v)))
        nb = (n + 63) // 64
        assert np.array_equal(cpu["kmean"][b].numpy().view(np.uint32), ref["kmean"][0].view(np.uint32))
        assert np.array_equal(cpu["sv"][b].numpy().view(np.uint32), ref["sv"][0].view(np.uint32))
        for name in ("qq", "kq"):
            assert np.array_equal(cpu[name][b, :, :n].numpy(), ref[name][0]), (b, name)
        for name in ("sq", "sk"):
            assert np.array_equal(cpu[name][b, :, :nb].numpy().view(np.uint32), ref[name][0].view(np.uint32))
        assert np.array_equal(cpu["vq_logical"][b, :, :n].numpy(), ref["vq"][0])


def test_sageattn_varlen_long_mix():
    """A long-context length mix (one long sequence, several short ones) in
    one call, against separate calls."""
    lens = [4096, 1000, 2500, 129, 64]
    H, d = 8, 128
    print(f"[gpu] sageattn_varlen lens={lens}", flush=True)
    q, k, v, cu = _packed(lens, H, d, "bf16", seed=17)
    o = attn.sageattn_varlen(q, k, v, cu, max(lens), causal=True)
    torch.cuda.synchronize()
    assert o.shape == q.shape and o.dtype == q.dtype
    for b, n in enumerate(lens):
        t0 = int(cu[b])
        o_ref = attn.sageattn(_seq(q, cu, b), _seq(k, cu, b), _seq(v, cu, b), causal=True)
        assert torch.equal(o[t0:t0 + n], o_ref[0].transpose(0, 1)), b


def test_packed_rejects_bad_bias_and_layout():
    q, k, v, cu = _packed([65, 10], 2, 64, "bf16", seed=1)
    prep = attn.sage8_prep_varlen(q, k, v, cu, 65)
    with pytest.raises(ValueError):  # nb must come from max_seqlen: ceil(65/64) = 2
        attn.fwd_sage8(prep, bias=torch.zeros((2, 2, 1, 1), device=DEV))
    with pytest.raises(ValueError):
        attn.fwd_sage8(prep, layout_like=torch.zeros((2, 2, 65, 64), device=DEV))
    with pytest.raises(ValueError):
        attn.sage8_prep_varlen(q, k, v, cu.long(), 65)


def test_packed_against_oracle():
    """One packed batch held to the oracle directly: each sequence's rows
    against the kernel-precision model of the recipe fed the oracle's own
    quantisation of that sequence alone (reading: each sequence is prepared
    on its own; max abs 1e-3, the contiguous path's bar), and against the
    exact fp64 attention of that sequence (cosine >= 0.999 where it has at
    least 64 keys)."""
    lens, H, d = [70, 1, 200, 129], 2, 128
    q, k, v, cu = _packed(lens, H, d, "bf16", seed=29)
    o = attn.sageattn_varlen(q, k, v, cu, max(lens), causal=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        qs, ks, vs = (_seq(x, cu, b).float().cpu().numpy() for x in (q, k, v))
        ref = oracle.sage8_prepare(qs, ks, vs)
        rows = np.array([(0, h, i) for h in range(H) for i in range(n)], dtype=np.int64)
        o_emu, _ = oracle.sage8_emulate_rows_fp32(ref, rows, causal=True, scale=1 / d ** 0.5)
        t0 = int(cu[b])
        got = o[t0:t0 + n].transpose(0, 1).reshape(-1, d).double().cpu().numpy()
        m = workloads.error_metrics(got, o_emu)
        assert m["max_abs"] <= 1e-3 and m["mean_abs"] <= 2e-5, (b, m)
        if n >= 64:
            o_ref, _ = oracle.attn_rows(qs, ks, vs, rows, causal=True, scale=1 / d ** 0.5)
            m_ref = workloads.error_metrics(got, o_ref)
            print(f"    packed sequence {b} (n={n}) vs fp32 model: {m}; vs fp64 attention: {m_ref}", flush=True)
            assert m_ref["cos"] >= 0.999, (b, m_ref)


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("qk", ["int8", "fp8"])
@pytest.mark.parametrize("keep", [None, 0.3])
def test_packed_with_block_bias(d, qk, keep):
    """A block bias [B,H,nb,nb] (nb from the longest length) on packed
    sequences: sequence b takes bias[b,h,i,j] for its blocks counted from its
    own first token, so its rows of O and its LSE are bit for bit those of
    the contiguous forward on it alone with the bias slice
    bias[b:b+1, :, :nb_b, :nb_b] (gates with and without gated-off blocks)."""
    lens = [130, 0, 64, 257, 1, 200]
    H = 2
    q, k, v, cu = _packed(lens, H, d, "bf16", seed=900 + d)
    N = max(lens)
    nb = (N + 63) // 64
    g = torch.randn((len(lens), H, nb, nb), generator=torch.Generator("cpu").manual_seed(77 + d))
    bias = workloads.gate_bias(g, keep=keep).to(DEV)
    print(f"[gpu] sage8 varlen bias d={d} qk={qk} keep={keep}", flush=True)
    prep = attn.sage8_prep_varlen(q, k, v, cu, N, qk=qk)
    for causal in (False, True):
        o, lse = attn.fwd_sage8(prep, causal=causal, bias=bias, return_lse=True)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all()
        for b, n in enumerate(lens):
            if n == 0:
                continue
            ref = attn.sage8_prep(_seq(q, cu, b), _seq(k, cu, b), _seq(v, cu, b), qk=qk)
            nbb = (n + 63) // 64
            bb = bias[b:b + 1, :, :nbb, :nbb].contiguous()
            o_ref, l_ref = attn.fwd_sage8(ref, causal=causal, bias=bb, return_lse=True)
            t0 = int(cu[b])
            assert torch.equal(o[t0:t0 + n], o_ref[0].transpose(0, 1)), (b, causal)
            assert torch.equal(lse[b, :, :n], l_ref[0]), (b, causal)

