"""GPU parity of the strided / packed-sequence forward (fp16 / bf16) against
the fp64 oracle, which takes contiguous [B,H,N,d] copies of the same rounded
inputs.  Bar as for the contiguous forward: max abs <= 1e-2, mean abs <=
1e-3, LSE within ln(1 + 2^-8) + 2^-12 (the inputs here are bf16)."""
import math

import numpy as np
import pytest
import torch

import bit_attention_attn_amd as attn
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MAX_ABS, MEAN_ABS, LSE_TOL = 1e-2, 1e-3, math.log1p(2.0 ** -8) + 2.0 ** -12


def _check(o, lse, q, k, v, causal, scale, label):
    """o, lse from the GPU; q, k, v CPU [B,H,N,d] (any dtype)."""
    qn, kn, vn = (t.float().contiguous().numpy() for t in (q, k, v))
    o_ref, l_ref = oracle.attn_full(qn, kn, vn, causal=causal, scale=scale)
    got = o.double().cpu().numpy()
    err = np.abs(got - o_ref)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (label, err.max(), err.mean())
    if lse is not None:
        assert np.abs(lse.double().cpu().numpy() - l_ref).max() <= LSE_TOL, label


@pytest.mark.parametrize("N", [65, 300])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_token_major_layout(N, d, causal):
    """[B,N,H,d] tensors passed as their [B,H,N,d] transposed views."""
    B, H = 2, 3
    g = torch.Generator("cpu").manual_seed(N * 7 + d + causal)
    x = [torch.randn((B, N, H, d), generator=g).to(torch.bfloat16) for _ in range(3)]
    q, k, v = (t.to(DEV).transpose(1, 2) for t in x)
    print(f"[gpu] strided token-major N={N} d={d} causal={causal}", flush=True)
    o, lse = attn.fwd_strided(q, k, v, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    assert o.stride() == q.stride()
    _check(o, lse, *(t.transpose(1, 2) for t in x), causal, 1 / math.sqrt(d), "token-major")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("out", ["same", "f32"])
def test_fused_qkv_views(dtype, out):
    """q, k, v as views of one [B,N,3,H,d] projection output."""
    B, N, H, d = 2, 200, 2, 128
    g = torch.Generator("cpu").manual_seed(5)
    qkv = torch.randn((B, N, 3, H, d), generator=g).to(workloads.torch_dtype(dtype))
    dev = qkv.to(DEV)
    q, k, v = (dev[:, :, i].transpose(1, 2) for i in range(3))
    print(f"[gpu] strided fused-qkv {dtype} out={out}", flush=True)
    o = attn.fwd_strided(q, k, v, causal=True, out_dtype=torch.float32 if out == "f32" else None)
    torch.cuda.synchronize()
    _check(o, None, *(qkv[:, :, i].transpose(1, 2) for i in range(3)), True, 1 / math.sqrt(d), "fused")


def test_strided_matches_contiguous_entry():
    """On contiguous tensors the strided entry gives the same result as the
    contiguous one (the same arithmetic in the same order)."""
    inp = workloads.make_inputs(2, 4, 333, 128, "bf16", seed=8)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    for causal in (False, True):
        o1 = attn.fwd(q, k, v, causal=causal)
        o2 = attn.fwd_strided(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_sequences(d, causal):
    """Sequences of lengths 1, 63, 64, 200, 513, 77 packed along the token
    axis; each attends only within itself."""
    lens = [1, 63, 64, 200, 513, 77]
    H = 2
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    g = torch.Generator("cpu").manual_seed(17 + d + causal)
    x = [torch.randn((total, H, d), generator=g).to(torch.bfloat16) for _ in range(3)]
    q, k, v = (t.to(DEV) for t in x)
    print(f"[gpu] varlen d={d} causal={causal}", flush=True)
    o, lse = attn.fwd_varlen(q, k, v, torch.from_numpy(cu).to(DEV), max(lens), causal=causal,
                             return_lse=True)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        seq = [t[s0:s1].transpose(0, 1).unsqueeze(0) for t in x]  # [1,H,n,d]
        _check(o[s0:s1].transpose(0, 1).unsqueeze(0), lse[b:b + 1, :, :n], *seq, causal,
               1 / math.sqrt(d), f"seq {b} (n={n})")


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("keep", [None, 0.3])
def test_packed_sequences_with_block_bias(d, causal, keep):
    """A block bias [B,H,nb,nb] (nb from the longest length) on packed
    sequences: sequence b takes bias[b,h,i,j] for its blocks counted from its
    own first token.  Each sequence against the oracle with its bias slice
    bias[b:b+1, :, :nb_b, :nb_b], and bit for bit against the contiguous
    forward on it alone with that slice (gates with and without gated-off
    blocks; the diagonal block is always kept)."""
    lens = [1, 63, 64, 200, 513, 0, 77]
    H = 2
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total, N = int(cu[-1]), max(lens)
    nb = (N + 63) // 64
    g = torch.Generator("cpu").manual_seed(31 + d + causal)
    x = [torch.randn((total, H, d), generator=g).to(torch.bfloat16) for _ in range(3)]
    bias = workloads.gate_bias(torch.randn((len(lens), H, nb, nb), generator=g), keep=keep)
    q, k, v = (t.to(DEV) for t in x)
    print(f"[gpu] varlen bias d={d} causal={causal} keep={keep}", flush=True)
    o, lse = attn.fwd_varlen(q, k, v, torch.from_numpy(cu).to(DEV), N, causal=causal, return_lse=True,
                             bias=bias.to(DEV))
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        if n == 0:
            continue
        s0, s1 = int(cu[b]), int(cu[b + 1])
        nbb = (n + 63) // 64
        bb = bias[b:b + 1, :, :nbb, :nbb].contiguous()
        seq = [t[s0:s1].transpose(0, 1).unsqueeze(0) for t in x]  # [1,H,n,d]
        qn, kn, vn = (t.float().contiguous().numpy() for t in seq)
        o_ref, l_ref = oracle.attn_full(qn, kn, vn, causal=causal, scale=1 / math.sqrt(d), bias=bb.numpy())
        got = o[s0:s1].transpose(0, 1).unsqueeze(0).double().cpu().numpy()
        err = np.abs(got - o_ref)
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (b, n, err.max(), err.mean())
        assert np.abs(lse[b:b + 1, :, :n].double().cpu().numpy() - l_ref).max() <= LSE_TOL, (b, n)
        o1, l1 = attn.fwd(*(t.to(DEV).contiguous() for t in seq), causal=causal, bias=bb.to(DEV),
                          return_lse=True)
        assert torch.equal(o[s0:s1], o1[0].transpose(0, 1)), (b, n)
        assert torch.equal(lse[b, :, :n], l1[0]), (b, n)


def test_strided_with_bias_matches_contiguous_entry():
    """A token-major layout with a gate bias gives the contiguous entry's
    result with the same bias, bit for bit."""
    inp = workloads.make_inputs(2, 3, 333, 128, "bf16", seed=9, gate=True, gate_keep=0.5)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    bias = inp["bias"].to(DEV)
    qt, kt, vt = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
    for causal in (False, True):
        o1 = attn.fwd(q, k, v, causal=causal, bias=bias)
        o2 = attn.fwd_strided(qt, kt, vt, causal=causal, bias=bias)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2.contiguous())


def test_packed_sequences_empty_and_padded_lse():
    """A zero-length sequence in the middle is allowed; O rows of the other
    sequences are unaffected."""
    lens = [100, 0, 130]
    H, d = 2, 64
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    g = torch.Generator("cpu").manual_seed(3)
    x = [torch.randn((total, H, d), generator=g).to(torch.bfloat16) for _ in range(3)]
    q, k, v = (t.to(DEV) for t in x)
    o = attn.fwd_varlen(q, k, v, torch.from_numpy(cu).to(DEV), max(lens), causal=True)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        if n == 0:
            continue
        s0, s1 = int(cu[b]), int(cu[b + 1])
        seq = [t[s0:s1].transpose(0, 1).unsqueeze(0) for t in x]
        _check(o[s0:s1].transpose(0, 1).unsqueeze(0), None, *seq, True, 1 / math.sqrt(d), f"seq {b}")


def test_packed_sequences_longer_than_max_seqlen_are_rejected():
    """The kernels clamp a sequence to max_seqlen, which would leave the rest
    of its rows unwritten: the binding checks the offsets first."""
    H, d = 2, 64
    x = torch.randn((100, H, d), generator=torch.Generator("cpu").manual_seed(3)).to(torch.bfloat16).to(DEV)
    cu = torch.tensor([0, 30, 100], dtype=torch.int32, device=DEV)   # lengths 30 and 70
    for fn in (attn.fwd_varlen, attn.sageattn_varlen):
        with pytest.raises(ValueError):
            fn(x, x, x, cu, 64)
        with pytest.raises(ValueError):
            fn(x, x, x, torch.tensor([0, 70, 50], dtype=torch.int32, device=DEV), 70)  # decreasing
        with pytest.raises(ValueError):
            fn(x, x, x, torch.tensor([0, 70, 101], dtype=torch.int32, device=DEV), 70)  # past the tokens
    o = attn.fwd_varlen(x, x, x, cu, 70)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
