"""Every output buffer a kernel writes sits between two canary bands.

Each entry point is called through the C ABI with its outputs (O, LSE, the
gradients and the bias gradient, the 8-bit workspace) carved out of larger
buffers whose 4 KiB before and after the region hold a fixed pattern.
After the call the bands must be untouched bit for bit (no kernel writes
outside the region it owns, also on ragged shapes, masked tails and packed
sequences), and the region must hold the binding's own result for the same
call bit for bit (so the call ran and wrote all of it).
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import bit_attention_attn_amd as attn
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BAND = 4096  # bytes of canary on each side
PATTERN = 0xA5


class Padded:
    """A tensor view of `shape` inside a byte buffer with canary bands."""

    def __init__(self, shape, dtype):
        elem = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) * elem
        self.raw = torch.full((BAND + n + BAND,), PATTERN, dtype=torch.uint8, device=DEV)
        self.n = n
        self.t = self.raw[BAND:BAND + n].view(dtype).view(shape)

    def ptr(self):
        return ctypes.c_void_p(self.t.data_ptr())

    def bands_intact(self):
        torch.cuda.synchronize()
        return bool((self.raw[:BAND] == PATTERN).all()) and bool((self.raw[BAND + self.n:] == PATTERN).all())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


SHAPES = [(1, 2, 200, 64, False, False), (2, 2, 333, 128, True, False), (1, 3, 190, 96, True, True),
          (1, 2, 257, 128, False, True)]


@pytest.mark.parametrize("B,H,N,d,causal,with_bias", SHAPES)
@pytest.mark.parametrize("out", ["same", "f32"])
def test_forward_16bit(B, H, N, d, causal, with_bias, out):
    inp = workloads.make_inputs(B, H, N, d, "bf16", seed=N + d, gate=with_bias, gate_keep=0.5)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    bias = inp["bias"].to(DEV) if with_bias else None
    odt = torch.bfloat16 if out == "same" else torch.float32
    o, lse = Padded((B, H, N, d), odt), Padded((B, H, N), torch.float32)
    L = attn.lib()
    st = L.attn_fwd_bf16(_p(q), _p(k), _p(v), o.ptr(), lse.ptr(), B, H, N, d, int(causal), 1.0 / math.sqrt(d),
                         _p(bias), attn.DTYPE_F32 if out == "f32" else attn.DTYPE_BF16, _stream())
    assert st == 0, st
    assert o.bands_intact() and lse.bands_intact()
    o_ref, l_ref = attn.fwd(q, k, v, causal=causal, scale=1.0 / math.sqrt(d), bias=bias, out_dtype=odt,
                            return_lse=True)
    assert torch.equal(o.t, o_ref) and torch.equal(lse.t, l_ref)


@pytest.mark.parametrize("d", [64, 128])
def test_forward_packed_with_bias(d):
    lens = [1, 63, 130, 0, 77]
    H, N = 2, max(lens)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    total, B, nb = sum(lens), len(lens), (N + 63) // 64
    g = torch.Generator("cpu").manual_seed(d)
    q, k, v = (torch.randn((total, H, d), generator=g).to(torch.bfloat16).to(DEV) for _ in range(3))
    bias = workloads.gate_bias(torch.randn((B, H, nb, nb), generator=g), keep=0.5).to(DEV)
    o, lse = Padded((total, H, d), torch.bfloat16), Padded((B, H, N), torch.float32)
    strides = []
    for t in (q, k, v, o.t):
        strides += [0, t.stride(1), t.stride(0)]
    arr = (ctypes.c_longlong * 12)(*strides)
    st = attn.lib().attn_fwd_strided_bf16(_p(q), _p(k), _p(v), o.ptr(), lse.ptr(), B, H, N, d, arr, _p(cu), 1,
                                          1.0 / math.sqrt(d), _p(bias), attn.DTYPE_BF16, _stream())
    assert st == 0, st
    assert o.bands_intact() and lse.bands_intact()
    o_ref, l_ref = attn.fwd_varlen(q, k, v, cu, N, causal=True, return_lse=True, bias=bias)
    assert torch.equal(o.t, o_ref)
    for b, n in enumerate(lens):
        assert torch.equal(lse.t[b, :, :n], l_ref[b, :, :n])


@pytest.mark.parametrize("B,H,N,d,causal,with_bias", SHAPES)
@pytest.mark.parametrize("qk", ["int8", "fp8", "pv16"])
def test_8bit_preparation_and_forward(B, H, N, d, causal, with_bias, qk):
    inp = workloads.make_inputs(B, H, N, d, "bf16", seed=3 * N + d, outliers=True, gate=with_bias)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    bias = inp["bias"].to(DEV) if with_bias else None
    L = attn.lib()
    need = L.attn_sage8_workspace_size(B, H, N, d)
    ws = Padded((need,), torch.uint8)
    prep_fn = L.attn_k_smooth_quant_fp8qk if qk == "fp8" else L.attn_k_smooth_quant
    st = prep_fn(_p(q), _p(k), _p(v), attn.DTYPE_BF16, B, H, N, d, ws.ptr(), need, _stream())
    assert st == 0, st
    assert ws.bands_intact()
    o, lse = Padded((B, H, N, d), torch.bfloat16), Padded((B, H, N), torch.float32)
    if qk == "pv16":
        st = L.attn_fwd_sage8_pv16(ws.ptr(), _p(v), attn.DTYPE_BF16, o.ptr(), lse.ptr(), B, H, N, d, int(causal),
                                   1.0 / math.sqrt(d), _p(bias), attn.DTYPE_BF16, _stream())
    else:
        fn = L.attn_fwd_sage8_fp8qk if qk == "fp8" else L.attn_fwd_sage8
        st = fn(ws.ptr(), o.ptr(), lse.ptr(), B, H, N, d, int(causal), 1.0 / math.sqrt(d), _p(bias),
                attn.DTYPE_BF16, _stream())
    assert st == 0, st
    assert o.bands_intact() and lse.bands_intact() and ws.bands_intact()
    prep = attn.sage8_prep(q, k, v, qk="fp8" if qk == "fp8" else "int8")
    if qk == "pv16":
        o_ref, l_ref = attn.fwd_sage8_pv16(prep, v, causal=causal, bias=bias, return_lse=True)
    else:
        o_ref, l_ref = attn.fwd_sage8(prep, causal=causal, bias=bias, return_lse=True)
    assert torch.equal(o.t, o_ref) and torch.equal(lse.t, l_ref)


@pytest.mark.parametrize("B,H,N,d,causal,with_bias", SHAPES)
def test_backward(B, H, N, d, causal, with_bias):
    inp = workloads.make_inputs(B, H, N, d, "bf16", seed=5 * N + d, gate=with_bias)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    bias = inp["bias"].to(DEV) if with_bias else None
    o, lse_t = attn.fwd(q, k, v, causal=causal, bias=bias, return_lse=True)
    dout = torch.randn(q.shape, generator=torch.Generator("cpu").manual_seed(N)).to(torch.bfloat16).to(DEV)
    L = attn.lib()
    wsb = L.attn_bwd_workspace_size(B, H, N, d)
    ws = Padded((wsb,), torch.uint8)
    nb = (N + 63) // 64
    dq, dk, dv = (Padded((B, H, N, d), torch.bfloat16) for _ in range(3))
    db = Padded((B, H, nb, nb), torch.float32) if with_bias else None
    st = L.attn_bwd_bf16(_p(q), _p(k), _p(v), _p(o), attn.DTYPE_BF16, _p(dout), _p(lse_t), dq.ptr(), dk.ptr(),
                         dv.ptr(), db.ptr() if db else None, B, H, N, d, int(causal), 1.0 / math.sqrt(d),
                         _p(bias), attn.DTYPE_BF16, ws.ptr(), wsb, _stream())
    assert st == 0, st
    for t in (dq, dk, dv, ws) + ((db,) if db else ()):
        assert t.bands_intact()
    ref = attn.bwd(q, k, v, o, dout, lse_t, causal=causal, bias=bias, return_dbias=with_bias)
    assert torch.equal(dq.t, ref[0]) and torch.equal(dk.t, ref[1]) and torch.equal(dv.t, ref[2])
    if with_bias:
        assert torch.equal(db.t, ref[3])
