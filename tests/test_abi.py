"""The C ABI: the library loads, exports every function include/attn.h
declares, and rejects invalid arguments with the documented status before any
HIP call (so these run without a GPU; no call here reaches a launch)."""
import ctypes
import os
import re

import pytest
import torch

import bit_attention_attn_amd as attn

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "attn.h")

OK, E_NULL, E_SHAPE, E_HEADDIM, E_DTYPE, E_ALIGN, E_ARG, E_WS, E_DEV, E_HIP = range(10)
F16, BF16, F32 = 0, 1, 2
FAKE = 0x100000  # 16- and 256-byte aligned, never dereferenced: every call below fails validation first


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = attn.lib()
    names = _declared_functions()
    assert {"attn_fwd_f16", "attn_fwd_bf16", "attn_fwd_strided_f16", "attn_fwd_strided_bf16",
            "attn_bwd_workspace_size", "attn_bwd_f16", "attn_bwd_bf16",
            "attn_k_smooth_quant_fp8qk", "attn_fwd_sage8_fp8qk",
            "attn_k_smooth_quant_strided", "attn_fwd_sage8_strided",
            "attn_sage8_workspace_size", "attn_k_smooth_quant", "attn_sage8_workspace_layout",
            "attn_fwd_sage8", "attn_fwd_sage8_pv16", "attn_status_str", "attn_abi_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert L.attn_abi_version() == 9
    for s in range(10):
        assert len(attn.status_str(s)) > 4


def _fwd(fn, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, H=1, N=64, d=64, causal=0, scale=0.125,
         bias=None, out=BF16):
    return fn(q, k, v, o, lse, B, H, N, d, causal, scale, bias, out, None)


@pytest.mark.parametrize("name,dt", [("attn_fwd_bf16", BF16), ("attn_fwd_f16", F16)])
def test_fwd_validation(name, dt):
    fn = getattr(attn.lib(), name)
    assert _fwd(fn, q=None, out=dt) == E_NULL
    assert _fwd(fn, o=None, out=dt) == E_NULL
    assert _fwd(fn, B=0, out=dt) == E_SHAPE
    assert _fwd(fn, N=0, out=dt) == E_SHAPE
    assert _fwd(fn, H=-1, out=dt) == E_SHAPE
    assert _fwd(fn, d=80, out=dt) == E_HEADDIM
    assert _fwd(fn, d=256, out=dt) == E_HEADDIM
    assert _fwd(fn, B=1 << 10, H=1 << 10, N=1 << 10, d=128, out=dt) == E_SHAPE  # 2^37 elements
    assert _fwd(fn, causal=2, out=dt) == E_ARG
    assert _fwd(fn, scale=float("nan"), out=dt) == E_ARG
    assert _fwd(fn, scale=float("inf"), out=dt) == E_ARG
    assert _fwd(fn, out=F16 if dt == BF16 else BF16) == E_DTYPE
    assert _fwd(fn, out=7) == E_DTYPE
    assert _fwd(fn, q=FAKE + 8, out=dt) == E_ALIGN
    assert _fwd(fn, o=FAKE + 2, out=dt) == E_ALIGN
    assert _fwd(fn, lse=FAKE + 2, out=dt) == E_ALIGN


def test_sage8_validation():
    L = attn.lib()
    assert L.attn_sage8_workspace_size(1, 1, 64, 80) == 0
    assert L.attn_sage8_workspace_size(1, 1, 64, 96) > 0
    assert L.attn_sage8_workspace_size(0, 1, 64, 64) == 0
    need = L.attn_sage8_workspace_size(1, 2, 100, 64)
    assert need >= 3 * 2 * 128 * 64  # three 8-bit tensors padded to 128 rows
    prep = L.attn_k_smooth_quant
    assert prep(None, FAKE, FAKE, BF16, 1, 2, 100, 64, FAKE, need, None) == E_NULL
    assert prep(FAKE, FAKE, FAKE, F32, 1, 2, 100, 64, FAKE, need, None) == E_DTYPE
    assert prep(FAKE, FAKE, FAKE, BF16, 1, 2, 100, 80, FAKE, need, None) == E_HEADDIM
    assert prep(FAKE, FAKE, FAKE, BF16, 1, 2, 100, 64, None, need, None) == E_WS
    assert prep(FAKE, FAKE, FAKE, BF16, 1, 2, 100, 64, FAKE, need - 1, None) == E_WS
    assert prep(FAKE, FAKE, FAKE, BF16, 1, 2, 100, 64, FAKE + 16, need, None) == E_ALIGN
    fwd8 = L.attn_fwd_sage8
    assert fwd8(None, FAKE, None, 1, 2, 100, 64, 0, 0.1, None, BF16, None) == E_WS
    assert fwd8(FAKE, None, None, 1, 2, 100, 64, 0, 0.1, None, BF16, None) == E_NULL
    assert fwd8(FAKE, FAKE, None, 1, 2, 100, 64, 3, 0.1, None, BF16, None) == E_ARG
    assert fwd8(FAKE, FAKE, None, 1, 2, 100, 64, 0, 0.1, None, 9, None) == E_DTYPE
    assert fwd8(FAKE + 64, FAKE, None, 1, 2, 100, 64, 0, 0.1, None, BF16, None) == E_ALIGN


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device error; a GPU is visible")
def test_no_device_is_an_error_not_a_fallback():
    assert _fwd(attn.lib().attn_fwd_bf16) == E_DEV


def test_python_binding_rejects_cpu_tensors():
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.fwd(q, q, q)
    # packed sequences: [total,H,d] tensors and int32 offsets on q's device
    qp = torch.zeros((8, 1, 64), dtype=torch.bfloat16)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    for fn in (attn.fwd_varlen, attn.sage8_prep_varlen, attn.sageattn_varlen):
        with pytest.raises(ValueError):
            fn(qp, qp, qp, cu, 8)
    with pytest.raises(ValueError):
        attn.sage8_prep_varlen(qp, qp, qp, cu, 8, qk="int4")


def _strided(fn, strides, q=FAKE, o=FAKE, cu=None, B=1, H=2, N=64, d=64, causal=0, out=BF16, bias=None):
    arr = None if strides is None else (ctypes.c_longlong * 12)(*strides)
    return fn(q, FAKE, FAKE, o, None, B, H, N, d, arr, cu, causal, 0.125, bias, out, None)


@pytest.mark.parametrize("name,dt", [("attn_fwd_strided_bf16", BF16), ("attn_fwd_strided_f16", F16)])
def test_strided_validation(name, dt):
    fn = getattr(attn.lib(), name)
    # a [B,N,H,d] token-major layout: batch N*H*d, head d, token H*d
    good = [64 * 2 * 64, 64, 2 * 64] * 4
    assert _strided(fn, None, out=dt) == E_NULL
    assert _strided(fn, good, q=None, out=dt) == E_NULL
    assert _strided(fn, good, d=80, out=dt) == E_HEADDIM
    assert _strided(fn, good, out=F16 if dt == BF16 else BF16) == E_DTYPE
    bad = list(good); bad[4] = -64
    assert _strided(fn, bad, out=dt) == E_ARG          # negative stride
    bad = list(good); bad[7] = 68
    assert _strided(fn, bad, out=dt) == E_ALIGN        # rows not 16-byte aligned
    bad = list(good); bad[11] = 32
    assert _strided(fn, bad, out=dt) == E_ARG          # token stride < d
    bad = list(good); bad[2] = 1 << 28
    assert _strided(fn, bad, N=1 << 12, out=dt) == E_SHAPE  # byte offsets beyond 32 bits
    assert _strided(fn, good, cu=FAKE + 2, out=dt) == E_ALIGN
    assert _strided(fn, good, causal=3, out=dt) == E_ARG
    assert _strided(fn, good, bias=FAKE + 2, out=dt) == E_ALIGN  # bias not 4-byte aligned


def _bwd(fn, q=FAKE, o=FAKE, lse=FAKE, dq=FAKE, dbias=None, B=1, H=2, N=100, d=64, causal=0,
         scale=0.125, grad=BF16, ws=FAKE, wsb=1 << 20, odt=None):
    return fn(q, FAKE, FAKE, o, grad if odt is None else odt, FAKE, lse, dq, FAKE, FAKE, dbias, B, H, N, d,
              causal, scale, None, grad, ws, wsb, None)


@pytest.mark.parametrize("name,dt", [("attn_bwd_bf16", BF16), ("attn_bwd_f16", F16)])
def test_bwd_validation(name, dt):
    L = attn.lib()
    fn = getattr(L, name)
    assert L.attn_bwd_workspace_size(1, 2, 100, 64) == 1024  # 200 fp32 rows, rounded to 256 bytes
    assert L.attn_bwd_workspace_size(1, 2, 100, 96) == 1024
    assert L.attn_bwd_workspace_size(1, 2, 100, 80) == 0      # no such head dimension
    assert _bwd(fn, q=None, grad=dt) == E_NULL
    assert _bwd(fn, lse=None, grad=dt) == E_NULL
    assert _bwd(fn, dq=None, grad=dt) == E_NULL
    assert _bwd(fn, B=0, grad=dt) == E_SHAPE
    assert _bwd(fn, d=80, grad=dt) == E_HEADDIM
    assert _bwd(fn, causal=2, grad=dt) == E_ARG
    assert _bwd(fn, scale=float("nan"), grad=dt) == E_ARG
    assert _bwd(fn, grad=F16 if dt == BF16 else BF16, odt=dt) == E_DTYPE
    assert _bwd(fn, grad=dt, odt=F16 if dt == BF16 else BF16) == E_DTYPE
    assert _bwd(fn, ws=None, grad=dt) == E_WS
    assert _bwd(fn, wsb=1023, grad=dt) == E_WS
    assert _bwd(fn, ws=FAKE + 16, grad=dt) == E_ALIGN
    assert _bwd(fn, o=FAKE + 8, grad=dt) == E_ALIGN
    assert _bwd(fn, dbias=FAKE + 2, grad=dt) == E_ALIGN


def test_fp8qk_validation():
    L = attn.lib()
    need = L.attn_sage8_workspace_size(1, 2, 100, 64)
    prep = L.attn_k_smooth_quant_fp8qk
    assert prep(None, FAKE, FAKE, BF16, 1, 2, 100, 64, FAKE, need, None) == E_NULL
    assert prep(FAKE, FAKE, FAKE, BF16, 1, 2, 100, 80, FAKE, need, None) == E_HEADDIM  # d = 64, 96 or 128
    assert prep(FAKE, FAKE, FAKE, F32, 1, 2, 100, 64, FAKE, need, None) == E_DTYPE
    assert prep(FAKE, FAKE, FAKE, BF16, 1, 2, 100, 64, FAKE, need - 1, None) == E_WS
    fwd8 = L.attn_fwd_sage8_fp8qk
    assert fwd8(None, FAKE, None, 1, 2, 100, 64, 0, 0.1, None, BF16, None) == E_WS
    assert fwd8(FAKE, FAKE, None, 1, 2, 100, 80, 0, 0.1, None, BF16, None) == E_HEADDIM
    assert fwd8(FAKE, FAKE, None, 1, 2, 100, 64, 3, 0.1, None, BF16, None) == E_ARG


def test_sage8_strided_validation():
    """Argument checks of the strided 8-bit pair (all run before any device
    call, so they hold without a GPU)."""
    L = attn.lib()
    ll = ctypes.c_longlong
    B, H, N, d = 1, 2, 100, 64
    need = L.attn_sage8_workspace_size(B, H, N, d)
    contig = [H * N * d, N * d, d] * 3
    nhd = [N * H * d, d, H * d] * 3
    prep = L.attn_k_smooth_quant_strided

    def p(st, fmt=0, dd=d, ws=FAKE, nb=need, q=FAKE, cu=None):
        arr = (ll * 9)(*st) if st is not None else None
        return prep(q, FAKE, FAKE, BF16, B, H, N, dd, arr, cu, fmt, ws, nb, None)

    assert p(None) == E_NULL
    assert p(contig, q=None) == E_NULL
    assert p(contig, fmt=3) == E_ARG
    assert p(contig, fmt=2, dd=80) == E_HEADDIM      # INT8 Q/K only: checked like the INT8 format
    assert p(contig, fmt=1, dd=80) == E_HEADDIM      # FP8 scores: d = 64, 96 or 128
    assert p(contig, nb=need - 1) == E_WS
    assert p(nhd[:2] + [d - 8] + nhd[3:]) == E_ARG    # token stride below d
    assert p(nhd[:1] + [d + 4] + nhd[2:]) == E_ALIGN  # not a multiple of 8 elements
    assert p([-8] + nhd[1:]) == E_ARG
    big = (1 << 31) // (N + 256) // 8 * 8 + 8          # (N + 256) rows no longer fit 32-bit byte offsets
    assert p(nhd[:5] + [big] + nhd[6:]) == E_SHAPE
    assert p(nhd, cu=FAKE + 2) == E_ALIGN             # cu_seqlens not 4-byte aligned
    fwd8 = L.attn_fwd_sage8_strided

    def f(st, fmt=0, dd=d, o=FAKE, cu=None, bias=None):
        arr = (ll * 3)(*st) if st is not None else None
        return fwd8(FAKE, o, None, B, H, N, dd, arr, cu, 0, 0.125, bias, BF16, fmt, None)

    assert f(None) == E_NULL
    assert f([N * H * d, d, H * d], o=None) == E_NULL
    assert f([N * H * d, d, H * d], fmt=5) == E_ARG
    assert f([N * H * d, d, H * d], fmt=2) == E_ARG  # a Q/K-only workspace has no FP8 V
    assert f([N * H * d, d, 8]) == E_ARG              # token stride below d
    assert f([N * H * d, d + 2, H * d]) == E_ALIGN
    assert f([N * H * d, d, H * d], fmt=1, dd=80) == E_HEADDIM
    assert f([0, d, H * d], cu=FAKE, bias=FAKE + 2) == E_ALIGN  # packed sequences: the bias is checked too
    assert f([0, d, H * d], cu=FAKE + 2) == E_ALIGN


def test_bias_size_bounds():
    """A block bias [B,H,nb,nb] is bounded: nb below 32768 (one head's gates
    addressed with 32-bit byte offsets) and B*H*nb*nb below 2^31 elements.
    Past either bound every entry point that takes a bias (or its gradient)
    returns ATTN_ERR_SHAPE instead of reading a wrapped descriptor."""
    L = attn.lib()
    n_max = 64 * 32767             # nb = 32767: the largest accepted
    n_over = n_max + 1             # nb = 32768: nb*nb*4 = 2^32
    for fn in (L.attn_fwd_bf16, L.attn_fwd_f16):
        assert _fwd(fn, bias=FAKE, N=n_over, d=64, out=BF16 if fn is L.attn_fwd_bf16 else F16) == E_SHAPE
        # at the bound the bias check passes and the next check (causal) fails
        assert _fwd(fn, bias=FAKE, N=n_max, d=64, causal=2,
                    out=BF16 if fn is L.attn_fwd_bf16 else F16) == E_ARG
        # 3 heads of 32767^2 gates exceed 2^31 elements
        assert _fwd(fn, bias=FAKE, H=3, N=n_max, d=64, out=BF16 if fn is L.attn_fwd_bf16 else F16) == E_SHAPE
        # without a bias the same shape is not limited by it
        assert _fwd(fn, N=n_over, d=64, causal=2, out=BF16 if fn is L.attn_fwd_bf16 else F16) == E_ARG
    good = [n_over * 64, n_over * 64, 64] * 4
    for name, dt in (("attn_fwd_strided_bf16", BF16), ("attn_fwd_strided_f16", F16)):
        fn = getattr(L, name)
        assert _strided(fn, good, N=n_over, bias=FAKE, out=dt) == E_SHAPE
        assert _strided(fn, good, N=n_max, bias=FAKE, causal=2, out=dt) == E_ARG
    for fwd8 in (L.attn_fwd_sage8, L.attn_fwd_sage8_fp8qk):
        assert fwd8(FAKE, FAKE, None, 1, 1, n_over, 64, 0, 0.1, FAKE, BF16, None) == E_SHAPE
        assert fwd8(FAKE, FAKE, None, 1, 1, n_max, 64, 2, 0.1, FAKE, BF16, None) == E_ARG
    for name in ("attn_bwd_bf16", "attn_bwd_f16"):
        fn = getattr(L, name)
        dt = BF16 if name.endswith("bf16") else F16
        assert _bwd(fn, dbias=FAKE, B=1, H=1, N=n_over, grad=dt, wsb=1 << 30) == E_SHAPE


def test_strided_tail_rows_must_be_addressable():
    """The 16-bit strided forward reads whole 64-row key blocks, up to 63
    rows past N: (N + 64) rows of the token stride must fit 32-bit byte
    offsets, not only N of them."""
    L = attn.lib()
    ts = 1 << 20                                   # token stride (elements)
    N = 2000                                       # N*ts*2 < 2^32 <= (N+64)*ts*2
    assert N * ts * 2 < (1 << 32) <= (N + 64) * ts * 2
    good = [0, 64, ts] * 4
    for name, dt in (("attn_fwd_strided_bf16", BF16), ("attn_fwd_strided_f16", F16)):
        assert _strided(getattr(L, name), good, N=N, out=dt) == E_SHAPE


def test_sage8_pv16_validation():
    """INT8 scores with the 16-bit P V product: workspace, V, dtypes and the
    common checks, all before any device call."""
    fn = attn.lib().attn_fwd_sage8_pv16

    def f(ws=FAKE, v=FAKE, vdt=BF16, o=FAKE, N=100, d=64, causal=0, scale=0.1, bias=None, out=BF16):
        return fn(ws, v, vdt, o, None, 1, 2, N, d, causal, scale, bias, out, None)

    assert f(ws=None) == E_WS
    assert f(v=None) == E_NULL
    assert f(o=None) == E_NULL
    assert f(d=80) == E_HEADDIM
    assert f(N=0) == E_SHAPE
    assert f(causal=2) == E_ARG
    assert f(scale=float("nan")) == E_ARG
    assert f(vdt=F32, out=F32) == E_DTYPE
    assert f(vdt=F16, out=BF16) == E_DTYPE
    assert f(out=9) == E_DTYPE
    assert f(ws=FAKE + 16) == E_ALIGN
    assert f(v=FAKE + 8) == E_ALIGN
    assert f(o=FAKE + 4) == E_ALIGN
    assert f(bias=FAKE, N=64 * 32768) == E_SHAPE
