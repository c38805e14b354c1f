"""Fused attention forward for AMD MI355X (gfx950): Python binding.

A thin ctypes layer over ``libattn.so`` (the C ABI of ``include/attn.h``).
It only marshals arguments: every step of the computation runs in the HIP
kernels.  PyTorch supplies device memory and the current stream.  There is
no fallback: if the library is missing or a call fails, an exception is
raised.

    fwd(q, k, v, causal=False, scale=None, bias=None, out_dtype=None,
        return_lse=False)                       # fp16 / bf16 path
    fwd_strided(q, k, v, ...)                   # same, any layout with d contiguous
    fwd_varlen(q, k, v, cu_seqlens, max_seqlen, ...)  # packed sequences
    prep = sage8_prep(q, k, v)                  # 8-bit preparation
    fwd_sage8(prep, causal=False, ...)          # 8-bit forward
    sageattn(q, k, v, causal=False, ...)        # both 8-bit steps
    fwd_sage8_pv16(prep, v, causal=False, ...)  # INT8 scores, 16-bit P V
    sageattn_pv16(q, k, v, causal=False, ...)   # both steps of that variant
    sageattn_varlen(q, k, v, cu_seqlens, max_seqlen, ...)  # 8-bit, packed sequences

Tensors are [B, H, N, d] contiguous CUDA (HIP) tensors, d in {64, 96, 128}
on every path (INT8 or FP8 scores alike).
``bias`` is fp32 [B, H, ceil(N/64), ceil(N/64)]: an additive logit per
64-query x 64-key block in natural-log units (packed sequences: N is the
longest length and sequence b takes bias[b] counted from its first token).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["fwd", "fwd_strided", "fwd_varlen", "bwd", "bwd_noalloc", "attention", "sage8_prep", "sage8_prep_varlen", "fwd_sage8",
           "fwd_sage8_pv16", "sageattn_pv16", "sageattn", "sageattn_varlen", "AttnError", "Sage8Prepared", "sage8_workspace_views", "lib", "LIB_PATH",
           "status_str"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

DTYPE_F16, DTYPE_BF16, DTYPE_F32 = 0, 1, 2
_DTYPE_CODE = {torch.float16: DTYPE_F16, torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({status_str(status)})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libattn.so with argument types set.  Raises if it has not
    been built (``python __graft_entry__.py`` or ``bit_attention_attn_amd/build.py``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run bit_attention_attn_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    fwd_args = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, i, vp]
    for name in ("attn_fwd_f16", "attn_fwd_bf16"):
        fn = getattr(L, name)
        fn.argtypes = fwd_args
        fn.restype = i
    ll_p = ctypes.POINTER(ctypes.c_longlong)
    for name in ("attn_fwd_strided_f16", "attn_fwd_strided_bf16"):
        fn = getattr(L, name)
        fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, ll_p, vp, i, f, vp, i, vp]
        fn.restype = i
    L.attn_bwd_workspace_size.argtypes = [i, i, i, i]
    L.attn_bwd_workspace_size.restype = sz
    for name in ("attn_bwd_f16", "attn_bwd_bf16"):
        fn = getattr(L, name)
        fn.argtypes = [vp, vp, vp, vp, i, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, i, vp, sz, vp]
        fn.restype = i
    L.attn_bwd_noalloc.argtypes = [i, vp, vp, vp, vp, i, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, i, vp]
    L.attn_bwd_noalloc.restype = i
    L.attn_sage8_workspace_size.argtypes = [i, i, i, i]
    L.attn_sage8_workspace_size.restype = sz
    L.attn_k_smooth_quant.argtypes = [vp, vp, vp, i, i, i, i, i, vp, sz, vp]
    L.attn_k_smooth_quant.restype = i
    L.attn_sage8_workspace_layout.argtypes = [i, i, i, i, ctypes.POINTER(sz), i]
    L.attn_sage8_workspace_layout.restype = i
    L.attn_fwd_sage8.argtypes = [vp, vp, vp, i, i, i, i, i, f, vp, i, vp]
    L.attn_fwd_sage8.restype = i
    L.attn_k_smooth_quant_fp8qk.argtypes = L.attn_k_smooth_quant.argtypes
    L.attn_k_smooth_quant_fp8qk.restype = i
    L.attn_fwd_sage8_fp8qk.argtypes = L.attn_fwd_sage8.argtypes
    L.attn_fwd_sage8_fp8qk.restype = i
    L.attn_fwd_sage8_pv16.argtypes = [vp, vp, i, vp, vp, i, i, i, i, i, f, vp, i, vp]
    L.attn_fwd_sage8_pv16.restype = i
    L.attn_k_smooth_quant_strided.argtypes = [vp, vp, vp, i, i, i, i, i, ll_p, vp, i, vp, sz, vp]
    L.attn_k_smooth_quant_strided.restype = i
    L.attn_fwd_sage8_strided.argtypes = [vp, vp, vp, i, i, i, i, ll_p, vp, i, f, vp, i, i, vp]
    L.attn_fwd_sage8_strided.restype = i
    L.attn_status_str.argtypes = [i]
    L.attn_status_str.restype = ctypes.c_char_p
    L.attn_abi_version.argtypes = []
    L.attn_abi_version.restype = i
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().attn_status_str(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_qkv(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA (HIP) tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B,H,N,d] tensor")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    if k.dtype != q.dtype or v.dtype != q.dtype or q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q, k, v must share one dtype: float16 or bfloat16")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")


def _check_bias(bias, B, H, N, device):
    if bias is None:
        return None
    nb = (N + 63) // 64
    if (bias.dtype != torch.float32 or tuple(bias.shape) != (B, H, nb, nb)
            or not bias.is_contiguous() or bias.device != device):
        raise ValueError(f"bias must be a contiguous fp32 [B,H,{nb},{nb}] tensor on {device}")
    return bias


def fwd(q, k, v, causal=False, scale=None, bias=None, out_dtype=None, return_lse=False):
    """Fused attention forward on fp16/bf16 inputs.  Returns O (and LSE in
    natural-log units, fp32 [B,H,N], when return_lse)."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    bias = _check_bias(bias, B, H, N, q.device)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    fn = lib().attn_fwd_bf16 if q.dtype == torch.bfloat16 else lib().attn_fwd_f16
    with torch.cuda.device(q.device):
        st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)),
                float(scale), _ptr(bias), _DTYPE_CODE.get(out_dtype, -1), _stream(q.device))
    if st != 0:
        raise AttnError(st, fn.__name__)
    return (o, lse) if return_lse else o


def bwd(q, k, v, o, dout, lse, causal=False, scale=None, bias=None, grad_dtype=None, return_dbias=False):
    """Gradients of the fused forward: given the forward's inputs, its output
    o (q's dtype, or float32 for an exact row statistic D) and LSE, and
    dout = dL/dO, returns (dq, dk, dv), plus the fp32 gradient of the
    [B,H,nb,nb] block bias when return_dbias.  d must be 64, 96 or 128."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    for name, t, dts in (("o", o, (q.dtype, torch.float32)), ("dout", dout, (q.dtype,))):
        if not isinstance(t, torch.Tensor) or t.shape != q.shape or t.dtype not in dts or t.device != q.device \
                or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor like q")
    if not isinstance(lse, torch.Tensor) or lse.shape != (B, H, N) or lse.dtype != torch.float32 \
            or lse.device != q.device or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,H,N] tensor on q's device")
    bias = _check_bias(bias, B, H, N, q.device)
    grad_dtype = q.dtype if grad_dtype is None else grad_dtype
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = (torch.empty((B, H, N, d), dtype=grad_dtype, device=q.device) for _ in range(3))
    nb = (N + 63) // 64
    dbias = torch.empty((B, H, nb, nb), dtype=torch.float32, device=q.device) if return_dbias else None
    wsb = lib().attn_bwd_workspace_size(B, H, N, d)
    ws = torch.empty((max(wsb, 256),), dtype=torch.uint8, device=q.device)
    fn = lib().attn_bwd_bf16 if q.dtype == torch.bfloat16 else lib().attn_bwd_f16
    with torch.cuda.device(q.device):
        st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _DTYPE_CODE[o.dtype], _ptr(dout), _ptr(lse), _ptr(dq),
                _ptr(dk), _ptr(dv),
                _ptr(dbias), B, H, N, d, int(bool(causal)), float(scale), _ptr(bias),
                _DTYPE_CODE.get(grad_dtype, -1), _ptr(ws), ws.numel(), _stream(q.device))
    if st != 0:
        raise AttnError(st, fn.__name__)
    return (dq, dk, dv, dbias) if return_dbias else (dq, dk, dv)


def bwd_noalloc(q, k, v, o, dout, lse, causal=False, scale=None, bias=None, grad_dtype=None, return_dbias=False):
    """bwd() through attn_bwd_noalloc: the library takes its scratch from a
    fixed device array instead of a workspace (for callers that cannot
    allocate device memory; B*H*N at most ATTN_BWD_NOALLOC_MAX_ROWS, calls
    on one GPU must not overlap).  The outputs are allocated here, as in
    bwd(); the results are bwd()'s bit for bit."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    for name, t, dts in (("o", o, (q.dtype, torch.float32)), ("dout", dout, (q.dtype,))):
        if not isinstance(t, torch.Tensor) or t.shape != q.shape or t.dtype not in dts or t.device != q.device \
                or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor like q")
    if not isinstance(lse, torch.Tensor) or lse.shape != (B, H, N) or lse.dtype != torch.float32 \
            or lse.device != q.device or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,H,N] tensor on q's device")
    bias = _check_bias(bias, B, H, N, q.device)
    grad_dtype = q.dtype if grad_dtype is None else grad_dtype
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = (torch.empty((B, H, N, d), dtype=grad_dtype, device=q.device) for _ in range(3))
    nb = (N + 63) // 64
    dbias = torch.empty((B, H, nb, nb), dtype=torch.float32, device=q.device) if return_dbias else None
    fn = lib().attn_bwd_noalloc
    with torch.cuda.device(q.device):
        st = fn(_DTYPE_CODE[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(o), _DTYPE_CODE[o.dtype], _ptr(dout), _ptr(lse),
                _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias), B, H, N, d, int(bool(causal)), float(scale), _ptr(bias),
                _DTYPE_CODE.get(grad_dtype, -1), _stream(q.device))
    if st != 0:
        raise AttnError(st, fn.__name__)
    return (dq, dk, dv, dbias) if return_dbias else (dq, dk, dv)


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, bias, causal, scale):
        o, lse = fwd(q, k, v, causal=causal, scale=scale, bias=bias, return_lse=True)
        ctx.save_for_backward(q, k, v, o, lse, bias)
        ctx.causal, ctx.scale = causal, scale
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, o, lse, bias = ctx.saved_tensors
        need_db = bias is not None and ctx.needs_input_grad[3]
        g = bwd(q, k, v, o, dout.contiguous(), lse, causal=ctx.causal, scale=ctx.scale, bias=bias,
                return_dbias=need_db)
        return g[0], g[1], g[2], (g[3] if need_db else None), None, None


def attention(q, k, v, causal=False, scale=None, bias=None):
    """Differentiable fused attention (fp16/bf16, d = 64, 96 or 128): the forward
    kernel, and the backward kernels for torch.autograd (gradients for q, k,
    v and the block bias)."""
    return _Attention.apply(q, k, v, bias, bool(causal), scale)


def _strided_call(q, k, v, o, lse, B, H, N, d, strides, cu, causal, scale, out_dtype, bias=None):
    fn = lib().attn_fwd_strided_bf16 if q.dtype == torch.bfloat16 else lib().attn_fwd_strided_f16
    arr = (ctypes.c_longlong * 12)(*[int(x) for x in strides])
    with torch.cuda.device(q.device):
        st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, arr, _ptr(cu), int(bool(causal)),
                float(scale), _ptr(bias), _DTYPE_CODE.get(out_dtype, -1), _stream(q.device))
    if st != 0:
        raise AttnError(st, fn.__name__)


def _check_views(ts, ndim):
    for name, t in zip(("q", "k", "v"), ts):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dim() != ndim or t.stride(-1) != 1:
            raise ValueError(f"{name} must be a {ndim}-D CUDA (HIP) tensor with the last dimension contiguous")
    q = ts[0]
    if any(t.dtype != q.dtype for t in ts) or q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q, k, v must share one dtype: float16 or bfloat16")
    if any(t.device != q.device for t in ts):
        raise ValueError("q, k, v must be on one device")


def fwd_strided(q, k, v, causal=False, scale=None, out_dtype=None, return_lse=False, bias=None):
    """Fused attention forward on logical [B,H,N,d] tensors of any layout
    with d contiguous (e.g. x.transpose(1, 2) of a [B,N,H,d] tensor, or
    views of a fused QKV projection).  O has q's layout (empty_like); LSE is
    [B,H,N] fp32; bias as for fwd ([B,H,nb,nb] fp32)."""
    _check_views((q, k, v), 4)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same logical shape")
    B, H, N, d = q.shape
    bias = _check_bias(bias, B, H, N, q.device)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q, dtype=out_dtype)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    strides = []
    for t in (q, k, v, o):
        strides += [t.stride(0), t.stride(1), t.stride(2)]
    _strided_call(q, k, v, o, lse, B, H, N, d, strides, None, causal, scale, out_dtype, bias)
    return (o, lse) if return_lse else o


def _check_cu(cu_seqlens, device, max_seqlen=None, total=None):
    """Packed-sequence offsets: a contiguous int32 [B+1] tensor on the device.
    With max_seqlen and total, also the contract the kernels rely on (they
    clamp a longer sequence to max_seqlen and would leave the rest of its
    rows unwritten): offsets non-decreasing from 0 up to at most total,
    every length at most max_seqlen.  This reads the B+1 offsets back to the
    host (one small synchronous copy), which a stream being recorded into a
    graph cannot do: under capture the offsets are not read and the caller
    keeps that contract."""
    if (not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
            or cu_seqlens.device != device or not cu_seqlens.is_contiguous() or cu_seqlens.numel() < 2):
        raise ValueError("cu_seqlens must be a contiguous int32 [B+1] tensor on q's device")
    if max_seqlen is None:
        return
    if int(max_seqlen) < 1:
        raise ValueError("max_seqlen must be >= 1")
    if torch.cuda.is_current_stream_capturing():
        return
    cu = cu_seqlens.cpu()
    lens = cu[1:] - cu[:-1]
    if int(cu[0]) < 0 or bool((lens < 0).any()) or int(cu[-1]) > total:
        raise ValueError("cu_seqlens must be non-decreasing offsets into the packed token axis")
    if int(lens.max()) > int(max_seqlen):
        raise ValueError(f"a sequence is longer than max_seqlen ({int(lens.max())} > {int(max_seqlen)})")


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, scale=None, out_dtype=None, return_lse=False,
               bias=None):
    """Fused attention forward on packed sequences: q, k, v [total,H,d] (d
    contiguous), cu_seqlens int32 [B+1] on the device (sequence b is tokens
    cu_seqlens[b] .. cu_seqlens[b+1]-1, attending only within itself),
    max_seqlen the longest length.  O is [total,H,d] like q; LSE is
    [B,H,max_seqlen] fp32.  bias: [B,H,nb,nb] fp32 with nb =
    ceil(max_seqlen/64); sequence b takes bias[b,h,i,j] for its query block i
    and key block j, counted from its own first token."""
    _check_views((q, k, v), 3)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    total, H, d = q.shape
    _check_cu(cu_seqlens, q.device, max_seqlen, total)
    B = cu_seqlens.numel() - 1
    bias = _check_bias(bias, B, H, int(max_seqlen), q.device)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q, dtype=out_dtype)
    lse = torch.empty((B, H, max_seqlen), dtype=torch.float32, device=q.device) if return_lse else None
    strides = []
    for t in (q, k, v, o):
        strides += [0, t.stride(1), t.stride(0)]
    _strided_call(q, k, v, o, lse, B, H, int(max_seqlen), d, strides, cu_seqlens, causal, scale, out_dtype, bias)
    return (o, lse) if return_lse else o


class Sage8Prepared:
    """Workspace written by the 8-bit preparation, with the shape it was
    prepared for (the forward must use the same shape)."""

    def __init__(self, workspace, shape, in_dtype, qk="int8", cu_seqlens=None, total=None):
        self.workspace = workspace
        self.shape = tuple(shape)
        self.in_dtype = in_dtype
        self.qk = qk  # "int8", "fp8" (the FP8-QK variant) or "int8_no_v" (no V prepared)
        # packed sequences: the int32 [B+1] offsets and the packed token count
        self.cu_seqlens = cu_seqlens
        self.total = total


# "int8_no_v": the INT8 Q and K only (for fwd_sage8_pv16, which reads no FP8 V)
_QK_FORMAT = {"int8": 0, "fp8": 1, "int8_no_v": 2}


def sage8_prep(q, k, v, workspace=None, qk="int8"):
    """K smoothing and 8-bit quantisation of Q, K, V into a device workspace.
    q, k, v are logical [B,H,N,d] tensors, contiguous or any layout with d
    contiguous (e.g. x.transpose(1, 2) of a token-major [B,N,H,d] tensor).
    qk="fp8" quantises Q and K to e4m3 blocks (the FP8-QK variant, any of
    d = 64, 96, 128) instead of INT8; fwd_sage8 then uses FP8 scores.  qk="int8_no_v"
    prepares the INT8 Q and K only (the same codes), for fwd_sage8_pv16."""
    if qk not in _QK_FORMAT:
        raise ValueError('qk must be "int8", "fp8" or "int8_no_v"')
    contiguous = qk != "int8_no_v" and all(isinstance(t, torch.Tensor) and t.is_contiguous() for t in (q, k, v))
    if contiguous:
        _check_qkv(q, k, v)
    else:
        _check_views((q, k, v), 4)
        if k.shape != q.shape or v.shape != q.shape:
            raise ValueError("q, k, v must have the same logical shape")
    B, H, N, d = q.shape
    L = lib()
    need = L.attn_sage8_workspace_size(B, H, N, d)
    if need == 0:
        raise AttnError(2, "attn_sage8_workspace_size")
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        if contiguous:
            fn = L.attn_k_smooth_quant_fp8qk if qk == "fp8" else L.attn_k_smooth_quant
            st = fn(_ptr(q), _ptr(k), _ptr(v), _DTYPE_CODE[q.dtype], B, H, N, d,
                    _ptr(workspace), workspace.numel(), _stream(q.device))
        else:
            fn = L.attn_k_smooth_quant_strided
            arr = (ctypes.c_longlong * 9)(*[int(t.stride(i)) for t in (q, k, v) for i in range(3)])
            st = fn(_ptr(q), _ptr(k), _ptr(v), _DTYPE_CODE[q.dtype], B, H, N, d, arr, None, _QK_FORMAT[qk],
                    _ptr(workspace), workspace.numel(), _stream(q.device))
    if st != 0:
        raise AttnError(st, fn.__name__)
    return Sage8Prepared(workspace, (B, H, N, d), q.dtype, qk)


def sage8_prep_varlen(q, k, v, cu_seqlens, max_seqlen, workspace=None, qk="int8"):
    """8-bit preparation of packed sequences: q, k, v [total,H,d] (d
    contiguous), cu_seqlens int32 [B+1] on the device (sequence b is tokens
    cu_seqlens[b] .. cu_seqlens[b+1]-1), max_seqlen the longest length.  Each
    sequence is prepared on its own (its K mean, V scales and 64-row blocks),
    into slot b of a [B,H,max_seqlen,d] workspace."""
    if qk not in ("int8", "fp8"):
        raise ValueError('qk must be "int8" or "fp8"')
    _check_views((q, k, v), 3)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    total, H, d = q.shape
    _check_cu(cu_seqlens, q.device, max_seqlen, total)
    B, N = cu_seqlens.numel() - 1, int(max_seqlen)
    L = lib()
    need = L.attn_sage8_workspace_size(B, H, N, d)
    if need == 0:
        raise AttnError(2, "attn_sage8_workspace_size")
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    fn = L.attn_k_smooth_quant_strided
    arr = (ctypes.c_longlong * 9)(*[x for t in (q, k, v) for x in (0, int(t.stride(1)), int(t.stride(0)))])
    with torch.cuda.device(q.device):
        st = fn(_ptr(q), _ptr(k), _ptr(v), _DTYPE_CODE[q.dtype], B, H, N, d, arr, _ptr(cu_seqlens), _QK_FORMAT[qk],
                _ptr(workspace), workspace.numel(), _stream(q.device))
    if st != 0:
        raise AttnError(st, fn.__name__)
    return Sage8Prepared(workspace, (B, H, N, d), q.dtype, qk, cu_seqlens=cu_seqlens, total=total)


def fwd_sage8(prep: Sage8Prepared, causal=False, scale=None, bias=None, out_dtype=None,
              return_lse=False, layout_like=None):
    """8-bit fused forward from a prepared workspace.  O is contiguous
    [B,H,N,d], or has the layout of the logical [B,H,N,d] tensor layout_like
    (torch.empty_like, so a token-major view gives a token-major O).  After
    sage8_prep_varlen, O is packed [total,H,d] and the LSE [B,H,max_seqlen];
    a bias [B,H,nb,nb] then gives sequence b the blocks bias[b,h,i,j]
    counted from its own first token."""
    B, H, N, d = prep.shape
    dev = prep.workspace.device
    packed = prep.cu_seqlens is not None
    if packed and layout_like is not None:
        raise ValueError("packed sequences take no layout_like")
    if prep.qk == "int8_no_v":
        raise ValueError("this preparation holds no FP8 V: use fwd_sage8_pv16")
    bias = _check_bias(bias, B, H, N, dev)
    out_dtype = prep.in_dtype if out_dtype is None else out_dtype
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if packed:
        o = torch.empty((prep.total, H, d), dtype=out_dtype, device=dev)
    elif layout_like is not None:
        if tuple(layout_like.shape) != (B, H, N, d):
            raise ValueError("layout_like must have the prepared [B,H,N,d] shape")
        o = torch.empty_like(layout_like, dtype=out_dtype, device=dev)
    else:
        o = torch.empty((B, H, N, d), dtype=out_dtype, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if return_lse else None
    with torch.cuda.device(dev):
        if o.is_contiguous() and not packed:
            fn = lib().attn_fwd_sage8_fp8qk if prep.qk == "fp8" else lib().attn_fwd_sage8
            st = fn(_ptr(prep.workspace), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)), float(scale),
                    _ptr(bias), _DTYPE_CODE.get(out_dtype, -1), _stream(dev))
        else:
            fn = lib().attn_fwd_sage8_strided
            ost = (0, o.stride(1), o.stride(0)) if packed else (o.stride(0), o.stride(1), o.stride(2))
            arr = (ctypes.c_longlong * 3)(*[int(x) for x in ost])
            st = fn(_ptr(prep.workspace), _ptr(o), _ptr(lse), B, H, N, d, arr, _ptr(prep.cu_seqlens),
                    int(bool(causal)), float(scale), _ptr(bias), _DTYPE_CODE.get(out_dtype, -1),
                    _QK_FORMAT[prep.qk], _stream(dev))
    if st != 0:
        raise AttnError(st, fn.__name__)
    return (o, lse) if return_lse else o


def sageattn(q, k, v, causal=False, scale=None, bias=None, out_dtype=None, return_lse=False, qk="int8",
             tensor_layout="HND"):
    """8-bit attention in one call (preparation, then the forward).
    tensor_layout "HND": q, k, v are [B,H,N,d]; "NHD": they are token-major
    [B,N,H,d] and O comes back token-major.  Either may be a strided view
    with d contiguous."""
    if tensor_layout not in ("HND", "NHD"):
        raise ValueError('tensor_layout must be "HND" or "NHD"')
    if tensor_layout == "NHD":
        q, k, v = (t.transpose(1, 2) for t in (q, k, v))
    prep = sage8_prep(q, k, v, qk=qk)
    res = fwd_sage8(prep, causal=causal, scale=scale, bias=bias, out_dtype=out_dtype,
                    return_lse=return_lse, layout_like=q)
    if tensor_layout == "NHD":
        return (res[0].transpose(1, 2), res[1]) if return_lse else res.transpose(1, 2)
    return res


def fwd_sage8_pv16(prep: Sage8Prepared, v, causal=False, scale=None, bias=None, out_dtype=None,
                   return_lse=False):
    """8-bit forward with INT8 scores from the prepared workspace (INT8
    format, contiguous preparation) and the 16-bit P V product with v, the
    contiguous [B,H,N,d] V that was prepared.  O is contiguous [B,H,N,d]."""
    B, H, N, d = prep.shape
    dev = prep.workspace.device
    if prep.qk not in ("int8", "int8_no_v") or prep.cu_seqlens is not None:
        raise ValueError("the 16-bit P V variant takes an INT8 preparation of unpacked sequences")
    if (not isinstance(v, torch.Tensor) or tuple(v.shape) != (B, H, N, d) or not v.is_contiguous()
            or v.dtype != prep.in_dtype or v.device != dev):
        raise ValueError("v must be the contiguous [B,H,N,d] V of the preparation, in its dtype")
    bias = _check_bias(bias, B, H, N, dev)
    out_dtype = prep.in_dtype if out_dtype is None else out_dtype
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, H, N, d), dtype=out_dtype, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if return_lse else None
    fn = lib().attn_fwd_sage8_pv16
    with torch.cuda.device(dev):
        st = fn(_ptr(prep.workspace), _ptr(v), _DTYPE_CODE[v.dtype], _ptr(o), _ptr(lse), B, H, N, d,
                int(bool(causal)), float(scale), _ptr(bias), _DTYPE_CODE.get(out_dtype, -1), _stream(dev))
    if st != 0:
        raise AttnError(st, fn.__name__)
    return (o, lse) if return_lse else o


def sageattn_pv16(q, k, v, causal=False, scale=None, bias=None, out_dtype=None, return_lse=False):
    """INT8 scores with the 16-bit P V product in one call: the 8-bit
    preparation of contiguous [B,H,N,d] q, k, v, then fwd_sage8_pv16."""
    _check_qkv(q, k, v)
    prep = sage8_prep(q, k, v, qk="int8_no_v")
    return fwd_sage8_pv16(prep, v, causal=causal, scale=scale, bias=bias, out_dtype=out_dtype,
                          return_lse=return_lse)


def sageattn_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, scale=None, out_dtype=None, return_lse=False,
                    qk="int8", bias=None):
    """8-bit attention on packed sequences in one call: q, k, v [total,H,d],
    cu_seqlens int32 [B+1] on the device, max_seqlen the longest length.  O
    is [total,H,d]; each sequence attends only within itself; bias as for
    fwd_varlen."""
    prep = sage8_prep_varlen(q, k, v, cu_seqlens, max_seqlen, qk=qk)
    return fwd_sage8(prep, causal=causal, scale=scale, bias=bias, out_dtype=out_dtype, return_lse=return_lse)


def sage8_workspace_views(prep: Sage8Prepared) -> dict:
    """Views of the prepared data inside the workspace (for inspection and
    tests): qq, kq int8 [B,H,Np,d]; sq, sk fp32 [B,H,nblk]; sv, kmean fp32
    [B,H,d]; vq uint8 e4m3 codes in the library's layout [B,H,nblk,d,64];
    vq_logical uint8 [B,H,Np,d] (the same codes in token order)."""
    B, H, N, d = prep.shape
    vals = (ctypes.c_size_t * 9)()
    if lib().attn_sage8_workspace_layout(B, H, N, d, vals, 9) != 9:
        raise AttnError(2, "attn_sage8_workspace_layout")
    off_qq, off_kq, off_vq, off_sq, off_sk, off_sv, off_km, np_, nblk = (int(x) for x in vals)
    ws = prep.workspace

    def region(off, count, dtype):
        nbytes = count * torch.tensor([], dtype=dtype).element_size()
        return ws[off:off + nbytes].view(dtype)

    out = dict(
        qq=region(off_qq, B * H * np_ * d, torch.int8).view(B, H, np_, d),
        kq=region(off_kq, B * H * np_ * d, torch.int8).view(B, H, np_, d),
        vq=region(off_vq, B * H * np_ * d, torch.uint8).view(B, H, nblk, d, 64),
        sq=region(off_sq, B * H * nblk, torch.float32).view(B, H, nblk),
        sk=region(off_sk, B * H * nblk, torch.float32).view(B, H, nblk),
        sv=region(off_sv, B * H * d, torch.float32).view(B, H, d),
        kmean=region(off_km, B * H * d, torch.float32).view(B, H, d),
    )
    # byte 32h + 16T + 4g + u of a row holds key 32T + 8g + 4h + u of the block
    pos = torch.empty(64, dtype=torch.long)
    for key in range(64):
        T, kin = key // 32, key % 32
        h, g, u = (kin // 4) % 2, kin // 8, kin % 4
        pos[key] = 32 * h + 16 * T + 4 * g + u
    vq = out["vq"][..., pos.to(ws.device)]                      # [B,H,nblk,d,64 keys]
    out["vq_logical"] = vq.permute(0, 1, 2, 4, 3).reshape(B, H, np_, d)
    return out
