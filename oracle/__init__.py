"""CPU oracle for the fused attention forward and its 8-bit variant.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  It is plain C (``attn_oracle.c``, ``sage8_oracle.c``) compiled with
gcc and driven through ctypes with numpy arrays; it shares no code with the
GPU library and never imports it.

Functions (each cites what it follows in the C source):

* ``attn_rows``      -- fp64 three-loop softmax(scale*Q K^T + bias) V for a
                        list of rows (page 4, "FlashAttention (TR)", the
                        attention formula of the section on standard
                        attention; bias: page 5, "SAS", log-form gate).
* ``row_probs``      -- the probability row P of one query (same passage).
* ``attn_bwd``       -- fp64 gradients dQ, dK, dV and of the block bias for
                        a given dO (page 3, "FlashAttention", glossary: the
                        backward pass recomputes instead of storing; page 5,
                        "SAS": the gate's gradient through the softmax).
* ``sage8_kmean``, ``sage8_quant_int8``, ``sage8_quant_v`` -- the 8-bit
                        preparation steps (page 1, "SageAttention",
                        "claim vs reality": K smoothing, INT8 Q/K, FP8).
* ``sage8_emulate_rows`` -- the blocked 8-bit forward modelled in fp64
                        (same passage: FP8 P, two-level accumulation).
* ``sage8_emulate_rows_fp32`` -- the same with the GPU kernel's fp32
                        decisions (lazy running maximum, P scale), for a
                        tight comparison with the GPU.
* ``sage8_qk8_rows`` -- INT8 scores (dequantised with the block scales) and
                        the exact softmax(.)V with the 16-bit V, in fp64: the
                        variant that quantises only the first product (same
                        passage of page 1).
* ``e4m3_encode``, ``e4m3_decode`` -- OCP FP8 E4M3 from its definition.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ATTN_ORACLE_LIB: another build of the same sources (the tests' sanitizer build)
_LIB_PATH = os.environ.get("ATTN_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_dbl = ctypes.c_double
_int = ctypes.c_int
_ptr = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.attn_oracle_rows.argtypes = [_ptr, _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64,
                                     _int, _dbl, _ptr, _i64, _ptr, _ptr, _int]
    lib.attn_oracle_rows.restype = _int
    lib.attn_oracle_row_probs.argtypes = [_ptr, _ptr, _ptr, _i64, _i64, _i64, _i64,
                                          _int, _dbl, _i64, _i64, _i64, _ptr]
    lib.attn_oracle_row_probs.restype = _int
    lib.attn_oracle_bwd.argtypes = [_ptr, _ptr, _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64,
                                    _int, _dbl, _ptr, _ptr, _ptr, _ptr, _int]
    lib.attn_oracle_bwd.restype = _int
    lib.attn_oracle_max_threads.argtypes = []
    lib.attn_oracle_max_threads.restype = _int
    lib.sage8_e4m3_encode.argtypes = [_dbl]
    lib.sage8_e4m3_encode.restype = ctypes.c_uint8
    lib.sage8_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.sage8_e4m3_decode.restype = _dbl
    lib.sage8_oracle_kmean.argtypes = [_ptr, _i64, _i64, _i64, _i64, _ptr]
    lib.sage8_oracle_kmean.restype = _int
    lib.sage8_oracle_quant_int8.argtypes = [_ptr, _ptr, _i64, _i64, _i64, _i64, _ptr, _ptr]
    lib.sage8_oracle_quant_int8.restype = _int
    lib.sage8_oracle_quant_fp8.argtypes = [_ptr, _ptr, _i64, _i64, _i64, _i64, _ptr, _ptr]
    lib.sage8_oracle_quant_fp8.restype = _int
    lib.sage8_oracle_quant_v.argtypes = [_ptr, _i64, _i64, _i64, _i64, _ptr, _ptr]
    lib.sage8_oracle_quant_v.restype = _int
    lib.sage8_oracle_emulate_rows.argtypes = [_ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr,
                                              _i64, _i64, _i64, _i64, _int, _dbl, _i64,
                                              _int, _ptr, _i64, _ptr, _ptr, _int, _int]
    lib.sage8_oracle_emulate_rows.restype = _int
    lib.sage8_oracle_emulate_rows_fp32.argtypes = [_ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr,
                                                   _i64, _i64, _i64, _i64, _int, ctypes.c_float,
                                                   _ptr, _i64, _ptr, _ptr, _int, _int]
    lib.sage8_oracle_emulate_rows_fp32.restype = _int
    lib.sage8_oracle_qk8_rows.argtypes = [_ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr,
                                          _i64, _i64, _i64, _i64, _int, _dbl,
                                          _ptr, _i64, _ptr, _ptr, _int]
    lib.sage8_oracle_qk8_rows.restype = _int
    _lib = lib
    return lib


def _f32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _rows(rows):
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    return r


def max_threads() -> int:
    return int(_load().attn_oracle_max_threads())


def attn_rows(q, k, v, rows, causal=False, scale=None, bias=None, nthreads=0):
    """fp64 attention for rows [(b,h,i), ...]; q,k,v are [B,H,N,d] arrays whose
    values are the rounded inputs (any float dtype; converted exactly to fp32).
    Returns (O [nrows,d] fp64, LSE [nrows] fp64, natural log)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, N, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nb = (N + 63) // 64
    if bias is not None:
        bias = _f32(bias)
        assert bias.shape == (B, H, nb, nb), bias.shape
    r = _rows(rows)
    out = np.zeros((r.shape[0], d), dtype=np.float64)
    lse = np.zeros((r.shape[0],), dtype=np.float64)
    rc = _load().attn_oracle_rows(_p(q), _p(k), _p(v), _p(bias), B, H, N, d, int(bool(causal)),
                                  float(scale), _p(r), r.shape[0], _p(out), _p(lse), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"attn_oracle_rows failed with code {rc}")
    return out, lse


def attn_full(q, k, v, causal=False, scale=None, bias=None, nthreads=0):
    """All rows: returns (O [B,H,N,d], LSE [B,H,N]) in fp64."""
    B, H, N, d = np.asarray(q).shape
    bb, hh, ii = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
    rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
    o, l = attn_rows(q, k, v, rows, causal=causal, scale=scale, bias=bias, nthreads=nthreads)
    return o.reshape(B, H, N, d), l.reshape(B, H, N)


def attn_bwd(q, k, v, dout, causal=False, scale=None, bias=None, nthreads=0):
    """fp64 gradients of sum(dout * O) for O = attention(q, k, v): returns
    (dq, dk, dv [B,H,N,d], dbias [B,H,nb,nb] or None when bias is None).
    All forward quantities are recomputed from the inputs."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, H, N, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape and dout.shape == q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nb = (N + 63) // 64
    if bias is not None:
        bias = _f32(bias)
        assert bias.shape == (B, H, nb, nb), bias.shape
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(q.shape, dtype=np.float64)
    dv = np.zeros(q.shape, dtype=np.float64)
    db = np.zeros((B, H, nb, nb), dtype=np.float64) if bias is not None else None
    rc = _load().attn_oracle_bwd(_p(q), _p(k), _p(v), _p(dout), _p(bias), B, H, N, d, int(bool(causal)),
                                 float(scale), _p(dq), _p(dk), _p(dv), _p(db), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"attn_oracle_bwd failed with code {rc}")
    return dq, dk, dv, db


def row_probs(q, k, b, h, i, causal=False, scale=None, bias=None):
    """The probability row P[b,h,i,:] (zeros where masked), fp64."""
    q, k = _f32(q), _f32(k)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if bias is not None:
        bias = _f32(bias)
    p = np.zeros((N,), dtype=np.float64)
    rc = _load().attn_oracle_row_probs(_p(q), _p(k), _p(bias), B, H, N, d, int(bool(causal)),
                                       float(scale), int(b), int(h), int(i), _p(p))
    if rc != 0:
        raise RuntimeError(f"attn_oracle_row_probs failed with code {rc}")
    return p


def e4m3_encode(x) -> np.ndarray:
    lib = _load()
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    flat, oflat = x.ravel(), out.ravel()
    for n in range(flat.size):
        oflat[n] = lib.sage8_e4m3_encode(float(flat[n]))
    return out


def e4m3_decode(c) -> np.ndarray:
    lib = _load()
    c = np.asarray(c, dtype=np.uint8)
    table = np.array([lib.sage8_e4m3_decode(i) for i in range(256)], dtype=np.float64)
    return table[c]


def sage8_kmean(k):
    k = _f32(k)
    B, H, N, d = k.shape
    out = np.zeros((B, H, d), dtype=np.float32)
    rc = _load().sage8_oracle_kmean(_p(k), B, H, N, d, _p(out))
    if rc != 0:
        raise RuntimeError(f"sage8_oracle_kmean failed with code {rc}")
    return out


def sage8_quant_int8(x, center=None):
    """Per-64-row-block INT8: returns (codes int8 [B,H,N,d], scales f32 [B,H,nb])."""
    x = _f32(x)
    B, H, N, d = x.shape
    if center is not None:
        center = _f32(center)
        assert center.shape == (B, H, d)
    nb = (N + 63) // 64
    codes = np.zeros((B, H, N, d), dtype=np.int8)
    scales = np.zeros((B, H, nb), dtype=np.float32)
    rc = _load().sage8_oracle_quant_int8(_p(x), _p(center), B, H, N, d, _p(codes), _p(scales))
    if rc != 0:
        raise RuntimeError(f"sage8_oracle_quant_int8 failed with code {rc}")
    return codes, scales


def sage8_quant_fp8(x, center=None):
    """Per-64-row-block e4m3 (the FP8-QK variant): returns (codes uint8
    [B,H,N,d], scales f32 [B,H,nb])."""
    x = _f32(x)
    B, H, N, d = x.shape
    if center is not None:
        center = _f32(center)
        assert center.shape == (B, H, d)
    nb = (N + 63) // 64
    codes = np.zeros((B, H, N, d), dtype=np.uint8)
    scales = np.zeros((B, H, nb), dtype=np.float32)
    rc = _load().sage8_oracle_quant_fp8(_p(x), _p(center), B, H, N, d, _p(codes), _p(scales))
    if rc != 0:
        raise RuntimeError(f"sage8_oracle_quant_fp8 failed with code {rc}")
    return codes, scales


def sage8_quant_v(v):
    """Per-channel e4m3: returns (codes uint8 [B,H,N,d], scales f32 [B,H,d])."""
    v = _f32(v)
    B, H, N, d = v.shape
    codes = np.zeros((B, H, N, d), dtype=np.uint8)
    scales = np.zeros((B, H, d), dtype=np.float32)
    rc = _load().sage8_oracle_quant_v(_p(v), B, H, N, d, _p(codes), _p(scales))
    if rc != 0:
        raise RuntimeError(f"sage8_oracle_quant_v failed with code {rc}")
    return codes, scales


def sage8_prepare(q, k, v, qk="int8"):
    """All three preparation steps; returns a dict of the quantised data.
    qk = "fp8" quantises Q and smoothed K to e4m3 blocks instead of INT8."""
    kmean = sage8_kmean(k)
    quant = sage8_quant_fp8 if qk == "fp8" else sage8_quant_int8
    qq, sq = quant(q)
    kq, sk = quant(k, kmean)
    vq, sv = sage8_quant_v(v)
    return dict(kmean=kmean, qq=qq, sq=sq, kq=kq, sk=sk, vq=vq, sv=sv, qk_fp8=qk == "fp8")


def sage8_emulate_rows(prep, rows, causal=False, scale=None, bias=None, kv_block=64,
                       p_mode=1, nthreads=0):
    """Blocked 8-bit forward on rows from the quantised data of sage8_prepare.
    Returns (O [nrows,d], LSE [nrows]) in fp64."""
    fp8 = bool(prep.get("qk_fp8", False))
    qq = np.ascontiguousarray(prep["qq"], dtype=np.uint8 if fp8 else np.int8)
    kq = np.ascontiguousarray(prep["kq"], dtype=np.uint8 if fp8 else np.int8)
    vq = np.ascontiguousarray(prep["vq"], dtype=np.uint8)
    sq, sk, sv = _f32(prep["sq"]), _f32(prep["sk"]), _f32(prep["sv"])
    B, H, N, d = qq.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if bias is not None:
        bias = _f32(bias)
    r = _rows(rows)
    out = np.zeros((r.shape[0], d), dtype=np.float64)
    lse = np.zeros((r.shape[0],), dtype=np.float64)
    km = _f32(prep["kmean"]) if prep.get("kmean") is not None else None
    rc = _load().sage8_oracle_emulate_rows(_p(qq), _p(kq), _p(vq), _p(sq), _p(sk), _p(sv),
                                           _p(km), _p(bias), B, H, N, d, int(bool(causal)), float(scale),
                                           int(kv_block), int(p_mode), _p(r), r.shape[0],
                                           _p(out), _p(lse), int(fp8), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"sage8_oracle_emulate_rows failed with code {rc}")
    return out, lse


def sage8_emulate_rows_fp32(prep, rows, causal=False, scale=None, bias=None, nthreads=0):
    """Blocked 8-bit forward with the kernel's fp32 decisions (64-key blocks,
    running maximum raised only past +2 in log2 units, P^ = e4m3(448*2^(t-m-2))).
    Returns (O [nrows,d], LSE [nrows]) in fp64."""
    fp8 = bool(prep.get("qk_fp8", False))
    qq = np.ascontiguousarray(prep["qq"], dtype=np.uint8 if fp8 else np.int8)
    kq = np.ascontiguousarray(prep["kq"], dtype=np.uint8 if fp8 else np.int8)
    vq = np.ascontiguousarray(prep["vq"], dtype=np.uint8)
    sq, sk, sv = _f32(prep["sq"]), _f32(prep["sk"]), _f32(prep["sv"])
    B, H, N, d = qq.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if bias is not None:
        bias = _f32(bias)
    r = _rows(rows)
    out = np.zeros((r.shape[0], d), dtype=np.float64)
    lse = np.zeros((r.shape[0],), dtype=np.float64)
    km = _f32(prep["kmean"]) if prep.get("kmean") is not None else None
    rc = _load().sage8_oracle_emulate_rows_fp32(_p(qq), _p(kq), _p(vq), _p(sq), _p(sk), _p(sv),
                                                _p(km), _p(bias), B, H, N, d, int(bool(causal)),
                                                float(np.float32(scale)), _p(r), r.shape[0],
                                                _p(out), _p(lse), int(fp8), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"sage8_oracle_emulate_rows_fp32 failed with code {rc}")
    return out, lse


def sage8_qk8_rows(prep, v, rows, causal=False, scale=None, bias=None, nthreads=0):
    """INT8 scores from the quantised Q and centred K of sage8_prepare (INT8
    format), then the exact softmax and the exact product with v (the 16-bit
    V, any float array [B,H,N,d]) in fp64.  Returns (O [nrows,d], LSE [nrows]);
    the LSE adds back the score shift of the K centring."""
    if prep.get("qk_fp8", False):
        raise ValueError("sage8_qk8_rows takes INT8 scores")
    qq = np.ascontiguousarray(prep["qq"], dtype=np.int8)
    kq = np.ascontiguousarray(prep["kq"], dtype=np.int8)
    sq, sk = _f32(prep["sq"]), _f32(prep["sk"])
    v = _f32(v)
    B, H, N, d = qq.shape
    assert v.shape == qq.shape and kq.shape == qq.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if bias is not None:
        bias = _f32(bias)
        assert bias.shape == (B, H, (N + 63) // 64, (N + 63) // 64), bias.shape
    km = _f32(prep["kmean"]) if prep.get("kmean") is not None else None
    r = _rows(rows)
    out = np.zeros((r.shape[0], d), dtype=np.float64)
    lse = np.zeros((r.shape[0],), dtype=np.float64)
    rc = _load().sage8_oracle_qk8_rows(_p(qq), _p(kq), _p(sq), _p(sk), _p(v), _p(km), _p(bias),
                                       B, H, N, d, int(bool(causal)), float(scale), _p(r), r.shape[0],
                                       _p(out), _p(lse), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"sage8_oracle_qk8_rows failed with code {rc}")
    return out, lse
