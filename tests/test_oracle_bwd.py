"""Pins of the fp64 oracle backward (CPU only).

The oracle's gradients (dQ, dK, dV, and the block-bias gradient that the
log-form gate of page 5, "SAS", needs) are checked against things other than
their own formulas:

* central finite differences of the *forward* oracle on inputs that are
  exact multiples of 2^-6, perturbed by 2^-12 (both exactly representable,
  so the differences see only the function);
* torch autograd in float64 through softmax(scale*Q K^T + bias) V on tiny
  inputs (a library routine on the same definition);
* exact identities: every row of dS sums to 0, so the key-sums of dK and
  the key-block sums of dbias vanish; the rows of P sum to 1, so the key-sum
  of dV is the query-sum of dO; a V constant over keys gives dQ = dK = 0.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _grid_inputs(shape, seed, lo=-2.0, hi=2.0):
    rng = np.random.default_rng(seed)
    return (np.round(rng.uniform(lo, hi, size=shape) * 64) / 64).astype(np.float32)


def _loss(q, k, v, dout, causal, scale, bias):
    o, _ = oracle.attn_full(q, k, v, causal=causal, scale=scale, bias=bias)
    return float(np.sum(o * dout.astype(np.float64)))


def _fd(fn, x, idx, eps=2.0 ** -12):
    """Central difference of fn at element idx of the float32 array x."""
    xp, xm = x.copy(), x.copy()
    xp[idx] += np.float32(eps)
    xm[idx] -= np.float32(eps)
    assert xp[idx] - x[idx] == np.float32(eps) and x[idx] - xm[idx] == np.float32(eps)
    return (fn(xp) - fn(xm)) / (2 * eps)


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences_qkv(causal):
    B, H, N, d = 1, 2, 9, 4
    q, k, v, dout = (_grid_inputs((B, H, N, d), s) for s in (1, 2, 3, 4))
    scale = 0.5
    dq, dk, dv, _ = oracle.attn_bwd(q, k, v, dout, causal=causal, scale=scale)
    worst = 0.0
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(x.shape):
            def fn(xx, name=name):
                a = dict(q=q, k=k, v=v)
                a[name] = xx
                return _loss(a["q"], a["k"], a["v"], dout, causal, scale, None)
            worst = max(worst, abs(_fd(fn, x, idx) - g[idx]))
    assert worst < 2e-6, worst


def test_finite_differences_bias():
    """The bias gradient, over several 64 x 64 blocks (N = 130: 3 blocks
    per side, ragged last block), causal."""
    B, H, N, d = 1, 1, 130, 4
    q, k, v, dout = (_grid_inputs((B, H, N, d), s, -1.0, 1.0) for s in (5, 6, 7, 8))
    bias = _grid_inputs((B, H, 3, 3), 9)
    scale = 0.75
    _, _, _, db = oracle.attn_bwd(q, k, v, dout, causal=True, scale=scale, bias=bias)
    for idx in np.ndindex(bias.shape):
        fd = _fd(lambda bb: _loss(q, k, v, dout, True, scale, bb), bias, idx)
        assert abs(fd - db[idx]) < 2e-6, (idx, fd, db[idx])
    # causal: key blocks above the diagonal block get no gradient
    assert db[0, 0, 0, 1] == 0.0 and db[0, 0, 0, 2] == 0.0 and db[0, 0, 1, 2] == 0.0


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd_float64(causal):
    B, H, N, d = 2, 2, 70, 8
    rng = np.random.default_rng(11)
    q, k, v, dout = (rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(4))
    bias = rng.standard_normal((B, H, 2, 2)).astype(np.float32)
    scale = 1 / math.sqrt(d)
    dq, dk, dv, db = oracle.attn_bwd(q, k, v, dout, causal=causal, scale=scale, bias=bias)
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, bias)]
    blk = torch.arange(N) // 64
    full_bias = t[3][:, :, blk][:, :, :, blk]
    s = scale * (t[0] @ t[1].transpose(-1, -2)) + full_bias
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ t[2]
    (o * torch.tensor(dout, dtype=torch.float64)).sum().backward()
    for mine, ref in ((dq, t[0].grad), (dk, t[1].grad), (dv, t[2].grad), (db, t[3].grad)):
        assert np.abs(mine - ref.numpy()).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_identities(causal):
    B, H, N, d = 1, 3, 150, 16
    rng = np.random.default_rng(12)
    q, k, v, dout = (rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(4))
    bias = rng.standard_normal((B, H, 3, 3)).astype(np.float32)
    dq, dk, dv, db = oracle.attn_bwd(q, k, v, dout, causal=causal, bias=bias)
    assert np.abs(dk.sum(axis=2)).max() < 1e-12
    assert np.abs(dv.sum(axis=2) - dout.astype(np.float64).sum(axis=2)).max() < 1e-11
    assert np.abs(db.sum(axis=3)).max() < 1e-12
    # V constant over keys: O does not depend on the scores
    vc = np.broadcast_to(rng.standard_normal((B, H, 1, d)).astype(np.float32), v.shape).copy()
    dq, dk, dv, db = oracle.attn_bwd(q, k, vc, dout, causal=causal, bias=bias)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12 and np.abs(db).max() < 1e-12


def test_single_key_and_masked_rows():
    """Causal row 0 sees one key (P = 1): dV[0] gets dO[0] in full and the
    row passes no gradient to Q.  A query block whose every key block is
    gated off (bias -inf) has O = 0 and passes no gradient anywhere."""
    B, H, N, d = 1, 1, 130, 4
    rng = np.random.default_rng(13)
    q, k, v, dout = (rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(4))
    dq, dk, dv, _ = oracle.attn_bwd(q[:, :, :1], k[:, :, :1], v[:, :, :1], dout[:, :, :1], causal=True)
    assert np.array_equal(dv[0, 0, 0], dout[0, 0, 0].astype(np.float64))
    assert not dq.any() and not dk.any()
    bias = np.zeros((B, H, 3, 3), dtype=np.float32)
    bias[0, 0, 1, :] = -np.inf
    dq, dk, dv, db = oracle.attn_bwd(q, k, v, dout, causal=False, bias=bias)
    assert not dq[0, 0, 64:128].any() and not db[0, 0, 1].any()
    dq2, dk2, dv2, _ = oracle.attn_bwd(q, k, v, np.where(np.arange(N)[None, None, :, None] // 64 == 1, 0, dout)
                                       .astype(np.float32), causal=False, bias=bias)
    assert np.abs(dk - dk2).max() == 0 and np.abs(dv - dv2).max() == 0
