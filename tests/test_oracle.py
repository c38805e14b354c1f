"""Pins for the fp64 attention oracle (CPU only).

The oracle is checked against things other than itself: hand-derived closed
forms (tests/golden/closed_forms.json), library routines on tiny inputs
(scipy softmax / logsumexp over an explicitly formed score matrix), and
invariants the mathematics fixes (rows of P sum to 1, shift invariance in K,
causal row 0 = V[0], Q = 0 gives means, permutation equivariance).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _rand(B, H, N, d, seed, grid=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((3, B, H, N, d))
    if grid:  # values on a 2^-6 grid: sums with small dyadic shifts stay exact
        x = np.round(x * 64) / 64
    return [a.astype(np.float32) for a in x]


def _library_attention(q, k, v, causal, scale, bias):
    """softmax(scale*QK^T + bias)V via numpy matmul and scipy softmax."""
    B, H, N, d = q.shape
    q64, k64, v64 = (a.astype(np.float64) for a in (q, k, v))
    s = scale * np.einsum("bhid,bhjd->bhij", q64, k64)
    if bias is not None:
        s = s + np.repeat(np.repeat(bias.astype(np.float64), 64, axis=2), 64, axis=3)[:, :, :N, :N]
    if causal:
        s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
    p = scipy.special.softmax(s, axis=-1)
    return p @ v64, scipy.special.logsumexp(s, axis=-1)


def _val(x):
    if isinstance(x, str):
        return {"ln2": math.log(2), "ln3": math.log(3), "ln4": math.log(4),
                "ln128": math.log(128), "ln256": math.log(256), "0": 0.0, "1": 1.0}[x]
    return float(x)


def test_golden_closed_forms():
    cases = json.load(open(GOLDEN))["cases"]
    assert len(cases) >= 5
    for c in cases:
        N, d = c["N"], c["d"]
        if c["name"] == "block_bias_one":
            q = np.zeros((1, 1, N, d), np.float32)
            k = (np.arange(N, dtype=np.float32) / 100).reshape(1, 1, N, d)
            v = np.where(np.arange(N) < 64, 1.0, 2.0).astype(np.float32).reshape(1, 1, N, d)
            bias = np.array([[_val(x) for x in row] for row in c["bias"]], np.float32)[None, None]
            o, lse = oracle.attn_full(q, k, v, causal=c["causal"], scale=_val(c["scale"]), bias=bias)
            exp_o = np.where(np.arange(N) < 64, c["expect_o"][0], c["expect_o"][1])
            exp_l = np.where(np.arange(N) < 64, _val(c["expect_lse"][0]), _val(c["expect_lse"][1]))
            np.testing.assert_allclose(o[0, 0, :, 0], exp_o, rtol=0, atol=1e-14)
            np.testing.assert_allclose(lse[0, 0], exp_l, rtol=0, atol=1e-13)
            continue
        q = np.array(c["q"], np.float32).reshape(1, 1, N, d)
        k = np.array(c["k"], np.float32).reshape(1, 1, N, d)
        v = np.array(c["v"], np.float32).reshape(1, 1, N, d)
        o, lse = oracle.attn_full(q, k, v, causal=c["causal"], scale=_val(c["scale"]))
        np.testing.assert_allclose(o[0, 0], np.array(c["expect_o"]), rtol=0, atol=1e-13,
                                   err_msg=c["name"])
        np.testing.assert_allclose(lse[0, 0], [_val(x) for x in c["expect_lse"]], rtol=1e-15,
                                   atol=1e-12, err_msg=c["name"])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("N,d", [(37, 16), (130, 8), (1, 4)])
def test_matches_library_softmax(causal, with_bias, N, d):
    q, k, v = _rand(1, 2, N, d, seed=N * 7 + d)
    bias = None
    if with_bias:
        nb = (N + 63) // 64
        bias = np.random.default_rng(5).normal(0, 2, (1, 2, nb, nb)).astype(np.float32)
    scale = 0.37
    o, lse = oracle.attn_full(q, k, v, causal=causal, scale=scale, bias=bias)
    o_ref, lse_ref = _library_attention(q, k, v, causal, scale, bias)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_prob_rows_sum_to_one(causal):
    q, k, _ = _rand(1, 1, 50, 8, seed=3)
    for i in [0, 1, 17, 49]:
        p = oracle.row_probs(q, k, 0, 0, i, causal=causal, scale=0.9)
        assert abs(p.sum() - 1.0) < 1e-14
        assert (p >= 0).all() and (p <= 1).all()
        if causal:
            assert (p[i + 1:] == 0).all()
            assert (p[: i + 1] > 0).all()


@pytest.mark.parametrize("causal", [False, True])
def test_k_shift_invariance(causal):
    # K and the shift are on dyadic grids, so K + c is exact in fp32.
    q, k, v = _rand(1, 2, 40, 16, seed=11, grid=True)
    c = (np.round(np.random.default_rng(2).standard_normal(16) * 8) / 8).astype(np.float32)
    k2 = k + c
    assert np.array_equal(k2.astype(np.float64), k.astype(np.float64) + c.astype(np.float64))
    o1, l1 = oracle.attn_full(q, k, v, causal=causal, scale=0.25)
    o2, l2 = oracle.attn_full(q, k2, v, causal=causal, scale=0.25)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    # the LSE moves by scale * q.c, exactly the shift
    shift = 0.25 * np.einsum("bhid,d->bhi", q.astype(np.float64), c.astype(np.float64))
    np.testing.assert_allclose(l2, l1 + shift, rtol=0, atol=1e-11)


def test_causal_row0_is_v0():
    q, k, v = _rand(2, 3, 33, 8, seed=4)
    o, lse = oracle.attn_full(q, k, v, causal=True, scale=1.3)
    np.testing.assert_array_equal(o[:, :, 0, :], v[:, :, 0, :].astype(np.float64))
    s00 = 1.3 * np.einsum("bhd,bhd->bh", q[:, :, 0].astype(np.float64), k[:, :, 0].astype(np.float64))
    np.testing.assert_allclose(lse[:, :, 0], s00, rtol=0, atol=1e-13)


def test_q_zero_gives_means():
    _, k, v = _rand(1, 2, 70, 8, seed=5)
    q = np.zeros_like(k)
    o, _ = oracle.attn_full(q, k, v, causal=False, scale=0.5)
    mean = v.astype(np.float64).mean(axis=2, keepdims=True)
    np.testing.assert_allclose(o, np.broadcast_to(mean, o.shape), rtol=0, atol=1e-13)
    oc, _ = oracle.attn_full(q, k, v, causal=True, scale=0.5)
    prefix = np.cumsum(v.astype(np.float64), axis=2) / np.arange(1, 71)[None, None, :, None]
    np.testing.assert_allclose(oc, prefix, rtol=0, atol=1e-13)


def test_degenerate_cases():
    q, k, v = _rand(1, 1, 20, 8, seed=6)
    # N = 1: the only key gets weight 1
    o, _ = oracle.attn_full(q[:, :, :1], k[:, :, :1], v[:, :, :1], scale=3.0)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0].astype(np.float64))
    # constant V gives V
    vc = np.full_like(v, 1.5)
    o, _ = oracle.attn_full(q, k, vc, causal=False, scale=0.7)
    np.testing.assert_allclose(o, 1.5, rtol=0, atol=1e-14)
    # scale = 0 gives the mean of V
    o, lse = oracle.attn_full(q, k, v, causal=False, scale=0.0)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0].astype(np.float64).mean(0), (20, 8)),
                               rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(20), rtol=0, atol=1e-14)


def test_permutation_equivariance():
    q, k, v = _rand(1, 2, 45, 8, seed=8)
    perm = np.random.default_rng(9).permutation(45)
    o1, l1 = oracle.attn_full(q, k, v, causal=False, scale=0.4)
    o2, l2 = oracle.attn_full(q, k[:, :, perm], v[:, :, perm], causal=False, scale=0.4)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)
    # permuting queries permutes output rows
    o3, _ = oracle.attn_full(q[:, :, perm], k, v, causal=False, scale=0.4)
    np.testing.assert_allclose(o3, o1[:, :, perm], rtol=0, atol=1e-15)


def test_minus_inf_bias_selects_one_block():
    q, k, v = _rand(1, 1, 192, 8, seed=10)
    bias = np.full((1, 1, 3, 3), -np.inf, np.float32)
    bias[:, :, :, 1] = 0.0  # only key block 1 (keys 64..127) is visible
    o, lse = oracle.attn_full(q, k, v, causal=False, scale=0.3, bias=bias)
    o_ref, lse_ref = _library_attention(q, k[:, :, 64:128], v[:, :, 64:128], False, 0.3, None)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_fully_masked_row_convention():
    q, k, v = _rand(1, 1, 70, 8, seed=12)
    bias = np.zeros((1, 1, 2, 2), np.float32)
    bias[0, 0, 1, :] = -np.inf  # query block 1 (rows 64..69) sees nothing
    o, lse = oracle.attn_full(q, k, v, causal=False, scale=0.3, bias=bias)
    assert (o[0, 0, 64:] == 0).all()
    assert np.isneginf(lse[0, 0, 64:]).all()
    assert np.isfinite(o[0, 0, :64]).all()


def _online_blocked(q, k, v, causal, scale, bias, block):
    """The online-softmax update (running max m, running sum l, rescaled O;
    page 4, 'FlashAttention (TR)', online softmax section) in fp64, one key
    block at a time.  Used to pin that this update reproduces the plain
    definition exactly, for any block size."""
    B, H, N, d = q.shape
    q64, k64, v64 = (a.astype(np.float64) for a in (q, k, v))
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                m, l, acc = -np.inf, 0.0, np.zeros(d)
                jend = i + 1 if causal else N
                for j0 in range(0, jend, block):
                    j1 = min(j0 + block, jend)
                    s = scale * (k64[b, h, j0:j1] @ q64[b, h, i])
                    if bias is not None:
                        s = s + bias[b, h, i // 64, np.arange(j0, j1) // 64]
                    mn = max(m, s.max())
                    if mn == -np.inf:
                        continue
                    alpha = 0.0 if m == -np.inf else math.exp(m - mn)
                    p = np.exp(s - mn)
                    acc = acc * alpha + p @ v64[b, h, j0:j1]
                    l = l * alpha + p.sum()
                    m = mn
                o[b, h, i] = acc / l if l > 0 else 0.0
                lse[b, h, i] = m + math.log(l) if l > 0 else -np.inf
    return o, lse


@pytest.mark.parametrize("block", [1, 7, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_online_update_equals_definition(block, causal):
    q, k, v = _rand(1, 1, 150, 8, seed=13)
    bias = np.random.default_rng(14).normal(0, 1, (1, 1, 3, 3)).astype(np.float32)
    o, lse = oracle.attn_full(q, k, v, causal=causal, scale=0.6, bias=bias)
    ob, lb = _online_blocked(q, k, v, causal, 0.6, bias.astype(np.float64), block)
    np.testing.assert_allclose(ob, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lb, lse, rtol=0, atol=1e-12)


def test_rows_subset_matches_full():
    q, k, v = _rand(2, 3, 90, 16, seed=15)
    o, lse = oracle.attn_full(q, k, v, causal=True, scale=0.25)
    rows = workloads.parity_rows(2, 3, 90, seed=1, n_random=5)
    orow, lrow = oracle.attn_rows(q, k, v, rows, causal=True, scale=0.25)
    np.testing.assert_array_equal(orow, o[rows[:, 0], rows[:, 1], rows[:, 2]])
    np.testing.assert_array_equal(lrow, lse[rows[:, 0], rows[:, 1], rows[:, 2]])


def test_rejects_bad_rows():
    q, k, v = _rand(1, 1, 4, 2, seed=0)
    with pytest.raises(RuntimeError):
        oracle.attn_rows(q, k, v, [(0, 0, 4)])
    with pytest.raises(RuntimeError):
        oracle.attn_rows(q, k, v, [(1, 0, 0)])
