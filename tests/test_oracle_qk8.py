"""Pins for the oracle of the INT8-score variant with the 16-bit P V product
(``oracle.sage8_qk8_rows``; CPU only).

Pinned against the plain fp64 oracle (itself pinned by closed forms, scipy
and brute force) on inputs the quantisers represent exactly, so that the
quantised scores are the exact scores: any dropped scale, wrong block index,
transposed operand or missing LSE term fails.  The centring of K is pinned
through softmax shift invariance (page 1, "SageAttention", claim vs reality
section): with K + c the output is unchanged and the LSE moves by
scale * q.c, which the oracle must add back.
"""
import math

import numpy as np
import pytest

import oracle
import workloads


def _exact_blocks(rng, B, H, N, d, zero_mean=False):
    """Values x = code * 2^e per 64-row block with one code of +-127 in each
    block (so the block scale amax/127 is exactly 2^e and every code round
    trips), returned as fp32 [B,H,N,d].  zero_mean: the second half of the
    rows is the negated first half (column sums exactly 0; N a multiple of
    128 and the mirrored blocks share their exponent)."""
    nqk = (N + 63) // 64
    codes = rng.integers(-126, 127, (B, H, N, d))
    e = rng.integers(-8, -4, (B, H, nqk))
    for blk in range(nqk):
        codes[:, :, 64 * blk, blk % d] = 127 if blk % 2 == 0 else -127
    if zero_mean:
        half = N // 2
        e[:, :, nqk // 2:] = e[:, :, :nqk // 2]
        codes[:, :, half:] = -codes[:, :, :half]
    scale = np.repeat(2.0 ** e, 64, axis=2)[:, :, :N, None]
    return (codes * scale).astype(np.float32)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [64, 150, 200])
def test_exact_scores_equal_plain_oracle(causal, N):
    """Prepared through the oracle's own quantisers, exactly representable Q
    and zero-mean K give the exact attention, bias included."""
    rng = np.random.default_rng(N + causal)
    B, H, d = 1, 2, 64
    q = _exact_blocks(rng, B, H, N, d)
    k = _exact_blocks(rng, B, H, N, d)
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    prep = oracle.sage8_prepare(q, k, v)
    # the mean of K is not zero here: pass the prep without centring so the
    # codes are exact (kmean enters only the LSE)
    kq, sk = oracle.sage8_quant_int8(k)
    prep = dict(prep, kq=kq, sk=sk, kmean=None)
    assert np.array_equal(kq.astype(np.float64) * np.repeat(sk, 64, axis=2)[:, :, :N, None], k)
    nb = (N + 63) // 64
    bias = rng.normal(0, 1, (B, H, nb, nb)).astype(np.float32)
    rows = workloads.parity_rows(B, H, N, seed=N, n_random=20)
    o_ref, l_ref = oracle.attn_rows(q, k, v, rows, causal=causal, scale=0.3, bias=bias)
    o8, l8 = oracle.sage8_qk8_rows(prep, v, rows, causal=causal, scale=0.3, bias=bias)
    np.testing.assert_allclose(o8, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l8, l_ref, rtol=0, atol=1e-12)


def test_centring_is_added_back_to_the_lse():
    """K + c with zero-mean K: the preparation's K mean is exactly c, the
    centred K is exactly K, so O equals the exact attention of (Q, K + c)
    and the LSE differs from that of (Q, K) by scale * q.c, which the oracle
    restores."""
    rng = np.random.default_rng(11)
    B, H, N, d = 1, 2, 256, 64
    q = _exact_blocks(rng, B, H, N, d)
    k = _exact_blocks(rng, B, H, N, d, zero_mean=True)
    assert not k.sum(axis=2, dtype=np.float64).any()
    c = (rng.integers(-8, 9, (B, H, 1, d)) / 8.0).astype(np.float32)
    ks = (k + c).astype(np.float32)
    assert np.array_equal(ks.astype(np.float64) - c, k.astype(np.float64))  # exact in fp32
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    prep = oracle.sage8_prepare(q, ks, v)
    assert np.array_equal(prep["kmean"], np.broadcast_to(c[:, :, 0], (B, H, d)))
    rows = workloads.parity_rows(B, H, N, seed=3, n_random=16)
    scale = 0.25
    o_ref, l_ref = oracle.attn_rows(q, ks, v, rows, causal=True, scale=scale)
    o8, l8 = oracle.sage8_qk8_rows(prep, v, rows, causal=True, scale=scale)
    np.testing.assert_allclose(o8, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l8, l_ref, rtol=0, atol=1e-12)
    # the shift is not negligible: without it the LSE would be off
    _, l0 = oracle.attn_rows(q, k, v, rows, causal=True, scale=scale)
    assert np.abs(l_ref - l0).max() > 0.1


def test_single_visible_key_and_masked_rows():
    """Causal row 0 sees only key 0: O = V[0] exactly, LSE = its score; a
    query block gated off everywhere gives O = 0 and LSE = -inf."""
    inp = workloads.make_inputs(1, 1, 130, 64, "bf16", seed=9, gate=True)
    q, k, v = (inp[n].float().numpy() for n in ("q", "k", "v"))
    bias = inp["bias"].numpy()
    bias[0, 0, 1, :] = -math.inf
    prep = oracle.sage8_prepare(q, k, v)
    o8, l8 = oracle.sage8_qk8_rows(prep, v, [(0, 0, 0), (0, 0, 64), (0, 0, 127)], causal=True, scale=0.125,
                                   bias=bias)
    np.testing.assert_array_equal(o8[0], v[0, 0, 0].astype(np.float64))
    assert (o8[1:] == 0).all() and np.isneginf(l8[1:]).all()


@pytest.mark.parametrize("cfg_id", [4, 5])
def test_recipe_meets_the_8bit_tolerance(cfg_id):
    """On scaled-down copies of the outlier and DiT-gated workloads the
    INT8-score recipe sits well inside cos >= 0.999 and rel-L1 <= 2e-2
    against exact attention (the FP8 P and V recipe does not: about 0.035)."""
    cfg = workloads.CONFIGS[cfg_id]
    inp = workloads.make_inputs(1, 2, 1024, cfg["d"], "bf16", seed=cfg_id, outliers=cfg.get("outliers", False),
                                gate=cfg.get("gate_bias", False))
    q, k, v = (inp[n].float().numpy() for n in ("q", "k", "v"))
    bias = inp["bias"].numpy() if inp["bias"] is not None else None
    prep = oracle.sage8_prepare(q, k, v)
    rows = workloads.parity_rows(1, 2, 1024, seed=cfg_id, n_random=48)
    scale = 1 / math.sqrt(cfg["d"])
    o_ref, _ = oracle.attn_rows(q, k, v, rows, causal=cfg["causal"], scale=scale, bias=bias)
    o8, _ = oracle.sage8_qk8_rows(prep, v, rows, causal=cfg["causal"], scale=scale, bias=bias)
    m = workloads.error_metrics(o8, o_ref)
    assert m["cos"] >= 0.9995 and m["rel_l1"] <= 0.015, m
    assert m["rel_l1"] > 1e-4, m  # the INT8 scores really are quantised
