"""Pins for the 8-bit preparation oracle and the 8-bit emulator (CPU only).

Pinned against: torch's float8_e4m3fn casts (a library conversion) on every
code and on ties; exact round trips of values that are exact multiples of
the scale; the half-step error bound of rounding; numpy's fp64 mean; and, for
the emulator, the plain fp64 oracle on inputs the quantisers represent
exactly.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def test_e4m3_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9


def _torch_encode(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch():
    vals = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = np.sort(np.unique(vals[np.isfinite(vals)]))
    # every representable value round-trips
    np.testing.assert_array_equal(oracle.e4m3_encode(finite), _torch_encode(finite))
    # midpoints between neighbours: ties to even (all exact in fp32)
    mids = (finite[1:] + finite[:-1]) / 2
    assert np.array_equal(mids.astype(np.float32).astype(np.float64), mids)
    np.testing.assert_array_equal(oracle.e4m3_encode(mids), _torch_encode(mids))
    # random values over the whole range, including subnormals
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * np.exp2(rng.uniform(-12, 8.8, 20000))).astype(np.float32)
    x = x[np.abs(x) < 464]
    np.testing.assert_array_equal(oracle.e4m3_encode(x.astype(np.float64)), _torch_encode(x))


def test_e4m3_saturates():
    assert oracle.e4m3_encode([448.0, 463.9, 464.0, 1e6])[0] == 0x7E
    assert (oracle.e4m3_encode([448.0, 463.9, 464.0, 1e6]) == 0x7E).all()
    assert (oracle.e4m3_encode([-500.0, -1e9]) == 0xFE).all()
    assert oracle.e4m3_encode([float("nan")])[0] == 0x7F


def test_int8_exact_multiples_round_trip():
    rng = np.random.default_rng(1)
    B, H, N, d = 1, 2, 130, 16
    ints = rng.integers(-127, 128, (B, H, N, d))
    nb = (N + 63) // 64
    # one power-of-two step per 64-row block, and force each block's absmax to 127
    steps = 2.0 ** rng.integers(-6, 3, (B, H, nb))
    for b in range(B):
        for h in range(H):
            for blk in range(nb):
                ints[b, h, blk * 64, 0] = 127
    x = (ints * np.repeat(steps, 64, axis=2)[:, :, :N, None]).astype(np.float32)
    codes, scales = oracle.sage8_quant_int8(x)
    np.testing.assert_array_equal(codes, ints)
    np.testing.assert_array_equal(scales, steps.astype(np.float32))


def test_int8_error_bound_and_extremes():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 2, 200, 32)).astype(np.float32) * 3
    center = rng.standard_normal((2, 2, 32)).astype(np.float32)
    codes, scales = oracle.sage8_quant_int8(x, center)
    y = x - center[:, :, None, :]
    s = np.repeat(scales, 64, axis=2)[:, :, :200, None].astype(np.float64)
    err = np.abs(codes * s - y)
    assert (err <= s * 0.5 * (1 + 1e-6)).all()
    assert codes.max() <= 127 and codes.min() >= -127
    # each block's largest |y| maps to +-127
    for b in range(2):
        for h in range(2):
            for blk in range(4):
                sl = slice(blk * 64, min(blk * 64 + 64, 200))
                assert np.abs(codes[b, h, sl]).max() == 127
                amax = np.abs(y[b, h, sl]).max()
                assert scales[b, h, blk] == np.float32(amax) / np.float32(127)


def test_int8_zero_block():
    x = np.zeros((1, 1, 70, 8), np.float32)
    x[0, 0, 64:] = 1.0
    codes, scales = oracle.sage8_quant_int8(x)
    assert scales[0, 0, 0] == 1.0 and (codes[0, 0, :64] == 0).all()
    assert (codes[0, 0, 64:] == 127).all()


def test_kmean_matches_numpy():
    rng = np.random.default_rng(3)
    k = torch.from_numpy(rng.standard_normal((2, 3, 333, 16)) + 5).to(torch.bfloat16).float().numpy()
    ours = oracle.sage8_kmean(k)
    ref = k.astype(np.float64).mean(axis=2).astype(np.float32)
    np.testing.assert_array_equal(ours, ref)
    # the smoothed K has column means near 0
    _, _ = oracle.sage8_quant_int8(k, ours)
    assert np.abs((k - ours[:, :, None, :]).astype(np.float64).mean(axis=2)).max() < 1e-5


def test_quant_v_bounds():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((1, 2, 300, 16)).astype(np.float32)
    v[0, 1, :, 3] = 0.0
    codes, scales = oracle.sage8_quant_v(v)
    dec = oracle.e4m3_decode(codes) * scales[:, :, None, :]
    rel = np.abs(dec - v) / np.maximum(np.abs(v), 1e-30)
    big = np.abs(v) >= (2.0 ** -6) * scales[:, :, None, :]  # normal range of e4m3
    assert (rel[big] <= 2.0 ** -4 * (1 + 1e-6)).all()  # half a step of a 3-bit mantissa
    assert scales[0, 1, 3] == 1.0 and (codes[0, 1, :, 3] == 0).all()
    # the per-channel absmax maps to 448
    for h in range(2):
        for c in range(16):
            if c == 3 and h == 1:
                continue
            n = np.argmax(np.abs(v[0, h, :, c]))
            assert (codes[0, h, n, c] & 0x7F) == 0x7E


def _lossless_prep(B, H, N, d, seed):
    """Quantised data whose dequantised values are known exactly, plus those
    values as fp32 arrays."""
    rng = np.random.default_rng(seed)
    nqk = (N + 63) // 64
    qq = rng.integers(-127, 128, (B, H, N, d)).astype(np.int8)
    kq = rng.integers(-127, 128, (B, H, N, d)).astype(np.int8)
    sq = (2.0 ** rng.integers(-8, -5, (B, H, nqk))).astype(np.float32)
    sk = (2.0 ** rng.integers(-8, -5, (B, H, nqk))).astype(np.float32)
    vq = rng.integers(0, 256, (B, H, N, d)).astype(np.uint8)
    vq[(vq & 0x7F) == 0x7F] = 0x10  # no NaN codes
    sv = (2.0 ** rng.integers(-9, -7, (B, H, d))).astype(np.float32)
    q = qq * np.repeat(sq, 64, axis=2)[:, :, :N, None]
    k = kq * np.repeat(sk, 64, axis=2)[:, :, :N, None]
    v = oracle.e4m3_decode(vq) * sv[:, :, None, :]
    prep = dict(qq=qq, kq=kq, vq=vq, sq=sq, sk=sk, sv=sv)
    return prep, q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kv_block", [1, 64, 100])
def test_emulator_without_p_rounding_equals_oracle(causal, kv_block):
    prep, q, k, v = _lossless_prep(1, 2, 150, 16, seed=5)
    assert np.array_equal(q.astype(np.float64),
                          prep["qq"] * np.repeat(prep["sq"], 64, axis=2)[:, :, :150, None].astype(np.float64))
    bias = np.random.default_rng(6).normal(0, 1, (1, 2, 3, 3)).astype(np.float32)
    rows = workloads.parity_rows(1, 2, 150, seed=2, n_random=20)
    o_ref, l_ref = oracle.attn_rows(q, k, v, rows, causal=causal, scale=0.7, bias=bias)
    o_emu, l_emu = oracle.sage8_emulate_rows(prep, rows, causal=causal, scale=0.7, bias=bias,
                                             kv_block=kv_block, p_mode=0)
    np.testing.assert_allclose(o_emu, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_emu, l_ref, rtol=0, atol=1e-12)


def test_emulator_p_rounding_is_bounded():
    """With P rounded to e4m3 each weight moves by at most half a step of a
    3-bit mantissa (2^-4 relative) or one subnormal step; the output moves by
    no more than that bound applied to sum_j p_j |v_j| / l."""
    prep, q, k, v = _lossless_prep(1, 1, 128, 16, seed=7)
    rows = [(0, 0, i) for i in range(0, 128, 9)]
    o0, _ = oracle.sage8_emulate_rows(prep, rows, causal=False, scale=0.5, p_mode=0)
    o1, _ = oracle.sage8_emulate_rows(prep, rows, causal=False, scale=0.5, p_mode=1)
    for n, (_, _, i) in enumerate(rows):
        p = oracle.row_probs(q, k, 0, 0, i, causal=False, scale=0.5)
        # |dP^_j| <= 2^-4 * 448 p_j (normal range) or 2^-10 (half a subnormal
        # step); dividing by 448 l with l >= 1 in running-max units gives:
        bound = (p * 2.0 ** -4 + 2.0 ** -10 / 448) @ np.abs(v[0, 0].astype(np.float64))
        assert (np.abs(o1[n] - o0[n]) <= bound * 1.01 + 1e-12).all()
    assert np.abs(o1 - o0).max() > 0  # the rounding is really applied


def test_emulator_floor_on_outlier_workload():
    """The specified 8-bit recipe against the fp64 oracle on a scaled-down
    workload-4 distribution: cosine meets 0.999, while relative L1 sits near
    0.035 -- a property of FP8 V and FP8 P on i.i.d. values, not of a kernel."""
    inp = workloads.make_inputs(1, 2, 1024, 128, "bf16", seed=4, outliers=True)
    q, k, v = (inp[n].float().numpy() for n in ("q", "k", "v"))
    prep = oracle.sage8_prepare(q, k, v)
    rows = workloads.parity_rows(1, 2, 1024, seed=4, n_random=48)
    scale = 1 / math.sqrt(128)
    o_ref, _ = oracle.attn_rows(q, k, v, rows, causal=True, scale=scale)
    o_emu, _ = oracle.sage8_emulate_rows(prep, rows, causal=True, scale=scale, kv_block=64)
    m = workloads.error_metrics(o_emu, o_ref)
    assert m["cos"] >= 0.999, m
    assert 0.02 < m["rel_l1"] < 0.06, m


@pytest.mark.parametrize("causal", [False, True])
def test_fp32_emulator_closed_form_q_zero(causal):
    """Q = 0: every score is 0, so P = 2^(log2(448) - 2) = 112, which e4m3
    represents exactly; O is then the (prefix) mean of the dequantised V and
    LSE = ln(number of visible keys).  The fp32 model carries the integer
    scores as 12582912 + S, so the exponent argument of each (row, key block)
    may be off by a common amount of at most E = 3 ulp(12582912 |f|) (the
    roundings of g, kc and the maximum): the block's P scales by 2^e with
    |e| <= E, which moves O by at most (2^(2E) - 1) max|V| and the LSE by
    E ln 2 (plus fp32 rounding of the constants)."""
    prep, _, _, v = _lossless_prep(1, 2, 150, 16, seed=9)
    prep["qq"] = np.zeros_like(prep["qq"])
    rows = [(0, h, i) for h in range(2) for i in (0, 1, 63, 64, 65, 100, 149)]
    scale = 0.3
    o, lse = oracle.sage8_emulate_rows_fp32(prep, rows, causal=causal, scale=scale)
    c = np.float32(scale * math.log2(math.e))
    f = float(prep["sq"].max()) * float(prep["sk"].max()) * float(c)
    E = 3 * 2.0 ** (math.floor(math.log2(12582912.0 * f)) - 23)
    assert E < 1e-2
    vd = v.astype(np.float64)
    for n, (_, h, i) in enumerate(rows):
        ref = vd[0, h, : i + 1].mean(axis=0) if causal else vd[0, h].mean(axis=0)
        tol = (2.0 ** (2 * E) - 1) * np.abs(vd).max() + 1e-12
        np.testing.assert_allclose(o[n], ref, rtol=0, atol=tol)
        np.testing.assert_allclose(lse[n], math.log(i + 1 if causal else 150), rtol=0,
                                   atol=E * math.log(2) + 1e-6)


def test_fp32_emulator_matches_recipe_floor():
    """The kernel-precision emulator on a scaled-down workload-4 distribution
    against the fp64 oracle: same accuracy class as the fp64 model."""
    inp = workloads.make_inputs(1, 2, 1024, 128, "bf16", seed=4, outliers=True)
    q, k, v = (inp[n].float().numpy() for n in ("q", "k", "v"))
    prep = oracle.sage8_prepare(q, k, v)
    rows = workloads.parity_rows(1, 2, 1024, seed=4, n_random=48)
    scale = 1 / math.sqrt(128)
    o_ref, l_ref = oracle.attn_rows(q, k, v, rows, causal=True, scale=scale)
    o32, l32 = oracle.sage8_emulate_rows_fp32(prep, rows, causal=True, scale=scale)
    o64, _ = oracle.sage8_emulate_rows(prep, rows, causal=True, scale=scale)
    m = workloads.error_metrics(o32, o_ref)
    assert m["cos"] >= 0.999 and 0.02 < m["rel_l1"] < 0.06, m
    # the two models differ only in where P is rounded
    assert workloads.error_metrics(o32, o64)["rel_l1"] < 0.03
    # the LSE includes the shift that the centring of K removed
    assert np.abs(l32 - l_ref).max() < 0.05
    _, l64 = oracle.sage8_emulate_rows(prep, rows, causal=True, scale=scale)
    assert np.abs(l64 - l_ref).max() < 0.05


@pytest.mark.parametrize("which", ["fp64", "fp32"])
def test_normaliser_is_sum_of_unquantised_p(which):
    """Two keys whose probabilities stand in the ratio 2^-1.5.  Hand-derived:
    K centres to rows +-1 (codes +-127, both scales 1/127 after the centring
    by kmean = 1), Q = e_0 (code 127, scale 1/127), so S = +-127 and the
    scores differ by 2 * scale.  With scale = 0.75 ln 2 the weights are 1 and
    2^-1.5.  V = rows (1, 0) in channel 0 (scale 1/448, codes exact), so only
    key 0 (P^ exact: 448 in the fp64 model, 112 in the fp32 model) enters the
    numerator.  With l = sum of the unquantised weights, O[0] = 1 / (1 +
    2^-1.5) = 0.738796...; the sum of the quantised weights would give
    448 / (448 + 160) = 112 / (112 + 40) = 0.736842... (158.39 rounds to the
    e4m3 value 160, 39.60 to 40)."""
    d = 64
    q = np.zeros((1, 1, 2, d), np.float32)
    q[0, 0, :, 0] = 1.0
    k = np.zeros((1, 1, 2, d), np.float32)
    k[0, 0, 0, 0], k[0, 0, 1, 0] = 2.0, 0.0
    v = np.zeros((1, 1, 2, d), np.float32)
    v[0, 0, 0, 0] = 1.0
    prep = oracle.sage8_prepare(q, k, v)
    assert prep["kq"][0, 0, 0, 0] == 127 and prep["kq"][0, 0, 1, 0] == -127
    rows = np.array([[0, 0, 0]])
    scale = 0.75 * math.log(2.0)
    if which == "fp64":
        o, _ = oracle.sage8_emulate_rows(prep, rows, causal=False, scale=scale)
    else:
        o, _ = oracle.sage8_emulate_rows_fp32(prep, rows, causal=False, scale=scale)
    # (the fp32 model's offset shifts the exponent by <= 3 ulp(12582912 f) ~ 2e-4)
    assert abs(o[0, 0] - 1.0 / (1.0 + 2.0 ** -1.5)) < 1e-4
    assert abs(o[0, 0] - 448.0 / 608.0) > 1e-3
