"""GPU parity of the FP8-QK variant of the 8-bit path (Q and mean-centred K
in e4m3 blocks, S on the FP8 matrix instruction; P, V and the two-level
P V product as in the INT8 recipe).

Bars, each against code under oracle/ only:
  * preparation: bit-exact against the oracle's e4m3 block quantiser (codes
    and scales of Q and the centred K), and the unchanged K mean and V;
  * forward against the fp32-decision model of the blocked forward with
    e4m3 scores, fed the oracle's quantised data.  The model adds the exact
    FP8 products of a score and rounds once; gfx950's FP8 matrix instruction
    does not: on 32x32x64 tiles of these codes its sums sit up to about
    2^-12.3 of the largest product away from the exact sum, and most outputs
    differ from the correctly rounded one (tests/test_gpu_fp8_mfma.py).  A score that close to an
    e4m3 rounding boundary of P^ = e4m3(448*2^(t-m-2)) then takes the other
    code (a few elements in 10^3), and one code is at most 1/8 of that P^.
    The per-row bar is therefore 1e-3 plus two such flips on the row's
    largest model probability p_max, each moving O by at most
    (1/8) * p_max * 2 * max|v| (measured: at most 0.14 of that bound).  The
    share of rows with any flip grows with the keys per row (up to 7 of 258
    measured at N = 129), so the count check is a loose sanity bar: at most
    10% of the rows (at least 2) leave the 1e-3 band.  The LSE (from the fp32 scores, before any
    e4m3 rounding) keeps the INT8 path's bar;
  * forward against exact fp64 attention: within REL_L1_MARGIN rel-L1 and
    COS_MARGIN cosine of the fp64 model of the same recipe on the same rows
    (the kernel-precision model measured at most 0.0013 rel-L1 and 8.1e-5
    cosine from it on these inputs), and cosine >= 0.999 wherever that fp64
    model reaches 0.999 + COS_MARGIN.  The recipe's own error is about
    0.045-0.05 rel-L1 here, with cosine down to 0.9986 on the DiT-gated and
    the longer non-causal rows: there no kernel faithful to FP8 scores meets
    the 8-bit tolerance (pinned on the CPU in tests/test_oracle_fp8qk.py),
    which is why the INT8 recipe stays the default.
"""
import math

import numpy as np
import pytest
import torch

import bit_attention_attn_amd as attn
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
EMU_ROW_ABS, EMU_LSE = 1e-3, 1e-4
COS_MIN, REL_L1_MARGIN, COS_MARGIN = 0.999, 0.0025, 2e-4
FLIPS, CODE_STEP = 2, 1.0 / 8.0


def _model_pmax(ref, rows, causal, scale, bias):
    """Largest softmax probability of each row under the recipe's own
    dequantised e4m3 scores (the row constant from the K mean cancels)."""
    table = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    out = np.empty(len(rows))
    for r, (b, h, i) in enumerate(rows):
        n = i + 1 if causal else ref["kq"].shape[2]
        qv = table[ref["qq"][b, h, i]] * float(ref["sq"][b, h, i // 64])
        kb = np.arange(n) // 64
        kd = table[ref["kq"][b, h, :n]] * ref["sk"][b, h, kb].astype(np.float64)[:, None]
        s = scale * (kd @ qv)
        if bias is not None:
            s = s + bias[b, h, i // 64, kb]
        if not np.isfinite(s).any():
            out[r] = 0.0
            continue
        e = np.exp(s - s[np.isfinite(s)].max())
        out[r] = e.max() / e.sum()
    return out


def _prep_both(inp, qk="fp8"):
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    prep = attn.sage8_prep(q, k, v, qk=qk)
    ref = oracle.sage8_prepare(*(inp[n].float().numpy() for n in ("q", "k", "v")), qk=qk)
    return prep, ref


def _check(inp, causal, scale, rows=None, label="", check_oracle=True):
    B, H, N, d = inp["q"].shape
    print(f"[gpu] fp8qk {label} shape={(B, H, N, d)} causal={causal}", flush=True)
    prep, ref = _prep_both(inp)
    bias = inp["bias"].to(DEV) if inp["bias"] is not None else None
    o, lse = attn.fwd_sage8(prep, causal=causal, scale=scale, bias=bias, out_dtype=torch.float32,
                            return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    if rows is None:
        rows = np.array([(b, h, i) for b in range(B) for h in range(H) for i in range(N)], dtype=np.int64)
    got = workloads.gather_rows(o, rows)
    idx = torch.as_tensor(rows, device=DEV)
    got_l = lse[idx[:, 0], idx[:, 1], idx[:, 2]].double().cpu().numpy()
    bn = inp["bias"].numpy() if inp["bias"] is not None else None
    o_emu, l_emu = oracle.sage8_emulate_rows_fp32(ref, rows, causal=causal, scale=scale, bias=bn)
    m_emu = workloads.error_metrics(got, o_emu)
    fin = np.isfinite(l_emu)
    assert np.array_equal(fin, np.isfinite(got_l)), label
    lse_err = float(np.abs(got_l[fin] - l_emu[fin]).max()) if fin.any() else 0.0
    row_err = np.abs(got - o_emu).max(axis=1)
    vmax = np.abs(inp["v"].float().numpy()).max(axis=(2, 3))[rows[:, 0], rows[:, 1]]
    pmax = _model_pmax(ref, rows, causal, scale, bn)
    bound = EMU_ROW_ABS + FLIPS * CODE_STEP * pmax * 2.0 * vmax
    n_out = int((row_err > EMU_ROW_ABS).sum())
    print(f"    vs fp32 model: {m_emu} lse {lse_err:.2e}; rows past {EMU_ROW_ABS}: {n_out}"
          f"/{len(rows)}; worst row/bound {float((row_err / bound).max()):.3f}", flush=True)
    assert (row_err <= bound).all(), (label, m_emu, np.argmax(row_err / bound))
    assert n_out <= max(2, int(0.10 * len(rows))), (label, n_out)
    assert lse_err <= EMU_LSE, (label, lse_err)
    if check_oracle:
        qn, kn, vn = (inp[n].float().numpy() for n in ("q", "k", "v"))
        o_ref, _ = oracle.attn_rows(qn, kn, vn, rows, causal=causal, scale=scale, bias=bn)
        o_model, _ = oracle.sage8_emulate_rows(ref, rows, causal=causal, scale=scale, bias=bn)
        m_ref = workloads.error_metrics(got, o_ref)
        m_model = workloads.error_metrics(o_model, o_ref)
        print(f"    vs fp64 attention: {m_ref}; fp64 model of the recipe: {m_model}", flush=True)
        assert m_ref["rel_l1"] <= m_model["rel_l1"] + REL_L1_MARGIN, (label, m_ref, m_model)
        assert m_ref["cos"] >= m_model["cos"] - COS_MARGIN, (label, m_ref, m_model)
        if m_model["cos"] >= COS_MIN + COS_MARGIN:
            assert m_ref["cos"] >= COS_MIN, (label, m_ref, m_model)
    return o, rows


@pytest.mark.parametrize("N", [1, 63, 64, 65, 200, 300])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_prep_bit_exact(N, d, dtype):
    inp = workloads.make_inputs(2, 2, N, d, dtype, seed=5 * N + d, outliers=(N % 2 == 0))
    print(f"[gpu] fp8qk prep N={N} d={d} {dtype}", flush=True)
    prep, ref = _prep_both(inp)
    torch.cuda.synchronize()
    cpu = {k: v.cpu() for k, v in attn.sage8_workspace_views(prep).items()}
    for name in ("qq", "kq"):
        codes = cpu[name].numpy().view(np.uint8)
        assert np.array_equal(codes[:, :, :N], ref[name]), name
        assert not codes[:, :, N:].any(), f"{name} padding"
    nb = (N + 63) // 64
    for name in ("sq", "sk"):
        assert np.array_equal(cpu[name][:, :, :nb].numpy().view(np.uint32), ref[name].view(np.uint32)), name
    assert np.array_equal(cpu["kmean"].numpy().view(np.uint32), ref["kmean"].view(np.uint32))
    assert np.array_equal(cpu["vq_logical"][:, :, :N].numpy(), ref["vq"])


@pytest.mark.parametrize("N", [1, 17, 64, 65, 129, 300])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("with_bias", [False, True])
def test_small_sweep(N, d, causal, with_bias):
    inp = workloads.make_inputs(1, 2, N, d, "bf16", seed=N * 17 + d + causal, gate=with_bias)
    _check(inp, causal, 1 / math.sqrt(d), label=f"sweep N={N} d={d} bias={with_bias}", check_oracle=N >= 64)


@pytest.mark.parametrize("d", [96, 128])
def test_outliers_long_rows(d):
    inp = workloads.make_inputs(1, 2, 2048 + 37, d, "bf16", seed=23 + d, outliers=True)
    rows = workloads.parity_rows(1, 2, 2048 + 37, seed=23, n_random=32)
    _check(inp, True, 1 / math.sqrt(d), rows=rows, label=f"outliers N=2085 d={d}")


def test_block_sparse_and_scale_edges():
    inp = workloads.make_inputs(1, 2, 700, 64, "bf16", seed=29, gate=True, gate_keep=0.25)
    _check(inp, False, 0.125, label="sparse gates")
    inp = workloads.make_inputs(1, 2, 150, 128, "bf16", seed=31)
    for scale in (0.0, -0.125):
        _check(inp, True, scale, label=f"scale={scale}", check_oracle=scale != 0.0)


@pytest.mark.parametrize("cfg_id", [4, 5, 3])
def test_workload_sampled(cfg_id):
    cfg, inp = workloads.config_inputs(cfg_id)
    rows = workloads.parity_rows(cfg["B"], cfg["H"], cfg["N"], seed=cfg_id, n_random=24)
    _check(inp, cfg["causal"], 1 / math.sqrt(cfg["d"]), rows=rows, label=f"workload {cfg['name']}")


def test_int8_scores_beat_fp8_scores_on_outliers():
    """The comparison the variant exists for: on the channel-outlier workload
    the INT8 recipe is the more accurate one (page 1, "SageAttention": INT8
    for the first product), by the same margin as in the fp64 models."""
    cfg = workloads.CONFIGS[4]
    inp = workloads.make_inputs(1, 4, 4096, 128, "bf16", seed=4, outliers=True)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    rows = workloads.parity_rows(1, 4, 4096, seed=4, n_random=32)
    qn, kn, vn = (inp[n].float().numpy() for n in ("q", "k", "v"))
    o_ref, _ = oracle.attn_rows(qn, kn, vn, rows, causal=True)
    res = {}
    for qk in ("int8", "fp8"):
        o = attn.fwd_sage8(attn.sage8_prep(q, k, v, qk=qk), causal=True, out_dtype=torch.float32)
        torch.cuda.synchronize()
        res[qk] = workloads.error_metrics(workloads.gather_rows(o, rows), o_ref)
    print(f"    int8 scores: {res['int8']}; fp8 scores: {res['fp8']}", flush=True)
    assert res["int8"]["rel_l1"] < res["fp8"]["rel_l1"] and res["int8"]["cos"] > res["fp8"]["cos"]
    assert cfg["outliers"]


@pytest.mark.parametrize("d", [64, 96, 128])
def test_deterministic(d):
    """Two calls on the same FP8-QK workspace give the same O and LSE bit for
    bit (no NaN anywhere, so torch.equal compares every value)."""
    inp = workloads.make_inputs(2, 2, 700, d, "bf16", seed=70 + d, outliers=True)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    prep = attn.sage8_prep(q, k, v, qk="fp8")
    o1, l1 = attn.fwd_sage8(prep, causal=True, return_lse=True)
    o2, l2 = attn.fwd_sage8(prep, causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all() and torch.isfinite(l1).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
