"""GPU parity of the INT8-score variant with the 16-bit P V product
(``attn_fwd_sage8_pv16``).  Two bars, each against code under oracle/ only:

  * against the fp64 model of the variant (``oracle.sage8_qk8_rows``: the
    exact softmax of the dequantised INT8 scores times the exact 16-bit V),
    fed the oracle's own quantised data: the 16-bit path's bars, max abs
    <= 1e-2 and mean abs <= 1e-3, LSE within ln(1 + 2^-8) + 2^-12 for bf16
    (2e-3 for fp16).  After the scores the kernel's arithmetic is the 16-bit
    path's: P rounded to the input dtype, fp32 accumulation, one rounding of
    O.  The scores themselves are exact integers, dequantised in fp32
    (f = sq * sk * scale * log2 e, one rounding each, and the folded offset
    of 1.5 * 2^23 within a few ulp of it, far below these bars);
  * against the exact fp64 attention of the same rounded inputs: cosine
    >= 0.999 and relative L1 <= 2e-2, the 8-bit tolerance asked of the path.
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
MAX_ABS, MEAN_ABS = 1e-2, 1e-3
LSE_TOL = {torch.bfloat16: math.log1p(2.0 ** -8) + 2.0 ** -12, torch.float16: 2e-3}
COS_MIN, REL_L1_MAX = 0.999, 2e-2


def _check(inp, causal, scale, rows=None, out_dtype=torch.float32, label="", check_exact=True):
    B, H, N, d = inp["q"].shape
    print(f"[gpu] pv16 {label} shape={(B, H, N, d)} {inp['q'].dtype} causal={causal}", flush=True)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    bias = inp["bias"].to(DEV) if inp["bias"] is not None else None
    prep = attn.sage8_prep(q, k, v, qk="int8_no_v")  # INT8 Q and K only, as sageattn_pv16 prepares
    o, lse = attn.fwd_sage8_pv16(prep, v, causal=causal, scale=scale, bias=bias, out_dtype=out_dtype,
                                 return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all(), label
    if rows is None:
        rows = np.array([(b, h, i) for b in range(B) for h in range(H) for i in range(N)], dtype=np.int64)
    got = workloads.gather_rows(o, rows)
    idx = torch.as_tensor(rows, device=DEV)
    got_l = lse[idx[:, 0], idx[:, 1], idx[:, 2]].double().cpu().numpy()
    qn, kn, vn = (inp[n].float().numpy() for n in ("q", "k", "v"))
    bn = inp["bias"].numpy() if inp["bias"] is not None else None
    ref = oracle.sage8_prepare(qn, kn, vn)
    o_m, l_m = oracle.sage8_qk8_rows(ref, vn, rows, causal=causal, scale=scale, bias=bn)
    m = workloads.error_metrics(got, o_m)
    fin = np.isfinite(l_m)
    assert np.array_equal(fin, np.isfinite(got_l)), label
    lse_err = float(np.abs(got_l[fin] - l_m[fin]).max()) if fin.any() else 0.0
    print(f"    vs fp64 model of the variant: {m} lse {lse_err:.2e}", flush=True)
    assert m["max_abs"] <= MAX_ABS and m["mean_abs"] <= MEAN_ABS, (label, m)
    assert lse_err <= LSE_TOL[inp["q"].dtype], (label, lse_err)
    m_ref = None
    if check_exact:
        o_ref, _ = oracle.attn_rows(qn, kn, vn, rows, causal=causal, scale=scale, bias=bn)
        m_ref = workloads.error_metrics(got, o_ref)
        print(f"    vs fp64 attention: {m_ref}", flush=True)
        assert m_ref["cos"] >= COS_MIN and m_ref["rel_l1"] <= REL_L1_MAX, (label, m_ref)
    return o, lse, m, m_ref


FWD_N = [1, 17, 64, 65, 127, 128, 129, 200, 300]


@pytest.mark.parametrize("N", FWD_N)
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("with_bias", [False, True])
def test_small_sweep(N, d, causal, with_bias):
    inp = workloads.make_inputs(1, 2, N, d, "bf16", seed=N * 19 + d + causal, gate=with_bias)
    _check(inp, causal, 1 / math.sqrt(d), label=f"sweep N={N} d={d} bias={with_bias}", check_exact=N >= 64)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("out", ["same", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_dtypes(dtype, out, d):
    inp = workloads.make_inputs(2, 3, 333, d, dtype, seed=13 + d, outliers=True)
    tdt = workloads.torch_dtype(dtype)
    o, _, _, _ = _check(inp, True, 0.088, out_dtype=torch.float32 if out == "f32" else tdt,
                        label=f"{dtype}->{out} d={d}")
    assert o.dtype == (torch.float32 if out == "f32" else tdt)


def test_outliers_long_rows():
    inp = workloads.make_inputs(1, 2, 2048, 128, "bf16", seed=21, outliers=True)
    rows = workloads.parity_rows(1, 2, 2048, seed=21, n_random=32)
    _check(inp, True, 1 / math.sqrt(128), rows=rows, label="outliers N=2048")


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5])
def test_scale_edge_cases(scale):
    inp = workloads.make_inputs(1, 2, 150, 64, "bf16", seed=31)
    _check(inp, True, scale, label=f"scale={scale}", check_exact=scale != 0.5)


def test_fully_masked_rows():
    inp = workloads.make_inputs(1, 1, 192, 64, "bf16", seed=41, gate=True)
    inp["bias"][0, 0, 1, :] = -math.inf
    o, lse, _, _ = _check(inp, False, 0.125, label="masked", check_exact=False)
    assert (o[0, 0, 64:128] == 0).all()
    assert torch.isneginf(lse[0, 0, 64:128]).all()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_gates(d, causal):
    inp = workloads.make_inputs(1, 2, 700, d, "bf16", seed=5 * d + causal, gate=True, gate_keep=0.25)
    _check(inp, causal, 1 / math.sqrt(d), label=f"sparse d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_block_sparse_chunk_boundaries(d):
    inp, rows = workloads.chunk_gate_inputs(d, seed=350 + d)
    _check(inp, True, 1 / math.sqrt(d), rows=rows, label=f"sparse chunks d={d}")


def test_deterministic_and_one_call():
    inp = workloads.make_inputs(2, 2, 500, 128, "bf16", seed=61)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    o1 = attn.sageattn_pv16(q, k, v, causal=True)
    o2 = attn.fwd_sage8_pv16(attn.sage8_prep(q, k, v), v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_rejects_other_preparations():
    inp = workloads.make_inputs(1, 1, 100, 64, "bf16", seed=3)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    with pytest.raises(ValueError):
        attn.fwd_sage8_pv16(attn.sage8_prep(q, k, v, qk="fp8"), v)
    with pytest.raises(ValueError):
        attn.fwd_sage8_pv16(attn.sage8_prep(q, k, v), v.float())
    with pytest.raises(ValueError):  # no FP8 V in a Q/K-only preparation
        attn.fwd_sage8(attn.sage8_prep(q, k, v, qk="int8_no_v"))


@pytest.mark.parametrize("N", [1, 65, 300, 1000])
@pytest.mark.parametrize("d", [64, 96, 128])
def test_qk_only_prep_is_the_int8_prep(N, d):
    """The Q/K-only preparation writes exactly the INT8 preparation's Q and K
    codes, block scales and K mean (and the oracle's quantisers), and the
    variant gives the same output from either."""
    inp = workloads.make_inputs(2, 2, N, d, "bf16", seed=N + 3 * d, outliers=True)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    full = attn.sage8_prep(q, k, v)
    qko = attn.sage8_prep(q, k, v, qk="int8_no_v")
    vf, vo = attn.sage8_workspace_views(full), attn.sage8_workspace_views(qko)
    torch.cuda.synchronize()
    nb = (N + 63) // 64
    for name in ("qq", "kq", "kmean"):
        assert torch.equal(vf[name], vo[name]), name
    for name in ("sq", "sk"):
        assert torch.equal(vf[name][:, :, :nb].view(torch.int32), vo[name][:, :, :nb].view(torch.int32)), name
    ref = oracle.sage8_prepare(*(inp[n].float().numpy() for n in ("q", "k", "v")))
    assert np.array_equal(vo["qq"][:, :, :N].cpu().numpy(), ref["qq"])
    assert np.array_equal(vo["kq"][:, :, :N].cpu().numpy(), ref["kq"])
    o1 = attn.fwd_sage8_pv16(full, v, causal=True)
    o2 = attn.fwd_sage8_pv16(qko, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("with_bias", [False, True])
def test_long_sequence_tiling(causal, with_bias):
    """At d = 128 and N >= 16384 the kernel runs 4-wave workgroups three to a
    CU instead of 8-wave ones: a ragged length, with and without the causal
    mask and a block bias, on sampled rows."""
    N = 16384 + 77
    inp = workloads.make_inputs(1, 2, N, 128, "bf16", seed=71 + causal + 2 * with_bias, gate=with_bias)
    rows = workloads.parity_rows(1, 2, N, seed=7, n_random=16)
    _check(inp, causal, 1 / math.sqrt(128), rows=rows, out_dtype=torch.bfloat16, label=f"long N={N}")


@pytest.mark.parametrize("cfg_id", [4, 5, 2, 3])
def test_workload_sampled_rows(cfg_id):
    """Full-size workloads in the launch configuration the benchmark times:
    sampled rows against the variant's fp64 model and the exact attention."""
    cfg, inp = workloads.config_inputs(cfg_id)
    rows = workloads.parity_rows(cfg["B"], cfg["H"], cfg["N"], seed=cfg_id, n_random=24)
    _check(inp, cfg["causal"], 1 / math.sqrt(cfg["d"]), rows=rows, out_dtype=torch.bfloat16,
           label=f"workload {cfg['name']}")
