"""Issue costs of the instructions the attention kernels are built from, and
the shader clock under a full-chip matrix load, on gfx950.

The performance reasoning about the kernels (the 8-bit forward bound by its
per-score VALU work, the matrix unit's share of the datasheet peak) rests on
these figures; the probe kernels (tests/probes/issue_rate_probe.hip, built by
__graft_entry__.build()) measure them with the shader cycle counter on
independent instruction chains, so no instruction waits for the previous one,
and the LDS read bandwidth of one CU with the two read forms the kernels use
for their matrix operands, alone and feeding a stream of products.
The assertions hold only what the published peak rates fix (at most 32 fp32
FMA lanes per SIMD and cycle, so a wave64 VALU instruction of one SIMD takes
at least 2 cycles; a matrix instruction cannot beat the datasheet peak:
32 cycles for the 32x32x16 bf16 and 32x32x32 INT8 shapes, 64 for the 32x32x64
FP8 shape), that waves sharing a SIMD cannot run faster than one alone, and
generous upper limits; the measured values are printed (run with -s).
"""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libprobes.so")

# kind: (name, instructions per probe round per wave, lower bound, upper bound) in
# cycles per instruction for one wave alone on its SIMD
KINDS = {
    0: ("v_fma_f32", 64, 2.0, 12.0),
    1: ("v_exp_f32", 64, 2.0, 40.0),
    2: ("v_cvt_pk_fp8_f32", 64, 2.0, 40.0),
    3: ("mfma 32x32x16 bf16", 32, 31.0, 100.0),
    4: ("mfma 32x32x32 i8", 32, 31.0, 100.0),
    5: ("mfma 32x32x64 fp8", 32, 62.0, 200.0),
    13: ("mfma 32x32x16 bf16, each onto the previous result", 32, 31.0, 200.0),
}


def _lib():
    if not os.path.exists(LIB):
        raise FileNotFoundError(f"{LIB} is not built: run tests/probes/build.py (or __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    L.issue_rate_probe_run.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3
    L.issue_rate_probe_run.restype = ctypes.c_int
    return L


def _run(kind, wgs, waves, iters):
    L = _lib()
    n = wgs * waves
    cyc = torch.zeros(2 * n, dtype=torch.int64, device="cuda")
    sink = torch.zeros(64 * n, dtype=torch.float32, device="cuda")
    st = L.issue_rate_probe_run(kind, wgs, waves, iters, cyc.data_ptr(), sink.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0, st
    torch.cuda.synchronize()
    return cyc.cpu().numpy().astype(np.float64).reshape(n, 2)


def _alone(kind, iters):
    """Cycles per instruction of one wave alone on the chip (best of three)."""
    per_round = KINDS[kind][1] if kind in KINDS else 64
    _run(kind, 1, 1, 50)  # warm the code path
    return min(float(np.diff(_run(kind, 1, 1, iters)[0])[0]) for _ in range(3)) / (iters * per_round)


@pytest.mark.parametrize("kind", sorted(KINDS))
def test_single_wave_issue_cost(kind):
    name, per_round, lo, hi = KINDS[kind]
    cpi = _alone(kind, 8000 if per_round == 64 else 2000)
    print(f"    {name}: {cpi:.2f} shader cycles per wave64 instruction (one wave per SIMD)", flush=True)
    assert lo <= cpi <= hi


@pytest.mark.parametrize("per_simd", [2, 3, 4])
def test_waves_sharing_a_simd(per_simd):
    """4 * per_simd waves in one workgroup (per_simd waves on each SIMD): the
    VALU and the matrix unit belong to the SIMD, so the SIMD's cost per
    instruction is the workgroup's span (first start to last end) over the
    per_simd * count instructions each SIMD ran."""
    for kind in (0, 1, 2, 3):
        name, per_round, lo, _ = KINDS[kind]
        iters = 4000 if per_round == 64 else 1000
        alone = _alone(kind, iters)
        t = _run(kind, 1, 4 * per_simd, iters)
        simd = float(t[:, 1].max() - t[:, 0].min()) / (per_simd * iters * per_round)
        print(f"    {name}, {per_simd} waves per SIMD: {simd:.2f} cycles per instruction of the SIMD "
              f"(one wave alone: {alone:.2f})", flush=True)
        assert simd >= 0.95 * lo


def test_matrix_and_valu_overlap():
    """One bf16 32x32x16 product plus eight v_fma_f32 per step, on independent
    registers: how much of the VALU work hides behind the product."""
    mix = _alone(6, 1000) * 64 / 32
    mf = _alone(3, 1000)
    fma = _alone(0, 4000)
    serial = mf + 8 * fma
    print(f"    one product + 8 fma: {mix:.1f} cycles per step (product alone {mf:.1f}, "
          f"8 fma alone {8 * fma:.1f}, both in series {serial:.1f}); "
          f"{100 * (serial - mix) / (8 * fma):.0f}% of the VALU time hidden", flush=True)
    assert 0.95 * mf <= mix <= serial * 1.1


def test_matrix_and_exp_overlap():
    """One bf16 32x32x16 product plus four v_exp_f32 per step (independent
    registers): whether the exponentials hide behind the products."""
    mix = _alone(14, 1000) * 64 / 32
    mf = _alone(3, 1000)
    ex = _alone(1, 4000)
    serial = mf + 4 * ex
    print(f"    one product + 4 exp: {mix:.1f} cycles per step (product alone {mf:.1f}, "
          f"4 exp alone {4 * ex:.1f}, both in series {serial:.1f}); "
          f"{100 * (serial - mix) / (4 * ex):.0f}% of the exponential time hidden", flush=True)
    assert 0.95 * mf <= mix <= serial * 1.1


def test_exp_on_another_wave_of_the_simd():
    """Eight waves: the first four run bf16 products, the other four run
    exponentials for longer (three times the rounds), and each wave reports
    the SIMD it ran on.  The product waves' cycles per product against one
    product wave alone: whether exponentials on one wave slow the product
    stream of another wave on the same SIMD (within one wave they do not
    overlap, test_matrix_and_exp_overlap)."""
    L = _lib()
    iters = 1000
    alone = _alone(3, iters)
    ex = _alone(1, 4000)
    n = 8
    cyc = torch.zeros(2 * n, dtype=torch.int64, device="cuda")
    sink = torch.zeros(64 * n, dtype=torch.float32, device="cuda")
    for it in (50, iters):
        assert L.issue_rate_probe_run(15, 1, n, it, cyc.data_ptr(), sink.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
    t = cyc.cpu().numpy().astype(np.float64).reshape(n, 2)
    simd = sink[n:2 * n].cpu().numpy().astype(int)
    prod = [w for w in range(4) if any(simd[e] == simd[w] for e in range(4, 8))]
    assert prod, f"no product wave shares a SIMD with an exponential wave: {simd.tolist()}"
    cpp = [float(np.diff(t[w])[0]) / (iters * 32) for w in prod]
    # 6 exponentials per product of the partner wave (3 * 64 per 32 products)
    serial = alone + 6 * ex
    print(f"    SIMD of each wave {simd.tolist()}; product waves beside exponential waves: "
          f"{[round(x, 1) for x in cpp]} cycles per product (alone {alone:.1f}; in series with the "
          f"partner's exponentials {serial:.1f})", flush=True)
    assert all(0.95 * 31.0 <= x <= 1.1 * serial for x in cpp)


def test_exp_beside_fma():
    """v_exp_f32 and v_fma_f32 alternating on separate chains, one wave: the
    cost of the pair against the two alone."""
    pair = _alone(8, 4000)
    ex = _alone(1, 4000)
    fma = _alone(0, 4000)
    print(f"    exp + fma pair: {pair:.2f} cycles (exp alone {ex:.2f}, fma alone {fma:.2f}, "
          f"sum {ex + fma:.2f})", flush=True)
    assert max(ex, fma) * 0.95 <= pair <= (ex + fma) * 1.1


@pytest.mark.parametrize("kind", [9, 10])
def test_lds_read_bandwidth(kind):
    """LDS read bandwidth of one CU: one workgroup of 8 or 16 waves streaming
    16-byte reads (kind 9) or 8-byte transposing reads (kind 10) from
    consecutive addresses; bytes read by all waves over the workgroup's span."""
    name, per_instr = {9: ("ds_read_b128", 1024), 10: ("ds_read_b64_tr_b16", 512)}[kind]
    iters = 2000
    for waves in (8, 16):
        _run(kind, 1, waves, 50)
        t = _run(kind, 1, waves, iters)
        span = float(t[:, 1].max() - t[:, 0].min())
        bpc = waves * iters * 8 * per_instr / span
        print(f"    {name}, {waves} waves on one CU: {bpc:.1f} bytes per shader cycle", flush=True)
        assert 0.0 < bpc <= 512.0


@pytest.mark.parametrize("kind", [11, 12])
def test_lds_fed_product_stream(kind):
    """Back-to-back bf16 32x32x16 products whose A operand comes from LDS,
    read two products ahead (kind 11: 16-byte reads; kind 12: two 8-byte
    transposing reads per product), with one, two and four waves per SIMD:
    the cycles per product of each SIMD (32 would keep the matrix unit busy).
    One wave alone cannot hide its own read latency; a second wave on the
    SIMD covers it."""
    name = {11: "ds_read_b128", 12: "2x ds_read_b64_tr_b16"}[kind]
    iters = 500
    for per_simd in (1, 2, 4):
        waves = 4 * per_simd
        _run(kind, 1, waves, 20)
        t = _run(kind, 1, waves, iters)
        cpp = float(t[:, 1].max() - t[:, 0].min()) / (per_simd * iters * 16)
        print(f"    products fed by {name}, {per_simd} waves per SIMD: {cpp:.1f} cycles per product "
              f"({100 * 32 / cpp:.0f}% of the matrix unit)", flush=True)
        assert 31.0 <= cpp <= 96.0


def test_clock_under_full_matrix_load():
    """Every CU's SIMDs run bf16 products for ~0.1 s; shader cycles over the
    100 MHz real-time counter give the clock the chip sustains under that
    load (the datasheet peak assumes 2.4 GHz)."""
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    _run(7, 2 * cus, 8, 2000)  # ramp
    out = _run(7, 2 * cus, 8, 40000)
    ghz = out[:, 0] / out[:, 1] * 0.1
    print(f"    shader clock under a full bf16 matrix load on {cus} CUs: median {np.median(ghz):.3f} GHz "
          f"(min {ghz.min():.3f}, max {ghz.max():.3f}) over {len(ghz)} waves", flush=True)
    assert 0.8 <= float(np.median(ghz)) <= 2.45
