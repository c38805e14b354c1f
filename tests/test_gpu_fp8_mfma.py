"""How far gfx950's FP8 (e4m3) matrix instruction sums lie from the exact
sum of their products, on a tile of real codes.

The FP8-QK variant's parity bar rests on this distance: its fp32 model adds
the exact products of a score and rounds once, while the instruction does
not, so a score within that distance of an e4m3 rounding boundary of P^ can
take the neighbouring code.  The probe (tests/probes/fp8_mfma_probe.hip, a
single 32x32x64 product built by __graft_entry__.build()) runs one tile of
the FP8-QK preparation's Q and centred-K codes.  Measured on gfx950: every
output within 2^-12.58 (seed 4) and 2^-12.26 (seed 5) of the largest of its
64 products from the exact sum, and 70-74% of the outputs differ from the
correctly rounded sum; the test holds the distance under 2^-12.  (The FP8-QK bar itself counts e4m3 code flips per
row, which any such distance can cause near a rounding boundary; its own
tests check how many occur.)
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libprobes.so")


def _run(a_codes, b_codes):
    if not os.path.exists(LIB):
        raise FileNotFoundError(f"{LIB} is not built: run tests/probes/build.py (or __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    L.fp8_mfma_probe_run.argtypes = [ctypes.c_void_p] * 4
    L.fp8_mfma_probe_run.restype = ctypes.c_int
    a = torch.from_numpy(np.ascontiguousarray(a_codes, dtype=np.uint8)).cuda()
    b = torch.from_numpy(np.ascontiguousarray(b_codes, dtype=np.uint8)).cuda()
    d = torch.zeros((32, 32), dtype=torch.float32, device="cuda")
    assert L.fp8_mfma_probe_run(a.data_ptr(), b.data_ptr(), d.data_ptr(),
                                torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    return d.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("seed", [4, 5])
def test_fp8_products_sum_within_the_bar(seed):
    inp = workloads.make_inputs(1, 1, 64, 128, "bf16", seed=seed, outliers=True)
    prep = oracle.sage8_prepare(*(inp[n].float().numpy() for n in ("q", "k", "v")), qk="fp8")
    a = prep["qq"][0, 0, :32, :64]          # 32 query rows, 64 channels (e4m3 codes)
    b = prep["kq"][0, 0, 32:64, :64]        # 32 key rows, the same channels
    table = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    ad, bd = table[a], table[b]
    prods = ad[:, None, :] * bd[None, :, :]  # [32, 32, 64], exact in fp64
    exact = prods.sum(axis=2)                # exact in fp64 (64 products of 4-bit mantissas)
    got = _run(a, b)
    scale = np.abs(prods).max(axis=2)
    dev = np.abs(got - exact) / np.where(scale > 0, scale, 1.0)
    not_rne = int((got != exact.astype(np.float32).astype(np.float64)).sum())
    print(f"    max deviation 2^{np.log2(dev.max() + 1e-300):.2f} of the largest product; "
          f"{not_rne}/1024 outputs differ from the correctly rounded sum", flush=True)
    assert dev.max() <= 2.0 ** -12
