"""attn_bwd_noalloc: the backward with its scratch in the library's fixed
device array, for callers that cannot allocate.  Called through the C ABI
(the binding's bwd_noalloc only marshals arguments) and compared with the
existing entry point attn_bwd_bf16 / attn_bwd_f16 on the same inputs: the
kernels are the same, so the results must be identical bit for bit (the
bias gradient adds at most two values onto zero per element, so it too is
the same from run to run).  Two calls in a row, the second on a smaller
shape, so a result left in the shared array by the first call cannot leak
into the second."""
import ctypes

import pytest
import torch

import bit_attention_attn_amd as attn

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(B, H, N, d, dtype, causal, seed, with_bias):
    g = torch.Generator("cpu").manual_seed(seed)
    q, k, v, dout = (torch.randn((B, H, N, d), generator=g).to(dtype).to(DEV) for _ in range(4))
    nb = (N + 63) // 64
    bias = torch.randn((B, H, nb, nb), generator=g).to(DEV) if with_bias else None
    o, lse = attn.fwd(q, k, v, causal=causal, bias=bias, return_lse=True)
    return q, k, v, dout, o, lse, bias


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_noalloc_matches_workspace_entry_twice(dtype):
    shapes = [(2, 4, 700, 128, True, True), (1, 3, 150, 64, False, False)]  # second call smaller
    for n, (B, H, N, d, causal, with_bias) in enumerate(shapes):
        print(f"[gpu] bwd noalloc call {n}: {(B, H, N, d)} {dtype} causal={causal} bias={with_bias}", flush=True)
        q, k, v, dout, o, lse, bias = _inputs(B, H, N, d, dtype, causal, 100 + n, with_bias)
        ref = attn.bwd(q, k, v, o, dout, lse, causal=causal, bias=bias, return_dbias=True)
        got = attn.bwd_noalloc(q, k, v, o, dout, lse, causal=causal, bias=bias, return_dbias=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "dbias"), got, ref):
            assert torch.isfinite(b).all(), name
            assert torch.equal(a, b), (n, name, float((a.float() - b.float()).abs().max()))


def test_noalloc_rejects_more_rows_than_its_array():
    """B*H*N past ATTN_BWD_NOALLOC_MAX_ROWS (4,194,304) is ATTN_ERR_WORKSPACE,
    before any device work (the pointers are never dereferenced)."""
    fn = attn.lib().attn_bwd_noalloc
    fake = ctypes.c_void_p(0x100000)
    st = fn(1, fake, fake, fake, fake, 1, fake, fake, fake, fake, fake, None, 1, 1, 4194304 + 64, 64, 0, 0.125,
            None, 1, None)
    assert st == 7
