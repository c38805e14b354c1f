"""Entry points called from several host threads at once.

The library promises that concurrent calls from different host threads
(each on its own outputs and stream) are safe.  The host state it keeps is
a cache of resident workgroup slots per kernel and device, filled by the
first launch of each kernel (it sizes the persistent and heaviest-first
grids).  A child process, so that this cache starts empty, runs 8 threads
that each launch the bf16 forward, the 8-bit preparation and forward and
the backward on their own stream at the same moment.  Afterwards the main
thread repeats every call on the default stream.  Each thread's outputs must
equal the serial ones bit for bit.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import threading
import torch
import bit_attention_attn_amd as attn

THREADS = 8
dev = torch.device("cuda:0")
# causal shapes whose launches consult the slot cache (persistent grid,
# heaviest-first order), d = 128 and 64
SHAPES = [(1, 8, 2048, 128), (2, 4, 1024, 64)]
inputs = []
for t in range(THREADS):
    B, H, N, d = SHAPES[t % len(SHAPES)]
    g = torch.Generator(device=dev).manual_seed(t)
    q, k, v, do = (torch.randn((B, H, N, d), device=dev, dtype=torch.bfloat16, generator=g) for _ in range(4))
    inputs.append((q, k, v, do))
torch.cuda.synchronize()

def work(q, k, v, do):
    o, lse = attn.fwd(q, k, v, causal=True, return_lse=True)
    prep = attn.sage8_prep(q, k, v)
    o8 = attn.fwd_sage8(prep, causal=True)
    dq, dk, dv = attn.bwd(q, k, v, o, do, lse, causal=True)[:3]
    return [o, lse, o8, dq, dk, dv]

results = [None] * THREADS
errors = []
start = threading.Barrier(THREADS)

def run(t):
    try:
        s = torch.cuda.Stream(device=dev)
        with torch.cuda.stream(s):
            start.wait()
            out = work(*inputs[t])
        s.synchronize()
        results[t] = out
    except Exception as e:  # reported by the main thread
        errors.append(repr(e))

threads = [threading.Thread(target=run, args=(t,)) for t in range(THREADS)]
for th in threads:
    th.start()
for th in threads:
    th.join()
assert not errors, errors
torch.cuda.synchronize()
for t in range(THREADS):
    ref = work(*inputs[t])
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(results[t], ref)):
        assert torch.equal(a, b), (t, i)
print("threads: all outputs equal the serial calls")
"""


def test_concurrent_host_threads():
    print("[gpu] 8 host threads, forward + 8-bit + backward", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, capture_output=True, text=True, timeout=240)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "all outputs equal the serial calls" in r.stdout, tail
