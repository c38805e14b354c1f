"""The oracle's C code under the host sanitizers: AddressSanitizer and
UndefinedBehaviorSanitizer (every report fatal), single-threaded.

The oracle library is rebuilt from the same sources with the sanitizers
(oracle/build.py: build_sanitized) and a child Python process loads it in
place of the normal build (ATTN_ORACLE_LIB, with the ASan runtime preloaded),
then drives every entry point on small and edge-case shapes: a single row,
ragged block tails, causal masks, a bias with gated-off blocks, the backward,
the 8-bit preparation in both formats and its forward models, and all 256
e4m3 codes.  Any out-of-bounds access, use of freed memory or undefined
arithmetic (signed overflow, bad shifts, misaligned loads) aborts the child.
A second child plants an undersized output buffer to show that the harness
reports it.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import numpy as np
import oracle, workloads
assert oracle._LIB_PATH.endswith("liboracle_san.so"), oracle._LIB_PATH
table = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
for v in (0.0, 1e-9, 0.0019, 0.5, 1.0, 300.0, 448.0, 464.0, -3.25, float(table[1]), float(table[127])):
    oracle.e4m3_encode(v)
for (B, H, N, d, causal, gate, keep) in ((1, 1, 1, 64, False, False, None), (1, 2, 65, 64, True, True, None),
                                         (2, 1, 130, 96, True, True, 0.5), (1, 1, 70, 128, False, True, 0.3)):
    inp = workloads.make_inputs(B, H, N, d, "bf16", seed=N + d, gate=gate, gate_keep=keep, outliers=True)
    q, k, v = (inp[n].float().numpy() for n in ("q", "k", "v"))
    bias = inp["bias"].numpy() if inp["bias"] is not None else None
    rows = np.array([(b, h, i) for b in range(B) for h in range(H) for i in range(N)], dtype=np.int64)
    o, l = oracle.attn_rows(q, k, v, rows, causal=causal, bias=bias)
    assert np.isfinite(o).all()
    oracle.row_probs(q, k, 0, 0, N - 1, causal=causal, bias=bias)
    dout = np.ones_like(q)
    dq, dk, dv, db = oracle.attn_bwd(q, k, v, dout, causal=causal, bias=bias)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    for qk in ("int8", "fp8"):
        prep = oracle.sage8_prepare(q, k, v, qk=qk)
        o8, l8 = oracle.sage8_emulate_rows_fp32(prep, rows, causal=causal, bias=bias)
        o9, l9 = oracle.sage8_emulate_rows(prep, rows, causal=causal, bias=bias)
        assert np.isfinite(o8).all() and np.isfinite(o9).all()
print("sanitized oracle: all entry points ran")
"""


# A planted mistake: the output buffer of attn_oracle_rows one row short.  The
# sanitized build must stop the child at the first write past it.
CHILD_OVERFLOW = r"""
import ctypes
import numpy as np
import oracle
lib = oracle._load()
B, H, N, d = 1, 1, 128, 128
q = np.random.default_rng(0).standard_normal((B, H, N, d)).astype(np.float32)
rows = np.array([(0, 0, i) for i in range(N)], dtype=np.int64)
out = np.zeros(((N - 1) * d,), dtype=np.float64)
lse = np.zeros((N,), dtype=np.float64)
p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
lib.attn_oracle_rows(p(q), p(q), p(q), None, B, H, N, d, 0, 0.125, p(rows), N, p(out), p(lse), 1)
print("no report")
"""


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    from oracle import build as obuild
    lib = obuild.build_sanitized(str(tmp_path_factory.mktemp("san") / "liboracle_san.so"))
    env = dict(os.environ)
    env.update(ATTN_ORACLE_LIB=lib, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="1")
    return env


def _child(env, code):
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=600)


def test_oracle_under_asan_and_ubsan(sanitized):
    r = _child(sanitized, CHILD)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
    assert "all entry points ran" in r.stdout, tail


def test_sanitizer_catches_a_planted_overflow(sanitized):
    """The harness is live: a call with an output buffer one row short aborts
    with an AddressSanitizer heap-buffer-overflow report."""
    r = _child(sanitized, CHILD_OVERFLOW)
    assert r.returncode != 0 and "no report" not in r.stdout
    assert "AddressSanitizer: heap-buffer-overflow" in r.stderr, (r.stdout + r.stderr)[-3000:]
