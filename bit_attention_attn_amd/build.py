"""Build libattn.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Each source compiles to an object in parallel, then one shared library is
linked next to this file.  Always compiles from scratch when called.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libattn.so")

SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_sage8.hip", "attn_bwd.hip", "attn_bwd_kv.hip"]

ARCH = "gfx950"
# -packed-fp32-ops: no packed fp32 VALU instructions in device code.
# -amdgpu-mfma-vgpr-form: matrix results stay in VGPRs, where the softmax
# reads them, instead of AGPRs that need a copy per element.
# -fno-honor-nans: max/min of matrix results need no NaN-quieting copies (a
# NaN score still reaches the output through exp2); infinities stay honoured.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.exists(c) or c == "hipcc":
            return c
    return "hipcc"


# The key-side backward kernel holds two matrix accumulators of D/32 x 16
# registers each besides its operands: it keeps them in AGPRs instead.
NO_VGPR_FORM = {"attn_bwd_kv.hip"}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    flags = FLAGS
    if src in NO_VGPR_FORM:
        i = flags.index("-amdgpu-mfma-vgpr-form")
        flags = flags[:i - 1] + flags[i + 1:]
    cmd = [_hipcc(), *flags]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l and "(ignoring feature)" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
