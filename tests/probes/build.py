"""Build the test probes (tests/probes/libprobes.so) for gfx950 with hipcc.

Test infrastructure only: small kernels that measure properties of the
hardware the parity bars depend on.  The library under test never loads them.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["fp8_mfma_probe.hip", "issue_rate_probe.hip"]
LIB = os.path.join(HERE, "libprobes.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc", "-O2", "-std=c++17",
           "-fPIC", "-shared", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           *[os.path.join(HERE, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the test probes:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
