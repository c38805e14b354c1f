"""Build the CPU oracle library (oracle/liboracle.so) with gcc.

Test infrastructure only: the oracle is a plain fp64 C implementation used by
the tests, the smoke check and the benchmark's CPU-baseline leg.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["attn_oracle.c", "sage8_oracle.c"]
LIB = os.path.join(HERE, "liboracle.so")

# No fast-math and no FMA contraction: the quantisation steps must round
# exactly as written.
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


# Host sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer) for the
# tests: single-threaded (no OpenMP), every undefined-behaviour report fatal.
SAN_CFLAGS = ["-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
              "-Wall", "-Wextra", "-Wno-unknown-pragmas", "-fno-omit-frame-pointer",
              "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def build_sanitized(out_path: str, verbose: bool = False) -> str:
    srcs = [os.path.join(HERE, s) for s in SOURCES]
    cmd = ["gcc", *SAN_CFLAGS, *srcs, "-o", out_path, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out_path


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(HERE, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, *srcs, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
