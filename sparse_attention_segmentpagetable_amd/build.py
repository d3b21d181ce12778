"""Compile libsegpaged.so in-tree for gfx950 with hipcc (the HIP kernels, the
C-ABI and the host planner in one shared library), and libsegpaged_probe.so
(the rate probes of include/segpaged_probe.h, used for measurement only)."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "lib", "libsegpaged.so")
PROBE_LIB = os.path.join(PKG, "lib", "libsegpaged_probe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden",
    # no packed fp32 ops in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(sources, out, verbose):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)
    os.replace(tmp, out)
    return out


def build_library(verbose: bool = False) -> str:
    _compile(["probe.hip"], PROBE_LIB, verbose)
    return _compile(["planner.cpp", "kernels.hip", "select.hip"], LIB, verbose)


if __name__ == "__main__":
    print(build_library(verbose=True))
