"""Build libspecdec.so (the HIP kernels and their C ABI) in-tree for gfx950,
and libspecdec_debug.so: the same sources with SPECDEC_DEBUG_KNOBS, whose
kernels read the tuning and test switches from the environment (tests that
compare paths or force a wait timeout load it; the product library reads no
environment)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libspecdec.so")
DEBUG_LIB = os.path.join(LIBDIR, "libspecdec_debug.so")
SOURCES = ["stats.hip", "verify.hip", "truncate.hip", "tree.hip", "ngram.hip", "commit.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no contraction: the sampling pass recomputes the chunk masses bit for bit
    "-ffp-contract=off",
    # packed fp32 instructions stay off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _command(out: str, debug: bool):
    return [hipcc(), *HIPCC_FLAGS, *(["-DSPECDEC_DEBUG_KNOBS"] if debug else []), "-I", INCLUDE,
            "-o", out, *[os.path.join(CSRC, s) for s in SOURCES]]


def build(verbose: bool = False) -> str:
    """Compiles both libraries (two hipcc processes side by side)."""
    os.makedirs(LIBDIR, exist_ok=True)
    jobs = []
    for out, debug in ((LIB, False), (DEBUG_LIB, True)):
        cmd = _command(out + ".tmp", debug)
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    failed = False
    for out, proc in jobs:
        _, err = proc.communicate()
        # the host pass does not know the packed-fp32 feature name: not an error
        noise = [ln for ln in err.splitlines()
                 if ln.strip() and "packed-fp32-ops" not in ln and "hip-link" not in ln]
        if proc.returncode != 0:
            sys.stderr.write(err)
            failed = True
            continue
        if noise and verbose:
            sys.stderr.write("\n".join(noise) + "\n")
        os.replace(out + ".tmp", out)
    if failed:
        raise RuntimeError("hipcc failed to build libspecdec")
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
