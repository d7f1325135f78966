"""Build libdsa.so (HIP, gfx950) in-tree with hipcc.

    python -m long_context_lightning_amd.build

Every HIP source under csrc/ is compiled for gfx950 only, with packed-fp32
instructions disabled, into one shared library next to this file.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdsa.so")

SOURCES = ["api.hip", "indexer.hip", "topk.hip", "prefill.hip", "sparse_mla.hip", "quant.hip", "paged.hip", "mha.hip", "kl.hip"]

FLAGS = [
    "-O3",
    "-std=c++17",
    # no kernel relies on NaN propagation (masks use -inf, which stays
    # honoured); without this, IEEE mode canonicalises every fmaxf input
    "-fno-honor-nans",
    "--offload-arch=gfx950",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    "-fvisibility=hidden",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libdsa)")
    return exe


def build(verbose=False, extra_flags=()):
    """Compile libdsa.so; raises CalledProcessError on failure."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        sys.stderr.write(err + "\n")
        raise subprocess.CalledProcessError(res.returncode, cmd, res.stdout, err)
    if verbose and err.strip():
        sys.stderr.write(err + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
