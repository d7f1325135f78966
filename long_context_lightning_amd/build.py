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


def m0_violations(asm_text):
    """Lines of gfx950 device assembly that reference m0 outside an inline
    asm block.  The LDS-DMA helpers (dsa_internal.h) set m0 from inline asm
    right before each global_load_lds; the backend treats m0 as reserved and
    does not honour a clobber of it, so the kernels stay correct only while the
    compiler itself never reads or writes m0 in them (no LDS-DMA builtin,
    s_sendmsg, relative register moves, ...)."""
    import re
    implicit = re.compile(r"^\s*(v_movrel|s_movrel|s_sendmsg|v_interp|ds_gws|ds_append|ds_consume|ds_ordered_count|"
                          r"global_load_lds|buffer_load\S*\s.*\blds\b)")
    bad, in_asm = [], False
    for n, line in enumerate(asm_text.splitlines(), 1):
        if ";;#ASMSTART" in line:
            in_asm = True
        elif ";;#ASMEND" in line:
            in_asm = False
        else:
            code = line.split(";")[0]
            if not in_asm and ("m0" in code.replace(",", " ").split() or implicit.match(code)):
                bad.append((n, line.strip()))
    return bad


def check_m0(verbose=False):
    """Compile every source to gfx950 device assembly and fail if the
    compiler references m0 anywhere outside the inline asm blocks."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    def one(src):
        with tempfile.TemporaryDirectory() as d:
            out = os.path.join(d, src + ".s")
            cmd = [hipcc(), *[f for f in FLAGS if f not in ("-shared", "-fPIC")], "--cuda-device-only", "-S",
                   "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, src), "-o", out]
            res = subprocess.run(cmd, capture_output=True, text=True)
            if res.returncode != 0:
                raise subprocess.CalledProcessError(res.returncode, cmd, res.stdout, res.stderr)
            return src, m0_violations(open(out).read())

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        found = [r for r in ex.map(one, SOURCES) if r[1]]
    if found:
        msg = "; ".join(f"{src}: line {n}: {text}" for src, lines in found for n, text in lines[:3])
        raise RuntimeError(f"compiler-generated m0 use next to the inline-asm LDS copies: {msg}")
    if verbose:
        print(f"m0 check: no compiler use of m0 in {len(SOURCES)} sources", flush=True)


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
    check_m0(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
