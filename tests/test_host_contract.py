"""CPU checks of the host-side contract: the binding refuses to run without
the HIP library (there is no CPU fallback), and bench.py measures one GPU only,
refusing any other --gpus value before it touches a device."""

import os
import subprocess
import sys

import pytest

import long_context_lightning_amd as lcl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_binding_raises_without_the_library(tmp_path):
    saved = lcl._lib
    try:
        lcl._lib = None
        with pytest.raises(RuntimeError, match="not found"):
            lcl.load(str(tmp_path / "libdsa.so"))
        assert lcl._lib is None
    finally:
        lcl._lib = saved


@pytest.mark.parametrize("n", [0, 2, 8])
def test_bench_refuses_other_gpu_counts(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert f"--gpus {n} is not supported" in r.stderr
    assert r.stdout == ""
