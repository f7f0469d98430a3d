"""Host-side launch logic of the library, checked on the CPU.

tests/host/host_logic_check.hip includes the library source and checks,
without launching a kernel: the XCD-aware block -> tile mapping is a
bijection onto the work items with balanced XCD shares (also when the grid
was sized for more rows than the device finds), the split-count rule's
bounds, and that for every number of rows a chunk may hold after ignored
rows are dropped on the device, the dH grid covers its work and the split-K
partials fit the workspace the plan reserves for them."""

import os
import shutil
import subprocess

import pytest

from lm_head_linear_bf16_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "host_logic_check.hip")


def test_launch_logic(tmp_path):
    cc = build.hipcc()
    if shutil.which(cc) is None and not os.path.exists(cc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "host_logic_check")
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-O3", "-fPIC", "-shared")]
    r = subprocess.run([cc, *flags, "-O1", "-o", exe, SRC], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
