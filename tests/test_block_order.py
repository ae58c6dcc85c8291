"""The attention kernels' workgroup order (regrouped per XCD; strips with the
border strips last) is a bijection onto (query block, tile, head, batch), and
the launch-invariant division it decodes with matches plain integer division:
both checked on the host by compiling the device header into small programs."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_block_order_is_a_bijection(tmp_path):
    exe = tmp_path / "block_order_check"
    subprocess.run([HIPCC, "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "partial_context_patch_amd", "csrc"),
                    os.path.join(ROOT, "tests", "block_order_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, timeout=300)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_invariant_division_matches_integer_division(tmp_path):
    exe = tmp_path / "divby_check"
    subprocess.run([HIPCC, "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "partial_context_patch_amd", "csrc"),
                    os.path.join(ROOT, "tests", "divby_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, timeout=300)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")
