"""The launch geometry's rules, checked on the host: a small program compiled
against the library's own header runs make_geometry over a grid of shapes (the
tile floors, the 16-vector argmax tiles, the sampler's chunk rule, and the
filtered call's two workspace layouts)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "geometry", "geometry_check.hip")
CSRC = os.path.join(ROOT, "draft_token_verification_verify_amd", "csrc")


def test_geometry_rules(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "geometry_check")
    subprocess.run([hipcc, "-O1", "-std=c++17", "-I", CSRC, "-I", os.path.join(ROOT, "include"), SRC,
                    "-o", exe], check=True, capture_output=True, text=True, timeout=600)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "geometry: ok" in r.stdout
