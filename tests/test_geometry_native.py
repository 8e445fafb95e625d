"""Host check of the kernels' division-free block addressing (CPU only).

Builds tests/native/geometry_check.cpp with g++ against the library's own
geometry code and runs it: for every kernel row and key of many geometries,
block_position() must equal row_position() / key_position(), the maps the
layout builder (and so the bit-exact LUT tests) use.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_block_position_matches_maps(tmp_path):
    exe = tmp_path / "geometry_check"
    src = [os.path.join(ROOT, "tests", "native", "geometry_check.cpp"),
           os.path.join(ROOT, "factorized_sparse_self_amd", "csrc", "st_layout.cpp")]
    subprocess.run(["g++", "-O1", "-std=c++17", "-o", str(exe), *src], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")
