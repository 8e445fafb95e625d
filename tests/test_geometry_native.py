"""Host checks of the library's native host code (CPU only, g++).

geometry_check.cpp: the kernels' division-free block addressing.  For every
kernel row and key of many geometries, block_position() must equal
row_position() / key_position(), the maps the layout builder (and so the
bit-exact LUT tests) use.

layout_sanitize.cpp: the layout builder under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only), over every pattern and a grid of
ragged and degenerate (T, l, c) and summary sets, with every table copied into
buffers of exactly the advertised sizes and checked for structure.
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


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_layout_builder_under_sanitizers(tmp_path):
    exe = tmp_path / "layout_sanitize"
    src = [os.path.join(ROOT, "tests", "native", "layout_sanitize.cpp"),
           os.path.join(ROOT, "factorized_sparse_self_amd", "csrc", "st_layout.cpp")]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "factorized_sparse_self_amd", "csrc")]
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", *san, *inc, "-o", str(exe), *src], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.startswith("ok")
