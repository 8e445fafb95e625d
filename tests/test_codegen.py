"""Checks on the gfx950 code the HIP sources compile to (CPU only: hipcc cross-compiles).

- The LDS DMA helper sets M0 inside its inline asm and does not restore it; that is only
  sound while the compiler itself never uses M0 in these kernels.  The test fails if M0
  appears anywhere outside the inline asm blocks.
- The 16-bit (bf16 / fp16) kernels must not spill registers to scratch memory.
"""
import os
import re
import shutil
import subprocess

import pytest

from factorized_sparse_self_amd import build

SOURCES = ("st_fwd.hip", "st_bwd.hip")


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    """Device assembly of each source, compiled once per test module."""
    cache = {}

    def get(src):
        if src not in cache:
            cache[src] = _device_asm(tmp_path_factory.mktemp("asm"), src)
        return cache[src]
    return get


def _device_asm(tmp_path, src):
    cc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cc):
        pytest.skip("hipcc not available")
    out = tmp_path / (src + ".s")
    include = ["-I", os.path.join(os.path.dirname(build.PKG), "include"), "-I", build.CSRC]
    flags = [f for f in build.COMMON if f != "-fPIC"]
    cmd = [cc, *flags, *include, "-x", "hip", "--cuda-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    assert r.returncode == 0, r.stdout.decode(errors="replace")
    return out.read_text()


@pytest.mark.parametrize("src", SOURCES)
def test_m0_only_inside_inline_asm(device_asm, src):
    text = device_asm(src)
    assert ";;#ASMSTART" in text, "expected the LDS DMA inline asm in the bf16 kernels"
    outside = re.sub(r";;#ASMSTART.*?;;#ASMEND", "", text, flags=re.S)
    uses = [line.strip() for line in outside.splitlines()
            if re.search(r"\bm0\b", line) and not line.strip().startswith(";")]
    assert not uses, f"{src}: compiler-generated M0 uses: {uses[:5]}"


@pytest.mark.parametrize("src", SOURCES)
def test_16bit_kernels_do_not_spill(device_asm, src):
    text = device_asm(src)
    kernels = re.findall(r"\.name:\s+(\S*b16_kernel\S*)\n(.*?)\.wavefront_size", text, flags=re.S)
    assert kernels, "no 16-bit kernel metadata found"
    # both element types are instantiated
    assert any("DF16b" in n for n, _ in kernels) and any("DF16_" in n for n, _ in kernels)
    for name, meta in kernels:
        spill = int(re.search(r"\.vgpr_spill_count:\s+(\d+)", meta).group(1))
        scratch = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", meta).group(1))
        assert spill == 0 and scratch == 0, f"{name}: {spill} VGPR spills, {scratch} bytes of scratch"
