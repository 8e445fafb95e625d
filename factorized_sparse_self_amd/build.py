"""Build libst.so in-tree with hipcc for gfx950.

``python -m factorized_sparse_self_amd.build`` (or ``build()``) compiles every
source under ``csrc/`` and links ``factorized_sparse_self_amd/libst.so``.  It
always recompiles (no GPU is needed: hipcc cross-compiles the gfx950 code
objects on any host).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libst.so")
SOURCES = ["st_layout.cpp", "st_api.hip", "st_fwd.hip", "st_bwd.hip"]
ARCH = "gfx950"

COMMON = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the softmax reads them with VALU, and the
    # AGPR form would copy every fragment across register files
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # no NaN inputs are assumed (infinities are kept: masked logits are -inf),
    # which drops the NaN-quieting copies IEEE mode adds around every max
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libst.so")
    return path


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile all sources and link libst.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    include = ["-I", os.path.join(os.path.dirname(PKG), "include"), "-I", CSRC]
    procs = []
    objs = []
    t0 = time.time()
    for src in SOURCES:
        obj = os.path.join(BUILD, src.rsplit(".", 1)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *COMMON, *include, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        msg = "\n".join(f"--- {s} ---\n{t}" for s, t in failed)
        raise RuntimeError(f"libst build failed:\n{msg}")
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("libst link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
