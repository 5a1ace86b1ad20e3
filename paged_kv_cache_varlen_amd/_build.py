"""Build libpa.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m paged_kv_cache_varlen_amd._build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
PROBE_LIB = os.path.join(PKG, "libpa_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["kv_cache.hip", "blocks.hip", "mla.hip", "attend.hip", "pa_api.cpp"]
# Packed-FP32 VALU forms are kept out of the generated code on purpose.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# Per-source flags.  mla.hip: MFMA accumulators in VGPRs (the default form
# kept them in AGPRs and copied them through VGPRs around every stage, for the
# occasional rescale, at 172 extra VALU instructions per stage).
EXTRA = {"mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libpa.so.  Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    # the streaming-read probe (bench.py's measured ceiling): its own library
    probe_tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + COMMON + ["-shared", os.path.join(CSRC, "read_probe.hip"), "-o", probe_tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for read_probe.hip:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(probe_tmp, PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
