"""Build the gfx950 HIP library in-tree: gated_delta_rule_51_amd/libkda_mi355x.so.

Every translation unit is compiled with hipcc for gfx950 only.  Packed fp32
VALU instructions are disabled (``-target-feature -packed-fp32-ops``); hipcc's
host pass warns that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "libkda_mi355x.so")
SOURCES = ["api.cpp", "decode.hip", "decode_chunk.hip", "chunk_local.hip", "inter_chunk.hip", "inter_chunk_ws.hip", "layer.hip", "backward.hip",
           "cp.hip", "noalloc.hip", "checks.hip",
           "prefill_fused.hip"]
ARCH = "gfx950"
# Per-file additions.  chunk_local: matrix-core results in VGPRs (not AGPRs) --
# every result there is read by the vector ALU next, and the accumulator-register
# form cost a move per element.
EXTRA_FLAGS = {"chunk_local.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the KDA library needs ROCm's hipcc to build")


def flags() -> list:
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *flags(), *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking libkda_mi355x.so failed")
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY}")
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
