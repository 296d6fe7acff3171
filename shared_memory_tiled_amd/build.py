"""Builds libgemm_f32.so from the HIP sources in csrc/ (gfx950 only).

    python -m shared_memory_tiled_amd.build [--resource-usage]

Each source is compiled to an object under _build/ by hipcc, then the objects
are linked into shared_memory_tiled_amd/libgemm_f32.so.  Packed-FP32 VALU
instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgemm_f32.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


# Per-source extra flags.  mfma16_ksplit.hip: matrix instructions in their
# vector-register form -- with the accumulators in AGPRs the register
# allocator copied every accumulator before each matrix instruction of that
# kernel.
EXTRA_FLAGS = {"mfma16_ksplit.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def _compile(src: str, resource_usage: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip() and resource_usage:
        print(msgs)
    return obj


def build(resource_usage: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, resource_usage), sources))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(resource_usage="--resource-usage" in sys.argv))
