"""Builds libmoe.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

    python -m quantized_moe_expert_fp32_amd.build [-v]
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["abi.hip", "route.hip", "decode.hip", "prefill.hip", "prefill_fp8.hip", "combine.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")
# Packed fp32 VALU instructions are disabled for every device compile.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]
# Per-source extras. The grouped GEMM applies a per-group scale to each MFMA
# product on the VALU; MFMA results in VGPRs save a copy out of AGPRs per element.
SOURCE_FLAGS = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
                "route.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compiles every source (always, even when a library exists) and links LIB."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for src in SOURCES:
            obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
            objs.append(obj)
            cmd = [HIPCC] + FLAGS + SOURCE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
            jobs.append(ex.submit(_run, cmd, verbose))
        for j in jobs:
            j.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
