"""Compile libforkkv.so in-tree: host C++ with g++, HIP kernels with hipcc for gfx950.

    python -m lora_shared_prefix_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libforkkv.so")
MICROBENCH_LIB = os.path.join(PKG, "libforkkv_microbench.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

CPP_SOURCES = ["pool.cpp", "plan.cpp", "api.cpp", "caps.cpp"]
HIP_SOURCES = ["kernels_generic.hip", "kernels_mfma_decode.hip", "kernels_mfma_prefill.hip",
               "scratch.hip"]
ARCH = "gfx950"

CXXFLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
            f"-I{INCLUDE}", f"-I{ROCM}/include", f"-I{CSRC}"]
HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
            # packed fp32 VALU ops stay off on this target
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results in ordinary VGPRs: the decode kernel post-processes them on VALU
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wno-unused-parameter"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cmds = []
    objs = []
    for src in CPP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append(["g++", *CXXFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([f"{ROCM}/bin/hipcc", *HIPFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([f"{ROCM}/bin/hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    # device ceilings for the bench (a separate library: not part of the C ABI)
    tmp = MICROBENCH_LIB + ".tmp"
    _run([f"{ROCM}/bin/hipcc", *HIPFLAGS, "-shared", os.path.join(CSRC, "microbench.hip"),
          "-o", tmp])
    os.replace(tmp, MICROBENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
