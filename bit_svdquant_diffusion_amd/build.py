"""Build libsvdq.so in-tree: host pack code with g++ (no FP contraction), HIP
kernels with hipcc for gfx950, linked by hipcc into one shared library.

    python -m bit_svdquant_diffusion_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libsvdq.so")

HIP_SOURCES = ["svdq_stage1.hip", "svdq_gemm_int4.hip", "svdq_gemm_small.hip", "svdq_gemm_mxfp4.hip", "svdq_awq.hip",
               "svdq_pack_gpu.hip", "svdq_peak.hip", "svdq_api.hip"]
CPP_SOURCES = ["svdq_pack.cpp", "svdq_awq_pack.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off (plain float code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math", "-fvisibility=hidden",
    "-I" + INCLUDE, "-I" + CSRC,
]
# per-source extras: the few-token GEMM multiplies into VGPRs, so its INT4
# dequant reads the MFMA results without accumulator-register copies
HIP_EXTRA = {"svdq_gemm_small.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math", "-fvisibility=hidden",
             "-Wall", "-I" + INCLUDE, "-I" + CSRC]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libsvdq.so next to this file. Returns its path."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for s in CPP_SOURCES:
        o = os.path.join(BUILD_DIR, s + ".o")
        jobs.append(["g++"] + CXX_FLAGS + ["-c", os.path.join(CSRC, s), "-o", o])
    for s in HIP_SOURCES:
        o = os.path.join(BUILD_DIR, s + ".o")
        jobs.append([HIPCC] + HIP_FLAGS + HIP_EXTRA.get(s, []) + ["-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [os.path.join(BUILD_DIR, s + ".o") for s in CPP_SOURCES + HIP_SOURCES]
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + ["-lpthread"])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


SANITIZED_HOST_LIB = os.path.join(BUILD_DIR, "libsvdq_host_asan.so")


def build_host_sanitized() -> str:
    """The host-only part of the library (pack, unpack, LoRA extension, sizes
    and workspace queries) built by g++ with AddressSanitizer and
    UndefinedBehaviorSanitizer, every finding fatal. For tests that load it
    in a process started with libasan preloaded; no GPU code is in it."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = SANITIZED_HOST_LIB + ".tmp"
    _run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off", "-Wall",
          "-I" + INCLUDE, "-I" + CSRC] + [os.path.join(CSRC, s) for s in CPP_SOURCES] + ["-o", tmp, "-lpthread"])
    os.replace(tmp, SANITIZED_HOST_LIB)
    return SANITIZED_HOST_LIB


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized())
    else:
        p = build(verbose="-v" in sys.argv)
        print(p)
