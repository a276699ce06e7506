"""Ahead-of-time build of libqgemv.so for gfx950 (hipcc, in-tree).

``python -m moe_expert_gemv_amd.build`` compiles every source under ``csrc/``
and links ``moe_expert_gemv_amd/libqgemv.so``.  Object files go to
``_build/`` at the repository root.  The library is built for gfx950 only.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libqgemv.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

# Device code: gfx950 only, -O3, no fast-math (the activation quantizer needs
# a correctly rounded fp32 division).  Packed-fp32 instruction selection is
# switched off: hipcc would otherwise form v_pk_{add,mul,fma}_f32 on its own.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]

HIP_SOURCES = ["qg_api.hip", "k_gemv_nvfp4.hip", "k_gemv_q8.hip", "k_gemv_a8.hip", "k_gemv_fp8.hip",
               "k_gemv_kquant.hip", "k_dequant.hip", "k_moe.hip", "k_moe_prefill.hip", "k_prefill.hip",
               "k_prefill_a8.hip", "k_probe.hip"]
CXX_SOURCES = ["qg_host.cpp"]
# Per-source compiler options.  The int8 prefill reads every MFMA result back
# into VALU arithmetic; the VGPR form of the MFMA saves a v_accvgpr_read per
# output per block.
HIP_FILE_FLAGS = {"k_prefill_a8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass of hipcc does not know the packed-fp32 feature; that note is harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = False, jobs: int = 8) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    cmds, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmds.append([HIPCC, *HIP_FLAGS, *HIP_FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".cpp", ".host.o"))
        cmds.append([shutil.which("g++") or "g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, c) for c in cmds]
        for f in futs:
            f.result()
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
