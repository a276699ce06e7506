"""Ahead-of-time build of libqgemv.so for gfx950 (hipcc, in-tree).

``python -m moe_expert_gemv_amd.build`` compiles every source under ``csrc/``
and links ``moe_expert_gemv_amd/libqgemv.so``.  Object files go to
``_build/`` at the repository root.  The library is built for gfx950 only.

``python -m moe_expert_gemv_amd.build --sanitize`` builds a second copy,
``moe_expert_gemv_amd/libqgemv_sanitize.so``, whose host code (the packers,
the argument checks and dispatch of every entry point, the launch stubs) is
compiled with AddressSanitizer and UndefinedBehaviorSanitizer; device code is
built as usual.  It is for CPU-side checks: load it with the clang ASan
runtime preloaded (``sanitizer_runtime()``) and point the binding at it with
``QG_LIBRARY``.
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
# Sanitizer build: host code only (each flag behind -Xarch_host on hipcc lines;
# the device passes are untouched), no recovery so the first report aborts.
SANITIZE_LIB_PATH = os.path.join(HERE, "libqgemv_sanitize.so")
SAN_HOST = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
SAN_HIP_FLAGS = [f for flag in SAN_HOST for f in ("-Xarch_host", flag)] + ["-g"]
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")

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


def build(verbose: bool = False, jobs: int = 8, sanitize: bool = False) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    build_dir = os.path.join(BUILD_DIR, "sanitize") if sanitize else BUILD_DIR
    lib_path = SANITIZE_LIB_PATH if sanitize else LIB_PATH
    os.makedirs(build_dir, exist_ok=True)
    cmds, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        san = SAN_HIP_FLAGS if sanitize else []
        cmds.append([HIPCC, *HIP_FLAGS, *san, *HIP_FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(build_dir, src.replace(".cpp", ".host.o"))
        if sanitize:  # clang, so that host objects share one sanitizer runtime
            cmds.append([CLANGXX, *CXX_FLAGS, *SAN_HOST, "-g", "-c", os.path.join(CSRC, src), "-o", obj])
        else:
            cmds.append([shutil.which("g++") or "g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, c) for c in cmds]
        for f in futs:
            f.result()
    tmp = lib_path + ".tmp"
    link_san = SAN_HIP_FLAGS if sanitize else []
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_san, "-o", tmp, *objs])
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


def sanitizer_runtime() -> str:
    """The clang ASan runtime that a process loading the sanitizer build must
    preload (LD_PRELOAD)."""
    import glob

    found = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError("clang ASan runtime not found under " + ROCM)
    return found[-1]


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
