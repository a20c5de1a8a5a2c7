"""Builds libwfattn.so (HIP kernels + C ABI) in-tree with hipcc for gfx950.

    python -m wavefront_causal_attention_wf_amd.build_lib

Every call recompiles. The library lands next to this file, where the binding
(wfattn.py) loads it from.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libwfattn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["wf_attn.hip", "wf_paged.hip", "wf_rope.hip", "wf_fp8.hip", "wf_page_table.cpp", "wf_error.cpp"]

# Packed-FP32 VALU forms are kept out of the generated code (the device pass
# honours the flag; the host pass only warns that it does not know it).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # MFMA results in VGPRs: the softmax reads the score accumulators with
             # VALU ops, and the query fragments go to AGPRs instead.
             "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libwfattn.so)")


def build(verbose: bool = False) -> str:
    """Compile every source into LIB_PATH (atomically replaced). Returns the path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", *HIP_FLAGS, "-shared", "-I", INCLUDE, "-I", CSRC,
           "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build_host_page_table_test(out_path: str) -> str:
    """Host-only build (g++, AddressSanitizer + UBSan) of the page table and a small
    driver that replays a command script; used by the CPU tests."""
    gxx = shutil.which("g++")
    if not gxx:
        raise RuntimeError("g++ not found")
    driver = os.path.join(CSRC, "host_tests", "page_table_driver.cpp")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", INCLUDE, "-I", CSRC,
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
           driver, os.path.join(CSRC, "wf_page_table.cpp"), os.path.join(CSRC, "wf_error.cpp"),
           "-o", out_path]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"g++ failed:\n{res.stderr}")
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
