"""Builds libcsa_mi355x.so in-tree with hipcc for gfx950.

    python -m sparse_attention_17_amd.build        # compile + link

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection turned off (plain fp32 code must not be fused into v_pk_* ops on
this target).  The host-only C ABI (api.cpp) is compiled by the same driver.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcsa_mi355x.so")
SOURCES = ["api.cpp", "profile.cpp", "compress.hip", "indexer.hip", "attend.hip", "attend_v_f32.hip",
           "attend_v_bf16_64.hip", "attend_v_bf16_128.hip", "attend_v_pair_bf16_128.hip",
           "attend_v_kv8.hip", "proj.hip", "step_static.hip", "step_tail.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return p


def common_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(os.cpu_count() or 8, 16, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
