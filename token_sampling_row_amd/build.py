"""Build libtsr.so (the C-ABI sampler library) for gfx950 with hipcc.

Each kernel family is its own translation unit, compiled in parallel; the
objects are linked into token_sampling_row_amd/libtsr.so in-tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtsr.so")
ARCH = os.environ.get("TSR_OFFLOAD_ARCH", "gfx950")
SOURCES = ["k_sample_bf16.hip", "k_sample_f32.hip", "k_verify_f32.hip", "k_verify_bf16.hip",
           "k_greedy.hip", "k_misc.hip", "api.hip"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # no packed fp32 instructions (v_pk_add/mul/fma_f32) anywhere
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libtsr.so")
    return exe


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{p.stderr[-4000:]}")
    return obj, p.stderr


def spill_report(remarks: str) -> list[str]:
    """Kernels whose registers spill to scratch, from the resource-usage remarks."""
    bad, name = [], None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].split("[")[0].strip()
        elif "VGPRs Spill:" in line and name:
            n = int(line.split("VGPRs Spill:")[1].split("[")[0])
            if n:
                bad.append(f"{name}: {n} VGPRs spilled")
    return bad


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    remarks = "\n".join(r for _, r in results)
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write(remarks)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr[-4000:]}")
    os.replace(tmp, LIB)
    spills = spill_report(remarks)
    if verbose:
        print(f"built {LIB}")
        for s in spills:
            print("  spill:", s)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
