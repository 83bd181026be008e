"""Build libtsr.so (the C-ABI sampler library) for gfx950 with hipcc.

Every kernel instance (element type x chunks per thread) is compiled in a
generated translation unit of its own, in parallel; the dispatch units and the
C-ABI host layer only declare them. Everything links into
token_sampling_row_amd/libtsr.so, in-tree.

``build(trace=True)`` (``python build.py --trace``) builds the same sources with
TSR_TRACE=1 into libtsr_trace.so instead: per-wavefront phase stamps of the
sampler kernels and the two calls of include/tsr_trace.h (trace.py reads them).
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
BUILD = os.path.join(HERE, "_build")
GEN = os.path.join(BUILD, "gen")
LIB = os.path.join(HERE, "libtsr.so")
BUILD_TRACE = os.path.join(HERE, "_build_trace")
LIB_TRACE = os.path.join(HERE, "libtsr_trace.so")
ARCH = os.environ.get("TSR_OFFLOAD_ARCH", "gfx950")
ROW_NCS = (1, 2, 4, 8, 16, 24, 32, 38)      # must match kRowNcs in dispatch.hpp
VERIFY_NCS = (1, 2, 4, 8, 16)               # must match kVerifyNcs
VERIFY_WIDE_NCS = (24, 32, 38)              # must match kVerifyWideNcs
DISPATCH = ["k_greedy.hip", "k_beam.hip", "k_sample_f32.hip", "k_sample_bf16.hip", "k_verify_f32.hip",
            "k_verify_bf16.hip", "k_misc.hip", "api.hip"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
         # no packed fp32 instructions (v_pk_add/mul/fma_f32) anywhere
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libtsr.so")
    return exe


def instance_units() -> dict[str, str]:
    """name -> source of one translation unit per kernel instance."""
    head = '#define TSR_INSTANCE_UNIT 1\n#include "dispatch.hpp"\nnamespace tsr {\n'
    sample_args = "(const unsigned char*, long long, int, int, KParams, int32_t*, DiagPtrs);\n}\n"
    units = {}
    for dt in (0, 1):
        for nc in ROW_NCS:
            units[f"i_sample_{dt}_{nc}.hip"] = head + (
                f"template __global__ void sample_kernel<{dt}, {nc}, false, 0>" + sample_args)
            if dt == 1:   # the register-resident finish for wide kept sets (bf16)
                units[f"i_sample_wide_{dt}_{nc}.hip"] = head + (
                    f"template __global__ void sample_kernel<{dt}, {nc}, true, 0>" + sample_args)
            # an allowed-token set (1), a repetition penalty only (2); bf16
            # takes the wide finish as well
            wide = "true" if dt == 1 else "false"
            for ext, tag in ((1, "mask"), (2, "rep")):
                units[f"i_sample_{tag}_{dt}_{nc}.hip"] = head + (
                    f"template __global__ void sample_kernel<{dt}, {nc}, {wide}, {ext}>" + sample_args)
            units[f"i_beam_{dt}_{nc}.hip"] = head + (
                f"template __global__ void beam_kernel<{dt}, {nc}>(const unsigned char*, long long, "
                "int, int, int, const double*, BeamWs);\n}\n")
            units[f"i_greedy_{dt}_{nc}.hip"] = head + (
                f"template __global__ void greedy_kernel<{dt}, {nc}>(const unsigned char*, "
                "long long, int, int, int32_t*, int32_t*);\n}\n")
        for nc in VERIFY_NCS:
            # two rows per workgroup: no chunk maxima kept in registers
            units[f"i_verify_{dt}_{nc}.hip"] = "#define TSR_ROW_NO_CMAX 1\n" + head + (
                f"template __global__ void verify_kernel<{dt}, {nc}>(const unsigned char*, "
                "const unsigned char*, const int32_t*, int, int, int, KParams, VerifyWs);\n"
                f"template __global__ void tree_kernel<{dt}, {nc}>(const unsigned char*, "
                "const unsigned char*, const int32_t*, const int32_t*, int, int, int, KParams, "
                "VerifyWs, int32_t*, int32_t*, int32_t*, int32_t*);\n}\n")
        for nc in VERIFY_WIDE_NCS:
            for tree in ("false", "true"):
                units[f"i_vrows_{dt}_{nc}_{tree}.hip"] = head + (
                    f"template __global__ void verify_rows_kernel<{dt}, {nc}, {tree}>("
                    "const unsigned char*, const unsigned char*, const int32_t*, int, int, int, "
                    "KParams, VerifyWs);\n}\n")
        units[f"i_vfinish_{dt}.hip"] = head + (
            f"template __global__ void verify_finish_kernel<{dt}>(const unsigned char*, const "
            "unsigned char*, const int32_t*, int, int, KParams, VerifyWs, int32_t*, int32_t*, "
            "int32_t*);\n"
            f"template __global__ void verify_draw_kernel<{dt}>(const unsigned char*, const "
            "unsigned char*, int, int, KParams, VerifyWs, int32_t*);\n"
            f"template __global__ void tree_finish_kernel<{dt}>(const unsigned char*, const unsigned "
            "char*, const int32_t*, const int32_t*, int, int, KParams, VerifyWs, int32_t*, "
            "int32_t*, int32_t*, int32_t*);\n}\n")
        units[f"i_stream_{dt}.hip"] = head + (
            f"template __global__ void sample_kernel_stream<{dt}>(const unsigned char*, long long, "
            "int, KParams, int32_t*, DiagPtrs);\n"
            f"template __global__ void greedy_kernel_stream<{dt}>(const unsigned char*, long long, "
            "int, int32_t*, int32_t*);\n}\n")
    return units


def _compile(src_path: str, out_dir: str = BUILD, extra: tuple = ()) -> tuple[str, str]:
    obj = os.path.join(out_dir, os.path.basename(src_path) + ".o")
    cmd = [_hipcc(), *FLAGS, *extra, "-I", CSRC, "-Rpass-analysis=kernel-resource-usage", "-c",
           src_path, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src_path}:\n{p.stderr[-4000:]}")
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


def build(verbose: bool = False, jobs: int | None = None, trace: bool = False) -> str:
    out_dir, lib = (BUILD_TRACE, LIB_TRACE) if trace else (BUILD, LIB)
    extra = ("-DTSR_TRACE=1",) if trace else ()
    os.makedirs(GEN, exist_ok=True)
    os.makedirs(out_dir, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in DISPATCH]
    for name, text in instance_units().items():
        path = os.path.join(GEN, name)
        if not os.path.exists(path) or open(path).read() != text:
            with open(path, "w") as f:
                f.write(text)
        srcs.append(path)
    jobs = jobs or int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))
    # biggest units first so the pool drains evenly
    srcs.sort(key=lambda s: (not os.path.basename(s).startswith("i_sample"), s), reverse=False)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        results = list(ex.map(lambda s: _compile(s, out_dir, extra), srcs))
    objs = [o for o, _ in results]
    remarks = "\n".join(r for _, r in results)
    with open(os.path.join(out_dir, "resource_usage.txt"), "w") as f:
        f.write(remarks)
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr[-4000:]}")
    os.replace(tmp, lib)
    spills = spill_report(remarks)
    if verbose:
        print(f"built {lib} from {len(srcs)} units")
        for s in spills:
            print("  spill:", s)
    return lib


if __name__ == "__main__":
    build(verbose=True, trace="--trace" in sys.argv[1:])
    sys.exit(0)
