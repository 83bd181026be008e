"""A build of libtsr.so whose host layer (csrc/api.hip: argument checks,
handle set-up and teardown, dispatch) carries AddressSanitizer, and the
tests/asan/abi_driver.c program linked against it.

Only api.hip is compiled again, with the sanitizer on its host side (the
device code of every unit is built as usual); the kernel units' objects come
from the ordinary build (build.py), which runs first if they are missing. The
link and the driver use the ROCm clang directly, which adds the sanitizer's
runtime. CPU only: the driver checks every argument-error path and
sampler_init's failure path, which need no GPU.

  python -m token_sampling_row_amd.build_asan     # builds, runs the driver
"""
from __future__ import annotations

import os
import subprocess
import sys

from token_sampling_row_amd import build as B

BUILD_ASAN = os.path.join(B.HERE, "_build_asan")
LIB_ASAN = os.path.join(BUILD_ASAN, "libtsr_asan.so")
DRIVER_SRC = os.path.join(B.ROOT, "tests", "asan", "abi_driver.c")
DRIVER = os.path.join(BUILD_ASAN, "abi_driver")
CLANG = "/opt/rocm/llvm/bin/clang"
ROCM_LIB = "/opt/rocm/lib"
# the sanitizer on the host compilation only (never on GPU code)
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def _asan_runtime_dir() -> str:
    """The folder of the sanitizer's shared runtime in the ROCm clang."""
    res = subprocess.run([CLANG, "-print-resource-dir"], capture_output=True, text=True,
                         check=True).stdout.strip()
    for sub in ("lib/linux", "lib/x86_64-unknown-linux-gnu"):
        d = os.path.join(res, sub)
        if os.path.exists(os.path.join(d, "libclang_rt.asan-x86_64.so")) or \
                os.path.exists(os.path.join(d, "libclang_rt.asan.so")):
            return d
    raise RuntimeError(f"no AddressSanitizer runtime under {res}")


def _run(cmd: list[str], what: str) -> None:
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"{what} failed:\n{p.stderr[-4000:]}")


def build_asan() -> str:
    """Build libtsr_asan.so and the driver; returns the driver's path."""
    kernel_objs = [os.path.join(B.BUILD, os.path.basename(s) + ".o")
                   for s in [os.path.join(B.CSRC, d) for d in B.DISPATCH if d != "api.hip"]]
    kernel_objs += [os.path.join(B.BUILD, n + ".o") for n in B.instance_units()]
    if not all(os.path.exists(o) for o in kernel_objs):
        B.build()
    os.makedirs(BUILD_ASAN, exist_ok=True)
    api_obj = os.path.join(BUILD_ASAN, "api.hip.o")
    _run([B._hipcc(), *B.FLAGS, *HOST_ASAN, "-I", B.CSRC, "-c", os.path.join(B.CSRC, "api.hip"),
          "-o", api_obj], "hipcc (api.hip with the host sanitizer)")
    _run([CLANG + "++", "-shared", "-fPIC", "-fsanitize=address", "-shared-libsan", api_obj,
          *kernel_objs, f"-L{ROCM_LIB}", "-lamdhip64", f"-Wl,-rpath,{ROCM_LIB}",
          f"-Wl,-rpath,{_asan_runtime_dir()}", "-o", LIB_ASAN], "link of libtsr_asan.so")
    rt = _asan_runtime_dir()
    _run([CLANG, "-fsanitize=address", "-shared-libsan", "-fno-omit-frame-pointer", "-g", "-I",
          os.path.join(B.ROOT, "include"), DRIVER_SRC, LIB_ASAN, f"-Wl,-rpath,{BUILD_ASAN}",
          f"-Wl,-rpath,{ROCM_LIB}", f"-Wl,-rpath,{rt}", "-lm", "-o", DRIVER],
         "build of the driver")
    return DRIVER


def run_driver(driver: str) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    # the HIP runtime keeps process-lifetime allocations: leaks are not checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    return subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)


if __name__ == "__main__":
    p = run_driver(build_asan())
    sys.stdout.write(p.stdout)
    sys.stderr.write(p.stderr)
    sys.exit(p.returncode)
