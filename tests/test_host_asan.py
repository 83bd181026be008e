"""The host layer under AddressSanitizer (token_sampling_row_amd/build_asan.py):
every argument-error path of the C ABI and sampler_init's failure path run in
tests/asan/abi_driver.c against a build whose api.hip carries the sanitizer.
CPU only."""
import os
import shutil

import pytest

from token_sampling_row_amd import build_asan

pytestmark = pytest.mark.skipif(
    shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
    reason="needs the HIP toolchain")


def test_abi_error_paths_are_clean_under_asan():
    p = build_asan.run_driver(build_asan.build_asan())
    assert "AddressSanitizer" not in p.stderr, p.stderr[-4000:]
    assert p.returncode == 0, p.stdout + p.stderr[-4000:]
    assert "abi_driver: ok" in p.stdout
