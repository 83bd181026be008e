"""The C-ABI library loads and exports every entry point include/tsr.h declares
(no device work: these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import token_sampling_row_amd as tsr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsr.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:int|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tsr.library_path()):
        from token_sampling_row_amd import build
        build.build()
    return tsr.load_library()


def test_header_declares_the_entry_points():
    assert sorted(declared_functions()) == sorted(tsr.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", tsr.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, f"{name} is not an unmangled exported symbol"


def test_error_strings(lib):
    for code in range(5):
        assert lib.sampler_strerror(code)
    assert b"unknown" in lib.sampler_strerror(99)


def test_init_rejects_bad_arguments_before_touching_a_device(lib):
    h = ctypes.c_void_p()
    assert lib.sampler_init(None, 0, 1, 1, 1, 0) == 1
    assert lib.sampler_init(ctypes.byref(h), 0, 0, 10, 1, 0) == 1
    assert lib.sampler_init(ctypes.byref(h), 0, 10, 0, 1, 0) == 1
    assert lib.sampler_init(ctypes.byref(h), 0, 10, 10, 33, 0) == 1
    assert h.value is None


def test_calls_reject_null_handle(lib):
    p = tsr._Params(1.0, 0, 1.0, 0.0, 0)
    assert lib.sample_rows(None, None, 0, 1, 1, 1, ctypes.byref(p), 0, None, None, None) == 1
    assert lib.greedy_argmax(None, None, 0, 1, 1, 1, None, None, None) == 1
    assert lib.spec_verify(None, None, None, 0, None, 1, 1, 1, ctypes.byref(p), 0, None, None,
                           None, None) == 1
    assert lib.sampler_philox(None, None, 1, None, None) == 1
    assert lib.sample_rows_masked(None, None, 0, 1, 1, 1, None, 0, ctypes.byref(p), 0, None,
                                  None, None, None) == 1
    cs = tsr._Constraints(None, 0, None, 0, 0, 1.0, None)
    assert lib.sample_rows_ex(None, None, 0, 1, 1, 1, ctypes.byref(cs), ctypes.byref(p), 0, None,
                              None, None, None) == 1
    assert lib.beam_step(None, None, 0, 1, 4, 1, 1, None, None, None, None, None, None) == 1
    assert lib.sampler_destroy(None) == 0


def test_struct_layouts_match_the_header():
    """The ctypes mirrors of tsr_params, tsr_diag and tsr_constraints have the
    C layout (x86-64 alignment: doubles and pointers on 8 bytes)."""
    assert ctypes.sizeof(tsr._Params) == 40
    assert tsr._Params.top_p.offset == 16 and tsr._Params.filter_mode.offset == 32
    assert ctypes.sizeof(tsr._Diag) == 5 * 8
    assert ctypes.sizeof(tsr._Constraints) == 7 * 8
    assert tsr._Constraints.history_len.offset == 24 and tsr._Constraints.row_params.offset == 48


def test_binding_has_no_cpu_fallback(monkeypatch, tmp_path):
    """Without the library every call raises; nothing computes on the CPU."""
    monkeypatch.setenv("TSR_LIBRARY", str(tmp_path / "missing.so"))
    monkeypatch.setattr(tsr, "_lib", None)
    with pytest.raises(tsr.TsrUnavailable):
        tsr.Sampler(0)
