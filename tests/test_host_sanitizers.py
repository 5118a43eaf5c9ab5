"""Host sanitizer run of the C ABI: the validation layer (abi.hip) built with
AddressSanitizer and UndefinedBehaviorSanitizer on its host side, linked
against the library's kernels, driven through every error path by
tests/sanitize/abi_driver.cpp. No call reaches a GPU, so this runs anywhere
hipcc does."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int4_weight_quantized_amd", "csrc")


def test_abi_validation_under_asan_ubsan():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    from int4_weight_quantized_amd import ops
    if not os.path.exists(ops.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    libdir = os.path.dirname(ops.LIB_PATH)
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "abi_driver")
        # the sanitizers apply to host code only (-Xarch_host before each)
        cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=undefined",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
               f"-I{CSRC}", os.path.join(CSRC, "abi.hip"), os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"),
               f"-L{libdir}", "-lw4", f"-Wl,-rpath,{libdir}", "-o", exe]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stdout + res.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        out = run.stdout + run.stderr
        assert "AddressSanitizer" not in out and "runtime error" not in out, out
        assert run.returncode == 0, out


def test_driver_calls_every_declared_entry_point():
    """The sanitizer driver exercises the validation of every function the
    header declares, so a new entry point cannot skip the sanitizer run."""
    import re
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from test_host_abi import _declared_functions
    drv = open(os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")).read()
    missing = [f for f in _declared_functions() if not re.search(r"\b%s\s*\(" % f, drv)]
    assert not missing, missing
