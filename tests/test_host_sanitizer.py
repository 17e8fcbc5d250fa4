"""The C-ABI layer (csrc/mx_api.cpp) built with AddressSanitizer, LeakSanitizer and
UndefinedBehaviorSanitizer by the host compiler, against stand-ins for the device launchers
(tests/host_sanitizer/stubs.cpp), and driven through its validation, row chunking, workspace
layout and error mapping by tests/host_sanitizer/driver.cpp (177 checks of include/mx.h's stated
rules).  CPU only: nothing here touches a GPU or device memory."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "microscaling_fp4_weight_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitizer")
HIP_INCLUDE = "/opt/rocm/include"


def test_c_abi_under_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.exists(os.path.join(HIP_INCLUDE, "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the HIP headers")
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE,
             "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", HERE]
    objs = []
    for src in (os.path.join(CSRC, "mx_api.cpp"), os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([cxx] + flags + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(obj)
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run([cxx, "-fsanitize=address,undefined", "-o", exe] + objs, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "all " in r.stdout and "checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]
