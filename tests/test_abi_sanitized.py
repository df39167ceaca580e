"""The C ABI's host validation layer (m3_api.cpp) built by the host compiler
with AddressSanitizer and UndefinedBehaviorSanitizer, against host stand-ins
for the kernel side (tests/sanitize/m3_host_stubs.cpp), and driven through
every entry point's error and launch paths by a C program
(tests/sanitize/abi_driver.c, which also checks that mamba3.h is valid C).
Runs on the CPU; any sanitizer report or wrong status fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(not (shutil.which("g++") and shutil.which("gcc")
                                     and os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h"))),
                                reason="needs gcc/g++ and the ROCm headers")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_abi_layer_under_asan_and_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), "-D__HIP_PLATFORM_AMD__"]
    objs = []
    for src, comp, std in ((os.path.join(ROOT, "state_space_sequence_prefill_amd", "csrc", "m3_api.cpp"), "g++", "-std=c++17"),
                           (os.path.join(ROOT, "tests", "sanitize", "m3_host_stubs.cpp"), "g++", "-std=c++17"),
                           (os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"), "gcc", "-std=c11")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        run([comp, std, *SAN, "-Wall", *inc, "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "abi_driver")
    run(["g++", *SAN, *objs, "-o", exe, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
         "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    assert r.stdout.startswith("ok ")
