"""AddressSanitizer and UndefinedBehaviorSanitizer over the host-side C and
C++: the CPU oracle, the seeded input generator and librkv's host layer
(validation, workspace sizing, status strings, no-op paths), each built
from its committed sources with g++/gcc -fsanitize=address,undefined and
driven by a program under tests/sanitize/ that reaches every entry point,
the degenerate cases included. The library's kernels are not part of this
build (tests/sanitize/launch_stubs.cpp aborts if a launcher is reached); the
GPU tests cover them."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "redundancy_aware_compression_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def compile_(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]


def run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    report = r.stdout[-2000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, report
    return r.stdout


@pytest.fixture(scope="module")
def toolchain(tmp_path_factory):
    if shutil.which("g++") is None or shutil.which("gcc") is None:
        pytest.skip("g++/gcc not found")
    d = tmp_path_factory.mktemp("san")
    # the sanitizers are live: a planted heap overflow and a planted signed
    # overflow in throwaway programs are caught
    canaries = {
        "address": ("#include <stdlib.h>\nint main(int c, char** v){int*p=malloc(4*sizeof(int));"
                    "p[3+c]=1;int r=p[0];free(p);return r;}\n", "heap-buffer-overflow"),
        "undefined": ("#include <limits.h>\nint main(int c, char** v){int x=INT_MAX-1;x+=c+1;return x&1;}\n",
                      "signed integer overflow"),
    }
    for kind, (text, finding) in canaries.items():
        src = d / f"canary_{kind}.c"
        src.write_text(text)
        exe = str(d / f"canary_{kind}")
        r = subprocess.run(["gcc", "-O1", "-g", f"-fsanitize={kind}", "-fno-sanitize-recover=all", str(src), "-o",
                            exe], capture_output=True, text=True)
        if r.returncode != 0:
            pytest.skip("this toolchain cannot link the sanitizer runtimes: " + r.stderr[-500:])
        c = subprocess.run([exe], capture_output=True, text=True, env=ENV)
        assert c.returncode != 0 and finding in c.stderr, c.stderr[-2000:]
    return d


def test_oracle_and_generator_are_clean(toolchain):
    d = str(toolchain)
    compile_(["g++", *FLAGS, "-std=c++17", "-c", os.path.join(ROOT, "oracle", "rkv_oracle.cpp"), "-o", "oracle.o"], d)
    compile_(["gcc", *FLAGS, "-std=c11", "-c", os.path.join(ROOT, "synth", "rkv_synth.c"), "-o", "synth.o"], d)
    compile_(["g++", *FLAGS, "-std=c++17", "-I" + os.path.join(ROOT, "oracle"),
              os.path.join(SAN, "oracle_synth_checks.cpp"), "oracle.o", "synth.o", "-lm", "-o", "oracle_checks"], d)
    assert "every call clean" in run(os.path.join(d, "oracle_checks"))


def test_host_layer_is_clean(toolchain):
    if not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("HIP headers not found")
    d = str(toolchain)
    inc = ["-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"),
           "-I" + CSRC]
    for src, obj in ((os.path.join(CSRC, "rkv_api.cpp"), "api.o"), (os.path.join(SAN, "launch_stubs.cpp"), "stubs.o"),
                     (os.path.join(SAN, "host_checks.cpp"), "host.o")):
        compile_(["g++", *FLAGS, "-std=c++17", *inc, "-c", src, "-o", obj], d)
    compile_(["g++", *FLAGS, "host.o", "api.o", "stubs.o", "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
              "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", "host_checks"], d)
    assert "every call clean" in run(os.path.join(d, "host_checks"))
