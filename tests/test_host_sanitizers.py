"""The host argument checks under AddressSanitizer and UndefinedBehavior-
Sanitizer: the C-ABI layer (csrc/api.cpp, where every argument check lives)
is rebuilt with host-side sanitizers and linked with the library's regular
kernel objects, and the argument-check tests of test_abi.py run against that
library in a child process.  Any sanitizer report fails the run.  No GPU is
used: the checks reject the arguments before any launch."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(BUILD, "san")
KERNEL_OBJS = ["segments.hip.o", "pack.hip.o", "decode.hip.o", "linear.hip.o", "gemm.hip.o",
               "moe.hip.o", "noalloc.hip.o"]


def asan_runtime():
    found = glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return found[0] if found else None


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX) and asan_runtime()),
                    reason="ROCm compiler or sanitizer runtime missing")
def test_argument_checks_under_asan_and_ubsan():
    objs = [os.path.join(BUILD, o) for o in KERNEL_OBJS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects missing: run __graft_entry__.build() first")
    os.makedirs(OUT, exist_ok=True)
    api_obj = os.path.join(OUT, "api_san.o")
    lib = os.path.join(OUT, "libmlora_san.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
                    "-I", os.path.join(ROOT, "include"), "-x", "hip", "-c",
                    os.path.join(ROOT, "adapter_lora_amd", "csrc", "api.cpp"), "-o", api_obj],
                   check=True, capture_output=True, text=True)
    # the host link pulls in the sanitizer runtimes as shared libraries
    subprocess.run([CLANGXX, "-shared", "-fPIC", "-shared-libsan",
                    "-fsanitize=address,undefined", api_obj, *objs, "-L/opt/rocm/lib",
                    "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan_runtime(), MLORA_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run(["python", "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-x", "-p", "no:cacheprovider",
                        "-k", "argument_checks or host_only or rejects"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert " passed" in report
