"""Build libmlora.so (gfx950) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, then linked into adapter_lora_amd/libmlora.so next to
this file.  The benchmark's streaming reference kernel (stream_copy.hip) is
linked into its own libmlora_stream.so beside it.  Run `python adapter_lora_amd/build.py` (not `-m`: importing the
package loads the library) or __graft_entry__.build().
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libmlora.so")
STREAM_OUT = os.path.join(HERE, "libmlora_stream.so")
STREAM_SOURCES = ["stream_copy.hip"]
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["api.cpp", "segments.hip", "pack.hip", "decode.hip", "linear.hip", "gemm.hip", "moe.hip",
           "noalloc.hip"]
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if warn:
        sys.stderr.write(f"[{src}]\n{warn}\n")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + STREAM_SOURCES
    jobs = min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], STREAM_OUT)
    if verbose:
        print(f"built {OUT} and {STREAM_OUT}")
    return OUT


if __name__ == "__main__":
    build()
