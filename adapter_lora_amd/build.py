"""Build libmlora.so (gfx950) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, then linked into adapter_lora_amd/libmlora.so next to
this file.  The same sources compiled with MLORA_DEBUG (device-side checks
of the segment tables the table-form calls are given, reported as
LORA_DEVERR_TABLE) go into libmlora_debug.so; select it with
MLORA_LIB=<path> before importing the package.  The benchmark's streaming
reference kernel (stream_copy.hip) is linked into its own
libmlora_stream.so.  Run `python adapter_lora_amd/build.py` (not `-m`:
importing the package loads the library) or __graft_entry__.build().
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
DEBUG_OUT = os.path.join(HERE, "libmlora_debug.so")
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


def _compile(src: str, debug: bool = False) -> str:
    sub = os.path.join(BUILD_DIR, "debug") if debug else BUILD_DIR
    obj = os.path.join(sub, os.path.basename(src) + ".o")
    extra = ["-DMLORA_DEBUG"] if debug else []
    cmd = [HIPCC, *COMMON_FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
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
    os.makedirs(os.path.join(BUILD_DIR, "debug"), exist_ok=True)
    jobs = [(s, False) for s in SOURCES + STREAM_SOURCES] + [(s, True) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=max(1, min(len(jobs), os.cpu_count() or 4))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    n = len(SOURCES)
    _link(objs[:n], OUT)
    _link(objs[n:n + len(STREAM_SOURCES)], STREAM_OUT)
    _link(objs[n + len(STREAM_SOURCES):], DEBUG_OUT)
    if verbose:
        print(f"built {OUT}, {DEBUG_OUT} and {STREAM_OUT}")
    return OUT


if __name__ == "__main__":
    build()
