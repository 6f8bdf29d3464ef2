"""The MLORA_DEBUG library (libmlora_debug.so): valid segment tables give
the same exact results with a clear error word, and tables with an entry
outside the batch or the weight table set LORA_DEVERR_TABLE, skip exactly
the tile or segment that holds it, and write nothing else.  The library is
loaded by tests/debug_table_run.py in a child process (one library per
process); every corrupted entry points into padding rows of that script's
own buffers.  With MLORA_DEBUG_WAIT_FAULT=1 the same library makes every
bounded wait on an exchange slot miss and give up after a few polls
(tests/debug_wait_run.py): the decode and bf16 MoE launches then report
LORA_DEVERR_WAIT and still end normally."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEBUG_LIB = os.path.join(ROOT, "adapter_lora_amd", "libmlora_debug.so")


def test_debug_library_checks_tables():
    assert os.path.exists(DEBUG_LIB), "run __graft_entry__.build() first"
    print("debug table checks: child process on libmlora_debug.so", flush=True)
    env = dict(os.environ, MLORA_LIB=DEBUG_LIB)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "debug_table_run.py")],
                       env=env, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-3000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    assert res["lib"] == "libmlora_debug.so"
    TABLE = 4   # LORA_DEVERR_TABLE
    for name in ("tiles_valid", "decode_valid"):
        assert res[name] == {"err": 0, "padding_untouched": True, "rows_exact": True,
                             "skipped": 0}, (name, res[name])
    for name in ("tiles_corrupt", "decode_corrupt"):
        v = res[name]
        assert v["err"] == TABLE and v["padding_untouched"] and v["rows_exact"], (name, v)
        assert v["skipped"] > 0
    g = res["gemm_corrupt"]
    assert g == {"err": TABLE, "padding_untouched": True, "rows_exact": True,
                 "lost_row_unwritten": True}, g


def test_debug_library_wait_timeout_reported():
    assert os.path.exists(DEBUG_LIB), "run __graft_entry__.build() first"
    print("debug wait timeout: child process on libmlora_debug.so, forced misses", flush=True)
    env = dict(os.environ, MLORA_LIB=DEBUG_LIB, MLORA_DEBUG_WAIT_FAULT="1")
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "debug_wait_run.py")],
                       env=env, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-3000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    assert res["lib"] == "libmlora_debug.so" and res["returned"]
    WAIT = 1   # LORA_DEVERR_WAIT
    for name in ("decode_err", "moe_gate_up_err", "moe_down_err"):
        assert res[name] & WAIT, (name, res)
