"""The C-ABI library loads and exports every symbol include/mlora.h declares;
host-only entry points and argument checks work without a GPU (no compute
call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlora.h")
LIB = os.path.join(ROOT, "adapter_lora_amd", "libmlora.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["lora_build_segments", "lora_shrink", "lora_expand_add", "lora_shrink_expand_add",
              "lora_fused_decode", "lora_linear_fused",
              "lora_moe_align", "lora_moe_gate_up_add", "lora_moe_silu_and_mul",
              "lora_moe_down_add", "lora_moe_topk_reduce", "lora_workspace_size",
              "lora_status_string", "lora_read_device_error", "lora_table_plan",
              "lora_pack_adapter"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    assert os.path.exists(LIB), "run __graft_entry__.build() first"
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (lora_\w+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing


def test_debug_library_exports_the_same_boundary():
    """libmlora_debug.so (MLORA_DEBUG: device-side segment-table checks) is
    built beside the release library and exports the same symbols."""
    dbg = os.path.join(ROOT, "adapter_lora_amd", "libmlora_debug.so")
    assert os.path.exists(dbg), "run __graft_entry__.build() first"
    out = subprocess.run(["nm", "-D", "--defined-only", dbg], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (lora_\w+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing


def test_binding_signature_table_matches_header():
    from adapter_lora_amd import _abi
    assert sorted(_abi.SIGNATURES) == declared_functions()


def test_host_only_calls():
    from adapter_lora_amd import _abi
    import adapter_lora_amd as ml
    lib = _abi.lib
    assert lib.lora_abi_version() == _abi.MLORA_ABI_VERSION
    assert lib.lora_status_string(1) == b"invalid argument"
    rp, ao, bo, na, nb = ml.lora_table_plan([20, 16, 0, 64, 8], 2, 64, 96)
    assert rp == [32, 16, 0, 64, 16]
    # rank-group major: padded 16 slots first (1, then 4), then 32 (0), then 64 (3)
    assert ao[1] == 0 and ao[4] == 2 * 16 * 64 and ao[0] == 4 * 16 * 64
    assert ao[3] == ao[0] + 2 * 32 * 64
    assert na == ao[3] + 2 * 64 * 64
    assert bo[1] == 0 and bo[4] == 96 * 16 and bo[0] == 2 * 96 * 16 and nb == bo[3] + 96 * 64
    assert ml.lora_moe_align_capacity(256, 2, 8, 64) == 1024
    assert ml.lora_moe_align_capacity(3, 2, 2, 2) == 8


def test_argument_checks_fail_before_any_launch():
    from adapter_lora_amd import _abi
    lib = _abi.lib
    INV = _abi.LORA_INVALID_ARG
    null = ctypes.c_void_p(0)
    assert lib.lora_build_segments(null, null, -1, 4, null, null, null, null, null, null, null,
                                   8, null) == INV
    assert lib.lora_build_segments(null, null, 4, 0, null, null, null, null, null, null, null,
                                   8, null) == INV
    assert lib.lora_build_segments(null, null, 4, 4, null, null, null, null, null, null, null,
                                   8, null) == INV
    assert lib.lora_tile_capacity(130, 4) == 2 + 4 and lib.lora_tile_capacity(3, 20) == 3
    w = _abi.lora_weights_t()
    w.dtype, w.K, w.n_slices, w.L, w.r_max = 1, 100, 1, 4, 16     # K not a multiple of 8
    assert lib.lora_shrink_expand_add(ctypes.byref(w), null, 0, 1, None, null, 0, null, 0,
                                      null) == INV
    w.K = 128
    w.slice_offsets[0], w.slice_offsets[1] = 0, 128              # pointers still null
    assert lib.lora_expand_add(ctypes.byref(w), null, 1, None, null, 0, null) == INV
    assert lib.lora_workspace_size(ctypes.byref(w), 8) == 0      # invalid table -> 0
    # fused decode: more tokens than one launch groups on chip, then a table
    # request with a missing buffer (checked before the null weight pointers
    # would matter: both need no GPU)
    w2 = _abi.lora_weights_t()
    w2.dtype, w2.K, w2.n_slices, w2.L, w2.r_max = 1, 128, 1, 4, 16
    w2.slice_offsets[0], w2.slice_offsets[1] = 0, 128
    w2.A = w2.B = ctypes.c_void_p(256)
    w2.a_off = w2.b_off = ctypes.cast(ctypes.c_void_p(256), ctypes.POINTER(ctypes.c_int64))
    w2.rank = ctypes.cast(ctypes.c_void_p(256), ctypes.POINTER(ctypes.c_int32))
    args = [null] * 7
    assert lib.lora_fused_decode(ctypes.byref(w2), null, null, null, 128, 65, null, 128, *args, 8,
                                 null, 0, null) == _abi.LORA_UNSUPPORTED
    some = ctypes.c_void_p(256)
    assert lib.lora_fused_decode(ctypes.byref(w2), null, null, null, 128, 8, null, 128, some,
                                 null, null, null, null, null, null, 8, null, 0, null) == INV
    assert lib.lora_fused_decode(ctypes.byref(w2), null, null, null, 128, 8, null, 128, *args, 0,
                                 null, 0, null) == INV                            # ids null
    # allocation-free form: a table whose exchange slots exceed the fixed
    # array (256 + 8 * 64 * ceil(K / 1024) * n_slices * r_max bytes) is
    # refused before anything touches a device; one that fits gets as far as
    # the argument checks (ids null)
    w3 = _abi.lora_weights_t()
    w3.dtype, w3.K, w3.n_slices, w3.L, w3.r_max = 1, 16384, 4, 4, 64
    for s_ in range(5):
        w3.slice_offsets[s_] = 128 * s_
    w3.A, w3.B, w3.a_off, w3.b_off, w3.rank = w2.A, w2.B, w2.a_off, w2.b_off, w2.rank
    assert 256 + 8 * 64 * 16 * 4 * 64 > _abi.LORA_NOALLOC_SCRATCH_BYTES
    assert lib.lora_fused_decode_noalloc(ctypes.byref(w3), some, null, some, 16384, 8, some, 512,
                                         *args, 0, null, null) == _abi.LORA_UNSUPPORTED
    assert lib.lora_fused_decode_noalloc(ctypes.byref(w2), null, null, null, 128, 65, null, 128,
                                         *args, 0, null, null) == _abi.LORA_UNSUPPORTED
    assert lib.lora_fused_decode_noalloc(ctypes.byref(w2), null, null, some, 128, 8, some, 128,
                                         *args, 0, null, null) == INV               # ids null
    # fused base GEMM: fp32 tables are not on this path; a null base weight
    # or a short workspace is rejected before any launch
    w2.dtype = 0
    assert lib.lora_linear_fused(ctypes.byref(w2), some, 128, some, 128, 8, None, some, 128,
                                 some, 1 << 20, null) == _abi.LORA_UNSUPPORTED
    w2.dtype = 1
    seg = _abi.lora_segments_t()
    for f in ("sorted_idx", "seg_indptr", "req_to_lora", "num_segments", "tile_info",
              "tile_rows", "num_tiles"):
        setattr(seg, f, ctypes.cast(some, ctypes.POINTER(ctypes.c_int32)))
    seg.L, seg.max_tiles = 4, 8
    assert lib.lora_linear_fused(ctypes.byref(w2), null, 128, some, 128, 8, ctypes.byref(seg),
                                 some, 128, some, 1 << 20, null) == INV      # W null
    assert lib.lora_linear_fused(ctypes.byref(w2), some, 120, some, 128, 8, ctypes.byref(seg),
                                 some, 128, some, 1 << 20, null) == INV      # ldw < K
    assert lib.lora_linear_fused(ctypes.byref(w2), some, 128, some, 128, 8, ctypes.byref(seg),
                                 some, 128, some, 16, null) == INV           # workspace short
    # MoE align: capacity not a multiple of the block; then outputs missing
    assert lib.lora_moe_align(some, some, some, 4, 2, 8, 2, 64, 100, some, some, some,
                              null) == INV
    assert lib.lora_moe_align(some, some, some, 4, 2, 8, 2, 64, 128, null, some, some,
                              null) == INV
    assert lib.lora_moe_align(some, some, null, 4, 2, 8, 2, 64, 128, some, some, some,
                              null) == INV                                  # mask null
    assert lib.lora_moe_silu_and_mul(1, null, 0, null, 0, 4, 12, null) == INV   # I % 8
    assert lib.lora_moe_topk_reduce(1, null, 0, null, null, 0, 4, 0, 64, null) == INV
    assert lib.lora_table_plan(2, (ctypes.c_int32 * 2)(8, 65), 1, 64, 64,
                               (ctypes.c_int32 * 2)(), (ctypes.c_int64 * 2)(),
                               (ctypes.c_int64 * 2)(), ctypes.byref(ctypes.c_int64()),
                               ctypes.byref(ctypes.c_int64())) == INV           # rank > 64


# ------------------------------------------------------------------ binding checks
class _FakeTable:
    """Metadata of a table, enough for the binding's checks (which run before
    anything touches the device or the library)."""

    def __init__(self, dtype, K=64, N=32, L=4, cols=16):
        import torch
        self.dtype, self.K, self.N, self.L, self.cols = dtype, K, N, L, cols


def test_binding_rejects_mismatched_operands_before_any_launch():
    """An operand whose dtype differs from the table's (the kernels would
    store elements of the table's size into it), an x whose width is not K,
    a y narrower than N and a short S are refused by the binding itself."""
    import torch
    import adapter_lora_amd as ml
    bf, f32 = torch.bfloat16, torch.float32
    tb = _FakeTable(bf)
    ids = torch.zeros(4, dtype=torch.int32)
    x, y = torch.zeros(4, 64, dtype=bf), torch.zeros(4, 32, dtype=bf)
    for bad in [dict(x=x.float()), dict(y=y.float()), dict(x=torch.zeros(4, 72, dtype=bf)),
                dict(y=torch.zeros(4, 24, dtype=bf))]:
        args = dict(x=x, y=y)
        args.update(bad)
        with pytest.raises(ml.LoraError, match="weights are|columns"):
            ml.lora_fused_decode(tb, ids, args["x"], args["y"], None)
        with pytest.raises(ml.LoraError, match="weights are|columns"):
            ml.lora_shrink_expand_add(tb, args["x"], None, args["y"], None)
    with pytest.raises(ml.LoraError, match="weights are"):
        ml.lora_shrink(tb, x.float(), None, None, None)
    with pytest.raises(ml.LoraError, match="weights are"):
        ml.lora_linear_fused(tb, torch.zeros(32, 64, dtype=f32), x, None, y, None)
    with pytest.raises(ml.LoraError, match="S must hold"):
        ml.lora_expand_add(tb, torch.zeros(4 * 16 - 1, dtype=f32), None, y)
    with pytest.raises(ml.LoraError, match="weights are|columns"):
        ml.lora_embedding_decode(tb, ids, ids, y.float())
    # the same calls with matching operands get past these checks and stop
    # at the device check (CPU tensors), not at a dtype or shape complaint
    with pytest.raises(ml.LoraError, match="GPU|device"):
        ml.lora_fused_decode(tb, ids, x, y, None)
    with pytest.raises(ml.LoraError, match="GPU|device"):
        ml.lora_shrink_expand_add(tb, x, None, y, None)
    # MoE: caches of another dtype or width
    mw = type("W", (), dict(dtype=bf, H=64, I=32))()
    with pytest.raises(ml.LoraError, match="weights are"):
        ml.lora_moe_gate_up_add(mw, x, 2, None, torch.zeros(8, 64, dtype=f32), None)
    with pytest.raises(ml.LoraError, match="columns"):
        ml.lora_moe_gate_up_add(mw, x, 2, None, torch.zeros(8, 60, dtype=bf), None)
    with pytest.raises(ml.LoraError, match="weights are"):
        ml.lora_moe_down_add(mw, torch.zeros(8, 32, dtype=f32), 4, 2, None,
                             torch.zeros(8, 64, dtype=bf), None)
    with pytest.raises(ml.LoraError, match="weights are"):
        ml.lora_moe_silu_and_mul(torch.zeros(8, 64, dtype=bf), torch.zeros(8, 32, dtype=f32))
    with pytest.raises(ml.LoraError, match="weights are"):
        ml.lora_moe_topk_reduce(torch.zeros(8, 64, dtype=bf), torch.zeros(4, 2, dtype=f32),
                                torch.zeros(4, 64, dtype=f32))


ROCTX_PROBE = r"""
import ctypes, sys
sys.path.insert(0, %r)
from adapter_lora_amd import _abi
null = ctypes.c_void_p(0)
st = _abi.lib.lora_build_segments(null, null, -1, 4, null, null, null, null, null, null, null,
                                  8, null)
maps = open("/proc/self/maps").read()
print(st, int("rocprofiler-sdk-roctx" in maps))
"""


def roctx_library_present():
    return any(os.path.exists(os.path.join(d, n)) for d in ("/opt/rocm/lib",)
               for n in ("librocprofiler-sdk-roctx.so.1",))


@pytest.mark.skipif(not roctx_library_present(), reason="no roctx library on this host")
def test_roctx_ranges_are_opt_in():
    """MLORA_ROCTX=1 makes the first range-carrying call load the roctx
    library (looked up at run time); without it, nothing is loaded."""
    from adapter_lora_amd import _abi
    def run(env_value):
        env = dict(os.environ)
        env.pop("MLORA_ROCTX", None)
        if env_value is not None:
            env["MLORA_ROCTX"] = env_value
        out = subprocess.run(["python", "-c", ROCTX_PROBE % ROOT], env=env, capture_output=True,
                             text=True, timeout=120)
        assert out.returncode == 0, out.stderr
        st, loaded = out.stdout.split()
        assert int(st) == _abi.LORA_INVALID_ARG
        return int(loaded)
    assert run("1") == 1
    assert run(None) == 0
    assert run("0") == 0
