"""ctypes view of include/mlora.h: library loading, struct layouts and
function signatures.  Loading fails loudly when the library is missing; there
is no other implementation behind these names."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MLORA_LIB", os.path.join(HERE, "libmlora.so"))

LORA_OK, LORA_INVALID_ARG, LORA_UNSUPPORTED, LORA_HIP_ERROR = 0, 1, 2, 3
LORA_DEVERR_WAIT, LORA_DEVERR_BAD_ID, LORA_DEVERR_TABLE = 1, 2, 4
LORA_F32, LORA_BF16 = 0, 1
LORA_MAX_SLICES = 4
LORA_RANK_ALIGN = 16
LORA_MAX_RANK = 64
LORA_MAX_ADAPTERS = 1024
LORA_DECODE_MAX_M = 64
LORA_NOALLOC_SCRATCH_BYTES = 1 << 20
LORA_TILE_ROWS = 64
MLORA_ABI_VERSION = 5


class LoraError(RuntimeError):
    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"libmlora.so not built ({LIB_PATH}); run __graft_entry__.build() "
                      f"or python -m adapter_lora_amd.build")
lib = ctypes.CDLL(LIB_PATH)

P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64
PI32 = ctypes.POINTER(ctypes.c_int32)
PI64 = ctypes.POINTER(ctypes.c_int64)
SZ = ctypes.c_size_t


class lora_weights_t(ctypes.Structure):
    _fields_ = [("dtype", I32), ("K", I32), ("n_slices", I32), ("L", I32), ("r_max", I32),
                ("reserved", I32), ("slice_offsets", I64 * (LORA_MAX_SLICES + 1)),
                ("A", P), ("B", P), ("a_off", PI64), ("b_off", PI64), ("rank", PI32)]


class lora_segments_t(ctypes.Structure):
    _fields_ = [("sorted_idx", PI32), ("seg_indptr", PI32), ("req_to_lora", PI32),
                ("num_segments", PI32), ("tile_info", PI32), ("tile_rows", PI32),
                ("num_tiles", PI32), ("L", I32), ("max_tiles", I32)]


class lora_moe_weights_t(ctypes.Structure):
    _fields_ = [("dtype", I32), ("L", I32), ("E", I32), ("H", I32), ("I", I32), ("r", I32),
                ("shared_outer", I32),
                ("A_gu", P), ("B_gu", P), ("A_d", P), ("B_d", P), ("adapter_enabled", PI32)]


class lora_moe_align_t(ctypes.Structure):
    _fields_ = [("sorted_token_ids", PI32), ("expert_ids", PI32), ("ntpp", PI32),
                ("max_tokens_padded", I32), ("block_size_m", I32)]


PW = ctypes.POINTER(lora_weights_t)
PS = ctypes.POINTER(lora_segments_t)
PMW = ctypes.POINTER(lora_moe_weights_t)
PMA = ctypes.POINTER(lora_moe_align_t)

# name -> (restype, argtypes); this table is also the list of exported symbols
SIGNATURES = {
    "lora_abi_version": (I32, []),
    "lora_status_string": (ctypes.c_char_p, [I32]),
    "lora_workspace_size": (SZ, [PW, I32]),
    "lora_workspace_init": (I32, [P, SZ, P]),
    "lora_read_device_error": (I32, [P, PI32, P]),
    "lora_table_plan": (I32, [I32, PI32, I32, I32, I64, PI32, PI64, PI64, PI64, PI64]),
    "lora_pack_adapter": (I32, [I32, I32, I64, I32, I32, I32, P, P, P, P, P]),
    "lora_tile_capacity": (I32, [I32, I32]),
    "lora_build_segments": (I32, [P, P, I32, I32, P, P, P, P, P, P, P, I32, P]),
    "lora_shrink": (I32, [PW, P, I64, I32, PS, P, P, SZ, P]),
    "lora_expand_add": (I32, [PW, P, I32, PS, P, I64, P]),
    "lora_shrink_expand_add": (I32, [PW, P, I64, I32, PS, P, I64, P, SZ, P]),
    "lora_linear_fused": (I32, [PW, P, I64, P, I64, I32, PS, P, I64, P, SZ, P]),
    "lora_fused_decode": (I32, [PW, P, P, P, I64, I32, P, I64, P, P, P, P, P, P, P, I32, P, SZ,
                                P]),
    "lora_fused_decode_noalloc": (I32, [PW, P, P, P, I64, I32, P, I64, P, P, P, P, P, P, P, I32,
                                        P, P]),
    "lora_pack_embedding_adapter": (I32, [I32, I32, I64, I32, I32, P, P, P, P, P]),
    "lora_embedding_shrink": (I32, [PW, P, I32, PS, P, P]),
    "lora_embedding_decode": (I32, [PW, P, P, P, I32, P, I64, P, P, P, P, P, P, P, I32, P]),
    "lora_moe_align_capacity": (I32, [I32, I32, I32, I32]),
    "lora_moe_align": (I32, [P, P, P, I32, I32, I32, I32, I32, I32, P, P, P, P]),
    "lora_moe_workspace_size": (SZ, [PMW, I32]),
    "lora_moe_gate_up_add": (I32, [PMW, P, I64, I32, I32, PMA, P, I64, P, SZ, P]),
    "lora_moe_silu_and_mul": (I32, [I32, P, I64, P, I64, I32, I32, P]),
    "lora_moe_down_add": (I32, [PMW, P, I64, I32, I32, PMA, P, I64, P, SZ, P]),
    "lora_moe_topk_reduce": (I32, [I32, P, I64, P, P, I64, I32, I32, I32, P]),
}

for _name, (_res, _args) in SIGNATURES.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args

if lib.lora_abi_version() != MLORA_ABI_VERSION:
    raise ImportError("libmlora ABI version mismatch; rebuild the library")


def check(status: int, what: str) -> None:
    if status != LORA_OK:
        msg = lib.lora_status_string(status).decode()
        raise LoraError(f"{what}: {msg} (status {status})", status)
