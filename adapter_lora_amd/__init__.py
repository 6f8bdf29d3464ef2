"""Python binding of libmlora (dynamic multi-LoRA on MI355X / gfx950).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the path runs in the library's kernels.
The names match the C ABI in include/mlora.h.  There is no fallback: if the
library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch

from ._abi import (LORA_BF16, LORA_F32, LORA_MAX_ADAPTERS, LORA_MAX_RANK,
                   LORA_MAX_SLICES, LORA_DECODE_MAX_M, LORA_TILE_ROWS, LORA_DEVERR_WAIT,
                   LORA_DEVERR_BAD_ID, LORA_DEVERR_TABLE, LoraError, lib, lora_weights_t,
                   lora_segments_t, lora_moe_weights_t, lora_moe_align_t, check)

__all__ = [
    "LORA_BF16", "LORA_F32", "LORA_DEVERR_WAIT", "LORA_DEVERR_BAD_ID", "LORA_DEVERR_TABLE", "LoraError", "LoraTable",
    "Segments", "Workspace",
    "MoeWeights", "MoeAlign",
    "lora_build_segments", "lora_tile_capacity", "lora_shrink", "lora_expand_add",
    "lora_shrink_expand_add", "lora_fused_decode", "lora_fused_decode_noalloc",
    "lora_pack_embedding_adapter", "lora_embedding_shrink", "lora_embedding_decode",
    "lora_workspace_size", "lora_workspace_init", "lora_read_device_error",
    "lora_table_plan", "lora_pack_adapter",
    "lora_moe_align_capacity", "lora_moe_align", "lora_moe_workspace_size",
    "lora_moe_gate_up_add", "lora_moe_silu_and_mul", "lora_moe_down_add",
    "lora_moe_topk_reduce", "stream_handle",
]


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_cur_device = getattr(torch._C, "_cuda_getDevice", None)


def stream_handle(stream: Optional[torch.cuda.Stream] = None) -> int:
    """hipStream_t of `stream`, else of the current stream (read without
    building a Stream object: a decode call is short enough for the host side
    of a launch to matter)."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None and _cur_device is not None:
        return _raw_stream(_cur_device())
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return LORA_BF16
    if t == torch.float32:
        return LORA_F32
    raise LoraError(f"unsupported dtype {t}")


def _ptr(t: Optional[torch.Tensor]) -> int:
    """Device address of a tensor (0 for None), passed as a plain int: the
    argument types declared for the library convert it."""
    return 0 if t is None else t.data_ptr()


def _check_io(dtype: torch.dtype, **named) -> None:
    """Every operand shares the table's dtype (the kernels read and write
    elements of that size): checked before any launch, on the tensors'
    metadata only."""
    for name, t in named.items():
        if t is not None and t.dtype != dtype:
            raise LoraError(f"{name} is {t.dtype} but the weights are {dtype}")


def _cols(t: torch.Tensor, name: str, want: int, exact: bool = True) -> None:
    """A 2-D operand has `want` columns (exact) or at least `want`."""
    if t.dim() != 2:
        raise LoraError(f"{name} must be a 2-D tensor")
    w = t.shape[1]
    if (w != want) if exact else (w < want):
        raise LoraError(f"{name} has {w} columns, {'' if exact else 'at least '}{want} needed")


def _rows(t: torch.Tensor, name: str) -> int:
    """Leading dimension of a row-major 2-D device tensor."""
    if t.dim() != 2 or (t.numel() > 0 and t.stride(1) != 1):
        raise LoraError(f"{name} must be a 2-D tensor with unit column stride")
    if not t.is_cuda:
        raise LoraError(f"{name} must live on the GPU")
    return max(t.stride(0), t.shape[1])


# ------------------------------------------------------------------------- table
def lora_table_plan(ranks: Sequence[int], n_slices: int, K: int, N_total: int):
    L = len(ranks)
    r = (ctypes.c_int32 * L)(*ranks)
    rp = (ctypes.c_int32 * L)()
    ao = (ctypes.c_int64 * L)()
    bo = (ctypes.c_int64 * L)()
    na, nb = ctypes.c_int64(), ctypes.c_int64()
    check(lib.lora_table_plan(L, r, n_slices, K, N_total, rp, ao, bo, ctypes.byref(na),
                              ctypes.byref(nb)), "lora_table_plan")
    return list(rp), list(ao), list(bo), na.value, nb.value


def lora_pack_adapter(A_src: torch.Tensor, B_src: torch.Tensor, K: int, N_total: int,
                      n_slices: int, rank: int, rank_pad: int, A_dst: torch.Tensor,
                      B_dst: torch.Tensor, stream=None) -> None:
    check(lib.lora_pack_adapter(_dtype_code(A_src.dtype), K, N_total, n_slices, rank, rank_pad,
                                _ptr(A_src), _ptr(B_src), _ptr(A_dst), _ptr(B_dst),
                                stream_handle(stream)), "lora_pack_adapter")


def lora_pack_embedding_adapter(A_src: torch.Tensor, B_src: torch.Tensor, vocab: int, emb: int,
                                rank: int, rank_pad: int, A_dst: torch.Tensor,
                                B_dst: torch.Tensor, stream=None) -> None:
    check(lib.lora_pack_embedding_adapter(_dtype_code(A_src.dtype), vocab, emb, rank, rank_pad,
                                          _ptr(A_src), _ptr(B_src), _ptr(A_dst), _ptr(B_dst),
                                          stream_handle(stream)), "lora_pack_embedding_adapter")


class LoraTable:
    """Rank-grouped packed adapter table on the device (load time).

    A[i]: [n_slices * r_i, K] (slice s = rows [s*r_i, (s+1)*r_i)),
    B[i]: [N_total, r_i]; rank 0 (or None) marks an empty slot.
    embedding=True: an embedding table (K = vocab, one slice of width emb),
    A[i] [r_i, vocab] packed transposed for the lookup.
    """

    def __init__(self, A: Sequence[Optional[torch.Tensor]], B: Sequence[Optional[torch.Tensor]],
                 ranks: Sequence[int], slice_sizes: Sequence[int], K: int,
                 dtype: torch.dtype, device="cuda", stream=None, embedding: bool = False):
        self.L = len(ranks)
        if not (1 <= self.L <= LORA_MAX_ADAPTERS):
            raise LoraError("adapter count out of range")
        if not (1 <= len(slice_sizes) <= LORA_MAX_SLICES):
            raise LoraError("slice count out of range")
        self.K = int(K)
        self.n_slices = len(slice_sizes)
        self.slice_sizes = [int(n) for n in slice_sizes]
        self.N = int(sum(self.slice_sizes))
        self.dtype = dtype
        self.ranks = [int(r) for r in ranks]
        rp, ao, bo, na, nb = lora_table_plan(self.ranks, self.n_slices, self.K, self.N)
        self.rank_pad = rp
        self.r_max = max([16] + rp)
        self.A_table = torch.zeros(max(na, 8), dtype=dtype, device=device)
        self.B_table = torch.zeros(max(nb, 8), dtype=dtype, device=device)
        for i, r in enumerate(self.ranks):
            if r == 0:
                continue
            a = A[i].to(device=device, dtype=dtype).contiguous()
            b = B[i].to(device=device, dtype=dtype).contiguous()
            if tuple(a.shape) != (self.n_slices * r, self.K) or tuple(b.shape) != (self.N, r):
                raise LoraError(f"adapter {i}: bad A/B shape {tuple(a.shape)} {tuple(b.shape)}")
            if embedding:
                if self.n_slices != 1:
                    raise LoraError("an embedding table has one output slice")
                lora_pack_embedding_adapter(a, b, self.K, self.N, r, rp[i], self.A_table[ao[i]:],
                                            self.B_table[bo[i]:], stream)
            else:
                lora_pack_adapter(a, b, self.K, self.N, self.n_slices, r, rp[i],
                                  self.A_table[ao[i]:], self.B_table[bo[i]:], stream)
        self.a_off = torch.tensor(ao, dtype=torch.int64, device=device)
        self.b_off = torch.tensor(bo, dtype=torch.int64, device=device)
        self.rank_dev = torch.tensor(rp, dtype=torch.int32, device=device)
        off = [0]
        for n in self.slice_sizes:
            off.append(off[-1] + n)
        so = (ctypes.c_int64 * (LORA_MAX_SLICES + 1))(*(off + [0] * (LORA_MAX_SLICES + 1 - len(off))))
        self.c = lora_weights_t(_dtype_code(dtype), self.K, self.n_slices, self.L, self.r_max, 0,
                                so, _ptr(self.A_table), _ptr(self.B_table),
                                ctypes.cast(_ptr(self.a_off), ctypes.POINTER(ctypes.c_int64)),
                                ctypes.cast(_ptr(self.b_off), ctypes.POINTER(ctypes.c_int64)),
                                ctypes.cast(_ptr(self.rank_dev), ctypes.POINTER(ctypes.c_int32)))
        self.ref = ctypes.pointer(self.c)

    @property
    def cols(self) -> int:
        return self.n_slices * self.r_max


# ------------------------------------------------------------------------- segments
class Segments:
    """Device buffers of a segment table and its tile schedule for up to
    M_cap tokens and L slots."""

    def __init__(self, M_cap: int, L: int, device="cuda"):
        self.L = int(L)
        self.max_tiles = max(int(lib.lora_tile_capacity(M_cap, L)), 1)
        self.sorted_idx = torch.empty(max(M_cap, 1), dtype=torch.int32, device=device)
        self.seg_indptr = torch.empty(L + 1, dtype=torch.int32, device=device)
        self.req_to_lora = torch.empty(L, dtype=torch.int32, device=device)
        self.num_segments = torch.empty(1, dtype=torch.int32, device=device)
        self.tile_info = torch.empty(self.max_tiles * 4, dtype=torch.int32, device=device)
        self.tile_rows = torch.empty(self.max_tiles * LORA_TILE_ROWS, dtype=torch.int32,
                                     device=device)
        self.num_tiles = torch.empty(1, dtype=torch.int32, device=device)
        p32 = lambda t: ctypes.cast(_ptr(t), ctypes.POINTER(ctypes.c_int32))
        self.c = lora_segments_t(p32(self.sorted_idx), p32(self.seg_indptr), p32(self.req_to_lora),
                                 p32(self.num_segments), p32(self.tile_info), p32(self.tile_rows),
                                 p32(self.num_tiles), self.L, self.max_tiles)
        # the output pointers of a call that writes the table, in ABI order
        self.outs = tuple(_ptr(t) for t in (self.sorted_idx, self.seg_indptr, self.req_to_lora,
                                            self.num_segments, self.tile_info, self.tile_rows,
                                            self.num_tiles))
        self.ref = ctypes.pointer(self.c)


_NO_OUTS = (0,) * 7


def _ids_arg(ids: torch.Tensor) -> int:
    if ids.dtype != torch.int32 or not ids.is_cuda or ids.dim() != 1 or not ids.is_contiguous():
        raise LoraError("ids must be a contiguous 1-D int32 device tensor")
    return ids.shape[0]


def _mask_arg(adapter_enabled: Optional[torch.Tensor], L: int) -> ctypes.c_void_p:
    if adapter_enabled is None:
        return _ptr(None)
    t = adapter_enabled
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous() or t.numel() < L:
        raise LoraError("adapter_enabled must be a contiguous int32 device tensor of L entries")
    return _ptr(t)


def lora_build_segments(ids: torch.Tensor, seg: Segments, stream=None,
                        adapter_enabled: Optional[torch.Tensor] = None) -> None:
    M = _ids_arg(ids)
    if M > seg.sorted_idx.shape[0]:
        raise LoraError("segment buffers too small")
    check(lib.lora_build_segments(ids.data_ptr(), _mask_arg(adapter_enabled, seg.L), M, seg.L,
                                  *seg.outs, seg.max_tiles, stream_handle(stream)),
          "lora_build_segments")


def lora_tile_capacity(M: int, L: int) -> int:
    return int(lib.lora_tile_capacity(M, L))


# ------------------------------------------------------------------------- workspace
def lora_workspace_size(table: LoraTable, M: int) -> int:
    return int(lib.lora_workspace_size(ctypes.byref(table.c), M))


def lora_workspace_init(ws: torch.Tensor, stream=None) -> None:
    check(lib.lora_workspace_init(_ptr(ws), ws.numel(), stream_handle(stream)),
          "lora_workspace_init")


def lora_read_device_error(ws: torch.Tensor, stream=None) -> int:
    out = ctypes.c_int32()
    check(lib.lora_read_device_error(_ptr(ws), ctypes.byref(out), stream_handle(stream)),
          "lora_read_device_error")
    return out.value


class Workspace:
    """Zero-initialised device workspace (uint8) for a table and up to M tokens."""

    def __init__(self, nbytes: int, device="cuda", stream=None):
        self.buf = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        self.ptr, self.nbytes = _ptr(self.buf), self.buf.numel()
        lora_workspace_init(self.buf, stream)

    @classmethod
    def for_table(cls, table: LoraTable, M: int, device="cuda", stream=None):
        return cls(lora_workspace_size(table, M), device, stream)


# ------------------------------------------------------------------------- dense calls
def lora_shrink(table: LoraTable, x: torch.Tensor, seg: Segments, S: torch.Tensor,
                ws: Workspace, stream=None) -> None:
    _check_io(table.dtype, x=x)
    _cols(x, "x", table.K)
    ldx = _rows(x, "x")
    if S.dtype != torch.float32 or not S.is_contiguous() or S.numel() < x.shape[0] * table.cols:
        raise LoraError("S must be a contiguous fp32 [M, n_slices, r_max] tensor")
    check(lib.lora_shrink(ctypes.byref(table.c), _ptr(x), ldx, x.shape[0], ctypes.byref(seg.c),
                          _ptr(S), _ptr(ws.buf), ws.buf.numel(), stream_handle(stream)),
          "lora_shrink")


def lora_embedding_shrink(table: LoraTable, tokens: torch.Tensor, seg: Segments,
                          S: torch.Tensor, stream=None) -> None:
    """Embedding lookup side: S [M, r_max] (sorted rows) from the token ids."""
    M = _ids_arg(tokens)
    if S.dtype != torch.float32 or not S.is_contiguous() or S.numel() < M * table.cols:
        raise LoraError("S must be a contiguous fp32 [M, r_max] tensor")
    check(lib.lora_embedding_shrink(ctypes.byref(table.c), _ptr(tokens), M, ctypes.byref(seg.c),
                                    _ptr(S), stream_handle(stream)), "lora_embedding_shrink")


def lora_embedding_decode(table: LoraTable, ids: torch.Tensor, tokens: torch.Tensor,
                          y: torch.Tensor, seg: Optional[Segments] = None,
                          adapter_enabled: Optional[torch.Tensor] = None, stream=None) -> None:
    """One launch: y += B_i A_i[:, token] for up to 64 tokens (embedding
    LoRA), grouped by adapter on chip; writes the segment table into `seg`
    when given."""
    _check_io(table.dtype, y=y)
    _cols(y, "y", table.N, exact=False)
    M = _ids_arg(ids)
    if _ids_arg(tokens) != M or y.shape[0] != M:
        raise LoraError("ids, tokens and y must have the same number of rows")
    ldy = _rows(y, "y")
    if seg is not None:
        if seg.L != table.L or M > seg.sorted_idx.shape[0]:
            raise LoraError("segment buffers do not match the table or the batch")
        outs = [_ptr(seg.sorted_idx), _ptr(seg.seg_indptr), _ptr(seg.req_to_lora),
                _ptr(seg.num_segments), _ptr(seg.tile_info), _ptr(seg.tile_rows),
                _ptr(seg.num_tiles)]
        cap = seg.max_tiles
    else:
        outs = [_ptr(None)] * 7
        cap = 0
    check(lib.lora_embedding_decode(ctypes.byref(table.c), _ptr(ids),
                                    _mask_arg(adapter_enabled, table.L), _ptr(tokens), M, _ptr(y),
                                    ldy, *outs, cap, stream_handle(stream)),
          "lora_embedding_decode")


def lora_expand_add(table: LoraTable, S: torch.Tensor, seg: Segments, y: torch.Tensor,
                    stream=None) -> None:
    _check_io(table.dtype, y=y)
    _cols(y, "y", table.N, exact=False)
    if S.dtype != torch.float32 or not S.is_contiguous():
        raise LoraError("S must be a contiguous fp32 tensor")
    if S.numel() < y.shape[0] * table.cols:
        raise LoraError("S must hold [M, n_slices, r_max] values")
    ldy = _rows(y, "y")
    check(lib.lora_expand_add(ctypes.byref(table.c), _ptr(S), y.shape[0], ctypes.byref(seg.c),
                              _ptr(y), ldy, stream_handle(stream)), "lora_expand_add")


def lora_shrink_expand_add(table: LoraTable, x: torch.Tensor, seg: Segments, y: torch.Tensor,
                           ws: Workspace, stream=None) -> None:
    _check_io(table.dtype, x=x, y=y)
    _cols(x, "x", table.K)
    _cols(y, "y", table.N, exact=False)
    ldx, ldy = _rows(x, "x"), _rows(y, "y")
    if x.shape[0] != y.shape[0]:
        raise LoraError("x and y must have the same number of rows")
    check(lib.lora_shrink_expand_add(table.ref, x.data_ptr(), ldx, x.shape[0], seg.ref,
                                     y.data_ptr(), ldy, ws.ptr, ws.nbytes, stream_handle(stream)),
          "lora_shrink_expand_add")


def lora_linear_fused(table: LoraTable, W: torch.Tensor, x: torch.Tensor, seg: Segments,
                      y: torch.Tensor, ws: Workspace, stream=None) -> None:
    """y = x W^T + (x A_i^T) B_i^T per token (bf16), y overwritten; W is the
    base weight [N, K] with the table's slices stacked in order."""
    _check_io(table.dtype, W=W, x=x, y=y)
    _cols(W, "W", table.K)
    _cols(x, "x", table.K)
    _cols(y, "y", table.N, exact=False)
    if x.shape[0] != y.shape[0]:
        raise LoraError("x and y must have the same number of rows")
    if W.shape[0] != table.N:
        raise LoraError("W must have one row per output column of the table")
    ldw, ldx, ldy = _rows(W, "W"), _rows(x, "x"), _rows(y, "y")
    check(lib.lora_linear_fused(ctypes.byref(table.c), _ptr(W), ldw, _ptr(x), ldx, x.shape[0],
                                ctypes.byref(seg.c), _ptr(y), ldy, _ptr(ws.buf), ws.buf.numel(),
                                stream_handle(stream)),
          "lora_linear_fused")


def lora_fused_decode(table: LoraTable, ids: torch.Tensor, x: torch.Tensor, y: torch.Tensor,
                      ws: Workspace, seg: Optional[Segments] = None,
                      adapter_enabled: Optional[torch.Tensor] = None, stream=None) -> None:
    """One launch: y += (x A_id^T) B_id^T for up to 64 tokens, grouped by
    adapter on chip; when `seg` is given the launch also writes the batch's
    segment table there."""
    _check_io(table.dtype, x=x, y=y)
    _cols(x, "x", table.K)
    _cols(y, "y", table.N, exact=False)
    M = _ids_arg(ids)
    ldx, ldy = _rows(x, "x"), _rows(y, "y")
    if x.shape[0] != M or y.shape[0] != M:
        raise LoraError("ids, x and y must have the same number of rows")
    if seg is not None:
        if seg.L != table.L or M > seg.sorted_idx.shape[0]:
            raise LoraError("segment buffers do not match the table or the batch")
        outs, cap = seg.outs, seg.max_tiles
    else:
        outs, cap = _NO_OUTS, 0
    check(lib.lora_fused_decode(table.ref, ids.data_ptr(), _mask_arg(adapter_enabled, table.L),
                                x.data_ptr(), ldx, M, y.data_ptr(), ldy, *outs, cap, ws.ptr,
                                ws.nbytes, stream_handle(stream)), "lora_fused_decode")


def lora_fused_decode_noalloc(table: LoraTable, ids: torch.Tensor, x: torch.Tensor,
                              y: torch.Tensor, seg: Optional[Segments] = None,
                              adapter_enabled: Optional[torch.Tensor] = None,
                              error_word: Optional[torch.Tensor] = None, stream=None) -> None:
    """lora_fused_decode without a workspace, for callers that cannot
    allocate: the library's fixed per-GPU array holds the exchange slots.
    Allocates nothing here either; error bits are OR-ed into `error_word`
    (a one-element int32 device tensor) when given."""
    _check_io(table.dtype, x=x, y=y)
    _cols(x, "x", table.K)
    _cols(y, "y", table.N, exact=False)
    M = _ids_arg(ids)
    ldx, ldy = _rows(x, "x"), _rows(y, "y")
    if x.shape[0] != M or y.shape[0] != M:
        raise LoraError("ids, x and y must have the same number of rows")
    if error_word is not None and (error_word.dtype != torch.int32 or not error_word.is_cuda
                                   or error_word.numel() < 1):
        raise LoraError("error_word must be an int32 device tensor")
    if seg is not None:
        if seg.L != table.L or M > seg.sorted_idx.shape[0]:
            raise LoraError("segment buffers do not match the table or the batch")
        outs, cap = seg.outs, seg.max_tiles
    else:
        outs, cap = _NO_OUTS, 0
    check(lib.lora_fused_decode_noalloc(table.ref, ids.data_ptr(),
                                        _mask_arg(adapter_enabled, table.L), x.data_ptr(), ldx,
                                        M, y.data_ptr(), ldy, *outs, cap, _ptr(error_word),
                                        stream_handle(stream)), "lora_fused_decode_noalloc")


# ------------------------------------------------------------------------- MoE
class MoeWeights:
    """Dense per-expert LoRA stacks [L, E, r, H] / [L, E, 2I, r] / [L, E, r, I] / [L, E, H, r].
    Outer stacks shared by the experts (gate_up A [L, 1, r, H] and down B
    [L, 1, H, r]) are recognised from their single expert slot."""

    def __init__(self, A_gu, B_gu, A_d, B_d, adapter_enabled):
        self.A_gu, self.B_gu = A_gu.contiguous(), B_gu.contiguous()
        self.A_d, self.B_d = A_d.contiguous(), B_d.contiguous()
        self.enabled = adapter_enabled.to(torch.int32).contiguous()
        L, E, I2, r = self.B_gu.shape
        I = I2 // 2
        H = self.A_gu.shape[3]
        eo = self.A_gu.shape[1]
        self.shared_outer = eo == 1 and E > 1
        if tuple(self.A_gu.shape) != (L, eo, r, H) or eo not in (1, E) \
                or tuple(self.A_d.shape) != (L, E, r, I) or tuple(self.B_d.shape) != (L, eo, H, r):
            raise LoraError("inconsistent MoE LoRA shapes")
        self.L, self.E, self.r, self.H, self.I = L, E, r, H, I
        self.dtype = self.A_gu.dtype
        self.c = lora_moe_weights_t(_dtype_code(self.dtype), L, E, H, I, r,
                                    1 if self.shared_outer else 0, _ptr(self.A_gu),
                                    _ptr(self.B_gu), _ptr(self.A_d), _ptr(self.B_d),
                                    ctypes.cast(_ptr(self.enabled), ctypes.POINTER(ctypes.c_int32)))


def lora_moe_align_capacity(M: int, topk: int, E: int, block_size_m: int) -> int:
    return int(lib.lora_moe_align_capacity(M, topk, E, block_size_m))


class MoeAlign:
    def __init__(self, L: int, max_tokens_padded: int, block_size_m: int, device="cuda"):
        self.sorted_token_ids = torch.empty(L * max_tokens_padded, dtype=torch.int32, device=device)
        self.expert_ids = torch.empty(L * (max_tokens_padded // block_size_m), dtype=torch.int32,
                                      device=device)
        self.ntpp = torch.empty(L, dtype=torch.int32, device=device)
        self.L = L
        self.max_tokens_padded = max_tokens_padded
        self.block_size_m = block_size_m
        self.c = lora_moe_align_t(
            ctypes.cast(_ptr(self.sorted_token_ids), ctypes.POINTER(ctypes.c_int32)),
            ctypes.cast(_ptr(self.expert_ids), ctypes.POINTER(ctypes.c_int32)),
            ctypes.cast(_ptr(self.ntpp), ctypes.POINTER(ctypes.c_int32)),
            max_tokens_padded, block_size_m)


def lora_moe_align(topk_ids: torch.Tensor, ids: torch.Tensor, adapter_enabled: torch.Tensor,
                   E: int, out: MoeAlign, stream=None) -> None:
    M, topk = topk_ids.shape
    for t, n in ((topk_ids, "topk_ids"), (ids, "ids"), (adapter_enabled, "adapter_enabled")):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise LoraError(f"{n} must be a contiguous int32 device tensor")
    if ids.numel() != M or adapter_enabled.numel() < out.L:
        raise LoraError("ids must have M entries and adapter_enabled L")
    check(lib.lora_moe_align(_ptr(topk_ids), _ptr(ids), _ptr(adapter_enabled), M, topk, E,
                             out.L, out.block_size_m, out.max_tokens_padded,
                             _ptr(out.sorted_token_ids), _ptr(out.expert_ids), _ptr(out.ntpp),
                             stream_handle(stream)), "lora_moe_align")


def lora_moe_workspace_size(w: MoeWeights, max_tokens_padded: int) -> int:
    return int(lib.lora_moe_workspace_size(ctypes.byref(w.c), max_tokens_padded))


def lora_moe_gate_up_add(w: MoeWeights, x: torch.Tensor, topk: int, align: MoeAlign,
                         cache1: torch.Tensor, ws: Workspace, stream=None) -> None:
    _check_io(w.dtype, x=x, cache1=cache1)
    _cols(x, "x", w.H)
    _cols(cache1, "cache1", 2 * w.I, exact=False)
    if cache1.shape[0] < x.shape[0] * topk:
        raise LoraError("cache1 needs one row per (token, expert) pair")
    check(lib.lora_moe_gate_up_add(ctypes.byref(w.c), _ptr(x), _rows(x, "x"), x.shape[0], topk,
                                   ctypes.byref(align.c), _ptr(cache1), _rows(cache1, "cache1"),
                                   _ptr(ws.buf), ws.buf.numel(), stream_handle(stream)),
          "lora_moe_gate_up_add")


def lora_moe_silu_and_mul(cache1: torch.Tensor, cache2: torch.Tensor, stream=None) -> None:
    _check_io(cache1.dtype, cache2=cache2)
    P, I = cache2.shape
    _cols(cache1, "cache1", 2 * I, exact=False)
    if cache1.shape[0] < P:
        raise LoraError("cache1 has fewer rows than cache2")
    check(lib.lora_moe_silu_and_mul(_dtype_code(cache1.dtype), _ptr(cache1), _rows(cache1, "cache1"),
                                    _ptr(cache2), _rows(cache2, "cache2"), P, I,
                                    stream_handle(stream)), "lora_moe_silu_and_mul")


def lora_moe_down_add(w: MoeWeights, cache2: torch.Tensor, M: int, topk: int, align: MoeAlign,
                      cache3: torch.Tensor, ws: Workspace, stream=None) -> None:
    _check_io(w.dtype, cache2=cache2, cache3=cache3)
    _cols(cache2, "cache2", w.I)
    _cols(cache3, "cache3", w.H, exact=False)
    if cache2.shape[0] < M * topk or cache3.shape[0] < M * topk:
        raise LoraError("cache2 and cache3 need one row per (token, expert) pair")
    check(lib.lora_moe_down_add(ctypes.byref(w.c), _ptr(cache2), _rows(cache2, "cache2"), M, topk,
                                ctypes.byref(align.c), _ptr(cache3), _rows(cache3, "cache3"),
                                _ptr(ws.buf), ws.buf.numel(), stream_handle(stream)),
          "lora_moe_down_add")


def lora_moe_topk_reduce(cache3: torch.Tensor, topk_weights: torch.Tensor, out: torch.Tensor,
                         stream=None) -> None:
    M, topk = topk_weights.shape
    if topk_weights.dtype != torch.float32 or not topk_weights.is_contiguous():
        raise LoraError("topk_weights must be contiguous fp32")
    _check_io(cache3.dtype, out=out)
    _cols(cache3, "cache3", out.shape[1], exact=False)
    if out.shape[0] < M or cache3.shape[0] < M * topk:
        raise LoraError("out needs M rows and cache3 M * topk")
    check(lib.lora_moe_topk_reduce(_dtype_code(cache3.dtype), _ptr(cache3), _rows(cache3, "cache3"),
                                   _ptr(topk_weights), _ptr(out), _rows(out, "out"), M, topk,
                                   out.shape[1], stream_handle(stream)), "lora_moe_topk_reduce")
