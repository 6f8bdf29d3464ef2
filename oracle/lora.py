"""CPU oracle for dynamic multi-LoRA on a mixed batch (float64, per-token loops).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.  It shares no code with the HIP
library: it reads the per-adapter (unpacked) arrays, never the packed table.

Sources (the pages, by title and section):
  * "vLLM-Ascend dynamic LoRA operator" walkthrough (pwwt.cn), section 1.1:
    A is [r, K], B is [N, r]; y = x W^T + (x A^T) B^T.
  * same page, section 2.1: one id per token, -1 = no adapter; output rows
    are the base rows plus the token's own delta.
  * same page, section 2.2: two serial products S = x A^T, then S B^T.
  * same page, section 2.3: tokens clustered by lora id into a segment table
    (id, contiguous token range); per segment X_seg A_i^T then B_i^T, added
    to the y_base rows of those tokens.
  * same page, section 3.4: a -1 token's base row passes through unchanged.
  * same page, section 4.3: rank padded to a multiple of 16 with zero rows of
    A and zero columns of B.
  * SGLang "LoRA Layers" page, per-layer table: stacked QKV A (3r, in),
    B (q+2kv, r); gate/up A (2r, in), B (2*out, r); output_offset of the
    B-side call; rank-0 slot returns at once.
  * SGLang "LoRA + MoE" page, CUDA-graph section: an adapter_enabled mask
    switches adapters off without changing the captured shapes.

Readings where the pages are silent:
  * segment order: ascending adapter id; stable inside a segment;
  * -1 tokens are placed after every segment and belong to none;
  * adapters without tokens get no segment; buffer tails are filled
    (seg_indptr tail = M_valid, req_to_lora tail = -1);
  * stacked slices: A rows [s*r, (s+1)*r) and B rows [off_s, off_{s+1})
    belong to slice s; each slice has its own S columns;
  * rank-0 adapters behave like -1 for their tokens' outputs;
  * a token whose adapter is disabled in the enable mask is a token without
    an adapter (it is in no segment and its row passes through).
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def mask_ids(ids: Sequence[int], enabled, L: int) -> np.ndarray:
    """Apply an adapter enable mask (SGLang "LoRA + MoE" page, adapter_enabled):
    a token whose id is a slot with enabled == 0 becomes a token without an
    adapter (-1).  enabled=None leaves the ids as they are."""
    ids = np.asarray(ids, dtype=np.int64).copy()
    if enabled is None:
        return ids
    for m in range(ids.shape[0]):
        v = int(ids[m])
        if 0 <= v < L and int(enabled[v]) == 0:
            ids[m] = -1
    return ids


def build_segments(ids: Sequence[int], L: int,
                   enabled=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray, int]:
    """Token clustering by lora id into a segment table (Ascend walkthrough,
    section 2.3), after the enable mask (mask_ids).

    Steps:
      1. key(m) = ids[m] when 0 <= ids[m] < L, otherwise +inf (no adapter);
      2. sorted_idx = stable sort of 0..M-1 by key (ties keep token order);
      3. the ids present, ascending, become req_to_lora[0..S); seg_indptr[0]=0
         and seg_indptr[s+1] = seg_indptr[s] + count(req_to_lora[s]);
      4. tails: seg_indptr[s] = M_valid for S < s <= L, req_to_lora[s] = -1
         for S <= s < L.
    Returns (sorted_idx int32[M], seg_indptr int32[L+1], req_to_lora int32[L],
    num_segments).
    """
    ids = mask_ids(ids, enabled, L)
    M = ids.shape[0]
    valid = (ids >= 0) & (ids < L)
    key = np.where(valid, ids, np.iinfo(np.int64).max)
    sorted_idx = np.argsort(key, kind="stable").astype(np.int32)
    present = sorted(set(int(v) for v in ids[valid]))
    S = len(present)
    seg_indptr = np.zeros(L + 1, dtype=np.int32)
    req_to_lora = np.full(L, -1, dtype=np.int32)
    for s, a in enumerate(present):
        req_to_lora[s] = a
        seg_indptr[s + 1] = seg_indptr[s] + int(np.count_nonzero(ids == a))
    m_valid = int(seg_indptr[S])
    seg_indptr[S + 1:] = m_valid
    return sorted_idx, seg_indptr, req_to_lora, S


def tile_schedule(ids: Sequence[int], L: int, rows: int = 64, enabled=None):
    """Tile schedule over the segment table (Ascend walkthrough, section 2.4:
    which block belongs to which segment, and its rank, is worked out before
    the kernels run).  Segments in order, each cut into ceil(count / rows)
    tiles of consecutive sorted positions.
    Returns (info int32[T, 4] = (segment, adapter id, first position, rows),
    tile_rows int32[T, rows] = token index per row, -1 past the rows)."""
    sorted_idx, seg_indptr, req_to_lora, S = build_segments(ids, L, enabled)
    info, trows = [], []
    for s in range(S):
        beg, end = int(seg_indptr[s]), int(seg_indptr[s + 1])
        for p in range(beg, end, rows):
            n = min(rows, end - p)
            info.append([s, int(req_to_lora[s]), p, n])
            r = [-1] * rows
            r[:n] = [int(v) for v in sorted_idx[p:p + n]]
            trows.append(r)
    return (np.array(info, dtype=np.int32).reshape(-1, 4),
            np.array(trows, dtype=np.int32).reshape(-1, rows))


def slice_offsets(slice_sizes: Sequence[int]) -> List[int]:
    off = [0]
    for n in slice_sizes:
        off.append(off[-1] + int(n))
    return off


def lora_linear(x, ids, A: Sequence, B: Sequence, ranks: Sequence[int],
                slice_sizes: Sequence[int], y_base, enabled=None) -> np.ndarray:
    """y = y_base + per-token delta (Ascend walkthrough sections 1.1, 2.2,
    3.4; stacked slices per the SGLang "LoRA Layers" table).

    For each token m with adapter i = ids[m] (skipped when i is -1, out of
    range, or rank[i] == 0):
        for each slice s:
            S[s, j] = sum_k x[m, k] * A_i[s*r_i + j, k]          (j < r_i)
            y[m, n] = y_base[m, n] + sum_j S[s, j] * B_i[n, j]   (off_s <= n < off_{s+1})
    All arithmetic in float64.  Rows that get no delta are copied bit for bit.
    Disabled adapters (enable mask) count as -1.
    """
    x = _f64(x)
    y = np.array(y_base, dtype=np.float64, copy=True)
    M = x.shape[0]
    off = slice_offsets(slice_sizes)
    L = len(ranks)
    ids = mask_ids(ids, enabled, L)
    for m in range(M):
        i = int(ids[m])
        if i < 0 or i >= L or ranks[i] == 0:
            continue
        r = int(ranks[i])
        Ai = _f64(A[i])
        Bi = _f64(B[i])
        for s in range(len(slice_sizes)):
            # S[j] = sum_k x[m, k] * A_i[s*r + j, k]   (matrix-vector product)
            S = Ai[s * r:(s + 1) * r, :] @ x[m]
            # y[m, n] += sum_j S[j] * B_i[n, j]        for n in slice s
            y[m, off[s]:off[s + 1]] = y[m, off[s]:off[s + 1]] + Bi[off[s]:off[s + 1], :r] @ S
    return y


def lora_shrink(x, ids, A: Sequence, ranks: Sequence[int], n_slices: int,
                r_cols: int) -> np.ndarray:
    """S in sorted-row order (Ascend walkthrough section 2.3, first product of
    the segmented flow): for sorted position p of a token m with adapter i,
        S[p, s, j] = sum_k x[m, k] * A_i[s*r_i + j, k]   for j < r_i,
    and 0 for r_i <= j < r_cols (zero rank padding, section 4.3).
    Rows p >= M_valid are returned as zeros.  Shape [M, n_slices, r_cols]."""
    x = _f64(x)
    L = len(ranks)
    sorted_idx, seg_indptr, req_to_lora, S_cnt = build_segments(ids, L)
    M = x.shape[0]
    out = np.zeros((M, n_slices, r_cols))
    for s_id in range(S_cnt):
        i = int(req_to_lora[s_id])
        r = int(ranks[i])
        Ai = _f64(A[i])
        for p in range(seg_indptr[s_id], seg_indptr[s_id + 1]):
            m = int(sorted_idx[p])
            for s in range(n_slices):
                out[p, s, :r] = Ai[s * r:(s + 1) * r, :] @ x[m]
    return out


def lora_expand_add(S, ids, B: Sequence, ranks: Sequence[int], slice_sizes: Sequence[int],
                    y_base) -> np.ndarray:
    """Second product of the segmented flow (Ascend walkthrough section 2.3),
    with the B-side output offsets of the SGLang "LoRA Layers" page:
        y[m, off_s + n] = y_base[m, off_s + n] + sum_{j<r_i} S[p, s, j] * B_i[off_s + n, j]
    where p is the sorted position of token m.  S is [M, n_sl, >= r_max]."""
    S = _f64(S)
    y = np.array(y_base, dtype=np.float64, copy=True)
    L = len(ranks)
    sorted_idx, seg_indptr, req_to_lora, S_cnt = build_segments(ids, L)
    off = slice_offsets(slice_sizes)
    for s_id in range(S_cnt):
        i = int(req_to_lora[s_id])
        r = int(ranks[i])
        if r == 0:
            continue
        Bi = _f64(B[i])
        for p in range(seg_indptr[s_id], seg_indptr[s_id + 1]):
            m = int(sorted_idx[p])
            for s in range(len(slice_sizes)):
                y[m, off[s]:off[s + 1]] = (y[m, off[s]:off[s + 1]]
                                           + Bi[off[s]:off[s + 1], :r] @ S[p, s, :r])
    return y


def delta_rows(ids, ranks, enabled=None) -> np.ndarray:
    """Boolean mask of the rows that receive a delta."""
    L = len(ranks)
    ids = mask_ids(ids, enabled, L)
    ok = (ids >= 0) & (ids < L)
    out = np.zeros(ids.shape[0], dtype=bool)
    for m in np.nonzero(ok)[0]:
        out[m] = ranks[int(ids[m])] > 0
    return out


def embedding_add(tokens, ids, A: Sequence, B: Sequence, ranks: Sequence[int], vocab: int,
                  y_base, enabled=None) -> np.ndarray:
    """Embedding LoRA (SGLang "LoRA Layers" page, VocabParallelEmbeddingWithLoRA:
    the A side is an embedding lookup of A_i [r, vocab], the B side the usual
    product with B_i [emb, r] added to the base output).

    For each token m with adapter i = ids[m] (skipped when i is -1, out of
    range, disabled or rank[i] == 0) and token id t = tokens[m]:
        S[j] = A_i[j, t]                               (j < r_i)
        y[m, n] = y_base[m, n] + sum_j S[j] * B_i[n, j]
    A token id outside [0, vocab) gets no delta (the page masks such added
    tokens for the base lookup; LoRA for them is not supported there).
    float64; rows without a delta are copied bit for bit."""
    y = np.array(y_base, dtype=np.float64, copy=True)
    L = len(ranks)
    ids = mask_ids(ids, enabled, L)
    for m in range(y.shape[0]):
        i = int(ids[m])
        t = int(tokens[m])
        if i < 0 or i >= L or ranks[i] == 0 or t < 0 or t >= vocab:
            continue
        r = int(ranks[i])
        S = _f64(A[i])[:r, t]                  # the lookup: column t of A_i
        y[m] = y[m] + _f64(B[i])[:, :r] @ S
    return y


def linear_with_base(x, W, ids, A: Sequence, B: Sequence, ranks: Sequence[int],
                     slice_sizes: Sequence[int], enabled=None) -> np.ndarray:
    """The base layer and its LoRA delta together (Ascend walkthrough section
    1.1: y = x W^T + (x A^T) B^T; SGLang "LoRA Layers" page, structure
    diagram: base_output + lora_delta).  W is [N_tot, K].  The base product
    is one float64 matrix product; the delta is lora_linear's per-token loop
    on top of it."""
    y_base = _f64(x) @ _f64(W).T
    return lora_linear(x, ids, A, B, ranks, slice_sizes, y_base, enabled)
