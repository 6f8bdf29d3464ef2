"""CPU oracle for LoRA on a Mixture-of-Experts MLP (float64, per-pair loops).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.  It shares no code with the HIP
library.

Source: SGLang "LoRA + MoE" page —
  * structure diagram: gate/up base GEMM -> cache1; cache1 += LoRA delta
    before the activation; silu_and_mul -> cache2; down base GEMM -> cache3;
    cache3 += LoRA delta before the final reduce; then the output;
  * LoRAInfo: gate_up A [L, E(or 1), r, H], gate_up B [L, E, 2I, r],
    down A [L, E, r, I], down B [L, E(or 1), H, r]; adapter_enabled [L];
  * "MoE LoRA Alignment": tokens sorted per (adapter, expert) pair into a
    [max_loras, max_num_tokens_padded] table, one list per adapter, padded
    per block_size_m;
  * design rationale: adding the delta before the nonlinearity keeps
    (W + BA) x equivalence.

Readings where the page is silent:
  * a (token, expert) pair is flattened as f = m*topk + k (row f of cache1 /
    cache2 / cache3);
  * inside an adapter's list: experts ascending, pairs ascending; each
    (adapter, expert) bucket padded to a multiple of block_size_m with the
    sentinel P = M*topk; empty buckets add no block; expert_ids of unused
    blocks = -1; ntpp[l] = padded length; disabled adapters or adapters with
    no pairs get ntpp = 0 and a row of sentinels;
  * tokens with id -1 belong to no list;
  * gate_up A is shared by the gate and up halves; gate is the first half
    (columns [0, I)) of the 2I outputs;
  * routing weights are applied in the reduce, after both deltas;
  * experts_shared_outer_loras: the stacks whose LoRAInfo shape carries
    "num_experts_or_1" -- gate_up A and down B, the matrices on the hidden
    side -- have one expert slot shared by every expert; gate_up B and down
    A stay per expert.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def align_capacity(M: int, topk: int, E: int, block_size_m: int) -> int:
    """Upper bound on one adapter's padded list length: every pair once plus
    at most block_size_m - 1 padding slots per expert, rounded up to a block."""
    P = M * topk
    cap = P + E * (block_size_m - 1)
    return ((cap + block_size_m - 1) // block_size_m) * block_size_m


def moe_align(topk_ids, ids, adapter_enabled, L: int, E: int, block_size_m: int,
              max_tokens_padded: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Per-adapter (adapter, expert) alignment ("MoE LoRA Alignment").

    For each adapter slot l (enabled, with pairs): for e = 0..E-1 append the
    flat pairs f = m*topk + k, in increasing f, with ids[m] == l and
    topk_ids[m, k] == e; pad the bucket with the sentinel P up to a multiple
    of block_size_m and record expert e for each of its blocks.
    Returns sorted_token_ids int32[L, max_tokens_padded],
    expert_ids int32[L, max_tokens_padded // block_size_m], ntpp int32[L].
    """
    topk_ids = np.asarray(topk_ids)
    ids = np.asarray(ids)
    M, topk = topk_ids.shape
    P = M * topk
    nblk = max_tokens_padded // block_size_m
    sorted_ids = np.full((L, max_tokens_padded), P, dtype=np.int32)
    expert_ids = np.full((L, nblk), -1, dtype=np.int32)
    ntpp = np.zeros(L, dtype=np.int32)
    for l in range(L):
        if not adapter_enabled[l]:
            continue
        pos = 0
        for e in range(E):
            bucket = [m * topk + k for m in range(M) for k in range(topk)
                      if ids[m] == l and topk_ids[m, k] == e]
            if not bucket:
                continue
            padded = -(-len(bucket) // block_size_m) * block_size_m
            sorted_ids[l, pos:pos + len(bucket)] = bucket
            for b in range(pos // block_size_m, (pos + padded) // block_size_m):
                expert_ids[l, b] = e
            pos += padded
        ntpp[l] = pos
    return sorted_ids, expert_ids, ntpp


def _pair_adapter(ids, adapter_enabled, L, m):
    l = int(ids[m])
    if l < 0 or l >= L or not adapter_enabled[l]:
        return -1
    return l


def moe_gate_up_add(x, cache1, topk_ids, ids, adapter_enabled, A_gu, B_gu,
                    shared_outer: bool = False) -> np.ndarray:
    """Stage 1.5: cache1[f] += B_gu[l, e] @ (A_gu[l, e'] @ x[m]) for every pair
    f = m*topk + k with an enabled adapter l = ids[m], e = topk_ids[m, k];
    e' = e, or 0 when the outer stacks are shared (A_gu [L, 1, r, H])."""
    x = _f64(x)
    c1 = np.array(cache1, dtype=np.float64, copy=True)
    A_gu = _f64(A_gu)
    B_gu = _f64(B_gu)
    M, topk = np.asarray(topk_ids).shape
    L = A_gu.shape[0]
    for m in range(M):
        l = _pair_adapter(ids, adapter_enabled, L, m)
        if l < 0:
            continue
        for k in range(topk):
            e = int(topk_ids[m, k])
            s = A_gu[l, 0 if shared_outer else e] @ x[m]
            c1[m * topk + k] = c1[m * topk + k] + B_gu[l, e] @ s
    return c1


def silu(z) -> np.ndarray:
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def silu_and_mul(cache1) -> np.ndarray:
    """Stage 2: cache2[f, j] = silu(cache1[f, j]) * cache1[f, I + j]."""
    c1 = _f64(cache1)
    I = c1.shape[1] // 2
    out = np.empty((c1.shape[0], I))
    for f in range(c1.shape[0]):
        out[f] = silu(c1[f, :I]) * c1[f, I:]
    return out


def moe_down_add(cache2, cache3, topk_ids, ids, adapter_enabled, A_d, B_d,
                 shared_outer: bool = False) -> np.ndarray:
    """Stage 3.5: cache3[f] += B_d[l, e'] @ (A_d[l, e] @ cache2[f]), e' = e, or 0
    when the outer stacks are shared (B_d [L, 1, H, r])."""
    c2 = _f64(cache2)
    c3 = np.array(cache3, dtype=np.float64, copy=True)
    A_d = _f64(A_d)
    B_d = _f64(B_d)
    M, topk = np.asarray(topk_ids).shape
    L = A_d.shape[0]
    for m in range(M):
        l = _pair_adapter(ids, adapter_enabled, L, m)
        if l < 0:
            continue
        for k in range(topk):
            e = int(topk_ids[m, k])
            f = m * topk + k
            c3[f] = c3[f] + B_d[l, 0 if shared_outer else e] @ (A_d[l, e] @ c2[f])
    return c3


def topk_reduce(cache3, topk_weights) -> np.ndarray:
    """Final reduce: out[m] = sum_k w[m, k] * cache3[m*topk + k]."""
    c3 = _f64(cache3)
    w = _f64(topk_weights)
    M, topk = w.shape
    out = np.zeros((M, c3.shape[1]))
    for m in range(M):
        for k in range(topk):
            out[m] = out[m] + w[m, k] * c3[m * topk + k]
    return out
