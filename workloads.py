"""Seeded synthetic inputs for dynamic multi-LoRA on a mixed batch.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic: no products, no sorting of tokens
into segments, no alignment.  Both the oracle and the HIP path receive the
exact bytes produced here.

Workload shapes follow the pages:
  * dynamic LoRA on a mixed batch, decode example with ids [0, 2, -1] and
    ranks 16/32 (vLLM-Ascend LoRA operator walkthrough, section 3.4);
  * ranks usually 16..64, A is [r, K], B is [N, r] (same page, section 1.1);
  * stacked QKV / gate-up shapes A (3r, in), B (q+2kv, r) and A (2r, in),
    B (2*out, r) (SGLang "LoRA Layers" page, per-layer table);
  * MoE LoRA with per-expert gate_up / down A and B stacks
    (SGLang "LoRA + MoE" page, LoRAInfo).
Values: x ~ N(0,1); A, B ~ N(0, 0.02^2); y_base ~ N(0,1) unless a case says
otherwise.  Random draws use numpy's PCG64 with a fixed draw order.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


# ----------------------------------------------------------------------------
# storage rounding (input preparation only)
# ----------------------------------------------------------------------------
def bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  NaN/Inf never occur in the
    generated data (normal draws), so no special casing is needed.
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Tensor:
    """One input tensor: exact values (float64) plus the storage bytes."""

    dtype: str                 # "f32" or "bf16"
    values: np.ndarray         # float64 view of exactly what is stored
    storage: np.ndarray        # float32 or uint16 (bf16 bit patterns)

    @property
    def shape(self):
        return self.values.shape


def make_tensor(a32: np.ndarray, dtype: str) -> Tensor:
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == F32:
        return Tensor(dtype, a32.astype(np.float64), a32)
    if dtype == BF16:
        bits = bf16_bits(a32)
        return Tensor(dtype, bf16_to_f64(bits), bits)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# dense multi-LoRA linear case
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class LinearCase:
    name: str
    dtype: str
    M: int
    K: int
    slice_sizes: List[int]          # output width of each stacked slice
    ranks: List[int]                # true rank of each adapter slot (0 allowed)
    ids: np.ndarray                 # int32 [M]; -1 = no adapter
    x: Tensor                       # [M, K]
    A: List[Tensor]                 # per adapter: [n_sl * r_i, K]
    B: List[Tensor]                 # per adapter: [N_tot, r_i]
    y_base: Tensor                  # [M, N_tot]

    @property
    def n_slices(self) -> int:
        return len(self.slice_sizes)

    @property
    def N(self) -> int:
        return int(sum(self.slice_sizes))

    @property
    def L(self) -> int:
        return len(self.ranks)


def _adapter_weights(rng, K, slice_sizes, ranks, dtype, std, scale=1.0):
    A, B = [], []
    n_sl = len(slice_sizes)
    N = int(sum(slice_sizes))
    for r in ranks:
        a = (rng.standard_normal((n_sl * r, K), dtype=np.float32) * std * scale)
        b = (rng.standard_normal((N, r), dtype=np.float32) * std * scale)
        A.append(make_tensor(a, dtype))
        B.append(make_tensor(b, dtype))
    return A, B


def dirichlet_lengths(rng, total: int, parts: int) -> List[int]:
    """Split `total` into `parts` non-negative integers from a Dirichlet(1)
    draw, floored, with the remainder given to the largest fractional parts
    (ties to the lower index)."""
    w = rng.dirichlet(np.ones(parts))
    raw = w * total
    base = np.floor(raw).astype(np.int64)
    rem = int(total - base.sum())
    frac = raw - base
    order = sorted(range(parts), key=lambda i: (-frac[i], i))
    for i in order[:rem]:
        base[i] += 1
    return [int(v) for v in base]


def tiny_fp32(seed: int = 0) -> LinearCase:
    """M=8 tokens, K=N=256, 3 adapters with ranks {8,16,16}, ids uniform over
    {-1,0,1,2}; x, A, B, y_base ~ N(0,1)*0.1."""
    rng = np.random.default_rng(seed)
    M, K, N = 8, 256, 256
    ranks = [8, 16, 16]
    ids = rng.integers(-1, 3, size=M).astype(np.int32)
    x = make_tensor(rng.standard_normal((M, K), dtype=np.float32) * 0.1, F32)
    A, B = _adapter_weights(rng, K, [N], ranks, F32, 0.1)
    y = make_tensor(rng.standard_normal((M, N), dtype=np.float32) * 0.1, F32)
    return LinearCase("tiny_fp32", F32, M, K, [N], ranks, ids, x, A, B, y)


def decode_bf16(seed: int = 0, M: int = 32, K: int = 4096, N: int = 4096,
                L: int = 20, p_none: float = 0.1, dtype: str = BF16) -> LinearCase:
    """Decode: one token per sequence, 20 adapters with ranks drawn from
    {16,32,64}; each token is -1 with probability 0.1, else uniform over the
    adapters.  x ~ N(0,1), A, B ~ N(0, 0.02^2), y_base ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    ranks = [int(v) for v in rng.choice([16, 32, 64], size=L)]
    none = rng.random(M) < p_none
    ids = rng.integers(0, L, size=M).astype(np.int32)
    ids[none] = -1
    x = make_tensor(rng.standard_normal((M, K), dtype=np.float32), dtype)
    A, B = _adapter_weights(rng, K, [N], ranks, dtype, 0.02)
    y = make_tensor(rng.standard_normal((M, N), dtype=np.float32), dtype)
    return LinearCase(f"decode_{dtype}", dtype, M, K, [N], ranks, ids, x, A, B, y)


def prefill_bf16(seed: int = 0, M: int = 2048, K: int = 4096, N: int = 4096,
                 ranks=(16, 16, 32, 32, 64, 64, 16, 32), dtype: str = BF16) -> LinearCase:
    """Prefill: contiguous segments whose lengths are a Dirichlet(1) split of
    M (zero-length segments allowed), laid out in a seeded order of the
    adapters so that the ids are not already sorted."""
    rng = np.random.default_rng(seed)
    ranks = [int(r) for r in ranks]
    L = len(ranks)
    lengths = dirichlet_lengths(rng, M, L)
    order = rng.permutation(L)
    ids = np.concatenate([np.full(lengths[a], a, dtype=np.int32) for a in order])
    x = make_tensor(rng.standard_normal((M, K), dtype=np.float32), dtype)
    A, B = _adapter_weights(rng, K, [N], ranks, dtype, 0.02)
    y = make_tensor(rng.standard_normal((M, N), dtype=np.float32), dtype)
    return LinearCase(f"prefill_{dtype}", dtype, M, K, [N], ranks, ids.astype(np.int32),
                      x, A, B, y)


def mixed_ids(rng, M: int, n_decode: int, n_prefill_seqs: int, L: int) -> np.ndarray:
    """Mixed batch: n_decode decode tokens first (one per sequence), then the
    rest of M split over prefill sequences; one uniform adapter id per
    sequence (no -1)."""
    lengths = dirichlet_lengths(rng, M - n_decode, n_prefill_seqs)
    seq_ids = rng.integers(0, L, size=n_decode + n_prefill_seqs)
    parts = [np.array([seq_ids[i]], dtype=np.int32) for i in range(n_decode)]
    for j, ln in enumerate(lengths):
        parts.append(np.full(ln, seq_ids[n_decode + j], dtype=np.int32))
    return np.concatenate(parts).astype(np.int32)


def stacked_bf16(which: str, seed: int = 0, M: int = 512, K: int = 4096,
                 L: int = 12, slice_sizes=None, dtype: str = BF16) -> LinearCase:
    """Stacked-slice outputs on a mixed prefill+decode batch of M=512 tokens
    (32 decode tokens + 4 prefill sequences), 12 adapters with ranks in
    {16,32,64}.  which="qkv": slices [4096,1024,1024], A (3r, K);
    which="gate_up": slices [14336,14336], A (2r, K).  The two share the
    batch (ids and ranks) and use separate activations."""
    rng = np.random.default_rng(seed)
    ranks = [int(v) for v in rng.choice([16, 32, 64], size=L)]
    ids = mixed_ids(rng, M, 32, 4, L)
    if slice_sizes is None:
        slice_sizes = [4096, 1024, 1024] if which == "qkv" else [14336, 14336]
    # separate streams for the two layers so that each is reproducible alone
    sub = np.random.default_rng([seed, 1 if which == "qkv" else 2])
    x = make_tensor(sub.standard_normal((M, K), dtype=np.float32), dtype)
    A, B = _adapter_weights(sub, K, list(slice_sizes), ranks, dtype, 0.02)
    y = make_tensor(sub.standard_normal((M, int(sum(slice_sizes))), dtype=np.float32), dtype)
    return LinearCase(f"stacked_{which}_{dtype}", dtype, M, K, list(slice_sizes), ranks,
                      ids, x, A, B, y)


def random_linear(seed: int, M: int, K: int, slice_sizes, ranks, dtype: str,
                  p_none: float = 0.2, contiguous: bool = False,
                  x_std: float = 1.0, w_std: float = 0.02) -> LinearCase:
    """General seeded case for parity sweeps (ragged sizes, rank 0 slots)."""
    rng = np.random.default_rng(seed)
    L = len(ranks)
    if contiguous:
        lengths = dirichlet_lengths(rng, M, L + 1)
        order = list(rng.permutation(L + 1))
        ids = np.concatenate([np.full(lengths[i], (a if a < L else -1), dtype=np.int32)
                              for i, a in enumerate(order)]) if M else np.zeros(0, np.int32)
    else:
        ids = rng.integers(0, max(L, 1), size=M).astype(np.int32)
        ids[rng.random(M) < p_none] = -1
        if L == 0:
            ids[:] = -1
    x = make_tensor(rng.standard_normal((M, K), dtype=np.float32) * x_std, dtype)
    A, B = _adapter_weights(rng, K, list(slice_sizes), list(ranks), dtype, w_std)
    y = make_tensor(rng.standard_normal((M, int(sum(slice_sizes))), dtype=np.float32), dtype)
    return LinearCase(f"random_{seed}", dtype, M, K, list(slice_sizes), list(ranks),
                      ids.astype(np.int32), x, A, B, y)


def integer_linear(seed: int, M: int, K: int, slice_sizes, ranks, dtype: str) -> LinearCase:
    """Inputs in {-1, 0, 1} with small K and r: every partial sum is a small
    integer, exact in fp32, bf16 and fp64, so any summation order gives the
    same bits."""
    rng = np.random.default_rng(seed)
    L = len(ranks)
    n_sl = len(slice_sizes)
    N = int(sum(slice_sizes))
    ids = rng.integers(-1, L, size=M).astype(np.int32)
    tri = lambda shape: rng.integers(-1, 2, size=shape).astype(np.float32)
    x = make_tensor(tri((M, K)), dtype)
    A = [make_tensor(tri((n_sl * r, K)), dtype) for r in ranks]
    B = [make_tensor(tri((N, r)), dtype) for r in ranks]
    y = make_tensor(tri((M, N)), dtype)
    return LinearCase(f"integer_{seed}", dtype, M, K, list(slice_sizes), list(ranks), ids,
                      x, A, B, y)


def base_weight(seed: int, N: int, K: int, dtype: str = BF16, std: float = 0.02,
                integer: bool = False) -> Tensor:
    """Base layer weight W [N, K] (row n = output column n), N(0, std^2), or
    values in {-1, 0, 1} for the exact-arithmetic cases."""
    rng = np.random.default_rng([seed, 11])
    if integer:
        return make_tensor(rng.integers(-1, 2, size=(N, K)).astype(np.float32), dtype)
    return make_tensor(rng.standard_normal((N, K), dtype=np.float32) * std, dtype)


# ----------------------------------------------------------------------------
# embedding and LM-head LoRA (SGLang "LoRA Layers" page: the embedding's A
# side is a lookup of A (r, vocab), its B is (emb, r); the LM head is a dense
# LoRA linear whose output width is the vocabulary)
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class EmbeddingCase:
    name: str
    dtype: str
    M: int
    vocab: int
    emb: int
    ranks: List[int]
    ids: np.ndarray                 # int32 [M] adapter per token; -1 = none
    tokens: np.ndarray              # int32 [M] token ids (may lie outside [0, vocab))
    A: List[Tensor]                 # per adapter: [r_i, vocab]
    B: List[Tensor]                 # per adapter: [emb, r_i]
    y_base: Tensor                  # [M, emb]: the base embedding rows

    @property
    def L(self) -> int:
        return len(self.ranks)


def embedding_bf16(seed: int = 0, M: int = 32, vocab: int = 32000, emb: int = 4096,
                   L: int = 20, p_none: float = 0.1, ranks=None, dtype: str = BF16,
                   contiguous: bool = False, p_outside: float = 0.0) -> EmbeddingCase:
    """Embedding LoRA on a decode batch (ids as in the decode workload: ranks
    from {16,32,64}, 10% of tokens without an adapter) or, with contiguous,
    on a prefill batch of Dirichlet(1) segments.  Token ids are uniform over
    the vocabulary; a fraction p_outside of them is moved past its end.
    A, B ~ N(0, 0.02^2), y_base ~ N(0,1)."""
    rng = np.random.default_rng([seed, 7])
    if ranks is None:
        ranks = [int(v) for v in rng.choice([16, 32, 64], size=L)]
    ranks = [int(r) for r in ranks]
    L = len(ranks)
    if contiguous:
        lengths = dirichlet_lengths(rng, M, L)
        order = rng.permutation(L)
        ids = np.concatenate([np.full(lengths[a], a, dtype=np.int32) for a in order])
    else:
        ids = rng.integers(0, L, size=M).astype(np.int32)
        ids[rng.random(M) < p_none] = -1
    tokens = rng.integers(0, vocab, size=M).astype(np.int32)
    outside = rng.random(M) < p_outside
    tokens[outside] = vocab + rng.integers(0, 100, size=int(outside.sum())).astype(np.int32)
    A, B = [], []
    for r in ranks:
        A.append(make_tensor(rng.standard_normal((r, vocab), dtype=np.float32) * 0.02, dtype))
        B.append(make_tensor(rng.standard_normal((emb, r), dtype=np.float32) * 0.02, dtype))
    y = make_tensor(rng.standard_normal((M, emb), dtype=np.float32), dtype)
    return EmbeddingCase(f"embedding_{dtype}", dtype, M, vocab, emb, ranks, ids.astype(np.int32),
                         tokens, A, B, y)


def lm_head_bf16(seed: int = 0, M: int = 32, K: int = 4096, vocab: int = 32000,
                 L: int = 20, dtype: str = BF16) -> LinearCase:
    """LM-head LoRA on a decode batch: the decode workload with the output
    width set to the vocabulary (hidden 4096 -> 32000 logits)."""
    case = decode_bf16(seed, M=M, K=K, N=vocab, L=L, dtype=dtype)
    case.name = f"lm_head_{dtype}"
    return case


# ----------------------------------------------------------------------------
# MoE LoRA case
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class MoECase:
    name: str
    dtype: str
    M: int
    H: int
    I: int
    E: int
    topk: int
    L: int
    rank: int
    block_size_m: int
    ids: np.ndarray                 # int32 [M] per-token adapter (-1 = none)
    adapter_enabled: np.ndarray     # int32 [L]
    topk_ids: np.ndarray            # int32 [M, topk]
    topk_weights: np.ndarray        # float32 [M, topk]
    x: Tensor                       # [M, H]
    A_gu: Tensor                    # [L, E, r, H]  ([L, 1, r, H] when shared_outer)
    B_gu: Tensor                    # [L, E, 2I, r]
    A_d: Tensor                     # [L, E, r, I]
    B_d: Tensor                     # [L, E, H, r]  ([L, 1, H, r] when shared_outer)
    cache1: Tensor                  # [M*topk, 2I]   base gate/up output
    cache3: Tensor                  # [M*topk, H]    base down output
    shared_outer: bool = False      # outer (hidden-side) matrices shared by the experts


def _route(rng, M, E, topk):
    """Router stand-in: logits ~ N(0,1), softmax over all experts, top-k by
    probability (ties to the lower expert index), weights not renormalised."""
    logits = rng.standard_normal((M, E)).astype(np.float64)
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    idx = np.argsort(-p, axis=1, kind="stable")[:, :topk].astype(np.int32)
    w = np.take_along_axis(p, idx, axis=1).astype(np.float32)
    return idx, w


def moe_case(seed: int = 0, M: int = 256, H: int = 4096, I: int = 14336, E: int = 8,
             topk: int = 2, L: int = 4, rank: int = 16, block_size_m: int = 64,
             p_none: float = 0.0, dtype: str = BF16, enabled=None,
             shared_outer: bool = False) -> MoECase:
    """MoE-LoRA: top-2 routing over 8 experts, 4 adapters of rank 16 with
    per-expert gate_up and down A/B; cache1/cache3 stand in for the base
    expert GEMM outputs, ~N(0,1).  shared_outer: the gate_up A and down B
    stacks have one expert slot, shared by all experts (SGLang "LoRA + MoE"
    page, experts_shared_outer_loras)."""
    rng = np.random.default_rng(seed)
    topk_ids, topk_w = _route(rng, M, E, topk)
    ids = rng.integers(0, L, size=M).astype(np.int32)
    if p_none > 0:
        ids[rng.random(M) < p_none] = -1
    en = np.ones(L, np.int32) if enabled is None else np.asarray(enabled, np.int32)
    f = lambda shape, s: rng.standard_normal(shape, dtype=np.float32) * s
    x = make_tensor(f((M, H), 1.0), dtype)
    Eo = 1 if shared_outer else E
    A_gu = make_tensor(f((L, Eo, rank, H), 0.02), dtype)
    B_gu = make_tensor(f((L, E, 2 * I, rank), 0.02), dtype)
    A_d = make_tensor(f((L, E, rank, I), 0.02), dtype)
    B_d = make_tensor(f((L, Eo, H, rank), 0.02), dtype)
    c1 = make_tensor(f((M * topk, 2 * I), 1.0), dtype)
    c3 = make_tensor(f((M * topk, H), 1.0), dtype)
    name = f"moe_shared_outer_{dtype}" if shared_outer else f"moe_{dtype}"
    return MoECase(name, dtype, M, H, I, E, topk, L, rank, block_size_m, ids, en,
                   topk_ids, topk_w, x, A_gu, B_gu, A_d, B_d, c1, c3, shared_outer)


def integer_moe_case(seed: int, M: int, H: int, I: int, E: int = 4, topk: int = 2, L: int = 3,
                     rank: int = 16, block_size_m: int = 16, p_none: float = 0.15,
                     enabled=None, shared_outer: bool = False, a_d_nnz: int = 32) -> MoECase:
    """MoE-LoRA inputs whose whole chain is exact in fp32, in the S hi / lo
    bf16 pair and in one final rounding, so device and oracle agree bit for
    bit (the activation excepted, whose device output feeds the oracle's
    next stage):
      * x in {0, 1}; every gate/up A row one-hot (a single 1); every gate/up
        B row one-hot with sign +-1: the gate/up delta is in {-1, 0, 1};
      * cache1 gate half in {1, 2}, up half 0: after the delta the gate is in
        {0, ..., 3} and the up value in {-1, 0, 1}, so silu(gate) * up is 0
        or of magnitude in [0.7, 2.9] (bf16 steps of at least 2^-8);
      * down A rows with at most `a_d_nnz` entries +-1: the down S values are
        multiples of 2^-8 below 2^8 in magnitude (16 significant bits, exact
        as a bf16 hi / lo pair); down B and cache3 in {-1, 0, 1};
      * routing weights in {0.25, 0.5, 0.75, 1}."""
    rng = np.random.default_rng([seed, 23])
    topk_ids, _ = _route(rng, M, E, topk)
    topk_w = rng.choice(np.array([0.25, 0.5, 0.75, 1.0], np.float32), size=(M, topk))
    ids = rng.integers(0, L, size=M).astype(np.int32)
    ids[rng.random(M) < p_none] = -1
    en = np.ones(L, np.int32) if enabled is None else np.asarray(enabled, np.int32)
    Eo = 1 if shared_outer else E
    x = rng.integers(0, 2, size=(M, H)).astype(np.float32)
    A_gu = np.zeros((L, Eo, rank, H), np.float32)
    hot = rng.integers(0, H, size=(L, Eo, rank))
    np.put_along_axis(A_gu, hot[..., None], 1.0, axis=3)
    B_gu = np.zeros((L, E, 2 * I, rank), np.float32)
    hot = rng.integers(0, rank, size=(L, E, 2 * I))
    sign = rng.choice(np.array([-1.0, 1.0], np.float32), size=(L, E, 2 * I, 1))
    np.put_along_axis(B_gu, hot[..., None], sign, axis=3)
    A_d = np.zeros((L, E, rank, I), np.float32)
    for l in range(L):
        for e in range(E):
            for j in range(rank):
                pos = rng.choice(I, size=min(a_d_nnz, I), replace=False)
                A_d[l, e, j, pos] = rng.choice(np.array([-1.0, 1.0], np.float32), size=len(pos))
    B_d = rng.integers(-1, 2, size=(L, Eo, H, rank)).astype(np.float32)
    c1 = np.zeros((M * topk, 2 * I), np.float32)
    c1[:, :I] = rng.integers(1, 3, size=(M * topk, I))
    c3 = rng.integers(-1, 2, size=(M * topk, H)).astype(np.float32)
    mk = lambda a: make_tensor(a, BF16)
    return MoECase(f"moe_integer_{seed}", BF16, M, H, I, E, topk, L, rank, block_size_m, ids, en,
                   topk_ids, topk_w, mk(x), mk(A_gu), mk(B_gu), mk(A_d), mk(B_d), mk(c1), mk(c3),
                   shared_outer)


# ----------------------------------------------------------------------------
# named workloads (full sizes) and their small parity counterparts
# ----------------------------------------------------------------------------
FULL = {
    "tiny_fp32": lambda: tiny_fp32(0),
    "decode_bf16": lambda: decode_bf16(0),
    "prefill_bf16": lambda: prefill_bf16(0),
    "stacked_qkv_bf16": lambda: stacked_bf16("qkv", 0),
    "stacked_gate_up_bf16": lambda: stacked_bf16("gate_up", 0),
}


def describe(case) -> Dict[str, object]:
    if isinstance(case, LinearCase):
        return {"name": case.name, "M": case.M, "K": case.K, "slices": case.slice_sizes,
                "L": case.L, "dtype": case.dtype}
    return {"name": case.name, "M": case.M, "H": case.H, "I": case.I, "E": case.E,
            "topk": case.topk, "L": case.L, "rank": case.rank, "dtype": case.dtype}
