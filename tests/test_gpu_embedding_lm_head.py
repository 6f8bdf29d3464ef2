"""GPU parity of embedding LoRA and LM-head LoRA (SGLang "LoRA Layers" page:
VocabParallelEmbeddingWithLoRA, ParallelLMHeadWithLoRA) through the C ABI
against the fp64 oracle.

Embedding: segment table -> lora_embedding_shrink (lookup of the token's
column of A, into S) -> lora_expand_add, and the single launch
lora_embedding_decode (lookup inside the decode kernel's consumers).  The looked-up S values are bf16 or
fp32 weights widened to fp32, so S is compared bit for bit; y meets the
spec tolerance and the element-wise bound; rows without a delta (no
adapter, disabled adapter, rank 0, token id past the vocabulary) are
bit-identical to the base rows.

LM head: the dense path with the vocabulary as output width, decode (the
single-launch kernel) and larger batches (shrink + expand), including an
output offset into a wider logits buffer (one vocabulary shard of two).
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import lora as O
from tests.helpers import assert_close, table_for, to_dev, to_f64, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ml():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import adapter_lora_amd
    return adapter_lora_amd


def log(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- embedding
def run_embedding(ml, case, enabled=None):
    dt = torch_dtype(case.dtype)
    A = [to_dev(a) for a in case.A]
    B = [to_dev(b) for b in case.B]
    table = ml.LoraTable(A, B, case.ranks, [case.emb], case.vocab, dt, embedding=True)
    ids = torch.from_numpy(case.ids).cuda()
    toks = torch.from_numpy(case.tokens).cuda()
    en = None if enabled is None else torch.from_numpy(enabled).cuda()
    seg = ml.Segments(case.M, case.L)
    ml.lora_build_segments(ids, seg, adapter_enabled=en)
    S = torch.full((max(case.M, 1), table.cols), -7.0, dtype=torch.float32, device="cuda")
    ml.lora_embedding_shrink(table, toks, seg, S)
    y = to_dev(case.y_base)
    ml.lora_expand_add(table, S, seg, y)
    torch.cuda.synchronize()
    return to_f64(y), S.cpu().numpy().astype(np.float64), table


def check_embedding(ml, case, enabled=None):
    log(f"embedding {case.name} M={case.M} vocab={case.vocab} emb={case.emb} L={case.L} "
        f"mask={'none' if enabled is None else int(enabled.sum())}")
    got, S, table = run_embedding(ml, case, enabled)
    A = [a.values for a in case.A]
    B = [b.values for b in case.B]
    ref = O.embedding_add(case.tokens, case.ids, A, B, case.ranks, case.vocab,
                          case.y_base.values, enabled)
    # S: the lookup, bit for bit, in sorted order
    si, seg_ip, req, nseg = O.build_segments(case.ids, case.L, enabled)
    for s in range(nseg):
        i = int(req[s])
        r = case.ranks[i]
        for p in range(seg_ip[s], seg_ip[s + 1]):
            t = int(case.tokens[si[p]])
            exp = np.zeros(table.r_max)
            if 0 <= t < case.vocab:
                exp[:r] = A[i][:r, t]
            assert np.array_equal(S[p, :table.r_max], exp), (s, p)
    keep = ~O.delta_rows(case.ids, case.ranks, enabled)
    keep |= (case.tokens < 0) | (case.tokens >= case.vocab)
    assert np.array_equal(got[keep], case.y_base.values[keep]), "pass-through rows changed"
    assert_close(got, ref, case.dtype, case.y_base.values, case.name)


EMB_CASES = [
    ("decode_vocab32000", lambda: W.embedding_bf16(0)),
    ("decode_outside_tokens", lambda: W.embedding_bf16(1, M=48, vocab=5000, emb=1024, L=9,
                                                       p_outside=0.25)),
    ("prefill_contiguous", lambda: W.embedding_bf16(2, M=300, vocab=4000, emb=520,
                                                    ranks=[16, 48, 0, 64, 8], contiguous=True)),
    ("fp32", lambda: W.embedding_bf16(3, M=40, vocab=2000, emb=264, ranks=[16, 5, 33],
                                      dtype=W.F32, p_outside=0.1)),
    ("M1", lambda: W.embedding_bf16(4, M=1, vocab=800, emb=128, ranks=[64], p_none=0.0)),
]


@pytest.mark.parametrize("name,mk", EMB_CASES, ids=[c[0] for c in EMB_CASES])
def test_embedding_matches_oracle(ml, name, mk):
    check_embedding(ml, mk())


def test_embedding_with_mask_and_empty(ml):
    case = W.embedding_bf16(5, M=64, vocab=3000, emb=256, L=7, p_outside=0.1)
    check_embedding(ml, case, enabled=np.array([1, 0, 1, 1, 0, 1, 1], np.int32))
    case0 = W.embedding_bf16(6, M=0, vocab=800, emb=128, ranks=[16])
    got, _, _ = run_embedding(ml, case0)
    assert got.shape == (0, 128)


# ---------------------------------------------------------------- LM head
def oracle_y(case):
    return O.lora_linear(case.x.values, case.ids, [a.values for a in case.A],
                         [b.values for b in case.B], case.ranks, case.slice_sizes,
                         case.y_base.values)


def test_lm_head_decode_single_launch(ml):
    """Decode batch of 32 tokens, hidden 4096 -> 32000 logits, 20 adapters,
    one lora_fused_decode launch."""
    case = W.lm_head_bf16(0)
    log(f"lm_head decode M={case.M} K={case.K} N={case.N}")
    table = table_for(case)
    ids = torch.from_numpy(case.ids).cuda()
    x = to_dev(case.x)
    y = to_dev(case.y_base)
    seg = ml.Segments(case.M, case.L)
    ws = ml.Workspace.for_table(table, case.M)
    ml.lora_fused_decode(table, ids, x, y, ws, seg=seg)
    torch.cuda.synchronize()
    assert ml.lora_read_device_error(ws.buf) == 0
    got = to_f64(y)
    keep = ~O.delta_rows(case.ids, case.ranks)
    assert np.array_equal(got[keep], case.y_base.values[keep])
    assert_close(got, oracle_y(case), case.dtype, case.y_base.values, case.name)


def test_lm_head_vocab_shard_with_output_offset(ml):
    """One vocabulary shard of two (the page's output_offset of a
    column-parallel LM head): the table holds the shard's B rows, y is the
    second half of a [M, 2 * shard] logits buffer; the first half must stay
    untouched."""
    shard = 8000
    case = W.decode_bf16(8, M=24, K=2048, N=shard, L=6)
    log(f"lm_head shard M={case.M} K={case.K} shard={shard}")
    table = table_for(case)
    rng = np.random.default_rng(9)
    other = W.make_tensor(rng.standard_normal((case.M, shard), dtype=np.float32), W.BF16)
    logits = torch.cat([to_dev(other), to_dev(case.y_base)], dim=1).contiguous()
    y = logits[:, shard:]
    ids = torch.from_numpy(case.ids).cuda()
    ws = ml.Workspace.for_table(table, case.M)
    ml.lora_fused_decode(table, ids, to_dev(case.x), y, ws)
    torch.cuda.synchronize()
    assert ml.lora_read_device_error(ws.buf) == 0
    full = to_f64(logits)
    assert np.array_equal(full[:, :shard], other.values), "the other shard changed"
    assert_close(full[:, shard:], oracle_y(case), case.dtype, case.y_base.values, "shard")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lm_head_consumers_over_tile_groups(ml, dtype):
    """Outputs wide enough that each decode consumer takes several column
    tiles (two stacked slices of 20000 and 10136 columns, 20 adapters: two
    tiles per consumer, a one-tile group at the end of the first slice and a
    ragged last tile)."""
    ranks = [16] * 20 if dtype == "f32" else [16, 32, 64, 0, 48] * 4
    case = W.random_linear(27, 8, 256, [20000, 10136], ranks, W.F32 if dtype == "f32" else W.BF16)
    log(f"lm_head tile groups {dtype} M={case.M} K={case.K} N={case.N}")
    table = table_for(case)
    ids = torch.from_numpy(case.ids).cuda()
    y = to_dev(case.y_base)
    seg = ml.Segments(case.M, case.L)
    ws = ml.Workspace.for_table(table, case.M)
    ml.lora_fused_decode(table, ids, to_dev(case.x), y, ws, seg=seg)
    torch.cuda.synchronize()
    assert ml.lora_read_device_error(ws.buf) == 0
    got = to_f64(y)
    keep = ~O.delta_rows(case.ids, case.ranks)
    assert np.array_equal(got[keep], case.y_base.values[keep])
    assert_close(got, oracle_y(case), case.dtype, case.y_base.values, case.name)


@pytest.mark.parametrize("form", ["ids", "table"])
def test_lm_head_many_tokens_per_adapter(ml, form):
    """64 tokens over three adapters (ranks 16, 64, 48: about 20 tokens
    each, past the 16 token rows of the matrix-core consumers' first block
    and the 4 of the dot-product consumers' registers) at 150008 columns,
    so each consumer walks two tiles pipelined and the last tile is
    ragged; through the ids form and the table form."""
    case = W.random_linear(28, 64, 512, [150008], [16, 64, 48], W.BF16, p_none=0.05)
    log(f"lm_head many tokens {form} M={case.M} K={case.K} N={case.N}")
    table = table_for(case)
    ids = torch.from_numpy(case.ids).cuda()
    y = to_dev(case.y_base)
    seg = ml.Segments(case.M, case.L)
    ws = ml.Workspace.for_table(table, case.M)
    if form == "ids":
        ml.lora_fused_decode(table, ids, to_dev(case.x), y, ws, seg=seg)
    else:
        ml.lora_build_segments(ids, seg)
        ml.lora_shrink_expand_add(table, to_dev(case.x), seg, y, ws)
    torch.cuda.synchronize()
    assert ml.lora_read_device_error(ws.buf) == 0
    got = to_f64(y)
    keep = ~O.delta_rows(case.ids, case.ranks)
    assert np.array_equal(got[keep], case.y_base.values[keep])
    assert_close(got, oracle_y(case), case.dtype, case.y_base.values, case.name)


def test_lm_head_larger_batch(ml):
    """More than 64 rows (the segmented shrink + expand) at vocabulary width."""
    case = W.random_linear(26, 160, 1024, [32000], [16, 64, 32, 0, 48], W.BF16)
    log(f"lm_head batch M={case.M} K={case.K} N={case.N}")
    table = table_for(case)
    ids = torch.from_numpy(case.ids).cuda()
    seg = ml.Segments(case.M, case.L)
    ml.lora_build_segments(ids, seg)
    y = to_dev(case.y_base)
    ws = ml.Workspace.for_table(table, case.M)
    ml.lora_shrink_expand_add(table, to_dev(case.x), seg, y, ws)
    torch.cuda.synchronize()
    got = to_f64(y)
    keep = ~O.delta_rows(case.ids, case.ranks)
    assert np.array_equal(got[keep], case.y_base.values[keep])
    assert_close(got, oracle_y(case), case.dtype, case.y_base.values, case.name)


# ---------------------------------------------------------------- embedding, one launch
def run_embedding_decode(ml, case, enabled=None, reps=1):
    dt = torch_dtype(case.dtype)
    table = ml.LoraTable([to_dev(a) for a in case.A], [to_dev(b) for b in case.B], case.ranks,
                         [case.emb], case.vocab, dt, embedding=True)
    ids = torch.from_numpy(case.ids).cuda()
    toks = torch.from_numpy(case.tokens).cuda()
    en = None if enabled is None else torch.from_numpy(enabled).cuda()
    seg = ml.Segments(case.M, case.L)
    y = to_dev(case.y_base)
    for _ in range(reps):
        ml.lora_embedding_decode(table, ids, toks, y, seg=seg, adapter_enabled=en)
    torch.cuda.synchronize()
    return to_f64(y), seg


EMB_DECODE_CASES = [
    ("decode_vocab32000", lambda: W.embedding_bf16(0), None),
    ("outside_tokens_masked", lambda: W.embedding_bf16(1, M=48, vocab=5000, emb=1024, L=9,
                                                       p_outside=0.25),
     np.array([1, 1, 0, 1, 1, 1, 0, 1, 1], np.int32)),
    ("fp32_ragged", lambda: W.embedding_bf16(3, M=40, vocab=2000, emb=264, ranks=[16, 5, 33, 0],
                                             dtype=W.F32, p_outside=0.1), None),
    ("M64_one_adapter", lambda: W.embedding_bf16(7, M=64, vocab=1000, emb=512, ranks=[64],
                                                 p_none=0.0), None),
    ("M1", lambda: W.embedding_bf16(4, M=1, vocab=800, emb=128, ranks=[64], p_none=0.0), None),
]


@pytest.mark.parametrize("name,mk,enabled", EMB_DECODE_CASES,
                         ids=[c[0] for c in EMB_DECODE_CASES])
def test_embedding_decode_single_launch(ml, name, mk, enabled):
    case = mk()
    log(f"embedding decode {name} M={case.M} vocab={case.vocab} emb={case.emb} L={case.L}")
    reps = 2 if name == "fp32_ragged" else 1
    got, seg = run_embedding_decode(ml, case, enabled, reps)
    A = [a.values for a in case.A]
    B = [b.values for b in case.B]
    ref = O.embedding_add(case.tokens, case.ids, A, B, case.ranks, case.vocab,
                          case.y_base.values, enabled)
    if reps > 1:
        ref = case.y_base.values + reps * (ref - case.y_base.values)
    keep = ~O.delta_rows(case.ids, case.ranks, enabled)
    keep |= (case.tokens < 0) | (case.tokens >= case.vocab)
    assert np.array_equal(got[keep], case.y_base.values[keep]), "pass-through rows changed"
    assert_close(got, ref, case.dtype, case.y_base.values, name, roundings=reps)
    si, sp, req, n = O.build_segments(case.ids, case.L, enabled)
    assert np.array_equal(seg.sorted_idx[:case.M].cpu().numpy(), si)
    assert np.array_equal(seg.seg_indptr.cpu().numpy(), sp)
    assert int(seg.num_segments.cpu()[0]) == n
