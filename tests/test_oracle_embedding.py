"""Pins for the embedding-LoRA oracle (SGLang "LoRA Layers" page,
VocabParallelEmbeddingWithLoRA: A (rank, vocab) looked up by token id, B
(emb, rank) added to the base rows).

What pins it, besides itself:
  * a hand-worked fixture under tests/golden/;
  * the one-hot closed form: looking up column t of A is the product of A
    with the one-hot row of t, so the lookup equals the dense oracle fed
    one-hot token rows (a different code path: matrix-vector products over
    the whole vocabulary);
  * pass-through rows (no adapter, disabled adapter, token outside the
    vocabulary) and planted mutants that must fail these pins.
"""
import numpy as np
import pytest

import workloads as W
from oracle import lora as O


def vals(case):
    return [a.values for a in case.A], [b.values for b in case.B]


def one_hot_reference(case, enabled=None):
    x = np.zeros((case.M, case.vocab))
    for m, t in enumerate(case.tokens):
        if 0 <= t < case.vocab:
            x[m, t] = 1.0
    A, B = vals(case)
    return O.lora_linear(x, case.ids, A, B, case.ranks, [case.emb], case.y_base.values, enabled)


def test_golden(golden):
    g = golden("embedding_example.json")
    A = [np.array(a, float) for a in g["A"]]
    B = [np.array(b, float) for b in g["B"]]
    y = O.embedding_add(g["tokens"], np.array(g["ids"], np.int32), A, B, g["ranks"], g["vocab"],
                        np.array(g["y_base"], float))
    assert np.array_equal(y, np.array(g["y"], float))


@pytest.mark.parametrize("seed,dtype,contig", [(0, W.F32, False), (1, W.BF16, False),
                                               (2, W.BF16, True)])
def test_lookup_equals_one_hot_product(seed, dtype, contig):
    case = W.embedding_bf16(seed, M=40, vocab=300, emb=48, ranks=[16, 8, 0, 33, 64],
                            dtype=dtype, contiguous=contig, p_outside=0.1)
    A, B = vals(case)
    y = O.embedding_add(case.tokens, case.ids, A, B, case.ranks, case.vocab, case.y_base.values)
    ref = one_hot_reference(case)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_passthrough_rows_and_mask():
    case = W.embedding_bf16(3, M=60, vocab=200, emb=32, ranks=[16, 32, 0, 8],
                            p_outside=0.2)
    A, B = vals(case)
    enabled = np.array([1, 0, 1, 1], np.int32)
    y = O.embedding_add(case.tokens, case.ids, A, B, case.ranks, case.vocab, case.y_base.values,
                        enabled)
    ids = case.ids
    keep = (ids < 0) | (ids == 1) | (ids == 2) | (case.tokens >= case.vocab)
    assert keep.any() and (~keep).any()
    assert np.array_equal(y[keep], case.y_base.values[keep])
    ref = one_hot_reference(case, enabled)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def _mutant(kind):
    def f(tokens, ids, A, B, ranks, vocab, y_base):
        y = np.array(y_base, float, copy=True)
        for m in range(y.shape[0]):
            i, t = int(ids[m]), int(tokens[m])
            if kind == "token_position":
                t = m % vocab
            if i < 0 or ranks[i] == 0 or (kind != "no_range_check" and t >= vocab):
                continue
            r = ranks[i]
            S = np.asarray(A[i], float)[:r, t % vocab if kind == "no_range_check" else t]
            if kind == "b_transposed":
                d = (np.asarray(B[i], float)[:, :r] @ S[::-1])
            else:
                d = np.asarray(B[i], float)[:, :r] @ S
            y[m] += d
        return y
    return f


@pytest.mark.parametrize("kind", ["token_position", "no_range_check", "b_transposed"])
def test_mutants_caught(kind, golden):
    """A planted slip fails the fixture or the one-hot pin."""
    g = golden("embedding_example.json")
    impl = _mutant(kind)
    A = [np.array(a, float) for a in g["A"]]
    B = [np.array(b, float) for b in g["B"]]
    y = impl(g["tokens"], g["ids"], A, B, g["ranks"], g["vocab"], np.array(g["y_base"], float))
    caught = not np.array_equal(y, np.array(g["y"], float))
    case = W.embedding_bf16(4, M=30, vocab=100, emb=16, ranks=[16, 32], p_outside=0.2)
    Ac, Bc = vals(case)
    got = impl(case.tokens, case.ids, Ac, Bc, case.ranks, case.vocab, case.y_base.values)
    caught = caught or np.max(np.abs(got - one_hot_reference(case))) > 1e-9
    assert caught
