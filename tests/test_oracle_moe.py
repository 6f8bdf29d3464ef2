"""Pins for the MoE-LoRA oracle (SGLang "LoRA + MoE" page: structure
diagram, LoRAInfo, "MoE LoRA Alignment", design rationale).

What pins it, besides itself:
  * hand-worked fixtures under tests/golden/;
  * alignment: brute force on tiny shapes against a second definition built
    by bucketing pairs in a dict, plus invariants;
  * the staged pipeline against the merged-weight closed form with explicit
    base experts W13 / W2: sum_k w (W2 + B_d A_d) silu_mul((W13 + B_gu A_gu) x);
  * negative controls: a delta added after the activation, or after the
    reduce, gives a different answer;
  * silu against scipy's logistic function and its identities.
"""
import itertools

import numpy as np
import pytest
from scipy.special import expit

import workloads as W
from oracle import moe as O


def test_golden_pipeline(golden):
    g = golden("moe_example.json")
    arr = lambda k: np.array(g[k], float)
    tid = np.array(g["topk_ids"], np.int32)
    ids = np.array(g["ids"], np.int32)
    en = np.array(g["adapter_enabled"], np.int32)
    c1 = O.moe_gate_up_add(arr("x"), arr("cache1"), tid, ids, en, arr("A_gu"), arr("B_gu"))
    assert np.array_equal(c1, arr("cache1_out"))
    c2 = O.silu_and_mul(c1)
    assert np.allclose(c2, arr("cache2_out"), rtol=1e-13)
    c3 = O.moe_down_add(c2, arr("cache3"), tid, ids, en, arr("A_d"), arr("B_d"))
    assert np.allclose(c3, arr("cache3_out"), rtol=1e-13)
    out = O.topk_reduce(c3, arr("topk_weights"))
    assert np.allclose(out, arr("out"), rtol=1e-13)


def test_golden_align(golden):
    g = golden("moe_align_example.json")
    s, e, n = O.moe_align(np.array(g["topk_ids"]), np.array(g["ids"]),
                          np.array(g["adapter_enabled"]), g["L"], g["E"],
                          g["block_size_m"], g["max_tokens_padded"])
    assert s.tolist() == g["sorted_token_ids"]
    assert e.tolist() == g["expert_ids"]
    assert n.tolist() == g["ntpp"]
    assert O.align_capacity(g["M"], g["topk"], g["E"], g["block_size_m"]) == g["max_tokens_padded"]


def bucket_definition(topk_ids, ids, enabled, L, E, bs, cap):
    """Second definition: a dict keyed by (adapter, expert) of pair lists."""
    M, topk = topk_ids.shape
    P = M * topk
    buckets = {}
    for m in range(M):
        for k in range(topk):
            l = int(ids[m])
            if 0 <= l < L and enabled[l]:
                buckets.setdefault((l, int(topk_ids[m, k])), []).append(m * topk + k)
    rows, experts, ntpp = [], [], []
    for l in range(L):
        row, ex = [], []
        for e in range(E):
            lst = buckets.get((l, e), [])
            if lst:
                pad = (-len(lst)) % bs
                row += lst + [P] * pad
                ex += [e] * ((len(lst) + pad) // bs)
        ntpp.append(len(row))
        rows.append(row + [P] * (cap - len(row)))
        experts.append(ex + [-1] * (cap // bs - len(ex)))
    return rows, experts, ntpp


def test_align_brute_force_tiny():
    L, E, topk, bs = 2, 3, 2, 2
    for M in range(0, 4):
        cap = O.align_capacity(M, topk, E, bs)
        pairs = [p for p in itertools.permutations(range(E), topk)]
        for choice in itertools.product(pairs, repeat=M):
            tid = np.array(choice, np.int32).reshape(M, topk)
            for ids in itertools.product(range(-1, L), repeat=M):
                ids = np.array(ids, np.int32)
                for en in ([1, 1], [0, 1]):
                    s, e, n = O.moe_align(tid, ids, en, L, E, bs, cap)
                    rs, re_, rn = bucket_definition(tid, ids, en, L, E, bs, cap)
                    assert s.tolist() == rs and e.tolist() == re_ and n.tolist() == rn


@pytest.mark.parametrize("seed", range(3))
def test_align_invariants(seed):
    case = W.moe_case(seed, M=97, H=8, I=8, E=8, topk=2, L=4, rank=4, block_size_m=16,
                      p_none=0.2, enabled=[1, 0, 1, 1])
    cap = O.align_capacity(case.M, case.topk, case.E, case.block_size_m)
    s, e, n = O.moe_align(case.topk_ids, case.ids, case.adapter_enabled, case.L, case.E,
                          case.block_size_m, cap)
    P = case.M * case.topk
    bs = case.block_size_m
    seen = []
    for l in range(case.L):
        assert n[l] % bs == 0 and n[l] <= cap
        used = n[l] // bs
        assert np.all(np.diff(e[l, :used]) >= 0)
        assert np.all(e[l, used:] == -1) and np.all(s[l, n[l]:] == P)
        for b in range(used):
            blk = s[l, b * bs:(b + 1) * bs]
            real = blk[blk < P]
            assert real.size > 0
            assert np.all(np.diff(real) > 0)
            for f in real:
                m, k = divmod(int(f), case.topk)
                assert case.ids[m] == l and case.topk_ids[m, k] == e[l, b]
            seen += real.tolist()
    expect = [m * case.topk + k for m in range(case.M) for k in range(case.topk)
              if case.ids[m] >= 0 and case.adapter_enabled[case.ids[m]]]
    assert sorted(seen) == sorted(expect)


def test_silu():
    z = np.linspace(-30, 30, 1001)
    assert np.allclose(O.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(O.silu(-z), O.silu(z) - z, atol=1e-12)


def tiny_moe(seed=0, shared_outer=False):
    rng = np.random.default_rng(seed)
    M, H, I, E, topk, L, r = 16, 64, 128, 4, 2, 3, 16
    case = W.moe_case(seed, M=M, H=H, I=I, E=E, topk=topk, L=L, rank=r, block_size_m=8,
                      p_none=0.2, dtype=W.F32, shared_outer=shared_outer)
    W13 = rng.standard_normal((E, 2 * I, H)) * 0.1
    W2 = rng.standard_normal((E, H, I)) * 0.1
    return case, W13, W2


def staged(case, W13, W2, gate_up_after_act=False, down_after_reduce=False):
    x = case.x.values
    M, topk = case.topk_ids.shape
    c1 = np.zeros((M * topk, W13.shape[1]))
    for m in range(M):
        for k in range(topk):
            c1[m * topk + k] = W13[case.topk_ids[m, k]] @ x[m]
    if gate_up_after_act:
        c2 = O.silu_and_mul(c1)
        d = O.moe_gate_up_add(x, np.zeros_like(c1), case.topk_ids, case.ids,
                              case.adapter_enabled, case.A_gu.values, case.B_gu.values,
                              case.shared_outer)
        I = c2.shape[1]
        c2 = c2 + d[:, :I] * d[:, I:]
    else:
        c1 = O.moe_gate_up_add(x, c1, case.topk_ids, case.ids, case.adapter_enabled,
                               case.A_gu.values, case.B_gu.values, case.shared_outer)
        c2 = O.silu_and_mul(c1)
    c3 = np.zeros((M * topk, W2.shape[1]))
    for m in range(M):
        for k in range(topk):
            c3[m * topk + k] = W2[case.topk_ids[m, k]] @ c2[m * topk + k]
    if down_after_reduce:
        out = O.topk_reduce(c3, case.topk_weights)
        d = O.moe_down_add(c2, np.zeros_like(c3), case.topk_ids, case.ids,
                           case.adapter_enabled, case.A_d.values, case.B_d.values,
                           case.shared_outer)
        for m in range(M):
            out[m] += d[m * topk:(m + 1) * topk].sum(axis=0)
        return out
    c3 = O.moe_down_add(c2, c3, case.topk_ids, case.ids, case.adapter_enabled,
                        case.A_d.values, case.B_d.values, case.shared_outer)
    return O.topk_reduce(c3, case.topk_weights)


def merged(case, W13, W2):
    """(W + B A) per expert and adapter, applied as one MLP per token."""
    x = case.x.values
    M, topk = case.topk_ids.shape
    I = W2.shape[2]
    out = np.zeros((M, W2.shape[1]))
    for m in range(M):
        l = int(case.ids[m])
        on = 0 <= l < case.L and case.adapter_enabled[l]
        for k in range(topk):
            e = int(case.topk_ids[m, k])
            eo = 0 if case.shared_outer else e        # outer stacks: one shared slot
            w13 = W13[e] + (case.B_gu.values[l, e] @ case.A_gu.values[l, eo] if on else 0)
            w2 = W2[e] + (case.B_d.values[l, eo] @ case.A_d.values[l, e] if on else 0)
            h = w13 @ x[m]
            a = h[:I] / (1 + np.exp(-h[:I])) * h[I:]
            out[m] += case.topk_weights[m, k] * (w2 @ a)
    return out


@pytest.mark.parametrize("shared_outer", [False, True])
@pytest.mark.parametrize("seed", range(3))
def test_pipeline_equals_merged_weights(seed, shared_outer):
    case, W13, W2 = tiny_moe(seed, shared_outer)
    got = staged(case, W13, W2)
    ref = merged(case, W13, W2)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_negative_controls():
    case, W13, W2 = tiny_moe(1)
    ref = merged(case, W13, W2)
    tol = 1e-3 * np.max(np.abs(ref))
    assert np.max(np.abs(staged(case, W13, W2, gate_up_after_act=True) - ref)) > tol
    assert np.max(np.abs(staged(case, W13, W2, down_after_reduce=True) - ref)) > tol


def test_disabled_adapters_leave_caches():
    case = W.moe_case(2, M=12, H=16, I=24, E=4, topk=2, L=2, rank=4, block_size_m=4,
                      enabled=[0, 0], dtype=W.F32)
    c1 = O.moe_gate_up_add(case.x.values, case.cache1.values, case.topk_ids, case.ids,
                           case.adapter_enabled, case.A_gu.values, case.B_gu.values)
    assert np.array_equal(c1, case.cache1.values)
    c2 = O.silu_and_mul(c1)
    c3 = O.moe_down_add(c2, case.cache3.values, case.topk_ids, case.ids,
                        case.adapter_enabled, case.A_d.values, case.B_d.values)
    assert np.array_equal(c3, case.cache3.values)


def test_topk_reduce_weights():
    rng = np.random.default_rng(3)
    c3 = rng.standard_normal((10, 6))
    w = rng.random((5, 2))
    out = O.topk_reduce(c3, w)
    assert np.allclose(out, w[:, :1] * c3[0::2] + w[:, 1:] * c3[1::2], rtol=1e-14)


def _replicated(case):
    """The same adapters with the shared outer stacks copied into every
    expert slot (an unshared case)."""
    import dataclasses
    rep = lambda t: W.Tensor(t.dtype, np.repeat(t.values, case.E, axis=1),
                             np.repeat(t.storage, case.E, axis=1))
    return dataclasses.replace(case, A_gu=rep(case.A_gu), B_d=rep(case.B_d), shared_outer=False)


def _chain(case, gate_up=None, down=None):
    gate_up = gate_up or O.moe_gate_up_add
    down = down or O.moe_down_add
    c1 = gate_up(case.x.values, case.cache1.values, case.topk_ids, case.ids,
                 case.adapter_enabled, case.A_gu.values, case.B_gu.values, case.shared_outer)
    c3 = down(O.silu_and_mul(c1), case.cache3.values, case.topk_ids, case.ids,
              case.adapter_enabled, case.A_d.values, case.B_d.values, case.shared_outer)
    return c1, c3


def test_shared_outer_equals_replicated_stacks():
    """experts_shared_outer_loras (SGLang "LoRA + MoE" page): sharing the
    gate_up A and down B slot equals copying it into every expert slot."""
    case = W.moe_case(4, M=20, H=32, I=48, E=4, topk=2, L=3, rank=8, block_size_m=4,
                      p_none=0.1, dtype=W.F32, shared_outer=True)
    assert case.A_gu.shape[1] == 1 and case.B_d.shape[1] == 1 and case.B_gu.shape[1] == 4
    got = _chain(case)
    ref = _chain(_replicated(case))
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_shared_outer_mutant_caught():
    """Planted slip: the inner stacks (gate_up B, down A) shared instead of the
    outer ones; the replicated-stack pin rejects it."""
    case = W.moe_case(5, M=20, H=32, I=48, E=4, topk=2, L=2, rank=8, block_size_m=4,
                      dtype=W.F32, shared_outer=True)

    def gate_up_inner(x, c1, tid, ids, en, A, B, shared):
        Bs = np.repeat(B[:, :1], B.shape[1], axis=1)          # inner slot 0 for all
        As = np.repeat(A, B.shape[1], axis=1)
        return O.moe_gate_up_add(x, c1, tid, ids, en, As, Bs)

    got = _chain(case, gate_up=gate_up_inner)
    ref = _chain(_replicated(case))
    assert not np.allclose(got[0], ref[0])
