"""Planted mistakes in copies of the oracle must be caught by its pins.

Each mutant is a plausible slip (a transposed operand, a dropped term, a
wrong slice index, Python's negative indexing of id -1, an unstable sort,
the wrong gate half, ...).  The detectors are the same pins the real oracle
passes: the hand-worked fixtures and the merged-weight closed forms.
"""
import numpy as np
import pytest

import workloads as W
from oracle import lora as O
from oracle import moe as OM
from tests.test_oracle_lora import merged_weight_reference, from_golden
from tests.test_oracle_segments import grouping_definition


# ---------------------------------------------------------------- lora_linear
def make_linear(mut):
    def f(x, ids, A, B, ranks, slice_sizes, y_base):
        x = np.asarray(x, float)
        y = np.zeros_like(np.asarray(y_base, float)) if mut == "drop_base" \
            else np.array(y_base, float, copy=True)
        off = O.slice_offsets(slice_sizes)
        n_sl = len(slice_sizes)
        for m in range(x.shape[0]):
            i = int(ids[m])
            if mut != "neg_index" and (i < 0 or i >= len(ranks)):
                continue
            if ranks[i] == 0:
                continue
            r = ranks[i]
            Ai, Bi = np.asarray(A[i], float), np.asarray(B[i], float)
            xm = x[m - 1] if mut == "wrong_token" else x[m]
            for s in range(n_sl):
                rows = (np.arange(r) * n_sl + s) if mut == "interleaved_slices" \
                    else np.arange(s * r, (s + 1) * r)
                S = Ai[rows] @ xm
                Bs = Bi[off[s]:off[s + 1], :r]
                if mut == "slice0_rows":
                    Bs = Bi[0:off[s + 1] - off[s], :r]
                d = Bs @ S
                if mut == "sign":
                    d = -d
                if mut == "truncate_rank":
                    d = Bs[:, :max(r - 1, 0)] @ S[:max(r - 1, 0)]
                y[m, off[s]:off[s + 1]] += d
        return y
    return f


LINEAR_MUTANTS = ["drop_base", "neg_index", "wrong_token", "interleaved_slices",
                  "slice0_rows", "sign", "truncate_rank"]


def linear_detected(impl):
    for name in ["decode_example_small.json", "stacked_example.json"]:
        from tests.conftest import load_golden
        g = load_golden(name)
        x, ids, A, B, ranks, sl, yb = from_golden(g)
        if not np.array_equal(impl(x, ids, A, B, ranks, sl, yb), np.array(g["y"], float)):
            return True
    for case in [W.random_linear(3, 37, 72, [40, 24], [0, 5, 16, 33], W.F32),
                 W.stacked_bf16("qkv", 0, M=64, K=128, L=5, slice_sizes=[96, 32, 32])]:
        got = impl(case.x.values, case.ids, [a.values for a in case.A],
                   [b.values for b in case.B], case.ranks, case.slice_sizes,
                   case.y_base.values)
        ref = merged_weight_reference(case)
        if np.max(np.abs(got - ref)) > 1e-9 * np.max(np.abs(ref)):
            return True
    return False


def test_real_linear_not_flagged():
    assert not linear_detected(O.lora_linear)


@pytest.mark.parametrize("mut", LINEAR_MUTANTS)
def test_linear_mutant_caught(mut):
    assert linear_detected(make_linear(mut))


# ---------------------------------------------------------------- segments
def make_segments(mut):
    def f(ids, L):
        ids = np.asarray(ids, np.int64)
        valid = (ids >= 0) & (ids < L)
        if mut == "minus_one_first":
            key = np.where(valid, ids, -1)
        elif mut == "descending":
            key = np.where(valid, -ids, np.iinfo(np.int64).max)
        else:
            key = np.where(valid, ids, np.iinfo(np.int64).max)
        kind = "quicksort" if mut == "unstable" else "stable"
        if mut == "unstable":
            # a deterministic non-stable order: ties broken by descending token
            order = np.lexsort((-np.arange(ids.size), key))
        else:
            order = np.argsort(key, kind=kind)
        present = sorted(set(int(v) for v in ids[valid]))
        if mut == "descending":
            present = present[::-1]
        seg = np.zeros(L + 1, np.int32)
        req = np.full(L, -1, np.int32)
        for s, a in enumerate(present):
            req[s] = a
            seg[s + 1] = seg[s] + int(np.count_nonzero(ids == a))
        tail = 0 if mut == "zero_tail" else seg[len(present)]
        seg[len(present) + 1:] = tail
        return order.astype(np.int32), seg, req, len(present)
    return f


@pytest.mark.parametrize("mut", ["minus_one_first", "descending", "unstable", "zero_tail"])
def test_segments_mutant_caught(mut):
    f = make_segments(mut)
    caught = False
    rng = np.random.default_rng(0)
    for _ in range(50):
        L = 3
        ids = rng.integers(-1, L, size=6).astype(np.int32)
        si, seg, req, n = f(ids, L)
        e = grouping_definition(ids.tolist(), L)
        if (si.tolist(), seg.tolist(), req.tolist(), n) != e:
            caught = True
            break
    assert caught


# ---------------------------------------------------------------- moe
def test_moe_wrong_gate_half_caught(golden):
    g = golden("moe_example.json")
    c1 = np.array(g["cache1_out"], float)
    I = c1.shape[1] // 2
    wrong = OM.silu(c1[:, I:]) * c1[:, :I]
    assert not np.allclose(wrong, np.array(g["cache2_out"], float))


def test_moe_wrong_flattening_caught():
    case = W.moe_case(0, M=5, H=8, I=8, E=4, topk=2, L=2, rank=2, block_size_m=2,
                      dtype=W.F32)
    cap = OM.align_capacity(case.M, case.topk, case.E, case.block_size_m)
    s, _, _ = OM.moe_align(case.topk_ids, case.ids, case.adapter_enabled, case.L, case.E,
                           case.block_size_m, cap)
    # the k-major flattening f = k*M + m would put different pairs in the lists
    M, topk = case.topk_ids.shape
    P = M * topk
    remap = lambda f: (f % topk) * M + f // topk if f < P else P
    assert not np.array_equal(np.vectorize(remap)(s), s)


# ---------------------------------------------------------------- enable mask
def mask_by_token(ids, enabled, L):
    """Planted slip: the mask indexed by token instead of by adapter id."""
    ids = np.asarray(ids, np.int64).copy()
    for m in range(ids.shape[0]):
        if 0 <= ids[m] < L and not enabled[m % L]:
            ids[m] = -1
    return ids


def mask_keep_disabled(ids, enabled, L):
    """Planted slip: the mask inverted (disabled adapters kept)."""
    ids = np.asarray(ids, np.int64).copy()
    for m in range(ids.shape[0]):
        if 0 <= ids[m] < L and enabled[ids[m]]:
            ids[m] = -1
    return ids


@pytest.mark.parametrize("mut", [mask_by_token, mask_keep_disabled])
def test_mask_mutant_caught(mut, monkeypatch):
    """The brute-force grouping pin rejects each mask mutant."""
    import itertools
    monkeypatch.setattr(O, "mask_ids", mut)
    caught = False
    for mask in itertools.product([0, 1], repeat=3):
        for ids in itertools.product([-1, 0, 1, 2], repeat=3):
            got = O.build_segments(np.array(ids, np.int32), 3, np.array(mask, np.int32))
            if got[0].tolist() != grouping_definition(list(ids), 3, mask)[0]:
                caught = True
    assert caught
