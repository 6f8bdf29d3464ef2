"""Pins for the dense multi-LoRA oracle (Ascend walkthrough sections 1.1,
2.2-2.3, 3.4, 4.3; SGLang "LoRA Layers" stacked shapes and rank-0 slot).

What pins it, besides itself:
  * hand-worked fixtures under tests/golden/;
  * the merged-weight closed form y = y_base + x (B A)^T (section 1.1) built
    as one fp64 matrix product per adapter and slice;
  * integer inputs where every intermediate is exact;
  * invariants: -1 / rank-0 rows pass through, linearity in x and in B,
    token permutation equivariance, zero rank-padding invariance, slices
    equal separate single-slice problems, shrink then expand equals the
    per-token loop.
"""
import numpy as np
import pytest

import workloads as W
from oracle import lora as O


def vals(case):
    return ([a.values for a in case.A], [b.values for b in case.B])


def merged_weight_reference(case):
    """y_base + x @ (B_s A_s)^T per adapter and slice, with whole-matrix
    products (no per-token loop)."""
    A, B = vals(case)
    y = case.y_base.values.copy()
    off = O.slice_offsets(case.slice_sizes)
    for i, r in enumerate(case.ranks):
        rows = np.nonzero(case.ids == i)[0]
        if r == 0 or rows.size == 0:
            continue
        for s in range(case.n_slices):
            Wd = B[i][off[s]:off[s + 1], :] @ A[i][s * r:(s + 1) * r, :]    # [n_s, K]
            y[np.ix_(rows, np.arange(off[s], off[s + 1]))] += case.x.values[rows] @ Wd.T
    return y


def run(case):
    A, B = vals(case)
    return O.lora_linear(case.x.values, case.ids, A, B, case.ranks, case.slice_sizes,
                         case.y_base.values)


def from_golden(g):
    return (np.array(g["x"], float), np.array(g["ids"], np.int32),
            [np.array(a, float) for a in g["A"]], [np.array(b, float) for b in g["B"]],
            g["ranks"], g["slice_sizes"], np.array(g["y_base"], float))


@pytest.mark.parametrize("name", ["decode_example_small.json", "stacked_example.json"])
def test_golden_linear(golden, name):
    g = golden(name)
    x, ids, A, B, ranks, sl, yb = from_golden(g)
    y = O.lora_linear(x, ids, A, B, ranks, sl, yb)
    assert np.array_equal(y, np.array(g["y"], float))


def test_golden_shrink(golden):
    g = golden("decode_example_small.json")
    x, ids, A, B, ranks, sl, yb = from_golden(g)
    S = O.lora_shrink(x, ids, A, ranks, 1, 2)
    assert np.array_equal(S, np.array(g["S_sorted"], float))


CASES = [
    lambda: W.tiny_fp32(0),
    lambda: W.decode_bf16(0, M=16, K=512, N=384, L=6),
    lambda: W.prefill_bf16(1, M=200, K=256, N=320, ranks=(16, 32, 64, 8, 0)),
    lambda: W.stacked_bf16("qkv", 0, M=64, K=128, L=5, slice_sizes=[96, 32, 32]),
    lambda: W.random_linear(3, 37, 72, [40, 24], [0, 5, 16, 33], W.F32),
]


@pytest.mark.parametrize("mk", CASES)
def test_merged_weight_closed_form(mk):
    case = mk()
    y = run(case)
    ref = merged_weight_reference(case)
    scale = max(1.0, float(np.max(np.abs(ref))))
    assert np.max(np.abs(y - ref)) <= 1e-12 * scale


def test_single_adapter_reduces_to_two_matmuls():
    rng = np.random.default_rng(5)
    M, K, N, r = 11, 40, 24, 7
    x = rng.standard_normal((M, K))
    A = rng.standard_normal((r, K))
    B = rng.standard_normal((N, r))
    yb = rng.standard_normal((M, N))
    y = O.lora_linear(x, np.zeros(M, np.int32), [A], [B], [r], [N], yb)
    assert np.allclose(y, yb + (x @ A.T) @ B.T, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
def test_integer_inputs_exact(seed, dtype):
    case = W.integer_linear(seed, 24, 96, [48, 16], [16, 3, 9], dtype)
    y = run(case)
    assert np.array_equal(y, np.round(y))
    assert np.array_equal(y, merged_weight_reference(case))


@pytest.mark.parametrize("mk", CASES)
def test_passthrough_rows_bit_identical(mk):
    case = mk()
    y = run(case)
    keep = ~O.delta_rows(case.ids, case.ranks)
    assert np.array_equal(y[keep], case.y_base.values[keep])


def test_rank_zero_slot_is_noop():
    case = W.random_linear(9, 30, 64, [32], [0, 16, 0], W.F32, p_none=0.0)
    y = run(case)
    rows = np.isin(case.ids, [0, 2])
    assert rows.any()
    assert np.array_equal(y[rows], case.y_base.values[rows])


def test_linearity_in_x_and_B():
    case = W.random_linear(4, 20, 48, [32], [16, 8], W.F32, p_none=0.1)
    A, B = vals(case)
    yb = case.y_base.values
    zero = np.zeros_like(yb)
    rng = np.random.default_rng(0)
    x1 = case.x.values
    x2 = rng.standard_normal(x1.shape)
    d = lambda x, Bs: O.lora_linear(x, case.ids, A, Bs, case.ranks, case.slice_sizes, zero)
    assert np.allclose(d(x1 + 2.0 * x2, B), d(x1, B) + 2.0 * d(x2, B), atol=1e-12)
    B2 = [rng.standard_normal(b.shape) for b in B]
    Bsum = [b + c for b, c in zip(B, B2)]
    assert np.allclose(d(x1, Bsum), d(x1, B) + d(x1, B2), atol=1e-12)
    # y_base enters additively
    assert np.allclose(O.lora_linear(x1, case.ids, A, B, case.ranks, case.slice_sizes, yb),
                       yb + d(x1, B), atol=1e-12)


def test_token_permutation_equivariance():
    case = W.random_linear(6, 33, 40, [24], [8, 16, 4], W.F32)
    A, B = vals(case)
    y = run(case)
    perm = np.random.default_rng(1).permutation(case.M)
    yp = O.lora_linear(case.x.values[perm], case.ids[perm], A, B, case.ranks,
                       case.slice_sizes, case.y_base.values[perm])
    assert np.allclose(yp, y[perm], rtol=0, atol=1e-13)


def test_zero_rank_padding_invariance():
    """Section 4.3: padding A rows and B columns with zeros to a multiple of
    16 leaves the result unchanged."""
    case = W.random_linear(7, 25, 64, [40, 8], [5, 20], W.F32)
    A, B = vals(case)
    y = run(case)
    n_sl = case.n_slices
    Ap, Bp, rp = [], [], []
    for a, b, r in zip(A, B, case.ranks):
        rh = -(-r // 16) * 16
        a2 = np.zeros((n_sl * rh, a.shape[1]))
        for s in range(n_sl):
            a2[s * rh:s * rh + r] = a[s * r:(s + 1) * r]
        b2 = np.zeros((b.shape[0], rh))
        b2[:, :r] = b
        Ap.append(a2), Bp.append(b2), rp.append(rh)
    yp = O.lora_linear(case.x.values, case.ids, Ap, Bp, rp, case.slice_sizes,
                       case.y_base.values)
    assert np.allclose(yp, y, rtol=0, atol=1e-12)


def test_slices_equal_separate_problems():
    case = W.random_linear(8, 21, 32, [16, 8, 8], [4, 8], W.F32)
    A, B = vals(case)
    y = run(case)
    off = O.slice_offsets(case.slice_sizes)
    for s in range(case.n_slices):
        As = [a[s * r:(s + 1) * r] for a, r in zip(A, case.ranks)]
        Bs = [b[off[s]:off[s + 1]] for b in B]
        ys = O.lora_linear(case.x.values, case.ids, As, Bs, case.ranks,
                           [case.slice_sizes[s]], case.y_base.values[:, off[s]:off[s + 1]])
        assert np.array_equal(ys, y[:, off[s]:off[s + 1]])


@pytest.mark.parametrize("mk", CASES)
def test_shrink_matches_segment_matmul_and_composes(mk):
    case = mk()
    A, B = vals(case)
    rmax = max([16] + [-(-r // 16) * 16 for r in case.ranks])
    S = O.lora_shrink(case.x.values, case.ids, A, case.ranks, case.n_slices, rmax)
    si, seg, req, n = O.build_segments(case.ids, case.L)
    for s_id in range(n):
        i = req[s_id]
        r = case.ranks[i]
        rows = si[seg[s_id]:seg[s_id + 1]]
        for s in range(case.n_slices):
            ref = case.x.values[rows] @ A[i][s * r:(s + 1) * r].T
            got = S[seg[s_id]:seg[s_id + 1], s, :r]
            assert np.allclose(got, ref, rtol=0, atol=1e-12 * max(1, np.abs(ref).max(initial=0)))
        assert np.all(S[seg[s_id]:seg[s_id + 1], :, r:] == 0)
    assert np.all(S[seg[n]:] == 0)
    y = O.lora_expand_add(S, case.ids, B, case.ranks, case.slice_sizes, case.y_base.values)
    ref = run(case)
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))


def test_enable_mask_matches_merged_weights_of_enabled_adapters():
    """With an enable mask (SGLang "LoRA + MoE" page, adapter_enabled), rows
    of disabled adapters pass through bit for bit and every other row equals
    the merged-weight closed form; an all-ones mask changes nothing."""
    case = W.random_linear(21, 40, 72, [48, 24], [16, 8, 32, 5], W.F32, p_none=0.1)
    A, B = vals(case)
    enabled = np.array([1, 0, 1, 0], np.int32)
    y = O.lora_linear(case.x.values, case.ids, A, B, case.ranks, case.slice_sizes,
                      case.y_base.values, enabled)
    off_rows = np.isin(case.ids, [1, 3])
    assert off_rows.any()
    assert np.array_equal(y[off_rows], case.y_base.values[off_rows])
    ref = merged_weight_reference(case)
    on = ~off_rows
    assert np.max(np.abs(y[on] - ref[on])) <= 1e-12 * np.max(np.abs(ref))
    y1 = O.lora_linear(case.x.values, case.ids, A, B, case.ranks, case.slice_sizes,
                       case.y_base.values, np.ones(4, np.int32))
    assert np.array_equal(y1, run(case))
    assert np.array_equal(O.delta_rows(case.ids, case.ranks, enabled),
                          O.delta_rows(case.ids, case.ranks) & on)
