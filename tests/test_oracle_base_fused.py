"""Pins for the oracle of the base layer fused with its LoRA delta
(Ascend walkthrough section 1.1, y = x W^T + (x A^T) B^T).

The oracle forms the base product and then adds the per-token delta; the
pins build each token's merged weight W + B_i A_i first (a different order
of the same mathematics) and check rows without a delta against the base
product alone.
"""
import numpy as np
import pytest

import workloads as W
from oracle import lora as O


def merged(case, Wb):
    x = case.x.values
    y = x @ Wb.T
    off = O.slice_offsets(case.slice_sizes)
    for m in range(case.M):
        i = int(case.ids[m])
        if i < 0 or i >= case.L or case.ranks[i] == 0:
            continue
        r = case.ranks[i]
        A, B = case.A[i].values, case.B[i].values
        Wm = Wb.copy()
        for s in range(case.n_slices):
            Wm[off[s]:off[s + 1]] += B[off[s]:off[s + 1], :r] @ A[s * r:(s + 1) * r]
        y[m] = Wm @ x[m]
    return y


@pytest.mark.parametrize("seed,slices", [(0, [48]), (1, [32, 16, 16])])
def test_equals_merged_weights(seed, slices):
    case = W.random_linear(seed, 30, 64, slices, [16, 8, 0, 32], W.F32)
    Wb = np.random.default_rng(50 + seed).standard_normal((case.N, case.K)) * 0.05
    got = O.linear_with_base(case.x.values, Wb, case.ids, [a.values for a in case.A],
                             [b.values for b in case.B], case.ranks, case.slice_sizes)
    ref = merged(case, Wb)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
    keep = ~O.delta_rows(case.ids, case.ranks)
    assert keep.any()
    assert np.array_equal(got[keep], (case.x.values @ Wb.T)[keep])


def test_integer_inputs_exact():
    case = W.integer_linear(3, 20, 48, [32], [16, 4], W.BF16)
    Wb = np.random.default_rng(7).integers(-1, 2, size=(case.N, case.K)).astype(float)
    got = O.linear_with_base(case.x.values, Wb, case.ids, [a.values for a in case.A],
                             [b.values for b in case.B], case.ranks, case.slice_sizes)
    assert np.array_equal(got, np.round(got))
    assert np.array_equal(got, merged(case, Wb))
