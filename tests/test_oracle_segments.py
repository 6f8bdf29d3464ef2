"""Pins for the oracle's segment table (Ascend walkthrough, section 2.3).

The oracle sorts with numpy's stable argsort; these tests pin it against a
hand-worked fixture, a second definition built from Python dict grouping,
brute force over every id map of small size, and invariants.
"""
import itertools

import numpy as np
import pytest

from oracle import lora as O


def grouping_definition(ids, L, enabled=None):
    """Independent definition: collect token lists per valid (and enabled)
    id in a dict, concatenate them by ascending id, then the tokens with no
    adapter."""
    groups = {}
    rest = []
    for m, v in enumerate(ids):
        if 0 <= v < L and (enabled is None or enabled[v]):
            groups.setdefault(v, []).append(m)
        else:
            rest.append(m)
    keys = sorted(groups)
    sorted_idx = [m for k in keys for m in groups[k]] + rest
    seg = [0]
    for k in keys:
        seg.append(seg[-1] + len(groups[k]))
    seg += [seg[-1]] * (L + 1 - len(seg))
    req = keys + [-1] * (L - len(keys))
    return sorted_idx, seg, req, len(keys)


@pytest.mark.parametrize("name", ["segments_example.json", "decode_example_small.json"])
def test_golden(golden, name):
    g = golden(name)
    si, seg, req, n = O.build_segments(g["ids"], g["L"])
    assert si.tolist() == g["sorted_idx"]
    assert seg.tolist() == g["seg_indptr"]
    assert req.tolist() == g["req_to_lora"]
    assert n == g["num_segments"]


@pytest.mark.parametrize("L", [1, 2, 3])
@pytest.mark.parametrize("M", [0, 1, 2, 3, 4])
def test_brute_force_all_maps(M, L):
    # every map over {-1, 0..L-1} plus one out-of-range id (treated as -1)
    values = list(range(-1, L)) + [L]
    for ids in itertools.product(values, repeat=M):
        ids = list(ids)
        si, seg, req, n = O.build_segments(np.array(ids, np.int32), L)
        e_si, e_seg, e_req, e_n = grouping_definition(ids, L)
        assert si.tolist() == e_si, ids
        assert seg.tolist() == e_seg, ids
        assert req.tolist() == e_req, ids
        assert n == e_n


@pytest.mark.parametrize("L", [1, 2, 3])
@pytest.mark.parametrize("M", [0, 1, 2, 3])
def test_brute_force_enable_masks(M, L):
    """Every id map and every enable mask: a disabled adapter's tokens join
    the tokens without an adapter (SGLang "LoRA + MoE" page, adapter_enabled)."""
    values = list(range(-1, L)) + [L]
    for mask in itertools.product([0, 1], repeat=L):
        for ids in itertools.product(values, repeat=M):
            ids = list(ids)
            got = O.build_segments(np.array(ids, np.int32), L, np.array(mask, np.int32))
            exp = grouping_definition(ids, L, mask)
            assert got[0].tolist() == exp[0], (ids, mask)
            assert got[1].tolist() == exp[1], (ids, mask)
            assert got[2].tolist() == exp[2], (ids, mask)
            assert got[3] == exp[3]


def test_enable_mask_hand_case():
    """ids [0, 2, -1, 1, 2], adapter 1 disabled: segments are adapter 0
    (token 0) and adapter 2 (tokens 1, 4); tokens 2 and 3 come last."""
    si, seg, req, n = O.build_segments([0, 2, -1, 1, 2], 3, [1, 0, 1])
    assert si.tolist() == [0, 1, 4, 2, 3]
    assert seg.tolist() == [0, 1, 3, 3]
    assert req.tolist() == [0, 2, -1]
    assert n == 2
    info, rows = O.tile_schedule([0, 2, -1, 1, 2], 3, rows=2, enabled=[1, 0, 1])
    assert info.tolist() == [[0, 0, 0, 1], [1, 2, 1, 2]]
    assert rows.tolist() == [[0, -1], [1, 4]]


@pytest.mark.parametrize("seed", range(6))
def test_invariants_random(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 64))
    M = int(rng.integers(0, 3000))
    ids = rng.integers(-1, L, size=M).astype(np.int32)
    si, seg, req, n = O.build_segments(ids, L)
    # permutation
    assert sorted(si.tolist()) == list(range(M))
    hist = np.bincount(ids[ids >= 0], minlength=L)
    assert n == int(np.count_nonzero(hist))
    # req_to_lora strictly increasing; segment sizes equal the histogram
    assert all(req[s] < req[s + 1] for s in range(n - 1))
    for s in range(n):
        a, b = seg[s], seg[s + 1]
        assert b - a == hist[req[s]]
        assert np.all(ids[si[a:b]] == req[s])
        assert np.all(np.diff(si[a:b]) > 0)        # stable
    mv = int(np.count_nonzero(ids >= 0))
    assert np.all(seg[n:] == mv)
    assert np.all(req[n:] == -1)
    assert np.all(ids[si[mv:]] < 0)
    assert np.all(np.diff(si[mv:]) > 0)


@pytest.mark.parametrize("seed", range(5))
def test_tile_schedule_invariants(seed):
    """Tiles cover every sorted position with an adapter exactly once, never
    straddle a segment, hold at most 64 rows, and their count respects the
    capacity bound floor(M/64) + min(L, M)."""
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 40))
    M = int(rng.integers(0, 3000))
    ids = rng.integers(-1, L, size=M).astype(np.int32)
    if seed == 0:
        ids[:] = 3 % L                      # one long segment
    info, rows = O.tile_schedule(ids, L)
    si, seg, req, n = O.build_segments(ids, L)
    assert len(info) <= M // 64 + min(L, M)
    covered = []
    for (s, a, p, cnt), r in zip(info, rows):
        assert 1 <= cnt <= 64 and req[s] == a
        assert seg[s] <= p and p + cnt <= seg[s + 1]
        assert np.array_equal(r[:cnt], si[p:p + cnt]) and np.all(r[cnt:] == -1)
        covered += list(range(p, p + cnt))
    assert covered == list(range(int(seg[n])))


def test_tile_schedule_hand_case():
    """ids [0, 2, 0, 1] (walkthrough section 2.3 example) with 2-row tiles:
    segment 0 -> tokens 0, 2 (one full tile); 1 -> token 3; 2 -> token 1."""
    info, rows = O.tile_schedule([0, 2, 0, 1], 3, rows=2)
    assert info.tolist() == [[0, 0, 0, 2], [1, 1, 2, 1], [2, 2, 3, 1]]
    assert rows.tolist() == [[0, 2], [3, -1], [1, -1]]
