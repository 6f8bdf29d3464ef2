"""GPU parity of the single-launch decode (lora_fused_decode) and of the
adapter enable mask, through the C ABI, against the fp64 oracle.

Gates: the segment table and tile schedule the launch writes are bit-exact
with the oracle's; y meets the benchmark spec's tolerance and the element-wise
bound of helpers.assert_close; rows without a delta (id -1, out of range,
rank 0, adapter disabled) are bit-identical to y_base.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import lora as O
from tests.helpers import assert_close, table_for, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ml():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import adapter_lora_amd
    return adapter_lora_amd


def log(msg):
    print(msg, flush=True)


def mask_for(L, seed, p_on=0.7):
    rng = np.random.default_rng(1000 + seed)
    m = (rng.random(L) < p_on).astype(np.int32)
    return m


def run_decode(ml, case, enabled=None, reps=1, with_table=True, expect_err=0):
    table = table_for(case)
    ids = torch.from_numpy(case.ids).cuda()
    seg = ml.Segments(case.M, case.L) if with_table else None
    en = None if enabled is None else torch.from_numpy(enabled).cuda()
    x = to_dev(case.x)
    y = to_dev(case.y_base)
    ws = ml.Workspace.for_table(table, case.M)
    for _ in range(reps):
        ml.lora_fused_decode(table, ids, x, y, ws, seg=seg, adapter_enabled=en)
    torch.cuda.synchronize()
    assert ml.lora_read_device_error(ws.buf) == expect_err
    return to_f64(y), seg


def check_table(seg, case, enabled):
    M, L = case.M, case.L
    ref = O.build_segments(case.ids, L, enabled)
    assert np.array_equal(seg.sorted_idx[:M].cpu().numpy(), ref[0])
    assert np.array_equal(seg.seg_indptr.cpu().numpy(), ref[1])
    assert np.array_equal(seg.req_to_lora.cpu().numpy(), ref[2])
    assert int(seg.num_segments.cpu()[0]) == ref[3]
    info, rows = O.tile_schedule(case.ids, L, enabled=enabled)
    nt = int(seg.num_tiles.cpu()[0])
    assert nt == len(info)
    assert np.array_equal(seg.tile_info.cpu().numpy().reshape(-1, 4)[:nt], info)
    assert np.array_equal(seg.tile_rows.cpu().numpy().reshape(-1, 64)[:nt], rows)


def check(ml, case, enabled=None, reps=1, expect_err=0):
    log(f"fused_decode {case.name} M={case.M} K={case.K} slices={case.slice_sizes} L={case.L} "
        f"mask={'none' if enabled is None else int(enabled.sum())}")
    got, seg = run_decode(ml, case, enabled, reps, expect_err=expect_err)
    check_table(seg, case, enabled)
    ref = O.lora_linear(case.x.values, case.ids, [a.values for a in case.A],
                        [b.values for b in case.B], case.ranks, case.slice_sizes,
                        case.y_base.values, enabled)
    if reps > 1:
        ref = case.y_base.values + reps * (ref - case.y_base.values)
    keep = ~O.delta_rows(case.ids, case.ranks, enabled)
    assert np.array_equal(got[keep], case.y_base.values[keep]), "pass-through rows changed"
    assert_close(got, ref, case.dtype, case.y_base.values, case.name, roundings=reps)


CASES = [
    ("cfg1_tiny_fp32", lambda: W.tiny_fp32(0)),
    ("cfg2_decode_bf16", lambda: W.decode_bf16(0)),
    ("decode_fp32", lambda: W.decode_bf16(3, M=24, K=1024, N=768, L=9, dtype=W.F32)),
    ("decode_ragged", lambda: W.random_linear(11, 13, 520, [328], [16, 48, 0, 5, 64], W.BF16)),
    ("decode_M1", lambda: W.random_linear(12, 1, 4096, [4096], [64], W.BF16, p_none=0.0)),
    ("decode_M64_one_adapter", lambda: W.random_linear(13, 64, 2048, [1024], [32], W.BF16,
                                                       p_none=0.0)),
    ("decode_slices", lambda: W.random_linear(14, 40, 1024, [512, 128, 136], [16, 32, 64, 40],
                                              W.BF16)),
    ("decode_slices_fp32", lambda: W.random_linear(15, 17, 264, [64, 48], [3, 17, 33], W.F32)),
    ("decode_M64_L40", lambda: W.random_linear(22, 64, 512, [256], [16, 32, 64, 0] * 10, W.BF16,
                                               p_none=0.05)),
]


@pytest.mark.parametrize("name,mk", CASES, ids=[c[0] for c in CASES])
def test_fused_decode_matches_oracle(ml, name, mk):
    check(ml, mk())


@pytest.mark.parametrize("name,mk", CASES[:4] + CASES[6:], ids=[c[0] for c in CASES[:4] + CASES[6:]])
def test_fused_decode_with_enable_mask(ml, name, mk):
    case = mk()
    check(ml, case, enabled=mask_for(case.L, 1))


def test_fused_decode_large_table(ml):
    """L = 300 slots: the mask and the rank / offset tables are read by id
    (the path for tables of more than 256 slots), and with L > M the units
    are numbered by segment; every other case here has L <= M, where each
    unit serves one adapter slot."""
    ranks = [16, 0, 32, 64, 8, 48] * 50
    case = W.random_linear(23, 48, 256, [136], ranks, W.BF16, p_none=0.1)
    case.ids[:] = np.random.default_rng(5).integers(-1, 300, size=48).astype(np.int32)
    check(ml, case)
    check(ml, case, enabled=mask_for(300, 2))


def test_fused_decode_repeated_calls(ml):
    """The exchange slots carry the launch's epoch, so repeated calls on one
    workspace each add a fresh delta and never read an earlier call's
    partial sums."""
    check(ml, W.decode_bf16(7, M=20, K=1536, N=512, L=6), reps=3)


def test_fused_decode_edge_cases(ml):
    # all tokens without an adapter, all adapters disabled, out-of-range ids
    case = W.random_linear(18, 50, 128, [64], [16, 32], W.BF16)
    case.ids[:] = -1
    check(ml, case)
    case = W.random_linear(24, 33, 256, [128], [16, 32, 64], W.BF16, p_none=0.0)
    check(ml, case, enabled=np.zeros(3, np.int32))
    case = W.random_linear(25, 20, 128, [64], [16, 16, 16, 16], W.F32)
    case.ids[:] = np.array([5, -1, 2, 9, -7, 2, 0, 4, 3, 3, 1, 100, -2, 0, 1, 2, 3, 4, 4, 0],
                           np.int32)
    # ids outside [-1, L) are treated as "no adapter" and reported
    check(ml, case, expect_err=ml.LORA_DEVERR_BAD_ID)
    # M = 0 writes the empty table and touches nothing else
    case0 = W.random_linear(19, 0, 128, [64], [16], W.BF16)
    got, seg = run_decode(ml, case0)
    assert got.shape == (0, 64)
    assert int(seg.num_segments.cpu()[0]) == 0 and int(seg.num_tiles.cpu()[0]) == 0
    assert np.array_equal(seg.seg_indptr.cpu().numpy(), [0, 0])
    assert np.array_equal(seg.req_to_lora.cpu().numpy(), [-1])


def test_fused_decode_without_table_and_reuse(ml):
    """Without table buffers the launch writes none; the table it writes
    when asked drives lora_shrink_expand_add on the same batch (another
    layer) to the same result."""
    case = W.decode_bf16(4, M=32, K=1024, N=512, L=7)
    got_no_table, _ = run_decode(ml, case, with_table=False)
    table = table_for(case)
    ids = torch.from_numpy(case.ids).cuda()
    seg = ml.Segments(case.M, case.L)
    x = to_dev(case.x)
    y1 = to_dev(case.y_base)
    y2 = to_dev(case.y_base)
    ws = ml.Workspace.for_table(table, case.M)
    ml.lora_fused_decode(table, ids, x, y1, ws, seg=seg)
    ml.lora_shrink_expand_add(table, x, seg, y2, ws)
    torch.cuda.synchronize()
    assert ml.lora_read_device_error(ws.buf) == 0
    assert torch.equal(y1, y2)
    assert np.array_equal(to_f64(y1), got_no_table)


MASKED_SEG_CASES = [
    ("wave", 50, 9, 31),
    ("wave_L300", 64, 300, 32),
    ("block", 700, 9, 33),
    ("block_L300", 5000, 300, 34),
]


@pytest.mark.parametrize("name,M,L,seed", MASKED_SEG_CASES, ids=[c[0] for c in MASKED_SEG_CASES])
def test_build_segments_with_mask_bit_exact(ml, name, M, L, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, L + 1, size=M).astype(np.int32)
    enabled = mask_for(L, 3)
    log(f"masked segments {name} M={M} L={L}")
    seg = ml.Segments(M, L)
    ml.lora_build_segments(torch.from_numpy(ids).cuda(), seg,
                           adapter_enabled=torch.from_numpy(enabled).cuda())
    torch.cuda.synchronize()
    ref = O.build_segments(ids, L, enabled)
    assert np.array_equal(seg.sorted_idx[:M].cpu().numpy(), ref[0])
    assert np.array_equal(seg.seg_indptr.cpu().numpy(), ref[1])
    assert np.array_equal(seg.req_to_lora.cpu().numpy(), ref[2])
    assert int(seg.num_segments.cpu()[0]) == ref[3]
    info, rows = O.tile_schedule(ids, L, enabled=enabled)
    nt = int(seg.num_tiles.cpu()[0])
    assert np.array_equal(seg.tile_info.cpu().numpy().reshape(-1, 4)[:nt], info)
    assert np.array_equal(seg.tile_rows.cpu().numpy().reshape(-1, 64)[:nt], rows)


def test_error_word_only_for_ids_outside_the_table(ml):
    """-1 is the ordinary "no adapter" id and reports nothing; one id past
    the table (or below -1) sets LORA_DEVERR_BAD_ID, its row is left as it
    was, and every other row still gets its delta."""
    case = W.decode_bf16(9, M=24, K=1024, N=512, L=6)
    case.ids[:] = np.where(case.ids >= 0, case.ids, -1)
    check(ml, case, expect_err=0)
    for bad in (6, 1000, -2):
        c2 = W.decode_bf16(9, M=24, K=1024, N=512, L=6)
        c2.ids[5] = bad
        check(ml, c2, expect_err=ml.LORA_DEVERR_BAD_ID)


def test_each_launch_tags_its_slots_afresh(ml):
    """The exchange slots are never emptied: each launch tags the slots it
    writes with a value of its own (from its dispatch), and consumers take
    only slots with their launch's tag.  Consecutive launches on one
    workspace leave different tags in the slot of sorted position 0,
    S column 0 (workspace: 256-byte header, then 64-bit {value, tag} slots
    [K chunk][position][column]); and a launch with new x after one with
    other x on the same workspace still matches the oracle for the new x
    (a stale partial sum would be taken before its producer rewrote it)."""
    case = W.decode_bf16(8, M=16, K=1024, N=512, L=5)
    case.ids[0] = 2                     # sorted position 0 has an adapter
    other = W.decode_bf16(11, M=16, K=1024, N=512, L=5)
    table = table_for(case)
    ws = ml.Workspace.for_table(table, case.M)
    slot0 = ws.buf[256:264].view(torch.int64)
    ids = torch.from_numpy(case.ids).cuda()
    tags = []
    for c in (other, case, other, case):
        x, y = to_dev(c.x), to_dev(case.y_base)
        ml.lora_fused_decode(table, ids, x, y, ws)
        torch.cuda.synchronize()
        tags.append(int(slot0.cpu()[0]) >> 32 & 0xffffffff)
    assert ml.lora_read_device_error(ws.buf) == 0
    assert all(t != 0 for t in tags) and len(set(tags)) == len(tags), tags
    ref = O.lora_linear(case.x.values, case.ids, [a.values for a in case.A],
                        [b.values for b in case.B], case.ranks, case.slice_sizes,
                        case.y_base.values)
    assert_close(to_f64(y), ref, case.dtype, case.y_base.values, "after other x")


# Inputs in {-1, 0, 1} (workloads.integer_linear): every S value and every
# delta is a small integer, exact in fp32 and in the S hi / lo bf16 pair, so
# the device result equals the oracle's rounded result bit for bit.  The
# cases cover the slot-mode view (L <= M), the segment view (L > M), the
# enable mask, the MFMA consumers (ranks above 16) and the VALU ones.
INT_CASES = [
    ("slot_mode_bf16", lambda: W.integer_linear(31, 32, 4096, [4096], [16, 64, 32, 0, 48] * 4,
                                                W.BF16), None),
    ("segments_L_gt_M_bf16", lambda: W.integer_linear(32, 20, 1032, [520, 264],
                                                      [16, 32, 64, 3] * 10, W.BF16), None),
    ("masked_bf16", lambda: W.integer_linear(33, 48, 2048, [1024], [64, 16, 32, 9, 64, 16],
                                             W.BF16), np.array([1, 0, 1, 1, 0, 1], np.int32)),
    ("slot_mode_fp32", lambda: W.integer_linear(34, 64, 520, [264, 136], [16, 33, 64], W.F32),
     None),
]


@pytest.mark.parametrize("name,mk,enabled", INT_CASES, ids=[c[0] for c in INT_CASES])
def test_fused_decode_integer_bit_exact(ml, name, mk, enabled):
    case = mk()
    log(f"fused_decode integer {name} M={case.M} K={case.K} L={case.L}")
    got, seg = run_decode(ml, case, enabled)
    check_table(seg, case, enabled)
    ref = O.lora_linear(case.x.values, case.ids, [a.values for a in case.A],
                        [b.values for b in case.B], case.ranks, case.slice_sizes,
                        case.y_base.values, enabled)
    ref = W.make_tensor(ref.astype(np.float32), case.dtype).values     # one rounding
    assert np.array_equal(got, ref)
