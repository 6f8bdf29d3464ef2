"""GPU parity: dense multi-LoRA through the C ABI against the fp64 oracle.

Gates (from the benchmark spec): segment tables bit-exact; float outputs
max|y - y_or| <= 2e-2 max|y_or| (bf16) or 1e-4 max|y_or| (fp32), plus a
tighter element-wise bound from the arithmetic (helpers.assert_close);
rows without a delta bit-identical to y_base; integer inputs bit-exact.
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


# ---------------------------------------------------------------- segments
def gpu_segments(ml, ids_np, L, enabled=None):
    ids = torch.from_numpy(ids_np.astype(np.int32)).cuda()
    seg = ml.Segments(len(ids_np), L)
    en = None if enabled is None else torch.from_numpy(enabled.astype(np.int32)).cuda()
    ml.lora_build_segments(ids, seg, adapter_enabled=en)
    torch.cuda.synchronize()
    M = len(ids_np)
    nt = int(seg.num_tiles.cpu()[0])
    return (seg.sorted_idx[:M].cpu().numpy(), seg.seg_indptr.cpu().numpy(),
            seg.req_to_lora.cpu().numpy(), int(seg.num_segments.cpu()[0]),
            seg.tile_info.cpu().numpy().reshape(-1, 4)[:nt],
            seg.tile_rows.cpu().numpy().reshape(-1, 64)[:nt])


SEG_CASES = [
    ("tiny", lambda: (W.tiny_fp32().ids, 3)),
    ("decode", lambda: (W.decode_bf16().ids, 20)),
    ("prefill", lambda: (W.prefill_bf16(M=2048, K=8, N=8).ids, 8)),
    ("stacked", lambda: (W.stacked_bf16("qkv", 0, K=8, slice_sizes=[8, 8, 8]).ids, 12)),
    ("moe_ids", lambda: (W.moe_case(0, H=8, I=8).ids, 4)),
    ("empty", lambda: (np.zeros(0, np.int32), 5)),
    ("all_none", lambda: (np.full(300, -1, np.int32), 7)),
    ("one_adapter", lambda: (np.full(1500, 3, np.int32), 4)),
    ("out_of_range", lambda: (np.array([5, -1, 2, 9, -7, 2, 0, 4], np.int32), 4)),
    ("big_random", lambda: (np.random.default_rng(1).integers(-1, 1024, 20000).astype(np.int32),
                            1024)),
    ("L1", lambda: (np.random.default_rng(2).integers(-1, 1, 777).astype(np.int32), 1)),
    # single-wavefront builder (M <= 64)
    ("wave_M64_L1024", lambda: (np.random.default_rng(3).integers(-1, 1024, 64).astype(np.int32),
                                1024)),
    ("wave_M64_L3", lambda: (np.random.default_rng(4).integers(-2, 5, 64).astype(np.int32), 3)),
    ("wave_M1", lambda: (np.array([5], np.int32), 8)),
    ("wave_M63_one_id", lambda: (np.full(63, 2, np.int32), 3)),
    ("wave_M65_block_path", lambda: (np.random.default_rng(5).integers(-1, 6, 65).astype(np.int32),
                                     6)),
    # adapter mask: disabled slots' tokens join the no-adapter bucket
    ("mask_block_M3000_L50", lambda: (np.random.default_rng(6).integers(-1, 50, 3000).astype(np.int32),
                                      50, (np.arange(50) % 3 != 1).astype(np.int32))),
    ("mask_block_uncached_M9000_L7",
     lambda: (np.random.default_rng(7).integers(-1, 7, 9000).astype(np.int32), 7,
              np.array([1, 0, 1, 1, 0, 1, 1], np.int32))),
    ("mask_wave_M40_L9", lambda: (np.random.default_rng(8).integers(-1, 9, 40).astype(np.int32),
                                  9, (np.arange(9) % 2).astype(np.int32))),
    ("mask_block_L1024_all_off",
     lambda: (np.random.default_rng(9).integers(-1, 1024, 5000).astype(np.int32), 1024,
              np.zeros(1024, np.int32))),
]


@pytest.mark.parametrize("name,mk", SEG_CASES, ids=[c[0] for c in SEG_CASES])
def test_segments_bit_exact(ml, name, mk):
    ids, L, *rest = mk()
    enabled = rest[0] if rest else None
    log(f"segments {name} M={len(ids)} L={L}")
    got = gpu_segments(ml, ids, L, enabled)
    ref = O.build_segments(ids, L, enabled)
    assert np.array_equal(got[0], ref[0])
    assert np.array_equal(got[1], ref[1])
    assert np.array_equal(got[2], ref[2])
    assert got[3] == ref[3]
    info, rows = O.tile_schedule(ids, L, enabled=enabled)
    assert np.array_equal(got[4], info)
    assert np.array_equal(got[5], rows)


# ---------------------------------------------------------------- full path
def run_fused(ml, case, reps=1):
    table = table_for(case)
    ids = torch.from_numpy(case.ids).cuda()
    seg = ml.Segments(case.M, case.L)
    ml.lora_build_segments(ids, seg)
    x = to_dev(case.x)
    y = to_dev(case.y_base)
    ws = ml.Workspace.for_table(table, case.M)
    for _ in range(reps):
        ml.lora_shrink_expand_add(table, x, seg, y, ws)
    torch.cuda.synchronize()
    assert ml.lora_read_device_error(ws.buf) == 0
    return to_f64(y)


def oracle_y(case):
    return O.lora_linear(case.x.values, case.ids, [a.values for a in case.A],
                         [b.values for b in case.B], case.ranks, case.slice_sizes,
                         case.y_base.values)


def check_case(ml, case, reps=1):
    log(f"{case.name} M={case.M} K={case.K} slices={case.slice_sizes} L={case.L}")
    got = run_fused(ml, case, reps)
    ref = oracle_y(case)
    if reps > 1:    # y += delta applied reps times
        ref = case.y_base.values + reps * (ref - case.y_base.values)
    keep = ~O.delta_rows(case.ids, case.ranks)
    assert np.array_equal(got[keep], case.y_base.values[keep]), "pass-through rows changed"
    return assert_close(got, ref, case.dtype, case.y_base.values, case.name, roundings=reps)


FUSED_CASES = [
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
    ("cfg3_prefill_bf16", lambda: W.prefill_bf16(0)),
    ("cfg4_stacked_qkv", lambda: W.stacked_bf16("qkv", 0)),
    ("cfg4_stacked_gate_up", lambda: W.stacked_bf16("gate_up", 0)),
    ("prefill_small_ragged", lambda: W.prefill_bf16(1, M=200, K=264, N=328,
                                                    ranks=(16, 32, 64, 8, 0))),
    ("prefill_random_ids", lambda: W.random_linear(16, 300, 1032, [200, 120], [16, 48, 64, 0, 24],
                                                   W.BF16)),
    ("prefill_fp32", lambda: W.random_linear(17, 150, 256, [96, 40], [16, 8, 0, 60], W.F32,
                                             contiguous=True)),
]


@pytest.mark.parametrize("name,mk", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_shrink_expand_add(ml, name, mk):
    check_case(ml, mk())


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("M", [8, 100])
def test_integer_inputs_bit_exact(ml, dtype, M):
    case = W.integer_linear(5, M, 96, [48, 16], [16, 3, 9], dtype)
    log(f"integer M={M} {dtype}")
    got = run_fused(ml, case)
    assert np.array_equal(got, oracle_y(case))


def test_repeated_calls_share_workspace(ml):
    """The decode exchange slots carry each launch's epoch, so a later call
    on the same workspace sees only its own partial sums (y gets 3 deltas)."""
    check_case(ml, W.decode_bf16(7, M=20, K=1536, N=512, L=6), reps=3)


def test_all_none_and_empty(ml):
    case = W.random_linear(18, 50, 128, [64], [16, 32], W.BF16)
    case.ids[:] = -1
    got = run_fused(ml, case)
    assert np.array_equal(got, case.y_base.values)
    case0 = W.random_linear(19, 0, 128, [64], [16], W.BF16)
    got0 = run_fused(ml, case0)
    assert got0.shape == (0, 64)


def test_shrink_matches_oracle_S(ml):
    for case in [W.prefill_bf16(2, M=300, K=1024, N=64, ranks=(16, 64, 32, 8)),
                 W.stacked_bf16("qkv", 1, M=96, K=512, L=5, slice_sizes=[64, 32, 32]),
                 W.random_linear(20, 77, 136, [32], [16, 0, 9], W.F32)]:
        log(f"shrink {case.name}")
        table = table_for(case)
        seg = ml.Segments(case.M, case.L)
        ml.lora_build_segments(torch.from_numpy(case.ids).cuda(), seg)
        S = torch.zeros(case.M, table.n_slices, table.r_max, dtype=torch.float32, device="cuda")
        ws = ml.Workspace.for_table(table, case.M)
        ml.lora_shrink(table, to_dev(case.x), seg, S, ws)
        torch.cuda.synchronize()
        pad_r = table.rank_pad
        A_pad = []
        for a, r, rp in zip(case.A, case.ranks, pad_r):
            ap = np.zeros((case.n_slices * rp, case.K))
            for s in range(case.n_slices):
                ap[s * rp:s * rp + r] = a.values[s * r:(s + 1) * r]
            A_pad.append(ap)
        ref = O.lora_shrink(case.x.values, case.ids, A_pad, pad_r, case.n_slices, table.r_max)
        mv = int(np.count_nonzero(O.delta_rows(case.ids, [max(r, 1) for r in case.ranks])))
        got = S.cpu().numpy().astype(np.float64)[:mv]
        scale = np.max(np.abs(ref[:mv])) if mv else 1.0
        # S is fp32 in both dtypes: only the accumulation order differs
        assert np.max(np.abs(got - ref[:mv]), initial=0) <= 1e-5 * scale


def test_expand_from_oracle_S(ml):
    """lora_expand_add alone, fed the oracle's S (rounded to fp32)."""
    case = W.stacked_bf16("gate_up", 2, M=160, K=256, L=6, slice_sizes=[520, 264])
    log(f"expand {case.name}")
    table = table_for(case)
    seg = ml.Segments(case.M, case.L)
    ml.lora_build_segments(torch.from_numpy(case.ids).cuda(), seg)
    S_or = O.lora_shrink(case.x.values, case.ids, [a.values for a in case.A], case.ranks,
                         case.n_slices, table.r_max)
    S32 = S_or.astype(np.float32)
    y = to_dev(case.y_base)
    ml.lora_expand_add(table, torch.from_numpy(S32).cuda(), seg, y)
    torch.cuda.synchronize()
    ref = O.lora_expand_add(S32.astype(np.float64), case.ids, [b.values for b in case.B],
                            case.ranks, case.slice_sizes, case.y_base.values)
    assert_close(to_f64(y), ref, case.dtype, case.y_base.values, "expand")


def run_with(ml, case, seg_cap=None, y_stride=None, sentinel=-7.0):
    """lora_shrink_expand_add with a segment table of capacity seg_cap tokens
    (more tiles than the batch needs: longer runs of output tiles per
    workgroup in the bf16 expand) and y as the first N columns of a
    [M, y_stride] buffer filled with a sentinel.  Returns y and the columns
    past N (which must keep the sentinel)."""
    table = table_for(case)
    seg = ml.Segments(seg_cap or case.M, case.L)
    ml.lora_build_segments(torch.from_numpy(case.ids).cuda(), seg)
    N = table.N
    dt = torch.bfloat16 if case.dtype == W.BF16 else torch.float32
    if y_stride is None:
        y = to_dev(case.y_base)
        pad = None
    else:
        big = torch.full((case.M, y_stride), sentinel, dtype=dt, device="cuda")
        big[:, :N] = to_dev(case.y_base)
        y, pad = big[:, :N], big[:, N:N + 64]
    ws = ml.Workspace.for_table(table, case.M)
    ml.lora_shrink_expand_add(table, to_dev(case.x), seg, y, ws)
    torch.cuda.synchronize()
    assert ml.lora_read_device_error(ws.buf) == 0
    return to_f64(y), (None if pad is None else pad.float().cpu().numpy())


@pytest.mark.parametrize("seg_cap", [20000, 60000])
def test_expand_long_tile_runs(ml, seg_cap):
    """Slices of 5 and 4 128-column tiles, each ending in a ragged tile (24
    and 8 columns): with a large schedule capacity the expand's units take
    runs of several tiles (one run per slice at 60000), odd and even
    lengths, so the two LDS buffers and register sets alternate across a
    run and its last tile loads nothing further."""
    case = W.random_linear(31, 150, 264, [536, 392], [16, 64, 32, 0, 48], W.BF16)
    log(f"long runs cap={seg_cap}")
    got, _ = run_with(ml, case, seg_cap=seg_cap)
    ref = oracle_y(case)
    keep = ~O.delta_rows(case.ids, case.ranks)
    assert np.array_equal(got[keep], case.y_base.values[keep])
    assert_close(got, ref, case.dtype, case.y_base.values, "long runs")


@pytest.mark.parametrize("stride", [4096, 1 << 24])
def test_expand_strided_y(ml, stride):
    """y inside a wider buffer: rows 4096 columns apart (the pipelined bf16
    expand) and 2^24 columns apart, 70 rows spanning 2.3 GB, past the 2 GiB
    that its 32-bit buffer offsets reach (the one-tile-per-workgroup
    expand).  The columns past N keep their sentinel."""
    case = W.random_linear(32, 70, 200, [328], [16, 32, 64], W.BF16, p_none=0.1)
    log(f"strided y stride={stride}")
    got, pad = run_with(ml, case, y_stride=stride)
    assert np.all(pad == -7.0), "columns past N were written"
    assert_close(got, oracle_y(case), case.dtype, case.y_base.values, f"stride {stride}")


def test_full_size_table_form_repeated(ml):
    """Full decode workload through the table form (lora_shrink_expand_add on
    a prebuilt table), 8 back-to-back calls on one workspace; every row is
    checked, the delta applied 8 times."""
    case = W.decode_bf16(0)
    check_case(ml, case, reps=8)


def test_full_size_bench_step(ml):
    """The step the benchmark times: lora_fused_decode (ids form, segment
    table written) on the full decode workload, input copies rotated over
    several packed tables, back to back on one workspace.  Every row of each
    copy's y is checked against the oracle, and each copy's segment table
    bit for bit."""
    case = W.decode_bf16(0)
    R = 3
    tables = [table_for(case) for _ in range(R)]
    ids = torch.from_numpy(case.ids).cuda()
    segs = [ml.Segments(case.M, case.L) for _ in range(R)]
    xs = [to_dev(case.x) for _ in range(R)]
    ys = [to_dev(case.y_base) for _ in range(R)]
    ws = ml.Workspace.for_table(tables[0], case.M)
    for i in range(2 * R):
        ml.lora_fused_decode(tables[i % R], ids, xs[i % R], ys[i % R], ws, seg=segs[i % R])
    torch.cuda.synchronize()
    assert ml.lora_read_device_error(ws.buf) == 0
    ref = oracle_y(case)
    ref2 = case.y_base.values + 2 * (ref - case.y_base.values)
    sref = O.build_segments(case.ids, case.L)
    for r in range(R):
        assert_close(to_f64(ys[r]), ref2, case.dtype, case.y_base.values, "bench step", roundings=2)
        assert np.array_equal(segs[r].sorted_idx[:case.M].cpu().numpy(), sref[0])
        assert np.array_equal(segs[r].seg_indptr.cpu().numpy(), sref[1])
