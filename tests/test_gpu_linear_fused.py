"""GPU parity of lora_linear_fused, the base layer and its LoRA delta in one
product (Ascend walkthrough section 1.1: y = x W^T + (x A^T) B^T; SGLang
"LoRA Layers" page: base output plus LoRA delta), against the fp64 oracle
linear_with_base.

Tolerance: the spec gate (max error <= 2e-2 max|y|) and an
element-wise bound from the arithmetic: one bf16 rounding of y (half an ulp,
<= 2^-8 |y|) plus fp32 summation of the K products of the base and of the
shrink and expand sums (gamma = 2 (K + 64) 2^-24 times the sums of absolute
products).  With inputs in {-1, 0, 1} every partial sum is a small integer,
exact in fp32 and bf16, so the result must equal the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import lora as O
from tests.helpers import TOL_BF16, table_for, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ml():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import adapter_lora_amd
    return adapter_lora_amd


def log(msg):
    print(msg, flush=True)


def run_fused(ml, case, Wt, enabled=None):
    table = table_for(case)
    ids = torch.from_numpy(case.ids).cuda()
    seg = ml.Segments(case.M, case.L)
    en = None if enabled is None else torch.from_numpy(enabled).cuda()
    ml.lora_build_segments(ids, seg, adapter_enabled=en)
    x = to_dev(case.x)
    y = torch.full((case.M, case.N), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = ml.Workspace.for_table(table, case.M)
    ml.lora_linear_fused(table, to_dev(Wt), x, seg, y, ws)
    torch.cuda.synchronize()
    return to_f64(y)


def abs_bound(case, Wt):
    """Sum over the products of absolute values: |x| |W|^T plus, per token
    with an adapter, (|x| |A_i|^T) |B_i|^T per slice."""
    ax = np.abs(case.x.values)
    b = ax @ np.abs(Wt.values).T
    off = O.slice_offsets(case.slice_sizes)
    for m in range(case.M):
        i = int(case.ids[m])
        if i < 0 or i >= case.L or case.ranks[i] == 0:
            continue
        r = case.ranks[i]
        A, B = np.abs(case.A[i].values), np.abs(case.B[i].values)
        for s in range(case.n_slices):
            sa = A[s * r:(s + 1) * r] @ ax[m]
            b[m, off[s]:off[s + 1]] += B[off[s]:off[s + 1], :r] @ sa
    return b


def check(ml, case, Wt):
    log(f"linear_fused {case.name} M={case.M} K={case.K} slices={case.slice_sizes} "
        f"ranks={case.ranks}")
    got = run_fused(ml, case, Wt)
    ref = O.linear_with_base(case.x.values, Wt.values, case.ids, [a.values for a in case.A],
                             [b.values for b in case.B], case.ranks, case.slice_sizes)
    assert not np.isnan(got).any(), "rows left unwritten"
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(got - ref)))
    assert err <= TOL_BF16 * scale, f"max err {err:.3e} > {TOL_BF16} * {scale:.3e}"
    gamma = 2.0 * (case.K + 64) * 2.0 ** -24
    bound = 2.0 ** -8 * np.abs(ref) + gamma * abs_bound(case, Wt) + 1e-30
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (f"{int(bad.sum())} elements beyond the element-wise bound; "
                           f"first at {np.argwhere(bad)[0].tolist()}")
    return got, ref


CASES = [
    # several row tiles per segment, a ragged last tile, rank-0 slot, tokens
    # without an adapter, stacked slices narrower than a column tile
    ("qkv_mixed", lambda: W.random_linear(40, 300, 1024, [512, 136, 136], [16, 64, 32, 0, 48],
                                          W.BF16)),
    # K not a multiple of the 32-wide stage, N not a multiple of 256
    ("ragged_K_N", lambda: W.random_linear(41, 77, 264, [200], [8, 24], W.BF16)),
    ("decode_rows", lambda: W.decode_bf16(42, M=32, K=4096, N=4096, L=20)),
    ("all_without_adapter", lambda: W.random_linear(43, 130, 512, [256], [16, 32], W.BF16,
                                                    p_none=1.0)),
    ("one_token", lambda: W.random_linear(44, 1, 512, [264], [64], W.BF16, p_none=0.0)),
    ("contiguous_segments", lambda: W.random_linear(45, 520, 768, [1024], [16, 16, 32, 64],
                                                    W.BF16, contiguous=True)),
    # 70 adapter slots (past one wavefront of slots: the segment search takes
    # two rounds of loads) and about 30 segments in each 128-row unit
    ("many_adapters", lambda: W.random_linear(48, 300, 256, [136], [16, 32, 0, 64, 16] * 14,
                                              W.BF16)),
    # K of one stage and of four stages (no steady-state loop iterations)
    ("K_one_stage", lambda: W.random_linear(49, 150, 64, [264], [16, 32], W.BF16)),
    ("K_four_stages", lambda: W.random_linear(50, 130, 200, [512], [64, 16, 32], W.BF16)),
]


@pytest.mark.parametrize("name,mk", CASES, ids=[c[0] for c in CASES])
def test_linear_fused_matches_oracle(ml, name, mk):
    case = mk()
    Wt = W.base_weight(100 + [c[0] for c in CASES].index(name), case.N, case.K)
    check(ml, case, Wt)


def test_linear_fused_strided_operands(ml):
    """x, W and y as column slices of wider buffers (leading dimensions past
    K and N): the padding must be neither read into the result nor written."""
    case = W.random_linear(51, 190, 320, [384], [16, 64, 32], W.BF16)
    Wt = W.base_weight(51, case.N, case.K)
    log(f"linear_fused strided M={case.M} K={case.K}")
    table = table_for(case)
    ids = torch.from_numpy(case.ids).cuda()
    seg = ml.Segments(case.M, case.L)
    ml.lora_build_segments(ids, seg)
    xw = torch.full((case.M, case.K + 40), float("nan"), dtype=torch.bfloat16, device="cuda")
    xw[:, :case.K] = to_dev(case.x)
    Ww = torch.full((case.N, case.K + 24), float("nan"), dtype=torch.bfloat16, device="cuda")
    Ww[:, :case.K] = to_dev(Wt)
    yw = torch.full((case.M, case.N + 56), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = ml.Workspace.for_table(table, case.M)
    ml.lora_linear_fused(table, Ww[:, :case.K], xw[:, :case.K], seg, yw[:, :case.N], ws)
    torch.cuda.synchronize()
    full = to_f64(yw)
    assert np.all(full[:, case.N:] == 7.0), "padding columns of y were written"
    got = full[:, :case.N]
    ref = O.linear_with_base(case.x.values, Wt.values, case.ids, [a.values for a in case.A],
                             [b.values for b in case.B], case.ranks, case.slice_sizes)
    assert not np.isnan(got).any()
    assert float(np.max(np.abs(got - ref))) <= TOL_BF16 * float(np.max(np.abs(ref)))
    gamma = 2.0 * (case.K + 64) * 2.0 ** -24
    assert not (np.abs(got - ref) > 2.0 ** -8 * np.abs(ref) + gamma * abs_bound(case, Wt)).any()


def test_linear_fused_integer_exact(ml):
    """Inputs in {-1, 0, 1}: bit-identical to the oracle."""
    case = W.integer_linear(46, 150, 200, [96, 40], [16, 3, 9, 0], W.BF16)
    Wt = W.base_weight(46, case.N, case.K, integer=True)
    log(f"linear_fused integer M={case.M} K={case.K}")
    got = run_fused(ml, case, Wt)
    ref = O.linear_with_base(case.x.values, Wt.values, case.ids, [a.values for a in case.A],
                             [b.values for b in case.B], case.ranks, case.slice_sizes)
    assert np.max(np.abs(ref)) <= 256
    assert np.array_equal(got, ref)


def test_linear_fused_with_enable_mask(ml):
    """Disabled adapters (segment table built with a mask) give their tokens
    the base product only."""
    case = W.random_linear(47, 200, 512, [384], [16, 64, 32, 48, 16], W.BF16)
    enabled = np.array([1, 0, 1, 0, 1], np.int32)
    Wt = W.base_weight(47, case.N, case.K)
    log(f"linear_fused masked M={case.M} K={case.K}")
    got = run_fused(ml, case, Wt, enabled)
    ref = O.linear_with_base(case.x.values, Wt.values, case.ids, [a.values for a in case.A],
                             [b.values for b in case.B], case.ranks, case.slice_sizes, enabled)
    scale = float(np.max(np.abs(ref)))
    assert float(np.max(np.abs(got - ref))) <= TOL_BF16 * scale
    gamma = 2.0 * (case.K + 64) * 2.0 ** -24
    masked = W.LinearCase(case.name, case.dtype, case.M, case.K, case.slice_sizes, case.ranks,
                          O.mask_ids(case.ids, enabled, case.L).astype(np.int32), case.x,
                          case.A, case.B, case.y_base)
    bound = 2.0 ** -8 * np.abs(ref) + gamma * abs_bound(masked, Wt)
    assert not (np.abs(got - ref) > bound).any()


def test_linear_fused_prefill_full_size(ml):
    """Prefill at full size (M=2048, K=N=4096, 8 adapters of ranks
    16/32/64, Dirichlet segment lengths), in the launch configuration the
    benchmark times; every 16th row against the oracle."""
    case = W.prefill_bf16(0)
    Wt = W.base_weight(0, case.N, case.K)
    log(f"linear_fused prefill M={case.M} K={case.K} N={case.N}")
    got = run_fused(ml, case, Wt)
    rows = np.arange(0, case.M, 16)
    sub = W.LinearCase("prefill_rows", case.dtype, len(rows), case.K, case.slice_sizes,
                       case.ranks, case.ids[rows],
                       W.Tensor(case.x.dtype, case.x.values[rows], case.x.storage[rows]),
                       case.A, case.B,
                       W.Tensor(case.y_base.dtype, case.y_base.values[rows],
                                case.y_base.storage[rows]))
    ref = O.linear_with_base(sub.x.values, Wt.values, sub.ids, [a.values for a in case.A],
                             [b.values for b in case.B], case.ranks, case.slice_sizes)
    g = got[rows]
    scale = float(np.max(np.abs(ref)))
    assert float(np.max(np.abs(g - ref))) <= TOL_BF16 * scale
    gamma = 2.0 * (case.K + 64) * 2.0 ** -24
    bound = 2.0 ** -8 * np.abs(ref) + gamma * abs_bound(sub, Wt)
    assert not (np.abs(g - ref) > bound).any()
    assert not np.isnan(got).any()


def test_linear_fused_rejects_fp32(ml):
    case = W.tiny_fp32(0)
    table = table_for(case)
    ids = torch.from_numpy(case.ids).cuda()
    seg = ml.Segments(case.M, case.L)
    ml.lora_build_segments(ids, seg)
    Wt = torch.zeros((case.N, case.K), dtype=torch.float32, device="cuda")
    y = torch.zeros((case.M, case.N), dtype=torch.float32, device="cuda")
    ws = ml.Workspace.for_table(table, case.M)
    with pytest.raises(ml.LoraError):
        ml.lora_linear_fused(table, Wt, to_dev(case.x), seg, y, ws)
