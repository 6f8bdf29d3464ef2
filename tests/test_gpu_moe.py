"""GPU parity: MoE-LoRA (alignment, gate/up delta, silu_and_mul, down delta,
top-k reduce) through the C ABI against the fp64 oracle.

Alignment is bit-exact.  Each float stage is checked in isolation on inputs
the oracle produced (rounded to the storage dtype by the test), and the
whole chain end to end."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import moe as O
from tests.helpers import assert_close, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ml():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import adapter_lora_amd
    return adapter_lora_amd


def log(msg):
    print(msg, flush=True)


def store(a64: np.ndarray, dtype: str) -> W.Tensor:
    """Round an oracle result to the storage dtype (test-side input prep)."""
    return W.make_tensor(a64.astype(np.float32), dtype)


def setup(ml, case):
    dev = lambda t: to_dev(t)
    w = ml.MoeWeights(dev(case.A_gu), dev(case.B_gu), dev(case.A_d), dev(case.B_d),
                      torch.from_numpy(case.adapter_enabled).cuda())
    cap = ml.lora_moe_align_capacity(case.M, case.topk, case.E, case.block_size_m)
    al = ml.MoeAlign(case.L, cap, case.block_size_m)
    ml.lora_moe_align(torch.from_numpy(case.topk_ids).cuda(), torch.from_numpy(case.ids).cuda(),
                          torch.from_numpy(case.adapter_enabled).cuda(), case.E, al)
    ws = ml.Workspace(ml.lora_moe_workspace_size(w, cap))
    return w, al, ws, cap


ALIGN_CASES = [
    ("cfg5", lambda: W.moe_case(0, H=8, I=8)),
    ("disabled_and_none", lambda: W.moe_case(1, M=97, H=8, I=8, L=4, p_none=0.3,
                                             enabled=[1, 0, 1, 1], block_size_m=16)),
    ("many_experts", lambda: W.moe_case(2, M=300, H=8, I=8, E=64, topk=4, L=3,
                                        block_size_m=32)),
    ("tiny", lambda: W.moe_case(3, M=3, H=8, I=8, E=2, topk=2, L=2, block_size_m=16)),
]


@pytest.mark.parametrize("name,mk", ALIGN_CASES, ids=[c[0] for c in ALIGN_CASES])
def test_align_bit_exact(ml, name, mk):
    case = mk()
    log(f"align {name}")
    cap = ml.lora_moe_align_capacity(case.M, case.topk, case.E, case.block_size_m)
    al = ml.MoeAlign(case.L, cap, case.block_size_m)
    ml.lora_moe_align(torch.from_numpy(case.topk_ids).cuda(), torch.from_numpy(case.ids).cuda(),
                          torch.from_numpy(case.adapter_enabled).cuda(), case.E, al)
    torch.cuda.synchronize()
    s, e, n = O.moe_align(case.topk_ids, case.ids, case.adapter_enabled, case.L, case.E,
                          case.block_size_m, cap)
    assert np.array_equal(al.sorted_token_ids.cpu().numpy().reshape(case.L, cap), s)
    assert np.array_equal(al.expert_ids.cpu().numpy().reshape(case.L, -1), e)
    assert np.array_equal(al.ntpp.cpu().numpy(), n)


MOE_CASES = [
    ("cfg5_moe_bf16", lambda: W.moe_case(0)),
    ("small_bf16_mixed", lambda: W.moe_case(4, M=70, H=520, I=264, E=6, topk=2, L=3, rank=32,
                                            block_size_m=16, p_none=0.2, enabled=[1, 1, 0])),
    ("small_fp32", lambda: W.moe_case(5, M=33, H=136, I=72, E=4, topk=2, L=2, rank=16,
                                      block_size_m=64, dtype=W.F32)),
    # gate/up output of 2I = 8208 columns: the wide (16 x 1024) expand tiles
    # with a ragged last tile of 16 columns; rank 64 (two K steps); blocks of
    # 32 rows with up to 2 row groups of 16
    ("wide_ragged_bf16", lambda: W.moe_case(7, M=150, H=264, I=4104, E=3, topk=2, L=2, rank=64,
                                            block_size_m=32)),
    # full 64-row blocks (two experts, one adapter): the wide expand's blocks
    # take two passes of 32 rows, the 64 x 256 tiles all their rows
    ("wide_full_blocks", lambda: W.moe_case(10, M=160, H=264, I=4104, E=2, topk=2, L=1, rank=16,
                                            block_size_m=64)),
    # the largest block size (256 rows): eight 32-row passes of the wide
    # expand, four 64-row passes of the narrow one, sixteen 16-row groups
    # in the shrink part; rank 32
    ("max_block_256", lambda: W.moe_case(11, M=300, H=264, I=4104, E=2, topk=2, L=1, rank=32,
                                         block_size_m=256)),
    # experts_shared_outer_loras: gate_up A and down B with one expert slot
    ("cfg5_shared_outer", lambda: W.moe_case(0, shared_outer=True)),
    ("shared_outer_fp32", lambda: W.moe_case(8, M=40, H=128, I=96, E=4, topk=2, L=3, rank=16,
                                             block_size_m=16, p_none=0.1, dtype=W.F32,
                                             shared_outer=True)),
    ("shared_outer_wide", lambda: W.moe_case(9, M=64, H=264, I=4104, E=6, topk=2, L=2, rank=32,
                                             block_size_m=16, shared_outer=True)),
]


@pytest.mark.parametrize("name,mk", MOE_CASES, ids=[c[0] for c in MOE_CASES])
def test_moe_stages_and_chain(ml, name, mk):
    case = mk()
    log(f"moe {name} M={case.M} H={case.H} I={case.I} E={case.E} L={case.L}")
    w, al, ws, cap = setup(ml, case)
    dt = case.dtype
    tid, ids, en = case.topk_ids, case.ids, case.adapter_enabled
    x = to_dev(case.x)
    # stage 1.5 on the seeded cache1
    c1 = to_dev(case.cache1)
    ml.lora_moe_gate_up_add(w, x, case.topk, al, c1, ws)
    torch.cuda.synchronize()
    ref1 = O.moe_gate_up_add(case.x.values, case.cache1.values, tid, ids, en, case.A_gu.values,
                             case.B_gu.values, case.shared_outer)
    got1 = to_f64(c1)
    assert_close(got1, ref1, dt, case.cache1.values, "gate_up")
    # stage 2 on the oracle's cache1, rounded to the storage dtype
    c1_in = store(ref1, dt)
    c2 = torch.empty(case.M * case.topk, case.I, dtype=c1.dtype, device="cuda")
    ml.lora_moe_silu_and_mul(to_dev(c1_in), c2)
    torch.cuda.synchronize()
    ref2 = O.silu_and_mul(c1_in.values)
    assert_close(to_f64(c2), ref2, dt, None, "silu_and_mul")
    # stage 3.5 on the oracle's cache2 and the seeded cache3
    c2_in = store(ref2, dt)
    c3 = to_dev(case.cache3)
    ml.lora_moe_down_add(w, to_dev(c2_in), case.M, case.topk, al, c3, ws)
    torch.cuda.synchronize()
    ref3 = O.moe_down_add(c2_in.values, case.cache3.values, tid, ids, en, case.A_d.values,
                          case.B_d.values, case.shared_outer)
    assert_close(to_f64(c3), ref3, dt, case.cache3.values, "down")
    # reduce on the oracle's cache3
    c3_in = store(ref3, dt)
    out = torch.empty(case.M, case.H, dtype=c1.dtype, device="cuda")
    wts = torch.from_numpy(case.topk_weights).cuda()
    ml.lora_moe_topk_reduce(to_dev(c3_in), wts, out)
    torch.cuda.synchronize()
    ref4 = O.topk_reduce(c3_in.values, case.topk_weights.astype(np.float64))
    assert_close(to_f64(out), ref4, dt, None, "topk_reduce")
    # whole chain on the device, against the oracle chain in fp64
    c1 = to_dev(case.cache1)
    c3 = to_dev(case.cache3)
    ml.lora_moe_gate_up_add(w, x, case.topk, al, c1, ws)
    ml.lora_moe_silu_and_mul(c1, c2)
    ml.lora_moe_down_add(w, c2, case.M, case.topk, al, c3, ws)
    ml.lora_moe_topk_reduce(c3, wts, out)
    torch.cuda.synchronize()
    r1 = ref1
    r3 = O.moe_down_add(O.silu_and_mul(r1), case.cache3.values, tid, ids, en, case.A_d.values,
                        case.B_d.values, case.shared_outer)
    r4 = O.topk_reduce(r3, case.topk_weights.astype(np.float64))
    assert_close(to_f64(out), r4, dt, None, "chain")
    assert ml.lora_read_device_error(ws.buf) == 0


def test_disabled_adapters_leave_caches(ml):
    case = W.moe_case(6, M=40, H=256, I=128, E=4, topk=2, L=2, enabled=[0, 0])
    w, al, ws, cap = setup(ml, case)
    c1 = to_dev(case.cache1)
    c3 = to_dev(case.cache3)
    c2 = to_dev(store(np.random.default_rng(0).standard_normal((case.M * 2, case.I)), W.BF16))
    ml.lora_moe_gate_up_add(w, to_dev(case.x), 2, al, c1, ws)
    ml.lora_moe_down_add(w, c2, case.M, 2, al, c3, ws)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(c1), case.cache1.values)
    assert np.array_equal(to_f64(c3), case.cache3.values)


# The whole chain on the device with exact arithmetic (workloads.
# integer_moe_case): gate/up delta, down delta and top-k reduce are bit-exact
# with the oracle's single rounding; the activation is checked to the
# tolerance and its device output is what the oracle's down stage reads, so
# every later stage is compared bit for bit.  Cases: the narrow expand, the
# wide (16 x 1024) expand with a ragged last tile (rank 32: the one-step
# build; rank 64: the two-step build of both expands), shared outer matrices
# with a disabled adapter.
INT_MOE_CASES = [
    ("narrow", lambda: W.integer_moe_case(1, M=90, H=264, I=64)),
    ("wide_ragged", lambda: W.integer_moe_case(2, M=70, H=136, I=4104, rank=32,
                                               block_size_m=32)),
    ("wide_rank64", lambda: W.integer_moe_case(4, M=60, H=136, I=4104, rank=64,
                                               block_size_m=32)),
    ("wide_full_blocks", lambda: W.integer_moe_case(5, M=120, H=136, I=4104, E=2, L=1,
                                                    block_size_m=64, p_none=0.0)),
    ("shared_outer_masked", lambda: W.integer_moe_case(3, M=50, H=264, I=136, shared_outer=True,
                                                       enabled=[1, 0, 1])),
]


@pytest.mark.parametrize("name,mk", INT_MOE_CASES, ids=[c[0] for c in INT_MOE_CASES])
def test_moe_chain_integer_bit_exact(ml, name, mk):
    case = mk()
    log(f"moe integer chain {name} M={case.M} H={case.H} I={case.I} E={case.E} L={case.L}")
    w, al, ws, cap = setup(ml, case)
    tid, ids, en = case.topk_ids, case.ids, case.adapter_enabled
    so = case.shared_outer
    bf = lambda a: W.make_tensor(a.astype(np.float32), W.BF16).values   # one rounding
    c1 = to_dev(case.cache1)
    c3 = to_dev(case.cache3)
    c2 = torch.empty(case.M * case.topk, case.I, dtype=c1.dtype, device="cuda")
    out = torch.empty(case.M, case.H, dtype=c1.dtype, device="cuda")
    wts = torch.from_numpy(case.topk_weights).cuda()
    ml.lora_moe_gate_up_add(w, to_dev(case.x), case.topk, al, c1, ws)
    ml.lora_moe_silu_and_mul(c1, c2)
    ml.lora_moe_down_add(w, c2, case.M, case.topk, al, c3, ws)
    ml.lora_moe_topk_reduce(c3, wts, out)
    torch.cuda.synchronize()
    r1 = O.moe_gate_up_add(case.x.values, case.cache1.values, tid, ids, en, case.A_gu.values,
                           case.B_gu.values, so)
    assert np.array_equal(to_f64(c1), bf(r1)), "gate/up"
    got2 = to_f64(c2)
    assert_close(got2, O.silu_and_mul(r1), W.BF16, None, "silu_and_mul")
    r3 = O.moe_down_add(got2, case.cache3.values, tid, ids, en, case.A_d.values, case.B_d.values,
                        so)
    got3 = to_f64(c3)
    assert np.array_equal(got3, bf(r3)), "down"
    r4 = O.topk_reduce(got3, case.topk_weights.astype(np.float64))
    assert np.array_equal(to_f64(out), bf(r4)), "top-k reduce"
    assert ml.lora_read_device_error(ws.buf) == 0
