"""The allocation-free decode entry point (lora_fused_decode_noalloc),
through the C ABI, against the workspace form it mirrors (lora_fused_decode)
on the same inputs.

Both run the same kernel with the same fixed summation order, so y and the
segment table must agree bit for bit; y is also held to the oracle's
tolerance.  Two calls in a row share the library's fixed array, the second
with a smaller batch and a smaller table (other K, N and adapters), and a
third repeats the first: nothing in the array needs clearing between calls.
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


def run_pair(ml, case):
    print(f"noalloc {case.name} M={case.M} K={case.K} N={case.N} L={case.L}", flush=True)
    table = table_for(case)
    ids = torch.from_numpy(case.ids).cuda()
    x = to_dev(case.x)
    y_ws, y_na = to_dev(case.y_base), to_dev(case.y_base)
    seg_ws, seg_na = ml.Segments(case.M, case.L), ml.Segments(case.M, case.L)
    ws = ml.Workspace.for_table(table, case.M)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ml.lora_fused_decode(table, ids, x, y_ws, ws, seg=seg_ws)
    ml.lora_fused_decode_noalloc(table, ids, x, y_na, seg=seg_na, error_word=err)
    torch.cuda.synchronize()
    assert ml.lora_read_device_error(ws.buf) == 0
    assert int(err.cpu()[0]) == 0
    assert torch.equal(y_na, y_ws)
    M = case.M
    for a, b in ((seg_na.sorted_idx[:M], seg_ws.sorted_idx[:M]),
                 (seg_na.seg_indptr, seg_ws.seg_indptr), (seg_na.req_to_lora, seg_ws.req_to_lora),
                 (seg_na.num_segments, seg_ws.num_segments), (seg_na.num_tiles, seg_ws.num_tiles)):
        assert torch.equal(a, b)
    ref = O.lora_linear(case.x.values, case.ids, [a.values for a in case.A],
                        [b.values for b in case.B], case.ranks, case.slice_sizes,
                        case.y_base.values)
    assert_close(to_f64(y_na), ref, case.dtype, case.y_base.values, case.name)
    keep = ~O.delta_rows(case.ids, case.ranks)
    assert np.array_equal(to_f64(y_na)[keep], case.y_base.values[keep])


def test_noalloc_matches_workspace_form(ml):
    run_pair(ml, W.decode_bf16(0))                                      # decode workload
    run_pair(ml, W.decode_bf16(5, M=9, K=1024, N=768, L=7))              # smaller, second
    run_pair(ml, W.decode_bf16(0))                                      # the first again


def test_noalloc_reports_bad_ids_into_error_word(ml):
    case = W.decode_bf16(6, M=12, K=512, N=256, L=4)
    case.ids[3] = 9                                       # outside [-1, L)
    table = table_for(case)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = to_dev(case.y_base)
    ml.lora_fused_decode_noalloc(table, torch.from_numpy(case.ids).cuda(), to_dev(case.x), y,
                                 error_word=err)
    torch.cuda.synchronize()
    assert int(err.cpu()[0]) == ml.LORA_DEVERR_BAD_ID
    ref = O.lora_linear(case.x.values, case.ids, [a.values for a in case.A],
                        [b.values for b in case.B], case.ranks, case.slice_sizes,
                        case.y_base.values)
    assert_close(to_f64(y), ref, case.dtype, case.y_base.values, "bad id")
