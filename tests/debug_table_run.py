"""Run by tests/test_gpu_debug_checks.py in a child process whose MLORA_LIB
names the library built with MLORA_DEBUG (a process loads one library).
Hands the table-form calls valid and deliberately corrupted segment tables
and prints one JSON line of findings.  Every corrupted entry points into
padding rows allocated past the batch, so even an unchecked access would
stay inside this script's own buffers.  Integer inputs (workloads.
integer_linear) make every expected value exact."""
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import adapter_lora_amd as ml  # noqa: E402
import workloads as W  # noqa: E402
from oracle import lora as O  # noqa: E402
from tests.helpers import table_for, to_dev, to_f64  # noqa: E402

PAD = 64
out = {"lib": os.path.basename(ml._abi.LIB_PATH)}


def padded(t):
    """Device copy of a [M, C] tensor inside a [M + PAD, C] buffer whose
    padding rows hold 7.0; returns (view of the first M rows, whole buffer)."""
    d = to_dev(t)
    full = torch.full((d.shape[0] + PAD, d.shape[1]), 7.0, dtype=d.dtype, device="cuda")
    full[: d.shape[0]] = d
    return full[: d.shape[0]], full


def bf(a):
    return W.make_tensor(a.astype(np.float32), W.BF16).values


def expected(case, skip_tokens, base=None):
    ids = case.ids.copy()
    ids[list(skip_tokens)] = -1
    A, B = [a.values for a in case.A], [b.values for b in case.B]
    if base is None:
        return bf(O.lora_linear(case.x.values, ids, A, B, case.ranks, case.slice_sizes,
                                case.y_base.values))
    return bf(O.linear_with_base(case.x.values, base.values, ids, A, B, case.ranks,
                                 case.slice_sizes))


def run_table_form(case, corrupt):
    table = table_for(case)
    seg = ml.Segments(case.M, case.L)
    ml.lora_build_segments(torch.from_numpy(case.ids).cuda(), seg)
    x, x_full = padded(case.x)
    y, y_full = padded(case.y_base)
    skip = corrupt(seg)
    ws = ml.Workspace.for_table(table, case.M)
    ml.lora_shrink_expand_add(table, x, seg, y, ws)
    torch.cuda.synchronize()
    err = ml.lora_read_device_error(ws.buf)
    pad_ok = bool(torch.all(y_full[case.M:].float() == 7.0).item())
    exact = bool(np.array_equal(to_f64(y), expected(case, skip)))
    return {"err": err, "padding_untouched": pad_ok, "rows_exact": exact, "skipped": len(skip)}


def tile_tokens(seg, t):
    n = int(seg.tile_info.view(-1, 4)[t, 3].item())
    return [int(v) for v in seg.tile_rows.view(-1, 64)[t, :n].cpu()]


def seg_tokens(seg, s):
    ip = seg.seg_indptr.cpu().numpy()
    return [int(v) for v in seg.sorted_idx[ip[s]:ip[s + 1]].cpu()]


# tile path (M > 64): shrink, reduce and expand over the tile schedule
big = W.integer_linear(61, 300, 520, [264, 136], [16, 32, 64, 48], W.BF16)
out["tiles_valid"] = run_table_form(big, lambda seg: [])


def corrupt_tiles(seg):
    skip = tile_tokens(seg, 0) + tile_tokens(seg, 1)
    rows = seg.tile_rows.view(-1, 64)
    rows[0, 3] = big.M + 5                               # a token past the batch
    info = seg.tile_info.view(-1, 4)
    info[1, 1] = big.L + 2                               # a slot past the table
    return skip


out["tiles_corrupt"] = run_table_form(big, corrupt_tiles)

# single-launch decode on a table (M <= 64): the segment view
small = W.integer_linear(62, 40, 1032, [520], [16, 64, 32, 16, 48], W.BF16)
out["decode_valid"] = run_table_form(small, lambda seg: [])


def corrupt_segment(seg):
    skip = seg_tokens(seg, 1)
    ip = seg.seg_indptr.cpu().numpy()
    seg.sorted_idx[int(ip[1])] = small.M + 3
    return skip


out["decode_corrupt"] = run_table_form(small, corrupt_segment)

# fused base GEMM: the sorted token list of its rows
fc = W.integer_linear(63, 200, 256, [264], [16, 64, 32], W.BF16)
Wt = W.base_weight(63, fc.N, fc.K, integer=True)
table = table_for(fc)
seg = ml.Segments(fc.M, fc.L)
ml.lora_build_segments(torch.from_numpy(fc.ids).cuda(), seg)
pos = int(seg.seg_indptr[1].item()) + 2                  # a row inside segment 1
lost = int(seg.sorted_idx[pos].item())
seg.sorted_idx[pos] = fc.M + 7
x, _ = padded(fc.x)
y = torch.zeros(fc.M, fc.N, dtype=torch.bfloat16, device="cuda")
y_full = torch.full((fc.M + PAD, fc.N), 7.0, dtype=torch.bfloat16, device="cuda")
y_full[: fc.M] = y
y = y_full[: fc.M]
ws = ml.Workspace.for_table(table, fc.M)
ml.lora_linear_fused(table, to_dev(Wt), x, seg, y, ws)
torch.cuda.synchronize()
got = to_f64(y)
ref = expected(fc, [], base=Wt)
keep = np.arange(fc.M) != lost
out["gemm_corrupt"] = {
    "err": ml.lora_read_device_error(ws.buf),
    "padding_untouched": bool(torch.all(y_full[fc.M:].float() == 7.0).item()),
    "rows_exact": bool(np.array_equal(got[keep], ref[keep])),
    "lost_row_unwritten": bool(np.all(got[lost] == 0.0)),
}
print(json.dumps(out), flush=True)
