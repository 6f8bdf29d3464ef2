"""HIP graph capture of the dense path (segment table + fused call, and the
single-launch decode with an adapter enable mask).

The kernels allocate nothing and keep their exchange state ready on the
device (slots tagged with an epoch that the last workgroup of each launch
advances), so a captured step replays correctly.  Each replay is preceded by
eager work on the captured buffers (new ids and x, y reset to its base) and
followed by a synchronisation, and every replay must equal the eager result
bit for bit (the kernels sum in a fixed order).
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.helpers import table_for, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ml():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import adapter_lora_amd
    return adapter_lora_amd


CASES = [
    ("decode", lambda s: W.decode_bf16(s, M=32, K=2048, N=1024, L=9)),
    ("prefill", lambda s: W.prefill_bf16(s, M=200, K=1024, N=520, ranks=(16, 64, 32, 0))),
]


@pytest.mark.parametrize("name,mk", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager(ml, name, mk):
    print(f"graph {name}", flush=True)
    cases = [mk(s) for s in range(3)]           # same shapes, different ids / x / y
    base = cases[0]
    table = table_for(base)
    M, L = base.M, base.L
    ids = torch.from_numpy(base.ids.copy()).cuda()
    x = to_dev(base.x)
    y = to_dev(base.y_base)
    seg = ml.Segments(M, L)
    ws = ml.Workspace.for_table(table, M)

    def step():
        ml.lora_build_segments(ids, seg)
        ml.lora_shrink_expand_add(table, x, seg, y, ws)

    # eager results for every input set
    eager = []
    for c in cases:
        ids.copy_(torch.from_numpy(c.ids))
        x.copy_(to_dev(c.x))
        y.copy_(to_dev(c.y_base))
        step()
        torch.cuda.synchronize()
        eager.append(y.clone())

    # capture on a side stream after a warm-up there
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(6):
        c = cases[rep % 3]
        ids.copy_(torch.from_numpy(c.ids))      # eager work between replays
        x.copy_(to_dev(c.x))
        y.copy_(to_dev(c.y_base))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager[rep % 3]), f"replay {rep} differs from the eager result"
    assert ml.lora_read_device_error(ws.buf) == 0


def test_graph_fused_decode_with_mask(ml):
    """Capture the single-launch decode once; each replay runs on new ids, x,
    y and a new adapter enable mask written into the captured buffers, and
    must equal the eager call bit for bit (segment table included)."""
    print("graph fused decode + mask", flush=True)
    cases = [W.decode_bf16(s, M=32, K=2048, N=1024, L=9) for s in range(3)]
    masks = [np.ones(9, np.int32), np.array([1, 0, 1, 1, 0, 1, 0, 1, 1], np.int32),
             np.zeros(9, np.int32)]
    base = cases[0]
    table = table_for(base)
    M, L = base.M, base.L
    ids = torch.from_numpy(base.ids.copy()).cuda()
    en = torch.from_numpy(masks[0].copy()).cuda()
    x = to_dev(base.x)
    y = to_dev(base.y_base)
    seg = ml.Segments(M, L)
    ws = ml.Workspace.for_table(table, M)

    def step():
        ml.lora_fused_decode(table, ids, x, y, ws, seg=seg, adapter_enabled=en)

    def load(i):
        c = cases[i % 3]
        ids.copy_(torch.from_numpy(c.ids))
        en.copy_(torch.from_numpy(masks[i % 3]))
        x.copy_(to_dev(c.x))
        y.copy_(to_dev(c.y_base))

    eager = []
    for i in range(3):
        load(i)
        step()
        torch.cuda.synchronize()
        eager.append((y.clone(), seg.sorted_idx.clone(), seg.seg_indptr.clone(),
                      seg.tile_rows.clone()))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(6):
        load(rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e = eager[rep % 3]
        assert torch.equal(y, e[0]), f"replay {rep}: y differs from the eager result"
        assert torch.equal(seg.sorted_idx, e[1]) and torch.equal(seg.seg_indptr, e[2])
        assert torch.equal(seg.tile_rows, e[3])
    assert ml.lora_read_device_error(ws.buf) == 0
