"""HIP graph capture of the dense path (segment table + fused call).

The kernels allocate nothing and clear their own exchange state (slots,
counters), so a captured step replays correctly.  Each replay is preceded by
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
