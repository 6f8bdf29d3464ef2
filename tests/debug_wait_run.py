"""Run by tests/test_gpu_debug_checks.py in a child process on the library
built with MLORA_DEBUG, with MLORA_DEBUG_WAIT_FAULT=1: every bounded wait on
an exchange slot then misses on purpose and gives up after a few polls.
Calls the single-launch decode and the two bf16 MoE delta calls once each
on small inputs and prints one JSON line: the workspace error word after
each call, and whether the call returned and synchronised normally.  The
kernels end normally; the outputs are not checked (their partial sums were
skipped)."""
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import adapter_lora_amd as ml  # noqa: E402
import workloads as W  # noqa: E402
from tests.helpers import table_for, to_dev  # noqa: E402

out = {"lib": os.path.basename(ml._abi.LIB_PATH),
       "fault": os.environ.get("MLORA_DEBUG_WAIT_FAULT")}

# single-launch decode (producers hand S to consumers through slots)
case = W.decode_bf16(3, M=8, K=512, N=256, L=3)
table = table_for(case)
seg = ml.Segments(case.M, case.L)
ws = ml.Workspace.for_table(table, case.M)
y = to_dev(case.y_base)
ml.lora_fused_decode(table, torch.from_numpy(case.ids).cuda(), to_dev(case.x), y, ws, seg=seg)
torch.cuda.synchronize()
out["decode_err"] = ml.lora_read_device_error(ws.buf)

# bf16 MoE deltas (one launch each: shrink part, then expand part polling)
mc = W.moe_case(2, M=24, H=128, I=64, E=3, topk=2, L=2, rank=16, block_size_m=16)
w = ml.MoeWeights(to_dev(mc.A_gu), to_dev(mc.B_gu), to_dev(mc.A_d), to_dev(mc.B_d),
                  torch.from_numpy(mc.adapter_enabled).cuda())
cap = ml.lora_moe_align_capacity(mc.M, mc.topk, mc.E, mc.block_size_m)
al = ml.MoeAlign(mc.L, cap, mc.block_size_m)
ml.lora_moe_align(torch.from_numpy(mc.topk_ids).cuda(), torch.from_numpy(mc.ids).cuda(),
                  torch.from_numpy(mc.adapter_enabled).cuda(), mc.E, al)
mws = ml.Workspace(ml.lora_moe_workspace_size(w, cap))
c1 = to_dev(mc.cache1)
ml.lora_moe_gate_up_add(w, to_dev(mc.x), mc.topk, al, c1, mws)
torch.cuda.synchronize()
out["moe_gate_up_err"] = ml.lora_read_device_error(mws.buf)
mws2 = ml.Workspace(ml.lora_moe_workspace_size(w, cap))
c2 = to_dev(W.make_tensor(np.ones((mc.M * mc.topk, mc.I), np.float32), W.BF16))
c3 = to_dev(mc.cache3)
ml.lora_moe_down_add(w, c2, mc.M, mc.topk, al, c3, mws2)
torch.cuda.synchronize()
out["moe_down_err"] = ml.lora_read_device_error(mws2.buf)
out["returned"] = True
print(json.dumps(out), flush=True)
