"""Benchmark of the dynamic multi-LoRA hot path on one MI355X.

Headline workload: decode, bf16, M=32 tokens (one per sequence), K=N=4096,
20 adapters with ranks drawn from {16,32,64}, 10% of tokens without an
adapter.  One step = lora_fused_decode on one batch: a single kernel launch
that groups the tokens by adapter, writes the batch's segment table and tile
schedule, and adds every token's delta.  The same work as two launches
(lora_build_segments, then lora_shrink_expand_add on the built table, the
form later layers of a model use) is reported beside it.  Inputs are
synthetic and seeded (workloads.py).

Protocol:
  * R copies of every input (packed weight table, x, y, ids, segment table)
    sized so that R copies exceed twice the 256 MB Infinity Cache; step i uses
    copy i % R, so each step reads its weights from HBM (cold MALL);
  * W warmup steps, then K timed steps between two device synchronisations;
    ms_per_step is the event time of the K steps on the launching stream
    (launch gaps included);
  * the dominant kernel is then launched K times back to back on the same
    rotation, bracketed by one HIP event pair on its stream; elapsed / K is
    its mean duration, and algorithmic bytes per launch / that duration gives
    the roofline figure against 8 TB/s;
  * a hand-written streaming kernel (adapter_lora_amd/csrc/stream_copy.hip)
    moving the decode step's byte mix (its reads, then its y writes) is timed
    the same way, at the decode launch's own grid and at the best grid of a
    sweep, as the practical ceiling; the same kernel copying 128 MB is the
    calibration kernel for the FETCH_SIZE / WRITE_SIZE counter runs;
  * HBM traffic per launch comes from those counter runs, kept as a summary
    under profiles/ with a hash of the kernel's sources; it is reported only
    while the sources still match the hash;
  * the same step is also captured as a HIP graph (one per input copy) and
    replayed, reported under "graph_replay" as context;
  * the oracle (fp64 CPU, one BLAS thread) is timed on the host on a bounded
    sample of each workload, median of three runs.
Other configurations (prefill, stacked QKV / gate-up, MoE, and the
LM-head and embedding LoRA decode cases: 32 tokens, 32000-token vocabulary,
4096 hidden) are measured the same way and reported under "extra" as
context; the headline line is the decode workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
METRIC = "LoRA-delta tokens/s; decode HBM GB/s and prefill MFMA TFLOP/s vs peak"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--only", default="",
                   help="comma list: decode,prefill,qkv,gate_up,moe,moe_shared,lm_head,embedding,"
                        "linear_fused")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    return p.parse_args()


# ----------------------------------------------------------------------------- helpers
def dev_tensor(t):
    import torch
    import workloads as W
    if t.dtype == W.BF16:
        return torch.from_numpy(t.storage.astype(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(t.storage).cuda()


def linear_bytes_flops(case):
    """Algorithmic bytes and FLOPs of one pass: each touched adapter's A and B
    read once, x rows of tokens with an adapter read once, their y rows read
    and written once (element size 2 for bf16)."""
    es = 2 if case.dtype == "bf16" else 4
    touched = sorted(set(int(i) for i in case.ids if 0 <= i < case.L and case.ranks[i] > 0))
    m_valid = int(sum(1 for i in case.ids if 0 <= i < case.L and case.ranks[i] > 0))
    w_bytes = sum(case.ranks[i] * (case.n_slices * case.K + case.N) * es for i in touched)
    act = m_valid * case.K * es + 2 * m_valid * case.N * es
    flops = sum(2 * case.ranks[int(i)] * (case.n_slices * case.K + case.N)
                for i in case.ids if 0 <= i < case.L and case.ranks[int(i)] > 0)
    return w_bytes + act, flops, m_valid, len(touched)


def run_timed(step, steps, warmup):
    """W untimed steps, then K steps between two synchronisations; returns
    (event ms per step on the launching stream, host wall ms per step)."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        step(warmup + i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return t0.elapsed_time(t1) / steps, wall / steps * 1e3


def back_to_back(launch, n):
    """Mean duration (ms) of `launch(i)` over n back-to-back launches bracketed
    by one event pair on the current stream (the stream the kernels use)."""
    import torch
    for i in range(min(n, 8)):
        launch(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(n):
        launch(i)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / n


_STREAM = None


def stream_lib():
    """The streaming reference kernel's library (built beside libmlora.so)."""
    global _STREAM
    if _STREAM is None:
        import ctypes
        path = os.path.join(ROOT, "adapter_lora_amd", "libmlora_stream.so")
        if not os.path.exists(path):
            raise SystemExit(f"{path} not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.mlora_stream.restype = ctypes.c_int
        lib.mlora_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        _STREAM = lib
    return _STREAM


def stream_time(rd_bytes, wr_bytes, n, grid=0, unroll=4, rotation=None):
    """Mean duration (ms) of the streaming kernel reading rd_bytes and writing
    wr_bytes, over n back-to-back launches on buffers rotated so that the
    reads miss the Infinity Cache."""
    import torch
    import adapter_lora_amd as ml
    lib = stream_lib()
    rd = (rd_bytes + 15) // 16 * 16
    wr = min((wr_bytes + 15) // 16 * 16, rd)
    R = rotation or max(2, min(64, int(np.ceil(2 * MALL_BYTES / rd))))
    src = [torch.randint(0, 255, (rd,), dtype=torch.uint8, device="cuda") for _ in range(R)]
    dst = [torch.empty(max(wr, 16), dtype=torch.uint8, device="cuda") for _ in range(R)]
    sh = ml.stream_handle()

    def launch(i):
        rc = lib.mlora_stream(src[i % R].data_ptr(), rd, dst[i % R].data_ptr(), wr, grid, unroll, sh)
        if rc != 0:
            raise RuntimeError(f"mlora_stream failed ({rc})")
    ms = back_to_back(launch, n)
    del src, dst
    return ms, R


def stream_ceiling(rd_bytes, wr_bytes, n, launch_grid):
    """The streaming kernel on the given byte mix: at `launch_grid` workgroups
    of 256 threads (unroll chosen so that one pass covers the reads; the
    better of two runs, one before and one after the sweep, since the first
    timed launches of a process can run on a cold clock), and the best of a
    sweep over loads in flight per thread (one pass each) and grid-stride
    launches of 256..2048 workgroups."""
    words = (rd_bytes + 15) // 16
    u_at = 1
    while u_at < 16 and launch_grid * 256 * u_at < words:
        u_at *= 2
    ms_at, R = stream_time(rd_bytes, wr_bytes, n, launch_grid, u_at)
    sweep = []
    for u in (1, 2, 4, 8, 16):
        sweep.append((stream_time(rd_bytes, wr_bytes, n, 0, u, R)[0], 0, u))
    for g in (256, 512, 1024, 2048):
        sweep.append((stream_time(rd_bytes, wr_bytes, n, g, 4, R)[0], g, 4))
    ms_at = min(ms_at, stream_time(rd_bytes, wr_bytes, n, launch_grid, u_at, R)[0])
    best = min(sweep)
    tot = rd_bytes + wr_bytes
    res = {"kernel": "k_stream (hand-written, stream_copy.hip)", "read_bytes": rd_bytes,
           "write_bytes": wr_bytes, "rotation": R,
           "at_launch_grid": {"workgroups": launch_grid, "unroll": u_at, "ms": ms_at,
                              "gbs": tot / (ms_at * 1e-3) / 1e9},
           "best": {"workgroups": best[1] or int(-(-words // (256 * best[2]))),
                    "unroll": best[2], "ms": best[0], "gbs": tot / (best[0] * 1e-3) / 1e9},
           "sweep_ms": {f"{'auto' if g == 0 else g}x{u}": round(m, 5) for m, g, u in sweep}}
    return res


def copy_calibration(n=20):
    """The streaming kernel copying 128 MB (read) into 128 MB (write): the
    kernel whose FETCH_SIZE / WRITE_SIZE readings calibrate the counter runs."""
    ms, R = stream_time(128 << 20, 128 << 20, n, 0, 4, rotation=2)
    return {"bytes": 256 << 20, "ms": ms, "gbs": (256 << 20) / (ms * 1e-3) / 1e9,
            "kernel": "k_stream copy, 128 MB read + 128 MB written"}


def decode_launch_grid(case):
    """Workgroups of the single-launch decode for this case: producers
    (slots x 16-row A blocks x 1024-wide K chunks), consumers (slots x
    256-column tiles), and the workgroup that writes the segment table."""
    s_max = min(case.L, case.M)
    r_max = max(16, max(-(-r // 16) * 16 for r in case.ranks))
    C = -(-case.K // 1024)
    tiles = sum(-(-n // 256) for n in case.slice_sizes)
    return s_max * (case.n_slices * r_max // 16) * C + s_max * tiles + 1


def strip_comments(text):
    """C/C++ source without its comments and blank lines (string literals in
    these sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def source_hash(files, read=None):
    """Hash of the code (comments stripped) of `files`, so that an edit to
    comments alone keeps a counter summary valid.  `read(path)` returns a
    file's text (default: the working tree)."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        if read is None:
            with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
                text = fh.read()
        else:
            text = read(f)
        h.update(strip_comments(text).encode())
    return h.hexdigest()[:16]


DECODE_SOURCES = ["adapter_lora_amd/csrc/decode.hip", "adapter_lora_amd/csrc/common.hpp",
                  "adapter_lora_amd/csrc/wave_groups.hpp", "adapter_lora_amd/csrc/kernels.hpp",
                  "include/mlora.h"]
TRAFFIC_SUMMARY = "profiles/decode_fused_traffic.md"


def measured_traffic():
    """HBM bytes per launch of the fused decode kernel from the committed
    counter summary, or None when it is absent or the sources changed since."""
    path = os.path.join(ROOT, TRAFFIC_SUMMARY)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    try:
        if vals["source_hash"] != source_hash(DECODE_SOURCES):
            return None
        return {"fetch_bytes": float(vals["fetch_bytes_per_launch"]),
                "write_bytes": float(vals["write_bytes_per_launch"]),
                "total_bytes": float(vals["traffic_bytes_per_launch"]),
                "calibration": vals.get("calibration", "")}
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------- dense
def bench_linear(case, steps, warmup, fused_kernel_name, single_launch=False):
    import torch
    import adapter_lora_amd as ml
    nbytes, flops, m_valid, touched = linear_bytes_flops(case)
    per_copy = nbytes + case.M * case.K * 2
    R = max(2, int(np.ceil(2 * MALL_BYTES / max(per_copy, 1))))
    A = [dev_tensor(a) for a in case.A]
    B = [dev_tensor(b) for b in case.B]
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    copies = []
    for r in range(R):
        table = ml.LoraTable(A, B, case.ranks, case.slice_sizes, case.K, dt)
        ids = torch.from_numpy(case.ids).cuda()
        seg = ml.Segments(case.M, case.L)
        copies.append((table, ids, seg, dev_tensor(case.x), dev_tensor(case.y_base)))
    ws = ml.Workspace.for_table(copies[0][0], case.M)
    del A, B
    torch.cuda.synchronize()

    def two_launch(i):
        table, ids, seg, x, y = copies[i % R]
        ml.lora_build_segments(ids, seg)
        ml.lora_shrink_expand_add(table, x, seg, y, ws)

    def table_kernel(i):
        table, ids, seg, x, y = copies[i % R]
        ml.lora_shrink_expand_add(table, x, seg, y, ws)

    def fused(i):
        table, ids, seg, x, y = copies[i % R]
        ml.lora_fused_decode(table, ids, x, y, ws, seg=seg)

    step = fused if single_launch else two_launch
    kernel = fused if single_launch else table_kernel
    ms_step, ms_wall = run_timed(step, steps, warmup)
    ms_kernel = back_to_back(kernel, steps)
    extra = {}
    if single_launch:
        # context: the two-launch form, and its product kernel alone on a
        # prebuilt table (the form every later layer of a batch runs)
        extra["ms_per_step_two_launch"], _ = run_timed(two_launch, steps, warmup)
        extra["ms_table_kernel_b2b"] = back_to_back(table_kernel, steps)
    # the same step captured as one HIP graph per input copy, replayed in turn
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(r)
        graphs.append(g)
    torch.cuda.synchronize()
    ms_graph, _ = run_timed(lambda i: graphs[i % R].replay(), steps, warmup)
    assert ml.lora_read_device_error(ws.buf) == 0, "device error during the bench"
    res = {
        "ms_per_step": ms_step, "ms_kernel_b2b": ms_kernel, "ms_wall_host": ms_wall,
        "ms_per_step_graph": ms_graph,
        "tokens_per_s": m_valid / (ms_step * 1e-3), "m_valid": m_valid, "M": case.M,
        "adapters_touched": touched, "alg_bytes": nbytes, "alg_flops": flops,
        "kernel": fused_kernel_name, "rotation_copies": R,
        "hbm_gbs": nbytes / (ms_kernel * 1e-3) / 1e9,
        "tflops": flops / (ms_kernel * 1e-3) / 1e12,
        **extra,
    }
    res["hbm_frac"] = res["hbm_gbs"] / HBM_PEAK_GBS
    res["mfma_frac"] = res["tflops"] / BF16_MFMA_PEAK_TFLOPS
    del copies, graphs
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- base + delta
def bench_linear_fused(case, steps, warmup):
    """The base layer fused with its delta on the prefill batch: step =
    lora_linear_fused (lora_shrink, then one MFMA product whose epilogue adds
    S B^T), segment table prebuilt.  FLOPs: 2 M K N for the base plus the
    delta's.  Context: the unfused form, torch.matmul (hipBLASLt) for the base
    product followed by lora_shrink_expand_add, and torch.matmul alone."""
    import torch
    import adapter_lora_amd as ml
    import workloads as W
    _, dflops, m_valid, touched = linear_bytes_flops(case)
    flops = 2.0 * case.M * case.K * case.N + dflops
    Wt = dev_tensor(W.base_weight(0, case.N, case.K))
    per_copy = (case.N * case.K + case.M * case.K + case.M * case.N) * 2
    R = max(2, int(np.ceil(2 * MALL_BYTES / per_copy)))
    A = [dev_tensor(a) for a in case.A]
    B = [dev_tensor(b) for b in case.B]
    table = ml.LoraTable(A, B, case.ranks, case.slice_sizes, case.K, torch.bfloat16)
    ids = torch.from_numpy(case.ids).cuda()
    seg = ml.Segments(case.M, case.L)
    ml.lora_build_segments(ids, seg)
    copies = [(Wt if r == 0 else Wt.clone(), dev_tensor(case.x),
               torch.empty((case.M, case.N), dtype=torch.bfloat16, device="cuda"))
              for r in range(R)]
    ws = ml.Workspace.for_table(table, case.M)
    torch.cuda.synchronize()

    def fused(i):
        w, x, y = copies[i % R]
        ml.lora_linear_fused(table, w, x, seg, y, ws)

    def unfused(i):
        w, x, y = copies[i % R]
        torch.matmul(x, w.t(), out=y)
        ml.lora_shrink_expand_add(table, x, seg, y, ws)

    def base_only(i):
        w, x, y = copies[i % R]
        torch.matmul(x, w.t(), out=y)

    ms_step, _ = run_timed(fused, steps, warmup)
    ms_unfused, _ = run_timed(unfused, steps, warmup)
    ms_base, _ = run_timed(base_only, steps, warmup)
    res = {
        "ms_per_step": ms_step, "ms_unfused_matmul_plus_delta": ms_unfused,
        "ms_matmul_base_only": ms_base, "M": case.M, "m_valid": m_valid,
        "adapters_touched": touched, "alg_flops": flops, "rotation_copies": R,
        "kernel": "k_shrink_dense + k_reduce_partials + k_gemm_lora",
        "tflops": flops / (ms_step * 1e-3) / 1e12,
        "tokens_per_s": case.M / (ms_step * 1e-3),
    }
    res["mfma_frac"] = res["tflops"] / BF16_MFMA_PEAK_TFLOPS
    del copies
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- embedding
def bench_embedding(case, steps, warmup):
    """Embedding LoRA on a decode batch: step = lora_embedding_decode, one
    launch (grouping, segment table, lookup and expand); the three-launch form
    (lora_build_segments + lora_embedding_shrink + lora_expand_add) is
    reported beside it.  Algorithmic bytes: the
    looked-up A rows and the B table of every touched adapter, the ids and
    token ids, and the y rows of tokens with a delta read and written."""
    import torch
    import adapter_lora_amd as ml
    es = 2 if case.dtype == "bf16" else 4
    valid = [m for m in range(case.M) if 0 <= case.ids[m] < case.L
             and case.ranks[case.ids[m]] > 0 and 0 <= case.tokens[m] < case.vocab]
    touched = sorted(set(int(case.ids[m]) for m in valid))
    b_bytes = sum(case.ranks[i] * case.emb * es for i in touched)
    a_bytes = sum(case.ranks[int(case.ids[m])] * es for m in valid)
    nbytes = b_bytes + a_bytes + 8 * case.M + 2 * len(valid) * case.emb * es
    R = max(2, min(12, int(np.ceil(2 * MALL_BYTES / max(b_bytes, 1)))))
    A = [dev_tensor(a) for a in case.A]
    B = [dev_tensor(b) for b in case.B]
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    copies = []
    for _ in range(R):
        table = ml.LoraTable(A, B, case.ranks, [case.emb], case.vocab, dt, embedding=True)
        seg = ml.Segments(case.M, case.L)
        S = torch.zeros(case.M, table.cols, dtype=torch.float32, device="cuda")
        copies.append((table, seg, S, dev_tensor(case.y_base)))
    del A, B
    ids = torch.from_numpy(case.ids).cuda()
    toks = torch.from_numpy(case.tokens).cuda()
    torch.cuda.synchronize()

    def three_launch(i):
        table, seg, S, y = copies[i % R]
        ml.lora_build_segments(ids, seg)
        ml.lora_embedding_shrink(table, toks, seg, S)
        ml.lora_expand_add(table, S, seg, y)

    def step(i):
        table, seg, S, y = copies[i % R]
        ml.lora_embedding_decode(table, ids, toks, y, seg=seg)

    ms_step, ms_wall = run_timed(step, steps, warmup)
    ms_kernels = back_to_back(step, steps)
    ms_three, _ = run_timed(three_launch, steps, warmup)
    res = {"ms_per_step": ms_step, "ms_kernel_b2b": ms_kernels, "ms_wall_host": ms_wall,
           "ms_per_step_three_launch": ms_three,
           "tokens_per_s": len(valid) / (ms_step * 1e-3), "m_valid": len(valid), "M": case.M,
           "adapters_touched": len(touched), "alg_bytes": nbytes, "rotation_copies": R,
           "hbm_gbs": nbytes / (ms_kernels * 1e-3) / 1e9,
           "kernel": "k_decode_fused<uint16_t> (lookup consumers)"}
    res["hbm_frac"] = res["hbm_gbs"] / HBM_PEAK_GBS
    del copies
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- MoE
def bench_moe(case, steps, warmup):
    import torch
    import adapter_lora_amd as ml
    es = 2
    P = case.M * case.topk
    pairs = [(int(case.ids[m]), int(case.topk_ids[m, k])) for m in range(case.M)
             for k in range(case.topk) if case.ids[m] >= 0 and case.adapter_enabled[case.ids[m]]]
    buckets = set(pairs)
    r, H, I = case.rank, case.H, case.I
    if case.shared_outer:
        # gate_up A and down B once per adapter; gate_up B and down A per bucket
        adapters = set(l for l, _ in buckets)
        w_bytes = len(buckets) * r * (2 * I + I) * es + len(adapters) * r * (H + H) * es
    else:
        w_bytes = len(buckets) * r * (H + 2 * I + I + H) * es
    act = len(pairs) * (H + 2 * 2 * I + I + 2 * H) * es
    nbytes = w_bytes + act
    flops = len(pairs) * 2 * r * (H + 2 * I + I + H)
    R = max(2, int(np.ceil(2 * MALL_BYTES / (w_bytes + act))))
    R = min(R, 12)
    en = torch.from_numpy(case.adapter_enabled).cuda()
    base = [dev_tensor(t) for t in (case.A_gu, case.B_gu, case.A_d, case.B_d)]
    copies = []
    for _ in range(R):
        w = ml.MoeWeights(*[t.clone() for t in base], en)
        copies.append((w, dev_tensor(case.x), dev_tensor(case.cache1), dev_tensor(case.cache3)))
    cap = ml.lora_moe_align_capacity(case.M, case.topk, case.E, case.block_size_m)
    al = ml.MoeAlign(case.L, cap, case.block_size_m)
    tid = torch.from_numpy(case.topk_ids).cuda()
    ids = torch.from_numpy(case.ids).cuda()
    wts = torch.from_numpy(case.topk_weights).cuda()
    c2 = torch.empty(P, I, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(case.M, H, dtype=torch.bfloat16, device="cuda")
    ws = ml.Workspace(ml.lora_moe_workspace_size(copies[0][0], cap))
    torch.cuda.synchronize()

    def step(i):
        w, x, c1, c3 = copies[i % R]
        ml.lora_moe_align(tid, ids, en, case.E, al)
        ml.lora_moe_gate_up_add(w, x, case.topk, al, c1, ws)
        ml.lora_moe_silu_and_mul(c1, c2)
        ml.lora_moe_down_add(w, c2, case.M, case.topk, al, c3, ws)
        ml.lora_moe_topk_reduce(c3, wts, out)

    def deltas(i):
        w, x, c1, c3 = copies[i % R]
        ml.lora_moe_gate_up_add(w, x, case.topk, al, c1, ws)
        ml.lora_moe_silu_and_mul(c1, c2)
        ml.lora_moe_down_add(w, c2, case.M, case.topk, al, c3, ws)

    ms_step, ms_wall = run_timed(step, steps, warmup)
    ms_deltas = back_to_back(deltas, steps)
    silu_bytes = P * 3 * I * es
    res = {
        "ms_per_step": ms_step, "ms_deltas_and_silu_b2b": ms_deltas, "ms_wall_host": ms_wall,
        "tokens_per_s": case.M / (ms_step * 1e-3), "pairs": len(pairs), "buckets": len(buckets),
        "alg_bytes_deltas": nbytes, "alg_bytes_silu": silu_bytes, "alg_flops": flops,
        "rotation_copies": R,
        "hbm_gbs": (nbytes + silu_bytes) / (ms_deltas * 1e-3) / 1e9,
    }
    res["hbm_frac"] = res["hbm_gbs"] / HBM_PEAK_GBS
    del copies
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- oracle
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(fn, units, seconds):
    """Median over three runs of units / second for `fn` repeated until each
    run has taken about seconds / 3, with the BLAS pool held to one thread
    (so that `cores` is what the oracle actually used)."""
    from threadpoolctl import threadpool_limits
    rates = []
    reps_tot, el_tot = 0, 0.0
    with threadpool_limits(limits=1):
        for _ in range(3):
            reps, t0 = 0, time.perf_counter()
            while True:
                fn()
                reps += 1
                el = time.perf_counter() - t0
                if el >= seconds / 3:
                    break
            rates.append(units * reps / el)
            reps_tot, el_tot = reps_tot + reps, el_tot + el
    return float(np.median(rates)), reps_tot, el_tot


def cpu_baseline_linear(case, seconds, tokens=None):
    """The dense oracle (fp64 per-token loop) on the first `tokens` tokens of
    the batch (all when None), as tokens with an adapter per second."""
    from oracle import lora as O
    M = case.M if tokens is None else min(tokens, case.M)
    A = [a.values for a in case.A]
    B = [b.values for b in case.B]
    x, ids, yb = case.x.values[:M], case.ids[:M], case.y_base.values[:M]
    m_valid = int(sum(1 for i in ids if 0 <= i < case.L and case.ranks[i] > 0))
    rate, reps, el = _oracle_rate(
        lambda: O.lora_linear(x, ids, A, B, case.ranks, case.slice_sizes, yb), m_valid, seconds)
    return {"value": rate, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} passes over {M} of the {case.M} tokens ({m_valid} with an "
                      f"adapter) in {el:.1f} s, median of 3 runs; fp64 numpy per-token loop, "
                      f"one BLAS thread",
            "cpu": cpu_model(), "host_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline_moe(case, seconds, tokens=32):
    """The MoE oracle's four stages (gate/up delta, silu-and-mul, down delta,
    top-k reduce) on the first `tokens` tokens, as tokens per second."""
    from oracle import moe as OM
    M, k = min(tokens, case.M), case.topk
    sl = slice(0, M * k)
    args = (case.topk_ids[:M], case.ids[:M], case.adapter_enabled)
    x, c1, c3 = case.x.values[:M], case.cache1.values[sl], case.cache3.values[sl]
    A_gu, B_gu, A_d, B_d = (t.values for t in (case.A_gu, case.B_gu, case.A_d, case.B_d))
    w = case.topk_weights[:M]

    def run():
        g = OM.moe_gate_up_add(x, c1, *args, A_gu, B_gu, case.shared_outer)
        c2 = OM.silu_and_mul(g)
        c3o = OM.moe_down_add(c2, c3, *args, A_d, B_d, case.shared_outer)
        OM.topk_reduce(c3o, w)
    rate, reps, el = _oracle_rate(run, M, seconds)
    return {"value": rate, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} passes over {M} of the {case.M} tokens (all four stages) in "
                      f"{el:.1f} s, median of 3 runs; fp64 numpy per-pair loop, one BLAS thread",
            "cpu": cpu_model(), "host_cpus": len(os.sched_getaffinity(0))}


# ----------------------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    only = set(s for s in args.only.split(",") if s)
    want = lambda k: not only or k in only

    results = {}
    dec_case = W.decode_bf16(0)
    cases = {}                      # workloads that also get an oracle timing
    if want("decode"):
        results["decode_bf16"] = bench_linear(dec_case, args.steps, args.warmup,
                                              "k_decode_fused<uint16_t>", single_launch=True)
    if want("prefill"):
        cases["prefill_bf16"] = (W.prefill_bf16(0), 64)
        results["prefill_bf16"] = bench_linear(cases["prefill_bf16"][0], args.steps, args.warmup,
                                               "k_shrink_dense + k_reduce_partials + k_expand_pipe")
    if want("qkv"):
        cases["stacked_qkv_bf16"] = (W.stacked_bf16("qkv", 0), 64)
        results["stacked_qkv_bf16"] = bench_linear(cases["stacked_qkv_bf16"][0], args.steps,
                                                   args.warmup, "shrink + reduce + expand")
    if want("gate_up"):
        cases["stacked_gate_up_bf16"] = (W.stacked_bf16("gate_up", 0), 32)
        results["stacked_gate_up_bf16"] = bench_linear(cases["stacked_gate_up_bf16"][0],
                                                       args.steps, args.warmup,
                                                       "shrink + reduce + expand")
    if want("moe"):
        cases["moe_bf16"] = (W.moe_case(0), 16)
        results["moe_bf16"] = bench_moe(cases["moe_bf16"][0], args.steps, args.warmup)
    if want("moe_shared"):
        results["moe_shared_outer_bf16"] = bench_moe(W.moe_case(0, shared_outer=True),
                                                     args.steps, args.warmup)
    if want("lm_head"):
        results["lm_head_decode_bf16"] = bench_linear(W.lm_head_bf16(0), args.steps, args.warmup,
                                                      "k_decode_fused<uint16_t>",
                                                      single_launch=True)
    if want("linear_fused"):
        results["prefill_base_fused_bf16"] = bench_linear_fused(W.prefill_bf16(0), args.steps,
                                                                args.warmup)
    if want("embedding"):
        results["embedding_decode_bf16"] = bench_embedding(W.embedding_bf16(0), args.steps,
                                                           args.warmup)

    head = results.get("decode_bf16")
    ceiling = None
    if head is not None:
        # the decode step's mix: everything it reads, then the y rows it writes
        wr = head["m_valid"] * dec_case.N * 2
        ceiling = stream_ceiling(head["alg_bytes"] - wr, wr, args.steps,
                                 decode_launch_grid(dec_case))
        ceiling["decode_kernel_over_ceiling_at_launch_grid"] = (
            head["ms_kernel_b2b"] / ceiling["at_launch_grid"]["ms"])
        ceiling["decode_kernel_over_best_ceiling"] = head["ms_kernel_b2b"] / ceiling["best"]["ms"]
    calib = copy_calibration()
    cpu = None
    if not args.no_cpu:
        if head is not None:
            cpu = cpu_baseline_linear(dec_case, args.cpu_seconds)
        for key, (case, tokens) in cases.items():
            f = cpu_baseline_moe if key.startswith("moe") else cpu_baseline_linear
            results[key]["cpu_baseline"] = f(case, args.cpu_seconds / 4, tokens)
    traffic = measured_traffic()
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"] if head else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"] if head else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_bf16: M=32 tokens, K=4096, N=4096, 20 adapters, ranks "
                               "from {16,32,64}, 10% tokens without adapter, seed 0",
                   "step": "lora_fused_decode (one launch: segment table + delta)",
                   "cold_mall_rotation": head["rotation_copies"] if head else None},
        "roofline": None if head is None else {
            "bound": "hbm", "achieved": head["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": head["hbm_frac"],
            "traffic": None if traffic is None else traffic["total_bytes"],
            "kernel": head["kernel"], "kernel_ms": head["ms_kernel_b2b"],
            "alg_bytes_per_launch": head["alg_bytes"],
            "vs_stream_ceiling": None if ceiling is None else {
                "at_launch_grid": ceiling["decode_kernel_over_ceiling_at_launch_grid"],
                "best": ceiling["decode_kernel_over_best_ceiling"],
                "note": "decode kernel time / time of the hand-written streaming kernel "
                        "moving the same bytes"},
            "traffic_detail": traffic},
        "cpu_baseline": cpu,
        "ceiling": ceiling,
        "counter_calibration_copy": calib,
        "graph_replay": None if head is None else {
            "ms_per_step": head["ms_per_step_graph"],
            "tokens_per_s": head["m_valid"] / (head["ms_per_step_graph"] * 1e-3),
            "note": "the same step captured as one HIP graph per input copy"},
        "two_launch": None if head is None else {
            "ms_per_step": head["ms_per_step_two_launch"],
            "tokens_per_s": head["m_valid"] / (head["ms_per_step_two_launch"] * 1e-3),
            "ms_table_kernel_b2b": head["ms_table_kernel_b2b"],
            "note": "lora_build_segments + lora_shrink_expand_add on the built table"},
        "extra": {k: v for k, v in results.items() if k != "decode_bf16"},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
