"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

  python rocprof_summary.py stats DIR "COMMAND" > profiles/<kernel>_<workload>.md
      per-kernel duration table from DIR's *_kernel_stats.csv
  python rocprof_summary.py mfma DIR "COMMAND" > profiles/<workload>_mfma.md
      per-kernel MFMA work and utilisation from one counter run of
      SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE
  python rocprof_summary.py durations "COMMAND_TEMPLATE" NAME=DIR ... > profiles/<file>.md
      per workload (one rocprofv3 --kernel-trace run each, COMMAND_TEMPLATE with
      {name} standing for NAME): launches, median, p10 and p90 of every
      library kernel's duration, grouped by kernel and grid size
  python rocprof_summary.py traffic_all "FETCH_TEMPLATE" "WRITE_TEMPLATE" NAME=FDIR,WDIR,BENCHJSON ...
      per workload: FETCH_SIZE and WRITE_SIZE bytes per step of the library's
      kernels (calibrated as below) against the workload's algorithmic bytes
      (alg_bytes of the bench line saved as BENCHJSON)
  python rocprof_summary.py traffic FETCH_DIR WRITE_DIR "FETCH_CMD" "WRITE_CMD" [WORKGROUPS] \\
      > profiles/decode_fused_traffic.md
      HBM bytes per launch of the fused decode kernel (only the dispatches with
      WORKGROUPS workgroups when given: the single-launch form) from two counter runs
      (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each scaled by what
      the same counter reads for the 256 MB streaming copy that bench.py runs
      (the hand-written k_stream kernel: 128 MB read, 128 MB written).

The traffic summary carries a hash of the decode kernel's sources (their
code, comments removed); bench.py reports the figure only while that hash
still matches.
"""
import csv
import glob
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DECODE_KERNEL = "k_decode_fused"
CALIB_KERNEL = "k_stream"
CALIB_BYTES = 256 << 20          # bench.copy_calibration(): 128 MB read + 128 MB written


def _rows(directory, suffix):
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    out = []
    for f in files:
        with open(f, newline="") as fh:
            out += list(csv.DictReader(fh))
    return out


def short(name):
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    if "(" in name:
        name = name[:name.index("(")]
    return name[:70]


def stats(directory, command):
    rows = _rows(directory, "kernel_stats.csv")
    print("# rocprofv3 kernel statistics\n")
    print(f"Command (from /tmp, `TMPDIR=/tmp`):\n\n```\n{command}\n```\n")
    print("| kernel | calls | mean µs | min µs | max µs | share % |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in sorted(rows, key=lambda r: -float(r.get("TotalDurationNs", 0))):
        print(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
              f"{float(r['Percentage']):.1f} |")


def _dur_us(r):
    return (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3


def _pct(v, q):
    v = sorted(v)
    if not v:
        return float("nan")
    i = q / 100 * (len(v) - 1)
    lo, hi = int(i), min(int(i) + 1, len(v) - 1)
    return v[lo] + (v[hi] - v[lo]) * (i - lo)


def durations(template, pairs):
    print("# Kernel durations per workload (rocprofv3 kernel trace)\n")
    print("One `rocprofv3 --kernel-trace` run of the benchmark per workload "
          "(from /tmp, `TMPDIR=/tmp`); the command, with `{name}` the workload:\n")
    print(f"```\n{template}\n```\n")
    print("Durations are the trace's start-to-end times of each dispatch, in µs, "
          "for the library's kernels and the streaming reference kernel; kernels are "
          "told apart by grid size (threads).  p10 / p90 are the 10th / 90th "
          "percentiles over all launches of the run (warm-up and timed steps, "
          "cold-MALL rotation).\n")
    print("| workload | kernel | grid | launches | median | p10 | p90 | mean |")
    print("|---|---|---:|---:|---:|---:|---:|---:|")
    for pair in pairs:
        name, d = pair.split("=", 1)
        rows = _rows(d, "kernel_trace.csv")
        groups = {}
        for r in rows:
            n = r["Kernel_Name"]
            if ("mlora" not in n and "k_stream" not in n) or "k_pack" in n or "k_fill" in n:
                continue
            key = (short(n), int(r.get("Grid_Size_X", r.get("Grid_Size", 0))))
            groups.setdefault(key, []).append(_dur_us(r))
        for (k, g), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            if len(v) < 20:
                continue
            print(f"| {name} | `{k}` | {g} | {len(v)} | {_pct(v, 50):.2f} | {_pct(v, 10):.2f} | "
                  f"{_pct(v, 90):.2f} | {sum(v) / len(v):.2f} |")


def _per_kernel_kib(rows, counter, keep):
    """Per (kernel, grid): list of the counter's value per dispatch, KiB."""
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter or not keep(r["Kernel_Name"]):
            continue
        key = (short(r["Kernel_Name"]), int(r.get("Grid_Size", r.get("Grid_Size_X", 0))),
               r["Dispatch_Id"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (k, g, _), v in per.items():
        out.setdefault((k, g), []).append(v)
    return out


def _calibration(rows, counter):
    """Bytes the counter reads per byte moved, from the 128 MB streaming copy."""
    half = CALIB_BYTES / 2
    cal = [v for v in _all(rows, counter, CALIB_KERNEL) if v * 1024 > 0.25 * half]
    if not cal:
        raise SystemExit(f"no calibration copy in the {counter} run")
    return (sum(cal) / len(cal)) * 1024 / half


def traffic_all(fetch_template, write_template, triples):
    import json
    print("# HBM traffic per workload (FETCH_SIZE, WRITE_SIZE)\n")
    print("Two counter runs of the benchmark per workload (from /tmp, `TMPDIR=/tmp`), "
          "with `{name}` the workload:\n")
    print(f"```\n{fetch_template}\n{write_template}\n```\n")
    print("Each counter (KiB per dispatch) is scaled by what it reads for the 128 MB "
          "streaming copy of the same run (`k_stream`, 128 MB read and 128 MB written).  "
          "Per kernel: bytes per dispatch, median over the run's dispatches.  Per "
          "workload: the step's kernels summed against the step's algorithmic bytes "
          "(the bench line's `alg_bytes`: every touched weight, x row and y row "
          "once).\n")
    print("| workload | kernel | grid | dispatches | fetch MB | write MB | in step |")
    print("|---|---|---:|---:|---:|---:|---|")
    summary = []
    for t in triples:
        name, rest = t.split("=", 1)
        fdir, wdir, bj, *sel = rest.split(",")
        # the step's kernels: "+"-separated name fragments, each optionally
        # "@grid" (threads); default every library kernel of the run
        picks = [q.split("@") for q in sel[0].split("+")] if sel else []

        def in_step(key):
            return not picks or any(q[0] in key[0] and (len(q) == 1 or int(q[1]) == key[1])
                                    for q in picks)
        fr = _rows(fdir, "counter_collection.csv")
        wr = _rows(wdir, "counter_collection.csv")
        ff, wf = _calibration(fr, "FETCH_SIZE"), _calibration(wr, "WRITE_SIZE")
        keep = lambda n: "mlora::" in n and "k_pack" not in n and "k_fill" not in n
        fk = _per_kernel_kib(fr, "FETCH_SIZE", keep)
        wk = _per_kernel_kib(wr, "WRITE_SIZE", keep)
        step_f = step_w = 0.0
        for key in sorted(set(fk) | set(wk), key=lambda kk: kk[0]):
            fv = sorted(fk.get(key, [0.0]))
            wv = sorted(wk.get(key, [0.0]))
            fb = fv[len(fv) // 2] * 1024 / ff
            wb = wv[len(wv) // 2] * 1024 / wf
            if len(fv) < 10:
                continue
            step = in_step(key)
            if step:
                step_f += fb
                step_w += wb
            print(f"| {name} | `{key[0]}` | {key[1]} | {len(fv)} | {fb / 1e6:.2f} | "
                  f"{wb / 1e6:.2f} |{' step' if step and picks else ''}")
        line = json.loads(open(bj).read().strip().splitlines()[-1])
        res = line.get("extra", {}).get(name) or {}
        alg = res.get("alg_bytes") or (res.get("alg_bytes_deltas", 0) + res.get("alg_bytes_silu", 0))
        if name == "decode_bf16":
            alg = line["roofline"]["alg_bytes_per_launch"]
        summary.append((name, step_f, step_w, alg))
    print("\n| workload | measured MB per step | algorithmic MB | measured / algorithmic |")
    print("|---|---:|---:|---:|")
    for name, f, w, alg in summary:
        ratio = "—" if not alg else f"{(f + w) / alg:.2f}"
        print(f"| {name} | {(f + w) / 1e6:.2f} | {'—' if not alg else f'{alg / 1e6:.2f}'} | "
              f"{ratio} |")


def _per_dispatch_kib(rows, counter, match, workgroups=None):
    vals = {}
    for r in rows:
        if workgroups is not None and int(r["Grid_Size"]) != workgroups * int(r["Workgroup_Size"]):
            continue
        if r["Counter_Name"] == counter and match in r["Kernel_Name"]:
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} values for kernels matching {match!r}")
    v = sorted(vals.values())
    return sum(v) / len(v), len(v), v[len(v) // 2]


def traffic(fetch_dir, write_dir, fetch_cmd, write_cmd, workgroups=None):
    import bench
    wg = None if workgroups is None else int(workgroups)
    fr = _rows(fetch_dir, "counter_collection.csv")
    wr = _rows(write_dir, "counter_collection.csv")
    kf, nkf, kf_med = _per_dispatch_kib(fr, "FETCH_SIZE", DECODE_KERNEL, wg)
    kw, nkw, kw_med = _per_dispatch_kib(wr, "WRITE_SIZE", DECODE_KERNEL, wg)
    # the streaming kernel also runs at the decode byte count; take the 128 MB copies
    half = CALIB_BYTES / 2
    cal = [v for v in _all(fr, "FETCH_SIZE", CALIB_KERNEL) if v * 1024 > 0.25 * half]
    calw = [v for v in _all(wr, "WRITE_SIZE", CALIB_KERNEL) if v * 1024 > 0.25 * half]
    f_fac = (sum(cal) / len(cal)) * 1024 / half
    w_fac = (sum(calw) / len(calw)) * 1024 / half
    fetch = kf * 1024 / f_fac
    write = kw * 1024 / w_fac
    print("# Fused decode kernel: HBM traffic per launch\n")
    print("Two counter runs over the decode benchmark (cold rotation of 50 input copies);")
    print("each counter is scaled by what it reads for the 256 MB bf16 streaming copy in")
    print("the same run (128 MB read, 128 MB written).\n")
    print(f"FETCH_SIZE run:\n\n```\n{fetch_cmd}\n```\n")
    print(f"WRITE_SIZE run:\n\n```\n{write_cmd}\n```\n")
    print(f"- kernel: `{DECODE_KERNEL}<uint16_t>`" +
          ("" if wg is None else f", dispatches of {wg} workgroups"))
    print(f"- dispatches: `{nkf}` (fetch run), `{nkw}` (write run)")
    print(f"- fetch_kib_per_dispatch_raw: `{kf:.1f}` (median {kf_med:.1f})")
    print(f"- write_kib_per_dispatch_raw: `{kw:.1f}` (median {kw_med:.1f})")
    print(f"- calibration: `copy 128 MB read reads {f_fac:.4f}x, 128 MB write reads {w_fac:.4f}x`")
    print(f"- fetch_bytes_per_launch: `{fetch:.0f}`")
    print(f"- write_bytes_per_launch: `{write:.0f}`")
    print(f"- traffic_bytes_per_launch: `{fetch + write:.0f}`")
    print(f"- source_hash: `{bench.source_hash(bench.DECODE_SOURCES)}`")


N_XCD = 8            # GRBM_GUI_ACTIVE is summed over the XCDs
N_SIMD = 256 * 4     # SQ_VALU_MFMA_BUSY_CYCLES is summed over the SIMDs
MOPS_FLOP = 512      # one MFMA MOP of SQ_INSTS_VALU_MFMA_MOPS_BF16


def mfma(directory, command):
    rows = _rows(directory, "counter_collection.csv")
    per = {}
    for r in rows:
        key = (short(r["Kernel_Name"]), r["Dispatch_Id"])
        per.setdefault(key, {})
        per[key][r["Counter_Name"]] = per[key].get(r["Counter_Name"], 0.0) + \
            float(r["Counter_Value"])
    kern = {}
    for (name, _), c in per.items():
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" not in c or c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] == 0:
            continue
        kern.setdefault(name, []).append(c)
    print("# MFMA work and utilisation per kernel\n")
    print(f"Counter run (from /tmp, `TMPDIR=/tmp`):\n\n```\n{command}\n```\n")
    print(f"FLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x {MOPS_FLOP}.  Busy = "
          f"SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {N_XCD} x {N_SIMD} SIMDs): the share "
          "of the kernel's cycles in which the matrix units were busy.  Clock = "
          "GRBM_GUI_ACTIVE per XCD over the same cycles, reported as cycles per dispatch.\n")
    print("| kernel | dispatches | GFLOP / dispatch | cycles / dispatch (per XCD) | MFMA busy % |")
    print("|---|---:|---:|---:|---:|")
    for name, cs in sorted(kern.items(), key=lambda kv: -sum(c["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
                                                             for c in kv[1])):
        n = len(cs)
        flop = sum(c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for c in cs) / n * MOPS_FLOP
        gui = sum(c.get("GRBM_GUI_ACTIVE", 0.0) for c in cs) / n / N_XCD
        busy = sum(c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for c in cs) / n
        pct = 100.0 * busy / (gui * N_SIMD) if gui else float("nan")
        print(f"| `{name}` | {n} | {flop / 1e9:.3f} | {gui:.0f} | {pct:.1f} |")


def _all(rows, counter, match):
    vals = {}
    for r in rows:
        if r["Counter_Name"] == counter and match in r["Kernel_Name"]:
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return list(vals.values())


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3])
    elif sys.argv[1] == "mfma":
        mfma(sys.argv[2], sys.argv[3])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:7])
    elif sys.argv[1] == "durations":
        durations(sys.argv[2], sys.argv[3:])
    elif sys.argv[1] == "traffic_all":
        traffic_all(sys.argv[2], sys.argv[3], sys.argv[4:])
    else:
        raise SystemExit(__doc__)
