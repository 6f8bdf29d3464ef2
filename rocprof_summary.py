"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

  python rocprof_summary.py stats DIR "COMMAND" > profiles/<kernel>_<workload>.md
      per-kernel duration table from DIR's *_kernel_stats.csv
  python rocprof_summary.py mfma DIR "COMMAND" > profiles/<workload>_mfma.md
      per-kernel MFMA work and utilisation from one counter run of
      SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE
  python rocprof_summary.py traffic FETCH_DIR WRITE_DIR "FETCH_CMD" "WRITE_CMD" [WORKGROUPS] \\
      > profiles/decode_fused_traffic.md
      HBM bytes per launch of the fused decode kernel (only the dispatches with
      WORKGROUPS workgroups when given: the single-launch form) from two counter runs
      (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each scaled by what
      the same counter reads for the 256 MB streaming copy that bench.py runs
      (the hand-written k_stream kernel: 128 MB read, 128 MB written).

The traffic summary carries a hash of the decode kernel's sources; bench.py
reports the figure only while that hash still matches.
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
    name = name.replace("void ", "")
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
    else:
        raise SystemExit(__doc__)
