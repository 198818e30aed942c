"""Measurement helpers: kernel-source hash and HBM traffic from rocprofv3 counters.

HBM bytes per launch of a kernel come from two rocprofv3 --pmc runs of the same
command (FETCH_SIZE, then WRITE_SIZE; both in KiB per dispatch), each scaled by the
factor that makes the same counter read the known size of a plain device-to-device
copy (bench.py --copy-calibration).

Per-kernel tables join such counter runs with the average durations of a kernel-trace
database of the same command (rocpd SQLite):
  mfma       MFMA utilisation (derived counter MfmaUtil: MFMA-busy cycles over all SIMDs'
             cycles while the GPU is active) and bf16 MFMA flops (SQ_INSTS_VALU_MFMA_MOPS_BF16
             x 512) per dispatch, with the achieved TFLOP/s against the 2.5 PFLOP/s dense peak
  bandwidth  HBM bytes per dispatch (calibrated FETCH_SIZE + WRITE_SIZE) over the traced
             duration, against the 8 TB/s peak

The kernel-only average duration of a class's kernel comes from the same database:
  trace      average duration and launch count of the kernels whose name contains S

usage:
  python -m flow_matching_dit_amd.measure trace --kernel-substr S --cls C --workload W \
      --db results.db --command "..." --out profiles/trace_C_W.json
  python -m flow_matching_dit_amd.measure traffic --kernel-substr S --cls C --workload W \
      --fetch fetch.csv --write write.csv --calib-fetch cf.csv --calib-write cw.csv \
      --calib-bytes N --out profiles/traffic_C_W.json
  python -m flow_matching_dit_amd.measure mfma --csv mfma.csv --trace results.db [--substr gemm]
  python -m flow_matching_dit_amd.measure bandwidth --fetch fetch.csv --write write.csv \
      --calib-fetch cf.csv --calib-write cw.csv --calib-bytes N --trace results.db [--substr gemm]
"""
import argparse
import csv
import hashlib
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("gemm.hip", "ops.hip", "kcommon.h"):
        with open(os.path.join(HERE, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _values(path, counter, substr):
    out = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter and substr in r["Kernel_Name"]:
            out.append(float(r["Counter_Value"]))
    return out


def traffic(args):
    cf = _values(args.calib_fetch, "FETCH_SIZE", args.calib_substr)
    cw = _values(args.calib_write, "WRITE_SIZE", args.calib_substr)
    if not cf or not cw:
        sys.exit("calibration copy kernel not found in the counter files")
    # the largest dispatch is the calibration copy (the rest are torch's small fills)
    f_fetch = args.calib_bytes / (max(cf) * 1024.0)
    f_write = args.calib_bytes / (max(cw) * 1024.0)
    fv = _values(args.fetch, "FETCH_SIZE", args.kernel_substr)
    wv = _values(args.write, "WRITE_SIZE", args.kernel_substr)
    if not fv or not wv:
        sys.exit("kernel not found in the counter files")
    fetch_b = statistics.fmean(fv) * 1024.0 * f_fetch
    write_b = statistics.fmean(wv) * 1024.0 * f_write
    res = {"class": args.cls, "workload": args.workload, "kernel_substr": args.kernel_substr,
           "dispatches": len(fv), "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
           "bytes_per_launch": fetch_b + write_b, "scale_fetch": f_fetch, "scale_write": f_write,
           "calib_bytes": args.calib_bytes, "kernel_source_hash": kernel_source_hash()}
    with open(args.out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0


def _by_kernel(path, counter):
    """counter value per dispatch, grouped by kernel name"""
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _trace_us(db_path):
    """average duration (us) and launch count per kernel name of a rocpd kernel-trace database"""
    import sqlite3
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, count(*), avg(duration) from kernels group by name").fetchall()
    return {n: (c, d / 1e3) for n, c, d in rows}


def _short(name):
    return name if len(name) < 90 else name[:87] + "..."


def _calib(args):
    cf = _values(args.calib_fetch, "FETCH_SIZE", args.calib_substr)
    cw = _values(args.calib_write, "WRITE_SIZE", args.calib_substr)
    if not cf or not cw:
        sys.exit("calibration copy kernel not found in the counter files")
    return args.calib_bytes / (max(cf) * 1024.0), args.calib_bytes / (max(cw) * 1024.0)


def mfma(args):
    util = _by_kernel(args.csv, "MfmaUtil")
    mops = _by_kernel(args.csv, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    tr = _trace_us(args.trace)
    rows = []
    for k, u in util.items():
        if args.substr not in k or k not in tr:
            continue
        fl = statistics.fmean(mops.get(k, [0.0])) * 512.0
        us = tr[k][1]
        rows.append((k, len(u), statistics.fmean(u), fl, us, fl / (us * 1e-6) / 1e12 if us > 0 else 0.0))
    rows.sort(key=lambda r: -r[3] * tr[r[0]][0])
    print("| kernel | dispatches | MfmaUtil % | bf16 MFMA GFLOP / dispatch | traced avg us | TFLOP/s | of 2.5 PF |")
    print("|---|---|---|---|---|---|---|")
    for k, n, u, fl, us, tf in rows:
        print(f"| `{_short(k)}` | {n} | {u:.1f} | {fl / 1e9:.2f} | {us:.2f} | {tf:.0f} | "
              f"{100.0 * tf / BF16_PEAK_TFLOPS:.1f}% |")


def bandwidth(args):
    f_fetch, f_write = _calib(args)
    fv, wv = _by_kernel(args.fetch, "FETCH_SIZE"), _by_kernel(args.write, "WRITE_SIZE")
    tr = _trace_us(args.trace)
    rows = []
    for k, f in fv.items():
        if args.substr not in k or k not in tr or k not in wv:
            continue
        fb = statistics.fmean(f) * 1024.0 * f_fetch
        wb = statistics.fmean(wv[k]) * 1024.0 * f_write
        us = tr[k][1]
        rows.append((k, len(f), fb, wb, us, (fb + wb) / (us * 1e-6) / 1e9 if us > 0 else 0.0))
    rows.sort(key=lambda r: -(r[2] + r[3]) * tr[r[0]][0])
    print(f"Calibration: FETCH_SIZE x {f_fetch:.2f}, WRITE_SIZE x {f_write:.2f} (plain copy of {args.calib_bytes} bytes).\n")
    print("| kernel | dispatches | fetched MB | written MB | traced avg us | GB/s | of 8 TB/s |")
    print("|---|---|---|---|---|---|---|")
    for k, n, fb, wb, us, gbs in rows:
        print(f"| `{_short(k)}` | {n} | {fb / 1e6:.2f} | {wb / 1e6:.2f} | {us:.2f} | {gbs:.0f} | "
              f"{100.0 * gbs / HBM_PEAK_GBS:.1f}% |")


def trace(args):
    import sqlite3
    db = sqlite3.connect(args.db)
    rows = db.execute("select name, count(*), avg(duration) from kernels group by name").fetchall()
    hits = [(n, c, d) for n, c, d in rows if args.kernel_substr in n]
    if len(hits) != 1:
        sys.exit(f"{len(hits)} kernel names contain {args.kernel_substr!r}; need exactly one")
    name, n, avg_ns = hits[0]
    res = {"class": args.cls, "workload": args.workload, "kernel": name, "launches": n,
           "avg_us": avg_ns / 1e3, "command": args.command, "kernel_source_hash": kernel_source_hash()}
    with open(args.out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    for k in ("kernel-substr", "cls", "workload", "fetch", "write", "calib-fetch", "calib-write", "out"):
        t.add_argument("--" + k, required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--calib-substr", default="copy")
    m = sub.add_parser("mfma")
    m.add_argument("--csv", required=True)
    m.add_argument("--trace", required=True)
    m.add_argument("--substr", default="gemm")
    b = sub.add_parser("bandwidth")
    for k in ("fetch", "write", "calib-fetch", "calib-write", "trace"):
        b.add_argument("--" + k, required=True)
    b.add_argument("--calib-bytes", type=int, required=True)
    b.add_argument("--calib-substr", default="copy")
    b.add_argument("--substr", default="gemm")
    tr = sub.add_parser("trace")
    for k in ("kernel-substr", "cls", "workload", "db", "command", "out"):
        tr.add_argument("--" + k, required=True)
    sub.add_parser("hash")
    args = ap.parse_args()
    if args.cmd == "traffic":
        traffic(args)
    elif args.cmd == "mfma":
        mfma(args)
    elif args.cmd == "bandwidth":
        bandwidth(args)
    elif args.cmd == "trace":
        trace(args)
    else:
        print(kernel_source_hash())


if __name__ == "__main__":
    main()
