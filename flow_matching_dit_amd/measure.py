"""Measurement helpers: kernel-source hash and HBM traffic from rocprofv3 counters.

HBM bytes per launch of a kernel come from two rocprofv3 --pmc runs of the same
command (FETCH_SIZE, then WRITE_SIZE; both in KiB per dispatch), each scaled by the
factor that makes the same counter read the known size of a plain device-to-device
copy (bench.py --copy-calibration).

usage:
  python -m flow_matching_dit_amd.measure traffic --kernel-substr S --cls C --workload W \
      --fetch fetch.csv --write write.csv --calib-fetch cf.csv --calib-write cw.csv \
      --calib-bytes N --out profiles/traffic_C_W.json
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


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    for k in ("kernel-substr", "cls", "workload", "fetch", "write", "calib-fetch", "calib-write", "out"):
        t.add_argument("--" + k, required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--calib-substr", default="copy")
    sub.add_parser("hash")
    args = ap.parse_args()
    if args.cmd == "traffic":
        traffic(args)
    else:
        print(kernel_source_hash())


if __name__ == "__main__":
    main()
