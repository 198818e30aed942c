"""Host logic of the measurement helpers (no GPU): the counter summaries join rocprofv3 counter
CSVs with a kernel-trace database by kernel name and apply the copy calibration."""
import csv
import sqlite3
from types import SimpleNamespace

import pytest

from flow_matching_dit_amd import measure

K1 = "void gr00t::gemm_dma_kernel<256, 128, 4, 4, 64, 3, 0, 8>(gr00t::GemmArgs, gr00t::Epi)"
K2 = "gr00t::copy_rows_kernel(float const*, long, float*, long, long, int, int)"
COPY = "__amd_rocclr_copyBuffer"


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})
    return str(path)


def _trace(path, rows):
    """rocpd-like database: a `kernels` table with name and duration (ns)"""
    db = sqlite3.connect(path)
    db.execute("create table kernels (name text, duration integer)")
    db.executemany("insert into kernels values (?, ?)", rows)
    db.commit()
    db.close()
    return str(path)


def _table(out):
    """rows of the markdown table printed by a summary: {kernel: [cells]}"""
    rows = {}
    for line in out.splitlines():
        if line.startswith("| `"):
            cells = [c.strip() for c in line.strip("|").split("|")]
            rows[cells[0].strip("`")] = cells[1:]
    return rows


def test_mfma_summary_rates(tmp_path, capsys):
    # two dispatches of K1: MfmaUtil 20 and 30 %, 2e9 and 4e9 MOPS/512 -> mean 3e9 * 512 flops
    c = _csv(tmp_path / "m.csv", [(K1, "MfmaUtil", 20.0), (K1, "MfmaUtil", 30.0),
                                  (K1, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2e9 / 512),
                                  (K1, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 4e9 / 512),
                                  (K2, "MfmaUtil", 0.0), (K2, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)])
    t = _trace(tmp_path / "t.db", [(K1, 10_000), (K1, 30_000), (K2, 3_000)])  # K1 averages 20 us
    measure.mfma(SimpleNamespace(csv=c, trace=t, substr="gemm"))
    rows = _table(capsys.readouterr().out)
    assert list(rows) == [K1]  # substring filter
    n, util, gflop, us, tfs, frac = rows[K1]
    assert (int(n), float(util), float(gflop), float(us)) == (2, 25.0, 3.0, 20.0)
    assert float(tfs) == pytest.approx(3e9 / 20e-6 / 1e12, abs=0.5)  # 150 TFLOP/s
    assert frac == "6.0%"


def test_bandwidth_summary_applies_copy_calibration(tmp_path, capsys):
    # calibration: a 1 MiB copy reads FETCH 512 KiB (x2) and WRITE 1024 KiB (x1); the largest
    # dispatch of the copy kernel is the calibration one
    cf = _csv(tmp_path / "cf.csv", [(COPY, "FETCH_SIZE", 4.0), (COPY, "FETCH_SIZE", 512.0)])
    cw = _csv(tmp_path / "cw.csv", [(COPY, "WRITE_SIZE", 1024.0)])
    f = _csv(tmp_path / "f.csv", [(K1, "FETCH_SIZE", 1000.0), (K1, "FETCH_SIZE", 3000.0), (K2, "FETCH_SIZE", 1.0)])
    w = _csv(tmp_path / "w.csv", [(K1, "WRITE_SIZE", 500.0), (K1, "WRITE_SIZE", 500.0), (K2, "WRITE_SIZE", 1.0)])
    t = _trace(tmp_path / "t.db", [(K1, 4_000), (K2, 1_000)])
    measure.bandwidth(SimpleNamespace(fetch=f, write=w, calib_fetch=cf, calib_write=cw, calib_bytes=1 << 20,
                                      calib_substr="copyBuffer", trace=t, substr="gr00t"))
    out = capsys.readouterr().out
    assert "FETCH_SIZE x 2.00, WRITE_SIZE x 1.00" in out
    rows = _table(out)
    assert list(rows) == [K1, K2]  # ordered by bytes x launches
    n, fetched, written, us, gbs, frac = rows[K1]
    fb, wb = 2000.0 * 1024 * 2, 500.0 * 1024  # mean KiB x calibration
    assert (int(n), float(fetched), float(written), float(us)) == (2, round(fb / 1e6, 2), round(wb / 1e6, 2), 4.0)
    assert float(gbs) == pytest.approx((fb + wb) / 4e-6 / 1e9, abs=0.5)


def test_bandwidth_without_calibration_copy_exits(tmp_path):
    cf = _csv(tmp_path / "cf.csv", [(K2, "FETCH_SIZE", 1.0)])
    args = SimpleNamespace(fetch=cf, write=cf, calib_fetch=cf, calib_write=cf, calib_bytes=1, calib_substr="copyBuffer",
                           trace=_trace(tmp_path / "t.db", []), substr="gr00t")
    with pytest.raises(SystemExit):
        measure.bandwidth(args)


def test_kernel_source_hash_is_stable():
    h = measure.kernel_source_hash()
    assert len(h) == 16 and h == measure.kernel_source_hash()
    int(h, 16)


def test_trace_averages_the_one_matching_kernel(tmp_path):
    import json
    db = _trace(tmp_path / "t.db", [(K1, 30000), (K1, 32000), (K2, 5000)])
    out = tmp_path / "trace.json"
    args = SimpleNamespace(db=db, kernel_substr="gemm_dma_kernel<256, 128", cls="ff_up", workload="w",
                           command="rocprofv3 ...", out=str(out))
    measure.trace(args)
    r = json.loads(out.read_text())
    assert r["launches"] == 2 and abs(r["avg_us"] - 31.0) < 1e-9 and r["kernel"] == K1
    assert r["kernel_source_hash"] == measure.kernel_source_hash()
    with pytest.raises(SystemExit):   # no kernel, or more than one, matches
        measure.trace(SimpleNamespace(**dict(vars(args), kernel_substr="gr00t::")))
