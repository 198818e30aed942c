#!/usr/bin/env python3
"""Summarise a rocprofv3 kernel-trace database (rocpd SQLite) per kernel name.

usage: rocpd_summary.py <results.db> [title]   -> markdown table on stdout
Columns: launches, total ms, average us, share, scratch bytes per lane (0 = no register
spills), LDS bytes, grid/block.
"""
import sqlite3
import sys


def main():
    db = sqlite3.connect(sys.argv[1])
    title = sys.argv[2] if len(sys.argv) > 2 else sys.argv[1]
    rows = db.execute(
        "select name, count(*), sum(duration), avg(duration), max(scratch_size), "
        "max(lds_size), max(grid_x), max(grid_y), max(grid_z), max(workgroup_x) from kernels group by name "
        "order by sum(duration) desc").fetchall()
    total = sum(r[2] for r in rows)
    print(f"# {title}\n")
    print(f"total kernel time {total / 1e6:.3f} ms over {sum(r[1] for r in rows)} launches\n")
    print("| kernel | launches | total ms | avg us | share | scratch B | lds B | grid (threads) x,y,z | block |")
    print("|---|---|---|---|---|---|---|---|---|")
    for name, n, tot, avg, scr, lds, gx, gy, gz, wx in rows:
        short = name if len(name) < 110 else name[:107] + "..."
        print(f"| `{short}` | {n} | {tot / 1e6:.3f} | {avg / 1e3:.2f} | {100.0 * tot / total:.1f}% | {scr} | "
              f"{lds} | {gx},{gy},{gz} | {wx} |")


if __name__ == "__main__":
    main()
