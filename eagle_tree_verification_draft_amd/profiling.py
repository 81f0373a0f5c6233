"""Summaries of rocprofv3 output for the committed profile notes.

    python -m eagle_tree_verification_draft_amd.profiling stats DIR
        Per-kernel call count / average / total from a --kernel-trace --stats
        run (the SQLite results db under DIR), as a markdown table.

    python -m eagle_tree_verification_draft_amd.profiling traffic \
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
        --copy-bytes N --kernels k_tree_attn_bf16,k_tree_attn_merge \
        --workload NAME --source FILE[,FILE...] [--command TEXT]
        HBM traffic per call of the named kernels from two --pmc runs
        (FETCH_SIZE, then WRITE_SIZE; csv output), each scaled by the factor
        that the same counter shows for a plain copy kernel of known size.
        Prints a text note whose 'source_sha256' line lets bench.py tell
        whether the kernel source changed since the counters were taken.

    python -m eagle_tree_verification_draft_amd.profiling mfma --pmc DIR \
        --kernels k_tree_attn_bf16 --workload NAME --source FILE[,FILE...] [--command TEXT]
        Matrix-core utilisation per dispatch of the named kernels from a
        --pmc run of MfmaUtil, SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE
        (MfmaUtil = busy cycles summed over the SIMDs / (GUI-active cycles x
        SIMD count), in percent), with the same source hash line.

All read rocprofv3's own output files only; nothing here touches the GPU.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import sqlite3
import sys


def _find(d, pattern):
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    if not hits:
        raise SystemExit(f"no {pattern} under {d}")
    return hits[0]


def stats(d, min_pct=0.5):
    """Per-kernel dispatch count, average, min, max and total duration, from
    the per-dispatch rows of the kernel-trace db (durations in ns)."""
    db = d if d.endswith(".db") else _find(d, "*.db")
    con = sqlite3.connect(db)
    rows = con.execute("select name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
                       "from kernels group by name order by sum(duration) desc").fetchall()
    grand = sum(r[5] for r in rows) or 1
    out = ["| kernel | calls | avg us | min us | max us | total us | % of GPU time |",
           "|---|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, tot in rows:
        pct = 100.0 * tot / grand
        short = name.split("(")[0]
        if "eagle::" not in short and pct < min_pct:
            continue
        if len(short) > 72:
            short = short[:72] + "..."
        out.append(f"| {short} | {calls} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | {tot / 1e3:.0f} "
                   f"| {pct:.1f} |")
    return "\n".join(out)


def source_hash(paths):
    """sha256 over the concatenated bytes of the given source files."""
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_note(path):
    """key: value lines of a traffic note (first ':' splits)."""
    out = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                out.setdefault(k.strip(), v.strip())
    return out


def _pmc_rows(d):
    """(kernel name, counter value) per dispatch from a --pmc csv run."""
    path = _find(d, "*counter_collection.csv")
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
            val = r.get("Counter_Value") or r.get("Counter-Value")
            if val is None:
                continue
            rows.append((name, float(val)))
    return rows


def _pmc_rows_by_counter(d):
    """(kernel name, counter name, value, duration ns) per dispatch from a --pmc csv run."""
    path = _find(d, "*counter_collection.csv")
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            rows.append((r.get("Kernel_Name", ""), r.get("Counter_Name", ""), float(r["Counter_Value"]),
                         int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return rows


def mfma(a):
    rows = _pmc_rows_by_counter(a.pmc)
    lines = []
    if a.command:
        lines.append(f"command: {a.command}")
    lines.append(f"workload: {a.workload}")
    lines.append(f"source: {a.source}")
    lines.append(f"source_sha256: {source_hash(a.source.split(','))}")
    util = None
    for k in a.kernels.split(","):
        sel = [r for r in rows if k in r[0]]
        if not sel:
            lines.append(f"kernel {k}: not found in the counter run")
            continue
        by = {}
        for name, cn, v, dur in sel:
            by.setdefault(cn, []).append((v, dur))
        avg = {cn: sum(v for v, _ in xs) / len(xs) for cn, xs in by.items()}
        durs = [d for _, d in by.get("MfmaUtil", by[next(iter(by))])]
        n = len(durs)
        lines.append(f"kernel {k}: dispatches {n}, average duration {sum(durs) / n / 1e3:.2f} us")
        for cn in sorted(avg):
            lines.append(f"  {cn}: {avg[cn]:.2f}")
        if util is None and "MfmaUtil" in avg:
            util = avg["MfmaUtil"] / 100.0
    if util is not None:
        lines.append(f"mfma_util: {util:.4f}")
    return "\n".join(lines)


def _per_dispatch(rows, key):
    vals = [v for n, v in rows if key in n]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def _largest(rows):
    """Average counter value of the dispatches of the kernel with the largest value."""
    best = max(rows, key=lambda r: r[1])
    return _per_dispatch(rows, best[0])[0], best[0]


def traffic(a):
    fetch, write = _pmc_rows(a.fetch), _pmc_rows(a.write)
    cf_kib, cf_name = _largest(_pmc_rows(a.copy_fetch))
    cw_kib, cw_name = _largest(_pmc_rows(a.copy_write))
    f_factor = a.copy_bytes / (cf_kib * 1024.0)
    w_factor = a.copy_bytes / (cw_kib * 1024.0)
    lines = []
    if a.command:
        lines.append(f"command: {a.command}")
    lines.append(f"workload: {a.workload}")
    lines.append(f"source: {a.source}")
    lines.append(f"source_sha256: {source_hash(a.source.split(','))}")
    lines.append(f"copy_kernel: {cf_name.split('(')[0][:80]}")
    lines.append(f"copy_bytes: {a.copy_bytes}")
    lines.append(f"copy_fetch_KiB_per_dispatch: {cf_kib:.1f}  factor {f_factor:.4f}")
    lines.append(f"copy_write_KiB_per_dispatch: {cw_kib:.1f}  factor {w_factor:.4f}")
    total = 0.0
    for k in a.kernels.split(","):
        fk, nf = _per_dispatch(fetch, k)
        wk, nw = _per_dispatch(write, k)
        if fk is None or wk is None:
            lines.append(f"kernel {k}: not found in the counter runs")
            continue
        fb, wb = fk * 1024.0 * f_factor, wk * 1024.0 * w_factor
        total += fb + wb
        lines.append(f"kernel {k}: dispatches {nf}/{nw}  FETCH_SIZE {fk:.1f} KiB  WRITE_SIZE {wk:.1f} KiB  "
                     f"-> {fb / 1e6:.3f} MB read + {wb / 1e6:.3f} MB written per dispatch")
    lines.append(f"traffic_bytes_per_call: {total:.0f}")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--kernels", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--source", required=True)
    t.add_argument("--command", default="")
    m = sub.add_parser("mfma")
    m.add_argument("--pmc", required=True)
    m.add_argument("--kernels", required=True)
    m.add_argument("--workload", required=True)
    m.add_argument("--source", required=True)
    m.add_argument("--command", default="")
    a = ap.parse_args(argv)
    print(stats(a.dir) if a.cmd == "stats" else traffic(a) if a.cmd == "traffic" else mfma(a))


if __name__ == "__main__":
    sys.exit(main())
