"""Turn rocprofv3 CSV output into the short summaries kept under profiles/.

Two kinds of summary:

* ``trace``: per-kernel call count and average / min / max duration from a
  ``--kernel-trace --stats --output-format csv`` run.
* ``pmc``: HBM bytes per launch of the attention kernel from one FETCH_SIZE
  run and one WRITE_SIZE run (KiB per dispatch), each scaled by the ratio
  bytes / counter measured on a plain device copy of known size in the same
  way, plus the hash of the kernel sources the counters were taken on (so the
  bench can drop the figure once the kernel changes).

Usage:
  python -m mla_decode_paged_split_amd.profile_summary trace <stats.csv> <out.md> "<command>"
  python -m mla_decode_paged_split_amd.profile_summary pmc <workload> <fetch.csv> <write.csv> \
      <copy_fetch.csv> <copy_write.csv> <algorithmic_bytes> <out.json> "<commands>"
"""

from __future__ import annotations

import csv
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = ["mla_decode_paged_split_amd/csrc/mla_device.hpp", "mla_decode_paged_split_amd/csrc/mla_decode.hip"]
ATTENTION = "mla_decode_kernel"
COPY_BYTES = 1 << 30


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def trace_summary(stats_csv: str, out_md: str, command: str) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [
        "# Kernel trace summary",
        "",
        f"Command: `{command}`",
        "",
        f"Kernel sources hash: `{kernel_source_hash()}`",
        "",
        "| kernel | calls | avg us | min us | max us | share |",
        "|---|---|---|---|---|---|",
    ]
    for r in rows:
        lines.append(
            f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
            f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |"
        )
    open(out_md, "w").write("\n".join(lines) + "\n")


def _per_dispatch(counter_csv: str, name_part: str, counter: str) -> list[float]:
    vals = []
    for r in csv.DictReader(open(counter_csv)):
        if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
            vals.append(float(r["Counter_Value"]))
    return vals


def pmc_summary(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, alg_bytes, out_json, commands):
    f = _per_dispatch(fetch_csv, ATTENTION, "FETCH_SIZE")
    w = _per_dispatch(write_csv, ATTENTION, "WRITE_SIZE")
    # the copy probe issues one torch copy kernel per iteration; take the larger dispatches (the 1 GiB copies)
    cf = _per_dispatch(copy_fetch_csv, "", "FETCH_SIZE")
    cw = _per_dispatch(copy_write_csv, "", "WRITE_SIZE")
    cf = sorted(cf)[len(cf) // 2:]
    cw = sorted(cw)[len(cw) // 2:]
    fetch_factor = COPY_BYTES / (statistics.median(cf) * 1024)
    write_factor = COPY_BYTES / (statistics.median(cw) * 1024)
    fetch_b = statistics.median(f) * 1024 * fetch_factor
    write_b = statistics.median(w) * 1024 * write_factor
    d = {
        "workload": workload,
        "kernel": ATTENTION,
        "kernel_source_hash": kernel_source_hash(),
        "fetch_kib_per_dispatch_median": statistics.median(f),
        "write_kib_per_dispatch_median": statistics.median(w),
        "dispatches": [len(f), len(w)],
        "copy_calibration": {
            "bytes_read": COPY_BYTES,
            "bytes_written": COPY_BYTES,
            "fetch_kib_median": statistics.median(cf),
            "write_kib_median": statistics.median(cw),
            "fetch_factor": fetch_factor,
            "write_factor": write_factor,
        },
        "hbm_read_bytes_per_launch": fetch_b,
        "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": fetch_b + write_b,
        "algorithmic_bytes_per_launch": alg_bytes,
        "traffic_over_algorithmic": (fetch_b + write_b) / alg_bytes,
        "commands": commands,
    }
    with open(out_json, "w") as fh:
        json.dump(d, fh, indent=2)
        fh.write("\n")


if __name__ == "__main__":
    kind = sys.argv[1]
    if kind == "trace":
        trace_summary(sys.argv[2], sys.argv[3], sys.argv[4])
    elif kind == "pmc":
        pmc_summary(sys.argv[2], *sys.argv[3:7], int(sys.argv[7]), sys.argv[8], sys.argv[9])
    else:
        raise SystemExit(__doc__)
