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
  python -m mla_decode_paged_split_amd.profile_summary trace <stats.csv> <out.md> "<command>" \
      [<trace.csv> <bench log>]
  python -m mla_decode_paged_split_amd.profile_summary pmc <workload> <fetch.csv> <write.csv> \
      <copy_fetch.csv> <copy_write.csv> <algorithmic_bytes> <out.json> "<commands>"
  python -m mla_decode_paged_split_amd.profile_summary mfma <counters.csv> <out.md> "<command>" <flops> <peak>
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


def trace_summary(stats_csv: str, out_md: str, command: str, trace_csv: str | None = None,
                  bench_log: str | None = None) -> None:
    """The --stats table, plus (with the per-dispatch trace and the bench's log) the attention launches of
    the bench's two timed regions, with the KV copies rotated: region 1 (whole steps back to back) and
    region 2 (attention launches back to back, the roofline's source).  The bench issues its settling
    steps, the warm-up, region 1, region 2, then diagnostics (per-launch events, one KV copy reused, ...),
    which the per-kernel table averages in but the region figures leave out."""
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [
        "# Kernel trace summary",
        "",
        f"Command: `{command}`",
        "",
        f"Kernel sources hash: `{kernel_source_hash()}`",
        "",
        "All dispatches (settling, warm-up, both timed regions and the diagnostics, some with one KV copy "
        "reused and so partly cache-warm):",
        "",
        "| kernel | calls | avg us | min us | max us | share |",
        "|---|---|---|---|---|---|",
    ]
    for r in rows:
        lines.append(
            f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
            f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |"
        )
    bench = None
    if bench_log:
        for line in open(bench_log):
            if line.startswith("{") and '"roofline"' in line:
                bench = json.loads(line)
    if trace_csv and bench:
        st = bench.get("settle", {})
        pre = int(st.get("timing_probe_steps", 0)) + int(st.get("steps", 0)) + int(bench["warmup"])
        k = int(bench["steps"])
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in csv.DictReader(open(trace_csv))
             if ATTENTION in r["Kernel_Name"]]
        for label, lo in (("region 1 (whole steps back to back)", pre),
                          ("region 2 (attention launches back to back; the roofline's source)", pre + k)):
            seg = d[lo:lo + k]
            if len(seg) == k:
                lines += [
                    "",
                    f"Attention launches of {label}, launches {lo + 1}-{lo + k} of {len(d)}: mean "
                    f"{statistics.mean(seg):.2f} us, median {statistics.median(seg):.2f} us, "
                    f"min {min(seg):.2f} us, max {max(seg):.2f} us.",
                ]
    if bench:
        r = bench["roofline"]
        lines += [
            "",
            f"The bench line of the same profiled run: step {bench['us_per_call']} us; attention launch "
            f"{r['kernel_avg_us']} us ({r.get('kernel_timing', 'HIP events')}), roofline frac {r['frac']}.",
        ]
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


def mfma_summary(counter_csv: str, out_md: str, command: str, flops_per_launch: int, mfma_peak_tflops: float) -> None:
    """MFMA busy share of the attention launch from SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES, GRBM_GUI_ACTIVE.

    GRBM_GUI_ACTIVE is summed over the 8 XCDs, so GRBM_GUI_ACTIVE / 8 is the launch's length in GPU cycles;
    SQ_VALU_MFMA_BUSY_CYCLES is taken as summed over the 1024 SIMDs (256 CUs x 4), so the busy share is
    MFMA_BUSY / (1024 * GRBM_GUI_ACTIVE / 8).  The algorithmic rate (flops / launch time / peak) is the
    cross-check of that reading."""
    vals: dict = {}
    for r in csv.DictReader(open(counter_csv)):
        if ATTENTION in r["Kernel_Name"]:
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    med = {k: statistics.median(v) for k, v in vals.items()}
    cycles = med["GRBM_GUI_ACTIVE"] / 8
    busy = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * cycles)
    lines = [
        "# MFMA utilisation of the attention launch",
        "",
        f"Command: `{command}`",
        "",
        f"Kernel sources hash: `{kernel_source_hash()}`",
        "",
        "| counter | median per dispatch |",
        "|---|---|",
    ] + [f"| {k} | {v:.0f} |" for k, v in sorted(med.items())] + [
        "",
        f"Launch length {cycles:.0f} GPU cycles (GRBM_GUI_ACTIVE / 8 XCDs); MFMA busy share "
        f"{busy:.3f} = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles).",
        f"Algorithmic: {flops_per_launch} flops per launch; at the launch length above and 2.4 GHz that is "
        f"{flops_per_launch / (cycles / 2.4e9) / 1e12:.0f} TFLOP/s, {flops_per_launch / (cycles / 2.4e9) / 1e12 / mfma_peak_tflops:.3f} "
        f"of the {mfma_peak_tflops:.0f} TFLOP/s dense peak of the P.V dtype.",
    ]
    open(out_md, "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    kind = sys.argv[1]
    if kind == "trace":
        trace_summary(sys.argv[2], sys.argv[3], sys.argv[4], *(sys.argv[5:7] + [None, None])[:2])
    elif kind == "mfma":
        mfma_summary(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5]), float(sys.argv[6]))
    elif kind == "pmc":
        pmc_summary(sys.argv[2], *sys.argv[3:7], int(sys.argv[7]), sys.argv[8], sys.argv[9])
    else:
        raise SystemExit(__doc__)
