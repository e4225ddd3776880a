"""Benchmark one MLA-decode step on one MI355X and print one JSON line.

A step is one pass of the whole path over one batch: one mla_decode_run
(work split, split attention and the merge of split partials).  With fp8
queries the attention kernel casts the bf16 Q itself (step a0 fused); with
--separate-q-cast the step is the standalone cast launch followed by the
run, and the amax-scaled workload runs the two launches of
mla_decode_quantize_q_dynamic before it.  The plan is made once: it does not
depend on the sequence lengths.

Inputs are seeded synthetic tensors of the workload's shapes, resident in HBM
before the timed region.  The KV pool and its indices are replicated R times
(R copies together >= 1 GiB) and the steps rotate through the copies, so a
step cannot be served from the 256 MB last-level cache left warm by the
previous step.

Before the warm-up the bench runs about --settle-ms of untimed back-to-back
steps: started after idle, the device runs the first ~25 ms of back-to-back
steps up to ~1.35x slower, then holds a steady rate (--transient prints that
start-up series as a diagnostic).  The timed steps measure the settled rate.

Throughput is reported as algorithmic HBM bytes per second: KV rows read
(576 B for fp8, 1152 B for bf16) + 4 B per page index + Q + bf16 output +
both indptrs (+ the last-page lengths when pages hold several rows).  The
split partials are implementation overhead and are not counted; their
traffic shows up in the FETCH_SIZE / WRITE_SIZE counters.  The roofline
object times the attention launch alone: K mla_decode_attend launches back to
back between two HIP events on its stream (average per launch; a pair of
events around every launch would add their own handling, about 1 us, which
the diagnostics report separately).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}  # MI355X dense
METRIC = "MLA decode µs/call + achieved HBM GB/s (% peak), bs=64 kv=8192 fp8 KV"
DEFAULT_WORKLOAD = "m_bf16q_fp8kv_b64_kv8192"
KERNEL_SOURCES = ["mla_decode_paged_split_amd/csrc/mla_device.hpp", "mla_decode_paged_split_amd/csrc/mla_decode.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(spec, case, q_elt: int) -> int:
    """Bytes one attention launch must move at least: every KV row once, its page index, Q, O, indptrs."""
    kv_elt = 1 if spec.kv_dtype == "fp8" else 2
    B = spec.batch
    total_q = case.total_q
    pages = int(case.kv_indptr[-1])
    n = case.total_kv * 576 * kv_elt + pages * 4 + total_q * 16 * 576 * q_elt + total_q * 16 * 512 * 2
    n += 2 * (B + 1) * 4 + (B * 4 if spec.page_size > 1 else 0)
    return n


def mfma_flops(case, causal: bool) -> int:
    """Multiply-adds of the two contractions (16 heads x (576 + 512) per row each token sees), times 2."""
    per_row = 2 * 16 * (576 + 512)
    rows = 0
    qo = case.qo_indptr.tolist()
    for b, L in enumerate(case.lengths.tolist()):
        ql = qo[b + 1] - qo[b]
        for i in range(ql):
            rows += max(0, min(L, L - ql + 1 + i)) if causal else L
    return rows * per_row


def workload_label(name, spec, opts) -> str:
    lens = f"kv{spec.kv_len}" if not spec.ragged_max else f"kv U[1,{spec.ragged_max}] permuted"
    extra = []
    if spec.q_lens is not None:
        extra.append(f"q_len={max(spec.q_lens)}" + (" causal" if opts.get("causal") else ""))
    if opts.get("logit_cap"):
        extra.append(f"logit_cap={opts['logit_cap']}")
    if opts.get("dynamic_q"):
        extra.append("amax-scaled Q cast")
    tail = (" " + " ".join(extra)) if extra else ""
    return f"{name}: MLA decode b{spec.batch} {lens} {spec.q_dtype}-Q {spec.kv_dtype}-KV page_size={spec.page_size}{tail}"


def load_traffic(workload: str):
    """HBM bytes per attention launch from the committed counter summary, if it matches the current kernel."""
    path = os.path.join(ROOT, "profiles", f"mla_decode_kernel_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(case, opts, budget_s: float, single_thread_s: float = 0.0):
    """Time the float64 oracle on whole sequences until about budget_s of CPU work (all host threads the
    numeric library uses), then, if single_thread_s > 0, again with one thread for about that long."""
    import oracle

    res = _cpu_oracle_rate(case, opts, budget_s)
    if single_thread_s > 0:
        try:
            from threadpoolctl import threadpool_limits

            with threadpool_limits(limits=1):
                one = _cpu_oracle_rate(case, opts, single_thread_s)
            res["single_thread"] = {"value": one["value"], "unit": "GB/s", "cores": 1, "sample": one["sample"]}
        except ImportError:  # pragma: no cover
            pass
    return res


def _cpu_oracle_rate(case, opts, budget_s: float):
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    spec = case.spec
    q_bits = case.q_bits().numpy()
    q_scale = None
    if spec.q_dtype == "fp8":
        if opts.get("dynamic_q"):
            q_bits, q_scale = oracle.quantize_q_dynamic(q_bits)
        else:
            q_bits, q_scale = oracle.bf16_bits_to_fp8_bits(q_bits), 1.0
    kv_bits = case.kv_bits().numpy()
    qo = case.qo_indptr.numpy()
    kvp = case.kv_indptr.numpy()
    idx = case.kv_indices.numpy()
    last = case.kv_last_page_len.numpy()
    kv_scale = float(case.kv_scale[0]) if case.kv_scale is not None else None
    # whole passes over the batch (at least one sequence, at least one pass when it fits the budget)
    done = []
    passes = 0
    t0 = time.perf_counter()
    while True:
        for b in range(spec.batch):
            oracle.mla_decode(q_bits, kv_bits, qo, kvp, idx, q_dtype=spec.q_dtype, kv_dtype=spec.kv_dtype,
                              q_scale=q_scale, kv_scale=kv_scale, sequences=[b], page_size=spec.page_size,
                              kv_last_page_len=last, causal=bool(opts.get("causal")),
                              logit_cap=float(opts.get("logit_cap", 0.0)))
            done.append(b)
            if time.perf_counter() - t0 >= budget_s:
                break
        else:
            passes += 1
            continue
        break
    dt = time.perf_counter() - t0
    lens = case.lengths.numpy()
    rows = int(sum(int(lens[b]) for b in done))
    kv_elt = 1 if spec.kv_dtype == "fp8" else 2
    q_elt = 1 if spec.q_dtype == "fp8" else 2
    toks = int(sum(int(qo[b + 1] - qo[b]) for b in done))
    nb = len(done)
    bytes_done = rows * (576 * kv_elt + 4) + toks * (16 * 576 * q_elt + 16 * 512 * 2) + nb * 8
    sample = (f"{passes} full passes + {nb - passes * spec.batch} sequences of the {spec.batch}-sequence "
              f"batch ({rows} KV rows), float64 numpy, {dt:.1f} s")
    return {
        "value": bytes_done / dt / 1e9,
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": sample,
        "us_per_call_extrapolated": dt / nb * spec.batch * 1e6,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--cpu-budget-single", type=float, default=4.0,
                    help="seconds of oracle work with one host thread (0: skip)")
    ap.add_argument("--rotate-bytes", type=float, default=2**30, help="KV bytes to rotate through (cache defeat)")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed back-to-back steps for about this long before the warm-up (clock settling)")
    ap.add_argument("--transient", action="store_true",
                    help="after the bench line, time 20-step blocks right after an idle second (diagnostic)")
    ap.add_argument("--num-units", type=int, default=0)
    ap.add_argument("--min-chunk", type=int, default=0)
    ap.add_argument("--flags", type=int, default=0)
    ap.add_argument("--separate-q-cast", action="store_true",
                    help="fp8-Q workloads: cast Q with mla_decode_quantize_q before each run instead of in the kernel")
    ap.add_argument("--probe-copy", action="store_true", help="time a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the decode path runs on a single device.",
              file=sys.stderr)
        return 2

    import torch

    from mla_decode_paged_split_amd import binding, synth

    dev = torch.device("cuda:0")

    if args.probe_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / 10
        print(json.dumps({"probe": "copy", "bytes_read": n, "bytes_written": n, "ms": dt * 1e3,
                          "GBps_read_plus_write": 2 * n / dt / 1e9}))
        return 0

    spec, opts = synth.workload(args.workload)
    case = synth.make_case(spec)
    kv_bytes_one = case.kv.numel() * case.kv.element_size()
    R = max(1, min(16, math.ceil(args.rotate_bytes / max(kv_bytes_one, 1))))

    q_bf16 = case.q_bf16.to(dev)
    kvs = [case.kv.to(dev) for _ in range(R)]
    idxs = [case.kv_indices.to(dev) for _ in range(R)]
    qo_indptr = case.qo_indptr.to(dev)
    kv_indptr = case.kv_indptr.to(dev)
    last = case.kv_last_page_len.to(dev) if spec.page_size > 1 else None
    kv_scale = case.kv_scale.to(dev) if case.kv_scale is not None else None
    fp8_q = spec.q_dtype == "fp8"
    dynamic_q = bool(opts.get("dynamic_q"))
    sep_cast = fp8_q and (args.separate_q_cast or dynamic_q)
    q_in = torch.empty(q_bf16.shape, dtype=torch.uint8, device=dev) if sep_cast else q_bf16
    q_scale = torch.ones(1, dtype=torch.float32, device=dev) if fp8_q else None
    scratch = torch.empty(binding.MLA_QUANT_DYNAMIC_SCRATCH_BYTES, dtype=torch.uint8, device=dev)
    out = torch.empty((case.total_q, 16, 512), dtype=torch.bfloat16, device=dev)
    flags = args.flags | (binding.MLA_FLAG_FUSED_Q_CAST if fp8_q and not sep_cast else 0)
    causal = bool(opts.get("causal"))
    flags |= binding.MLA_FLAG_CAUSAL if causal else 0
    max_q = max(spec.q_lens) if spec.q_lens is not None else 1
    dec = binding.Decoder(spec.batch, spec.q_dtype, spec.kv_dtype, dev, num_units=args.num_units,
                          min_chunk=args.min_chunk, flags=flags, page_size=spec.page_size,
                          max_q_len=max_q if max_q > 1 else 0, total_q=case.total_q,
                          logit_cap=float(opts.get("logit_cap", 0.0)))
    sm_scale = 1.0 / 24.0
    stream = torch.cuda.current_stream()

    def attend(i: int):
        r = i % R
        binding.mla_decode_attend(dec.plan, q_in, kvs[r], qo_indptr, kv_indptr, idxs[r], last, q_scale, kv_scale,
                                  sm_scale, out, None, stream)

    def step(i: int, ev=None, ev_merge=None):
        if dynamic_q:
            binding.mla_decode_quantize_q_dynamic(q_bf16, q_in, q_scale, scratch, stream)
        elif sep_cast:
            binding.mla_decode_quantize_q(q_bf16, q_in, stream)
        if ev is not None:
            ev[0].record(stream)
        attend(i)
        if ev is not None:
            ev[1].record(stream)
        if ev_merge is not None:
            ev_merge[0].record(stream)
        binding.mla_decode_merge(dec.plan, qo_indptr, kv_indptr, out, None, stream)
        if ev_merge is not None:
            ev_merge[1].record(stream)

    # every event is created before the warm-up, so no host work idles the GPU between the two timed regions
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    # Settling: after idle the device first runs back-to-back steps up to ~1.35x slower, for ~25 ms, until
    # its clocks settle at their sustained level.  The timed steps follow that many milliseconds of untimed
    # back-to-back steps (the count from the time of a few probe steps), then the W warm-up steps.
    settle_steps = 0
    probe_steps = 0
    if args.settle_ms > 0:
        probe_steps = 8
        for i in range(3):
            step(i)
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(5):
            step(i)
        t_end.record(stream)
        torch.cuda.synchronize()
        est_ms = max(t_start.elapsed_time(t_end) / 5, 1e-3)
        settle_steps = int(math.ceil(args.settle_ms / est_ms))
        for i in range(settle_steps):
            step(i)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region 1: whole steps back to back
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / args.steps

    # timed region 2: the attention launch alone, K launches back to back (the same inputs and KV copies as
    # the steps; with fp8 Q cast separately, the cast of region 1 is left in q_in) between two events on
    # its stream: the launch's average duration, as the profiler sees it plus the gap between launches
    t_start.record(stream)
    for i in range(args.steps):
        attend(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    kern_avg_ms = t_start.elapsed_time(t_end) / args.steps
    # diagnostic: whole steps again, with the attention launch bracketed by its own pair of events (each
    # pair adds the events' own handling, ~1 us, to what it encloses)
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    kern_ms = sorted(a.elapsed_time(b) for a, b in evs)
    kern_ev_avg_ms = sum(kern_ms) / len(kern_ms)
    kern_med_ms = kern_ms[len(kern_ms) // 2]
    kern_p10_ms = kern_ms[len(kern_ms) // 10]
    kern_p90_ms = kern_ms[(len(kern_ms) * 9) // 10]

    # diagnostics (not the contract figures): the attention launch with one KV copy reused (rows warm in
    # the last-level cache where they fit), the plan call, and a plain streaming read on the same device
    n_diag = min(args.steps, 50)
    for i in range(n_diag):
        step(0, evs[i])
    torch.cuda.synchronize()
    hot_ms = sorted(a.elapsed_time(b) for a, b in evs[:n_diag])
    hot_med_ms = hot_ms[len(hot_ms) // 2]
    # the merge launch alone (rotating KV copies as in the timed regions)
    for i in range(n_diag):
        step(i, None, evs[i])
    torch.cuda.synchronize()
    merge_ms = sorted(a.elapsed_time(b) for a, b in evs[:n_diag])
    merge_avg_ms = sum(merge_ms) / len(merge_ms)
    torch.cuda.synchronize()
    plan_t0 = time.perf_counter()
    for _ in range(20):
        binding.mla_decode_plan(dec.params, dec.workspace, stream)
    torch.cuda.synchronize()
    plan_us = (time.perf_counter() - plan_t0) / 20 * 1e6
    cast_us = None
    if fp8_q:  # step a0 on its own: the unit-scale cast and the amax-scaled one (two launches)
        q8 = torch.empty(q_bf16.shape, dtype=torch.uint8, device=dev)
        qs_tmp = torch.ones(1, dtype=torch.float32, device=dev)
        cast_us = {}
        for label, fn in (("unit_scale_one_launch", lambda: binding.mla_decode_quantize_q(q_bf16, q8, stream)),
                          ("amax_scaled_two_launches", lambda: binding.mla_decode_quantize_q_dynamic(q_bf16, q8, qs_tmp, scratch,
                                                                                        stream))):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            t_start.record(stream)
            for _ in range(n_diag):
                fn()
            t_end.record(stream)
            torch.cuda.synchronize()
            cast_us[label] = round(t_start.elapsed_time(t_end) / n_diag * 1e3, 2)
        del q8, qs_tmp
    probe = torch.ones(1 << 30, dtype=torch.uint8, device=dev)  # 1 GiB
    sink = torch.empty(binding.read_probe_sink_words(1 << 30), dtype=torch.int32, device=dev)
    for _ in range(3):
        binding.mla_read_probe(probe, sink, stream)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(10):
        binding.mla_read_probe(probe, sink, stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    probe_gbs = probe.numel() * 10 / (t_start.elapsed_time(t_end) * 1e-3) / 1e9
    del probe
    # the same probe over exactly the attention launch's algorithmic bytes (rounded up to 16), one launch per
    # slice, rotating over slices that together exceed the last-level cache: the plain read rate at this size,
    # start-up and tail included, as the attention launch pays them
    q_elt = 1 if sep_cast else 2  # the attention launch reads fp8 Q, or bf16 Q it casts itself
    alg_bytes = algorithmic_bytes(spec, case, q_elt)
    n_slice = (alg_bytes + 15) // 16 * 16
    n_rot = max(2, math.ceil(args.rotate_bytes / n_slice))
    slab = torch.ones(n_slice * n_rot, dtype=torch.uint8, device=dev)
    sink = torch.empty(binding.read_probe_sink_words(n_slice), dtype=torch.int32, device=dev)
    slices = [slab[i * n_slice:(i + 1) * n_slice] for i in range(n_rot)]
    for i in range(2 * n_rot):
        binding.mla_read_probe(slices[i % n_rot], sink, stream)
    torch.cuda.synchronize()
    for i in range(n_diag):
        evs[i][0].record(stream)
        binding.mla_read_probe(slices[i % n_rot], sink, stream)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    same_ms = sorted(a.elapsed_time(b) for a, b in evs[:n_diag])
    same_ev_avg_ms = sum(same_ms) / len(same_ms)
    t_start.record(stream)  # back to back, timed like the attention launch
    for i in range(n_diag):
        binding.mla_read_probe(slices[i % n_rot], sink, stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    same_avg_ms = t_start.elapsed_time(t_end) / n_diag
    del slab, slices, sink

    q_prep = 0
    if dynamic_q:
        q_prep = q_bf16.numel() * 5  # amax pass reads 2 B, cast pass reads 2 B and writes 1 B per value
    elif sep_cast:
        q_prep = q_bf16.numel() * 3
    step_bytes = alg_bytes + q_prep
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (kern_avg_ms * 1e-3) / 1e9
    flops = mfma_flops(case, causal)
    mfma_dtype = "fp8" if spec.q_dtype == "fp8" else "bf16"  # QK in fp8 for a8w8; P.V always bf16
    mfma_tflops = flops / (kern_avg_ms * 1e-3) / 1e12

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(ms_per_step * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if fp8_q else "bf16",
        "data": "synthetic",
        "config": {
            "workload": workload_label(args.workload, spec, opts),
            "batch": spec.batch,
            "q_seq_len": max_q,
            "kv_len": spec.kv_len if not spec.ragged_max else f"U[1,{spec.ragged_max}]",
            "total_kv_rows": case.total_kv,
            "q_dtype": spec.q_dtype,
            "kv_dtype": spec.kv_dtype,
            "heads": 16,
            "qk_dim": 576,
            "v_dim": 512,
            "page_size": spec.page_size,
            "causal": causal,
            "logit_cap": float(opts.get("logit_cap", 0.0)),
            "kv_copies_rotated": R,
            "num_units": int(dec.plan.params.num_units),
            "min_chunk": int(dec.plan.params.min_chunk),
            "fused_merge": bool(args.flags & binding.MLA_FLAG_FUSED_MERGE),
            "q_cast": (("amax-scaled, two launches" if dynamic_q else "separate launch") if sep_cast
                       else "in the attention kernel") if fp8_q else None,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": load_traffic(args.workload),
            "kernel": "mla_decode_kernel",
            "algorithmic_bytes_per_launch": alg_bytes,
            "kernel_avg_us": round(kern_avg_ms * 1e3, 2),
            "kernel_timing": f"{args.steps} attention launches back to back between two HIP events on its stream",
            "per_launch_events": {
                "avg_us": round(kern_ev_avg_ms * 1e3, 2),
                "median_us": round(kern_med_ms * 1e3, 2),
                "p10_us": round(kern_p10_ms * 1e3, 2),
                "p90_us": round(kern_p90_ms * 1e3, 2),
            },
            "mfma": {
                "flops_per_launch": flops,
                "achieved_tflops": round(mfma_tflops, 1),
                "peak_tflops": PEAK_MFMA_TFLOPS[mfma_dtype],
                "dtype": mfma_dtype,
                "frac": round(mfma_tflops / PEAK_MFMA_TFLOPS[mfma_dtype], 4),
            },
        },
        "diagnostics": {
            "attention_median_us_one_kv_copy_reused": round(hot_med_ms * 1e3, 2),
            "merge_avg_us_per_launch_events": round(merge_avg_ms * 1e3, 2),
            "step_minus_attention_us": round((ms_per_step - kern_avg_ms) * 1e3, 2),
            "plan_us_per_call_host": round(plan_us, 1),
            "q_cast_us": cast_us,
            "read_probe": {
                "kind": "mla_read_probe: one pass of 512-thread workgroups, four 16-byte non-temporal loads per "
                        "thread, over 1 GiB, same device",
                "GBps": round(probe_gbs, 1),
                "attention_frac_of_probe": round(achieved / probe_gbs, 4),
            },
            "read_probe_same_bytes": {
                "kind": "mla_read_probe over the attention launch's algorithmic bytes, one launch each, "
                        f"rotating over {n_rot} slices, back to back between two HIP events",
                "bytes": n_slice,
                "avg_us": round(same_avg_ms * 1e3, 2),
                "avg_us_per_launch_events": round(same_ev_avg_ms * 1e3, 2),
                "GBps": round(n_slice / (same_avg_ms * 1e-3) / 1e9, 1),
                "frac_of_peak": round(n_slice / (same_avg_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "attention_time_over_probe": round(kern_avg_ms / same_avg_ms, 4),
            },
        },
        "settle": {"ms": args.settle_ms, "steps": settle_steps, "timing_probe_steps": probe_steps},
        "wall_s_timed": round(wall, 4),
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case, opts, args.cpu_budget, args.cpu_budget_single)
    print(json.dumps(res), flush=True)
    if args.transient:
        # whole steps in blocks of 20 right after one idle second: the settling that the timed region skips
        blk, nblk = 20, max(1, int(math.ceil(60.0 / (ms_per_step * 20))))
        bev = [torch.cuda.Event(enable_timing=True) for _ in range(nblk + 1)]
        torch.cuda.synchronize()
        time.sleep(1.0)
        bev[0].record(stream)
        for b in range(nblk):
            for i in range(blk):
                step(b * blk + i)
            bev[b + 1].record(stream)
        torch.cuda.synchronize()
        series = [round(bev[b].elapsed_time(bev[b + 1]) / blk * 1e3, 2) for b in range(nblk)]
        print(json.dumps({"transient_us_per_step_20_step_blocks_after_idle": series,
                          "settled_us_per_step": round(ms_per_step * 1e3, 2)}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
