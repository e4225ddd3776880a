"""Full-size workloads in the launch configuration the bench times.

For each workload the GPU output is compared with the float64 oracle on
every sequence, and two properties are checked on every output: it is finite,
and each element lies within the range of its sequence's V column (the output
is a convex combination of V rows).
"""

import numpy as np
import pytest
import torch

import oracle
from mla_decode_paged_split_amd import binding, synth

from mla_cases import DevCase, Timer, assert_parity, log, oracle_ref, to64

pytestmark = pytest.mark.gpu

NAMES = list(synth.CONFIGS)


def convex_bound_ok(dc: DevCase, out: torch.Tensor) -> bool:
    """Every output row lies within the range of its sequence's V columns (a convex combination of V rows)."""
    case = dc.case
    kv = case.kv[:, :512]
    vals = kv.float() * (case.kv_scale if case.kv_scale is not None else 1.0)
    qo = case.qo_indptr.tolist()
    o = out.float().cpu()
    for b in range(dc.batch):
        rows = torch.from_numpy(oracle.paged_rows(case.kv_indptr.numpy(), case.kv_indices.numpy(), b,
                                                  case.spec.page_size, case.kv_last_page_len.numpy()))
        if rows.numel() == 0:
            continue
        hi = vals[rows].max(dim=0).values
        lo = vals[rows].min(dim=0).values
        slack = 2.0 ** -7 * torch.maximum(hi.abs(), lo.abs()) + 1e-6
        for t in range(qo[b], qo[b + 1]):
            if not bool(((o[t] <= hi + slack) & (o[t] >= lo - slack)).all()):
                log(f"  convex bound violated in sequence {b}, query row {t}")
                return False
    return True


@pytest.mark.parametrize("name", NAMES)
def test_full_config(gpu, name):
    spec = synth.CONFIGS[name]
    log(f"[config {name}]")
    with Timer("generate"):
        case = synth.make_case(spec)
    with Timer("to device"):
        dc = DevCase(case, gpu)
    # the launch configuration the bench times: one share per compute unit, separate merge launch,
    # fp8 Q cast inside the attention kernel
    out = dc.run(q_cast=spec.q_dtype == "fp8")
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    assert convex_bound_ok(dc, out)
    with Timer(f"oracle on all {case.spec.batch} sequences"):
        ref = oracle_ref(case)
    assert_parity(ref, to64(out), name)


@pytest.mark.parametrize("name", list(synth.FEATURE_WORKLOADS))
def test_full_feature_workload(gpu, name):
    spec, opts = synth.workload(name)
    log(f"[workload {name}]")
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    causal = bool(opts.get("causal"))
    cap = float(opts.get("logit_cap", 0.0))
    q_fp8 = None
    if opts.get("dynamic_q"):
        scratch = torch.empty(binding.MLA_QUANT_DYNAMIC_SCRATCH_BYTES, dtype=torch.uint8, device=gpu)
        binding.mla_decode_quantize_q_dynamic(dc.q_bf16, dc.q, dc.q_scale, scratch)
        q_fp8 = oracle.quantize_q_dynamic(case.q_bits().numpy())
        assert float(dc.q_scale.cpu()[0]) == q_fp8[1]
        out = dc.run(causal=causal, logit_cap=cap)
    else:
        out = dc.run(q_cast=spec.q_dtype == "fp8", causal=causal, logit_cap=cap)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    assert convex_bound_ok(dc, out)
    with Timer(f"oracle on all {case.spec.batch} sequences"):
        ref = oracle_ref(case, causal=causal, logit_cap=cap, q_fp8=q_fp8)
    assert_parity(ref, to64(out), name)
