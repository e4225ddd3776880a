"""Full-size workloads in the launch configuration the bench times.

For each workload the GPU output is compared with the float64 oracle on a
sample of sequences (first, middle, last, random ones and, for the ragged
case, the shortest and the longest), and two properties are checked on every
output: it is finite, and each element lies within the range of its
sequence's V column (the output is a convex combination of V rows).
"""

import zlib

import numpy as np
import pytest
import torch

from mla_decode_paged_split_amd import synth

from mla_cases import DevCase, Timer, assert_parity, log, oracle_ref, to64

pytestmark = pytest.mark.gpu

NAMES = list(synth.CONFIGS)


def sample_sequences(case, k_random=3, seed=0):
    B = case.spec.batch
    if B <= 8:
        return list(range(B))
    rng = np.random.default_rng(seed)
    picks = {0, 1, B // 2, B - 1, *rng.choice(B, size=k_random, replace=False).tolist()}
    lens = case.lengths.numpy()
    picks |= {int(lens.argmin()), int(lens.argmax())}
    return sorted(picks)


def convex_bound_ok(dc: DevCase, out: torch.Tensor) -> bool:
    kv = dc.kv[:, :512]
    vals = kv.float() * (dc.kv_scale if dc.kv_scale is not None else 1.0)
    indptr = dc.case.kv_indptr.tolist()
    o = out.float()
    ok = True
    for b in range(dc.batch):
        rows = dc.kv_indices[indptr[b]:indptr[b + 1]].long()
        hi = vals[rows].max(dim=0).values
        lo = vals[rows].min(dim=0).values
        slack = 2.0 ** -7 * torch.maximum(hi.abs(), lo.abs()) + 1e-6
        if not bool(((o[b] <= hi + slack) & (o[b] >= lo - slack)).all()):
            ok = False
            log(f"  convex bound violated in sequence {b}")
            break
    return ok


@pytest.mark.parametrize("name", NAMES)
def test_full_config(gpu, name):
    spec = synth.CONFIGS[name]
    log(f"[config {name}]")
    with Timer("generate"):
        case = synth.make_case(spec)
    with Timer("to device"):
        dc = DevCase(case, gpu)
    out = dc.run()  # the default plan: one share per compute unit, fused merge
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    assert convex_bound_ok(dc, out)
    seqs = sample_sequences(case, seed=zlib.crc32(name.encode()) % 1000)
    with Timer(f"oracle on {len(seqs)} sequences"):
        ref = oracle_ref(case, sequences=seqs)
    got = to64(out)
    assert_parity(ref[seqs], got[seqs], name)
