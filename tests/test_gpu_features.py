"""GPU parity of the widened decode forms against the float64 oracle.

Pages of several rows (mla_decode_run_paged with last-page lengths), several
query tokens per sequence with and without the causal rule, and the logit
soft-cap, each across the dtype pairs and work splits from one workgroup per
sequence down to 32-row shares, plus their combination.
"""

import numpy as np
import pytest
import torch

from mla_decode_paged_split_amd import binding, synth

from mla_cases import DevCase, assert_parity, log, oracle_ref, to64

pytestmark = pytest.mark.gpu

PAIRS = [("bf16", "bf16"), ("bf16", "fp8"), ("fp8", "fp8")]
SPLITS = [(1, 32, 0), (8, 32, 0), (256, 32, 0), (256, 32, 1)]  # (num_units, min_chunk, flags)


@pytest.mark.parametrize("ps", [2, 8, 16, 64])
@pytest.mark.parametrize("qd,kd", PAIRS)
def test_paged_parity(gpu, ps, qd, kd):
    lens = [1, ps - 1 if ps > 1 else 1, ps, ps + 1, 3 * ps + 5, 700, 2053]
    spec = synth.CaseSpec(batch=len(lens), q_dtype=qd, kv_dtype=kd, lengths=lens, permuted=True,
                          extra_pool_rows=5 * ps, page_size=ps, seed=2100 + ps + 7 * PAIRS.index((qd, kd)))
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    ref = oracle_ref(case)
    for units, chunk, flags in SPLITS:
        log(f"[paged ps={ps} {qd}/{kd} units={units} min_chunk={chunk} flags={flags}]")
        out = dc.run(num_units=units, min_chunk=chunk, flags=flags)
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"ps{ps} {qd}/{kd} u{units} f{flags}")


def test_paged_full_pages_match_run(gpu):
    # with every last page full, mla_decode_run and mla_decode_run_paged give identical bits
    spec = synth.CaseSpec(batch=4, q_dtype="bf16", kv_dtype="fp8", lengths=[16, 64, 160, 8], permuted=True,
                          page_size=8, seed=2200)
    dc = DevCase(synth.make_case(spec), gpu)
    a = dc.run(num_units=16, min_chunk=32, paged=True).cpu()
    b = dc.run(num_units=16, min_chunk=32, paged=False).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_page_size_one_ignores_last_page_len(gpu):
    # page size 1 with the sequence length passed as the last-page length (one page does this)
    spec = synth.CaseSpec(batch=3, q_dtype="bf16", kv_dtype="fp8", lengths=[5, 300, 64], permuted=True, seed=2300)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    a = dc.run(num_units=8, min_chunk=32).cpu()
    dc.kv_last_page_len = case.lengths.to(torch.int32).to(gpu)
    b = dc.run(num_units=8, min_chunk=32, paged=True).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


QL_CASES = [
    # lengths, tokens per sequence
    ([1, 40, 129, 2000, 3, 700], [1, 2, 2, 2, 2, 1]),
    ([5, 300, 1000, 2, 64, 9000], [4, 3, 1, 4, 2, 3]),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("qd,kd", PAIRS)
@pytest.mark.parametrize("ci", range(len(QL_CASES)))
def test_multi_token_parity(gpu, causal, qd, kd, ci):
    lens, q_lens = QL_CASES[ci]
    spec = synth.CaseSpec(batch=len(lens), q_dtype=qd, kv_dtype=kd, lengths=lens, q_lens=q_lens, permuted=True,
                          extra_pool_rows=13, seed=2400 + 10 * ci + PAIRS.index((qd, kd)))
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    ref = oracle_ref(case, causal=causal)
    for units, chunk, flags in SPLITS:
        log(f"[tokens {q_lens} causal={causal} {qd}/{kd} units={units} flags={flags}]")
        out = dc.run(num_units=units, min_chunk=chunk, flags=flags, causal=causal)
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"tokens causal={causal} {qd}/{kd} u{units} f{flags}")
    if causal and ci == 1:
        # token 0 of the 2-row sequence with 4 tokens sees no row: zeros
        t = int(case.qo_indptr[3])
        assert torch.equal(out[t].cpu().float(), torch.zeros(16, 512))


@pytest.mark.parametrize("qd,kd", PAIRS)
def test_general_kernel_matches_plain_decode(gpu, qd, kd):
    # a plan for several tokens (the general kernel: page arithmetic, soft-cap and token passes compiled
    # in) run on one-token sequences with pages of one row equals the plain-decode kernel bit for bit
    spec = synth.CaseSpec(batch=5, q_dtype=qd, kv_dtype=kd, lengths=[300, 1, 77, 1024, 45], permuted=True,
                          seed=2500)
    dc = DevCase(synth.make_case(spec), gpu)
    for units in (1, 16, 256):
        a = dc.run(num_units=units, min_chunk=32).cpu()
        b = dc.run(num_units=units, min_chunk=32, max_q_len=4).cpu()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), units


@pytest.mark.parametrize("cap", [1.0, 30.0])
@pytest.mark.parametrize("qd,kd", PAIRS)
def test_logit_cap_parity(gpu, cap, qd, kd):
    lens = [1, 33, 500, 2049]
    spec = synth.CaseSpec(batch=len(lens), q_dtype=qd, kv_dtype=kd, lengths=lens, permuted=True, seed=2600)
    case = synth.make_case(spec)
    # larger queries so the cap bends the scores (|s| ~ 4 before capping)
    case.q_bf16 = (case.q_bf16.float() * 4.0).to(torch.bfloat16)
    dc = DevCase(case, gpu)
    ref = oracle_ref(case, logit_cap=cap)
    plain = oracle_ref(case)
    assert np.max(np.abs(ref - plain)) > 1e-2  # the cap matters at these sizes
    for units, chunk, flags in SPLITS:
        out = dc.run(num_units=units, min_chunk=chunk, flags=flags, logit_cap=cap)
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"cap={cap} {qd}/{kd} u{units} f{flags}")


def test_everything_combined(gpu):
    lens = [3, 17, 1000, 4100, 64]
    q_lens = [2, 3, 1, 4, 2]
    spec = synth.CaseSpec(batch=len(lens), q_dtype="fp8", kv_dtype="fp8", lengths=lens, q_lens=q_lens, permuted=True,
                          extra_pool_rows=40, page_size=16, seed=2700)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    ref = oracle_ref(case, causal=True, logit_cap=5.0)
    for units, chunk, flags in SPLITS:
        out = dc.run(num_units=units, min_chunk=chunk, flags=flags, causal=True, logit_cap=5.0)
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"combined u{units} f{flags}")
    fused = dc.run(num_units=64, min_chunk=32, causal=True, logit_cap=5.0, q_cast=True)
    assert_parity(ref, to64(fused), "combined fused cast")
