"""Every attention-kernel form the dispatch can reach, against the float64 oracle.

The library picks one attention kernel per launch from five properties: the
dtype pair, whether the batch fits the kernel's in-LDS sequence table (1024
sequences) or not, the form (the plain decode with pages of one row, one
token and no soft-cap; the general form; the general form with the soft-cap),
and how many query tokens share one walk of the KV rows.  This file runs one
case for each reachable combination, through the C ABI, with the default
split over every compute unit and with 32-row shares, and compares the
sampled sequences with the oracle at the parity gate.  Batches beyond the
table use many short sequences, so the oracle stays fast.
"""

import numpy as np
import pytest
import torch

from mla_decode_paged_split_amd import synth

from mla_cases import DevCase, assert_parity, log, oracle_ref, to64

pytestmark = pytest.mark.gpu

PAIRS = [("bf16", "bf16"), ("bf16", "fp8"), ("fp8", "fp8")]
# (form, tokens per sequence): the general form is reached through pages of 8 rows with one token,
# or through several causal tokens per sequence with pages of one row
FORMS = [("plain", 1), ("general", 1), ("cap", 1), ("general", 2), ("cap", 2)]
TABLE = 1024  # sequences whose indptr values the attention kernel keeps in LDS


def _case(qd, kd, big, form, tokens, seed):
    rng = np.random.default_rng(seed)
    if big:
        batch = TABLE + 77
        lens = rng.integers(1, 60, size=batch).tolist()
    else:
        batch = 37
        lens = rng.integers(1, 400, size=batch).tolist()
        lens[3] = 2100  # one long sequence, split over several shares
    page = 8 if (form != "plain" and tokens == 1) else 1
    q_lens = rng.integers(1, 4, size=batch).tolist() if tokens > 1 else None
    spec = synth.CaseSpec(batch=batch, q_dtype=qd, kv_dtype=kd, lengths=lens, q_lens=q_lens, permuted=True,
                          extra_pool_rows=3 * page, page_size=page, seed=seed)
    return synth.make_case(spec)


@pytest.mark.parametrize("form,tokens", FORMS)
@pytest.mark.parametrize("big", [False, True], ids=["table", "beyond_table"])
@pytest.mark.parametrize("qd,kd", PAIRS)
def test_every_kernel_form(gpu, qd, kd, big, form, tokens):
    seed = 4000 + 100 * PAIRS.index((qd, kd)) + 10 * FORMS.index((form, tokens)) + (5 if big else 0)
    case = _case(qd, kd, big, form, tokens, seed)
    dc = DevCase(case, gpu)
    cap = 5.0 if form == "cap" else 0.0
    causal = tokens > 1
    if cap:  # larger queries so the cap bends the scores
        case.q_bf16 = (case.q_bf16.float() * 4.0).to(torch.bfloat16)
        dc = DevCase(case, gpu)
    batch = case.spec.batch
    seqs = sorted({0, 1, 3, batch // 2, batch - 1} | ({TABLE - 1, TABLE, TABLE + 1, TABLE + 40} if big else set()))
    qo = case.qo_indptr.tolist()
    rows = [t for b in seqs for t in range(qo[b], qo[b + 1])]
    ref = oracle_ref(case, sequences=seqs, causal=causal, logit_cap=cap)
    for units, chunk in ((0, 0), (256, 32)):
        log(f"[form {form} tokens={tokens} {qd}/{kd} batch={batch} page={case.spec.page_size} units={units}]")
        out = dc.run(num_units=units, min_chunk=chunk, causal=causal, logit_cap=cap, q_cast=qd == "fp8")
        torch.cuda.synchronize()
        got = to64(out)
        assert bool(np.all(np.isfinite(got[rows])))
        assert_parity(ref[rows], got[rows], f"{form}/{tokens} {qd}/{kd} big={big} u{units}")
