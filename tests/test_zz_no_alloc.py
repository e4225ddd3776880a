"""The entry point that allocates nothing (mla_decode_run_noalloc) against the plan-based one.

mla_decode_run_noalloc runs the same kernels as mla_decode_run_paged with the
library's own scratch array as the workspace, so with the same parameters its
output must equal that of mla_decode_run_paged bit for bit, and both must
match the float64 oracle.  Two calls in a row share the scratch array; the
second has a smaller input (fewer sequences, so its arrival counters overlap
where the first call left its split record).
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from mla_decode_paged_split_amd import binding, synth

from mla_cases import DevCase, assert_parity, log, oracle_ref, to64

pytestmark = pytest.mark.gpu


def _both(dc, flags, units=0, page_lens=None):
    """(no-alloc output, no-alloc lse, plan-based output, plan-based lse) for one case."""
    case = dc.case
    kw = dict(num_units=units, flags=flags, page_size=dc.page_size,
              max_q_len=dc.max_q_len if dc.max_q_len > 1 else 0, total_q=dc.total_q)
    params = binding.make_params(dc.batch, dc.q_dtype, dc.kv_dtype, **kw)
    last = dc.kv_last_page_len if dc.page_size > 1 else None
    out_n = torch.full((case.total_q, 16, 512), float("nan"), dtype=torch.bfloat16, device=dc.dev)
    lse_n = torch.full((case.total_q, 16), float("nan"), dtype=torch.float32, device=dc.dev)
    binding.mla_decode_run_noalloc(params, dc.q, dc.kv, dc.qo_indptr, dc.kv_indptr, dc.kv_indices, last, dc.q_scale,
                                   dc.kv_scale, oracle.SM_SCALE, out_n, lse_n)
    dec = binding.Decoder(dc.batch, dc.q_dtype, dc.kv_dtype, dc.dev, **kw)
    out_p = torch.full_like(out_n, float("nan"))
    lse_p = torch.full_like(lse_n, float("nan"))
    binding.mla_decode_run_paged(dec.plan, dc.q, dc.kv, dc.qo_indptr, dc.kv_indptr, dc.kv_indices, last, dc.q_scale,
                                 dc.kv_scale, oracle.SM_SCALE, out_p, lse_p)
    torch.cuda.synchronize()
    return out_n, lse_n, out_p, lse_p


@pytest.mark.parametrize("flags", [0, binding.MLA_FLAG_FUSED_MERGE])
def test_noalloc_matches_plan_based_run_twice(gpu, flags):
    rng = np.random.default_rng(7100)
    big = synth.CaseSpec(batch=80, q_dtype="bf16", kv_dtype="fp8", lengths=rng.integers(1, 3000, size=80).tolist(),
                         permuted=True, extra_pool_rows=11, seed=7101)
    small = synth.CaseSpec(batch=5, q_dtype="bf16", kv_dtype="fp8", lengths=[700, 1, 2049, 64, 300], permuted=True,
                           seed=7102)
    for spec in (big, small):  # the second call is the smaller one
        case = synth.make_case(spec)
        dc = DevCase(case, gpu)
        log(f"[no-alloc flags={flags} batch={spec.batch}]")
        out_n, lse_n, out_p, lse_p = _both(dc, flags)
        assert torch.equal(out_n.view(torch.int16), out_p.view(torch.int16))
        assert torch.equal(lse_n.view(torch.int32), lse_p.view(torch.int32))
        assert_parity(oracle_ref(case), to64(out_n), f"no-alloc batch {spec.batch} flags {flags}")


def test_noalloc_other_forms(gpu):
    # a8w8 with pages of 8 rows and several causal tokens (the general form), then the plain decode again
    spec = synth.CaseSpec(batch=6, q_dtype="fp8", kv_dtype="fp8", lengths=[3, 17, 1000, 4100, 64, 9],
                          q_lens=[2, 3, 1, 2, 2, 1], permuted=True, extra_pool_rows=40, page_size=8, seed=7200)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    # three tokens per sequence need 3 partial rows per slot: 64 shares keep the workspace inside the array
    out_n, _, out_p, _ = _both(dc, binding.MLA_FLAG_CAUSAL, units=64)
    assert torch.equal(out_n.view(torch.int16), out_p.view(torch.int16))
    assert_parity(oracle_ref(case, causal=True), to64(out_n), "no-alloc general form")
    spec2 = synth.CaseSpec(batch=3, q_dtype="bf16", kv_dtype="bf16", lengths=[5, 900, 33], seed=7201)
    case2 = synth.make_case(spec2)
    dc2 = DevCase(case2, gpu)
    out_n, _, out_p, _ = _both(dc2, 0)
    assert torch.equal(out_n.view(torch.int16), out_p.view(torch.int16))
    assert_parity(oracle_ref(case2), to64(out_n), "no-alloc bf16/bf16")


def test_noalloc_rejects_a_workspace_beyond_its_array(gpu):
    spec = synth.CaseSpec(batch=4, q_dtype="bf16", kv_dtype="fp8", lengths=[100, 200, 300, 400], seed=7300)
    dc = DevCase(synth.make_case(spec), gpu)
    params = binding.make_params(4, "bf16", "fp8", num_units=4096)  # 2 * 4096 partial slots: 256 MiB
    assert binding.mla_decode_workspace_size(params) > binding.MLA_NOALLOC_SCRATCH_BYTES
    out = torch.full((4, 16, 512), float("nan"), dtype=torch.bfloat16, device=gpu)
    code = binding.lib().mla_decode_run_noalloc(
        ctypes.byref(params), dc.q.data_ptr(), dc.kv.data_ptr(), dc.qo_indptr.data_ptr(), dc.kv_indptr.data_ptr(),
        dc.kv_indices.data_ptr(), None, None, dc.kv_scale.data_ptr(), oracle.SM_SCALE, out.data_ptr(), None,
        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert code == binding.MLA_ERR_WORKSPACE
    assert bool(torch.isnan(out.float()).all())  # nothing was launched
    # the largest accepted share count still runs
    params = binding.make_params(4, "bf16", "fp8", num_units=256)
    assert binding.mla_decode_workspace_size(params) <= binding.MLA_NOALLOC_SCRATCH_BYTES
    binding.mla_decode_run_noalloc(params, dc.q, dc.kv, dc.qo_indptr, dc.kv_indptr, dc.kv_indices, None, None,
                                   dc.kv_scale, oracle.SM_SCALE, out)
    torch.cuda.synchronize()
    assert_parity(oracle_ref(dc.case), to64(out), "no-alloc 256 units")
