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


# ------------------------------------------------------- amax-scaled Q cast

import oracle  # noqa: E402


def _dyn_cast(gpu, bits_np):
    src = torch.from_numpy(bits_np.astype(np.int16)).view(torch.bfloat16).to(gpu)
    dst = torch.empty(src.numel(), dtype=torch.uint8, device=gpu)
    scale = torch.full((1,), -1.0, dtype=torch.float32, device=gpu)
    scratch = torch.empty(binding.MLA_QUANT_DYNAMIC_SCRATCH_BYTES, dtype=torch.uint8, device=gpu)
    binding.mla_decode_quantize_q_dynamic(src.reshape(-1), dst, scale, scratch)
    torch.cuda.synchronize()
    return dst.cpu().numpy(), float(scale.cpu()[0])


@pytest.mark.parametrize("mag", [1e-3, 1.0, 37.0, 3e4])
@pytest.mark.parametrize("n", [16 * 576 * 3, 16 * 576 * 3 - 5, 999])
def test_dynamic_q_cast_bit_exact(gpu, mag, n):
    rng = np.random.default_rng(2800 + n)
    x = torch.from_numpy(rng.standard_normal(n).astype(np.float32) * mag).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().astype(np.uint16)
    bits[: min(n, 40)] = rng.integers(0, 1 << 16, size=min(n, 40))  # every exponent range, NaN / inf included
    codes, scale = _dyn_cast(gpu, bits)
    want_codes, want_scale = oracle.quantize_q_dynamic(bits)
    assert np.float32(scale) == np.float32(want_scale)
    bad = np.nonzero(codes != want_codes)[0]
    assert bad.size == 0, f"{bad.size} codes differ, first at {bad[0]}: bits {bits[bad[0]]:#06x} got {codes[bad[0]]:#x} want {want_codes[bad[0]]:#x}"


def test_dynamic_q_cast_unaligned_view(gpu):
    rng = np.random.default_rng(2900)
    x = torch.from_numpy(rng.standard_normal(5000).astype(np.float32) * 3.0).to(torch.bfloat16).to(gpu)
    src = x[3:-2]  # 6-byte offset: the element-by-element amax path
    dst = torch.empty(src.numel() + 1, dtype=torch.uint8, device=gpu)[1:]
    scale = torch.empty(1, dtype=torch.float32, device=gpu)
    scratch = torch.empty(binding.MLA_QUANT_DYNAMIC_SCRATCH_BYTES, dtype=torch.uint8, device=gpu)
    binding.mla_decode_quantize_q_dynamic(src, dst, scale, scratch)
    torch.cuda.synchronize()
    want_codes, want_scale = oracle.quantize_q_dynamic(src.cpu().view(torch.int16).numpy())
    assert float(scale.cpu()[0]) == want_scale
    assert np.array_equal(dst.cpu().numpy(), want_codes)


def test_dynamic_q_cast_degenerate(gpu):
    codes, scale = _dyn_cast(gpu, np.array([0x0000, 0x8000, 0x0000], dtype=np.uint16))
    assert scale == 1.0 and codes.tolist() == [0x00, 0x80, 0x00]
    codes, scale = _dyn_cast(gpu, np.zeros(0, dtype=np.uint16))
    assert scale == 1.0 and codes.size == 0
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x7F80, 0xFF80, 0x7FC1, 0xFFC1], dtype=np.uint16)  # 1, -2, .5, inf...
    codes, scale = _dyn_cast(gpu, bits)
    assert np.float32(scale) == np.float32(2.0) / np.float32(448.0)
    assert codes.tolist()[1] == 0xFE and codes.tolist()[3:] == [0x7F, 0xFF, 0x7F, 0xFF]


def test_decode_with_dynamic_q_scale(gpu):
    spec = synth.CaseSpec(batch=4, q_dtype="fp8", kv_dtype="fp8", lengths=[7, 300, 1500, 64], permuted=True,
                          seed=3000)
    case = synth.make_case(spec)
    case.q_bf16 = (case.q_bf16.float() * 60.0).to(torch.bfloat16)  # |q| up to ~300: the scale is not 1
    dc = DevCase(case, gpu)
    scratch = torch.empty(binding.MLA_QUANT_DYNAMIC_SCRATCH_BYTES, dtype=torch.uint8, device=gpu)
    binding.mla_decode_quantize_q_dynamic(dc.q_bf16, dc.q, dc.q_scale, scratch)
    codes, q_scale = oracle.quantize_q_dynamic(case.q_bits().numpy())
    assert float(dc.q_scale.cpu()[0]) == q_scale and q_scale != 1.0
    assert np.array_equal(dc.q.cpu().numpy().reshape(codes.shape), codes)
    ref = oracle.mla_decode(codes, case.kv_bits().numpy(), case.qo_indptr.numpy(), case.kv_indptr.numpy(),
                            case.kv_indices.numpy(), q_dtype="fp8", kv_dtype="fp8", q_scale=q_scale,
                            kv_scale=float(case.kv_scale[0]))
    for units in (1, 64):
        out = dc.run(num_units=units, min_chunk=32)
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"dynamic q_scale u{units}")


# ------------------------------------------------------------------- edge cases

def test_sequences_without_query_tokens(gpu):
    # q_len 0 for some sequences: nothing is computed for them, the other tokens are unaffected
    lens, q_lens = [100, 700, 5, 2000], [2, 0, 3, 0]
    spec = synth.CaseSpec(batch=4, q_dtype="bf16", kv_dtype="fp8", lengths=lens, q_lens=q_lens, permuted=True,
                          seed=3600)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    ref = oracle_ref(case, causal=True)
    for units, flags in ((1, 0), (64, 0), (64, 1)):
        out = dc.run(num_units=units, min_chunk=32, flags=flags, causal=True)
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"q_len 0 u{units} f{flags}")


def test_last_page_lengths_out_of_range_are_clamped(gpu):
    # last-page lengths of 0 and above the page size read as 1 and as a full page, as in the oracle
    spec = synth.CaseSpec(batch=4, q_dtype="fp8", kv_dtype="fp8", lengths=[40, 9, 64, 17], permuted=True,
                          page_size=16, extra_pool_rows=64, seed=3700)
    case = synth.make_case(spec)
    case.kv_last_page_len = torch.tensor([0, 99, -5, 16], dtype=torch.int32)
    dc = DevCase(case, gpu)
    ref = oracle_ref(case)  # the oracle clamps into [1, page_size] itself
    for units in (1, 8, 64):
        out = dc.run(num_units=units, min_chunk=32)
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"clamped last pages u{units}")


@pytest.mark.parametrize("ps", [256, 1024])
def test_large_pages(gpu, ps):
    lens = [1, ps - 3, ps + 1, 3 * ps]
    spec = synth.CaseSpec(batch=4, q_dtype="bf16", kv_dtype="fp8", lengths=lens, permuted=True, page_size=ps,
                          extra_pool_rows=ps, seed=3800 + ps)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    ref = oracle_ref(case)
    for units in (1, 16, 256):
        out = dc.run(num_units=units, min_chunk=32)
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"ps{ps} u{units}")


@pytest.mark.parametrize("qd,kd", PAIRS)
def test_most_tokens_per_sequence(gpu, qd, kd):
    """max_q_len 16, the most the library takes: eight two-token passes over each piece.  A 9-row sequence
    with 16 causal tokens leaves its first 7 tokens without a visible row (zeros); a long one is split."""
    lens, q_lens = [9, 3000, 600], [16, 16, 5]
    spec = synth.CaseSpec(batch=3, q_dtype=qd, kv_dtype=kd, lengths=lens, q_lens=q_lens, permuted=True,
                          extra_pool_rows=7, seed=3700 + PAIRS.index((qd, kd)))
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    ref = oracle_ref(case, causal=True)
    for units, flags in ((1, 0), (32, 0), (256, binding.MLA_FLAG_FUSED_MERGE)):
        log(f"[16 tokens {qd}/{kd} units={units} flags={flags}]")
        out = dc.run(num_units=units, min_chunk=32, flags=flags, causal=True, q_cast=qd == "fp8")
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"16 tokens {qd}/{kd} u{units} f{flags}")
        assert torch.equal(out[:7].cpu().float(), torch.zeros(7, 16, 512))
