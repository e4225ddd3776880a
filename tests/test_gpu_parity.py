"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Small cases span several 32-row tiles with ragged tails, every dtype pair,
and work splits from one workgroup per sequence down to 32-row shares (more
than 64 pieces per sequence).  Invariants that need no oracle are checked too:
split count, pool permutation, determinism, empty sequences, closed forms.
"""

import time

import numpy as np
import pytest
import torch

import oracle
from mla_decode_paged_split_amd import binding, synth

from mla_cases import DevCase, Timer, assert_parity, compare, log, oracle_ref, to64

pytestmark = pytest.mark.gpu

PAIRS = [("bf16", "bf16"), ("bf16", "fp8"), ("fp8", "fp8")]
PIECE_COST_ROWS = 256  # the split's per-sequence cost, in rows
LENGTHS = [1, 2, 31, 32, 33, 64, 100, 257, 513, 1000, 2053]
# (num_units, min_chunk, flags): one share for everything, a few shares, many
# shares, and 32-row shares (up to 65 pieces for the 2053-row sequence)
SPLITS = [(1, 32, 0), (8, 32, 0), (8, 32, 1), (256, 32, 0), (4096, 32, 0), (4096, 32, 1)]  # flag 1: fused merge


def test_device_facts(gpu):
    p = torch.cuda.get_device_properties(0)
    log(f"  device={p.name} gcn={getattr(p, 'gcnArchName', '?')} CUs={p.multi_processor_count} "
        f"mem={p.total_memory / 2**30:.0f}GiB")
    assert "gfx950" in getattr(p, "gcnArchName", "gfx950")


def test_quantize_q_exhaustive_bit_exact(gpu):
    codes = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16)
    src = codes.view(torch.bfloat16).to(gpu)
    dst = torch.empty(1 << 16, dtype=torch.uint8, device=gpu)
    binding.mla_decode_quantize_q(src, dst)
    torch.cuda.synchronize()
    expect = oracle.bf16_bits_to_fp8_bits(codes.numpy())
    got = dst.cpu().numpy()
    bad = np.nonzero(got != expect)[0]
    assert bad.size == 0, f"{bad.size} codes differ, first {hex(bad[0])}: got {got[bad[0]]:#x} want {expect[bad[0]]:#x}"


def test_quantize_q_unaligned_tail(gpu):
    codes = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16)
    big = codes.view(torch.bfloat16).to(gpu)
    src = big[1:-2]  # 2-byte offset: takes the element-by-element path
    dst_buf = torch.empty(src.numel() + 3, dtype=torch.uint8, device=gpu)
    dst = dst_buf[3:]
    binding.mla_decode_quantize_q(src, dst)
    torch.cuda.synchronize()
    expect = oracle.bf16_bits_to_fp8_bits(codes.numpy()[1:-2])
    assert np.array_equal(dst.cpu().numpy(), expect)


@pytest.mark.parametrize("qd,kd", PAIRS)
def test_parity_small_all_splits(gpu, qd, kd):
    spec = synth.CaseSpec(batch=len(LENGTHS), q_dtype=qd, kv_dtype=kd, lengths=LENGTHS, permuted=True,
                          extra_pool_rows=37, seed=100 + 10 * PAIRS.index((qd, kd)))
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    with Timer("oracle"):
        ref = oracle_ref(case)
    for units, chunk, flags in SPLITS:
        log(f"[parity {qd}/{kd} units={units} min_chunk={chunk} flags={flags}]")
        out = dc.run(num_units=units, min_chunk=chunk, flags=flags)
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"{qd}/{kd} u{units} c{chunk} f{flags}")


@pytest.mark.parametrize("qd,kd", PAIRS)
def test_split_count_invariance(gpu, qd, kd):
    """Any split gives the unsplit result up to the bf16 rounding of the softmax weights.

    The P.V product takes the weights p_i = 2^(x_i - m) rounded to bf16
    (relative error <= 2^-9 each), and m is each piece's own running max, so
    two splits round differently.  Elementwise the outputs can then differ by
    at most 2^-8 * max_i |v_i - O| (two roundings of each weight) plus one bf16
    rounding of each output (2^-9 |O|); that bound uses 2 max_i |v_i| for
    max_i |v_i - O|.  Statistically the weight errors average out, so the
    normwise difference must also stay below 5e-3.
    """
    spec = synth.CaseSpec(batch=4, q_dtype=qd, kv_dtype=kd, lengths=[4000, 129, 2049, 700], seed=300)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    vmax = np.zeros((4, 512))
    for b in range(4):
        rows = case.kv_indices[case.kv_indptr[b]:case.kv_indptr[b + 1]].long()
        v = case.kv[rows, :512].float() * (case.kv_scale if case.kv_scale is not None else 1.0)
        vmax[b] = v.abs().max(dim=0).values.double().numpy()
    base = to64(dc.run(num_units=1, min_chunk=32))  # one workgroup, nothing split
    for units in (2, 3, 7, 64, 1024):
        got = to64(dc.run(num_units=units, min_chunk=32))
        d = np.abs(got - base)
        bound = 2.0 ** -8 * 2 * vmax[:, None, :] + 2.0 ** -8 * np.abs(base) + 1e-6
        nrm = float(np.linalg.norm(got - base) / np.linalg.norm(base))
        log(f"  units={units}: max|diff|={d.max():.3e} normwise={nrm:.2e} max(diff/bound)={np.max(d / bound):.3f}")
        assert np.all(d <= bound) and nrm <= 5e-3


def test_pool_permutation_bit_identical(gpu):
    spec = synth.CaseSpec(batch=5, q_dtype="bf16", kv_dtype="fp8", lengths=[300, 1, 77, 1024, 45], seed=400)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    a = dc.run(num_units=16, min_chunk=64).cpu()
    g = torch.Generator().manual_seed(401)
    perm = torch.randperm(case.kv.shape[0], generator=g)
    moved = torch.empty_like(case.kv.view(torch.uint8))
    moved[perm] = case.kv.view(torch.uint8)
    case2 = synth.Case(spec, case.q_bf16, moved.view(torch.float8_e4m3fn), case.kv_scale, case.qo_indptr,
                       case.kv_indptr, perm[case.kv_indices.long()].to(torch.int32), case.lengths)
    b = DevCase(case2, gpu).run(num_units=16, min_chunk=64).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("flags", [0, 1])
def test_determinism(gpu, flags):
    spec = synth.CaseSpec(batch=6, q_dtype="fp8", kv_dtype="fp8", lengths=[5000, 3, 900, 4096, 64, 1500], seed=500)
    dc = DevCase(synth.make_case(spec), gpu)
    dec = dc.decoder(num_units=64, min_chunk=32, flags=flags)
    a = dc.run(dec).clone()
    b = dc.run(dec).clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("qd,kd", PAIRS)
def test_empty_sequences_give_zeros(gpu, qd, kd):
    lens = [0, 5, 0, 0, 100, 0]
    spec = synth.CaseSpec(batch=len(lens), q_dtype=qd, kv_dtype=kd, lengths=lens, seed=600)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    ref = oracle_ref(case)
    for units, chunk in ((1, 32), (4, 32), (64, 32)):
        out = to64(dc.run(num_units=units, min_chunk=chunk))
        for b, n in enumerate(lens):
            if n == 0:
                assert np.array_equal(out[b], np.zeros((16, 512)))
        assert_parity(ref, out, f"empties u{units}")


def test_all_sequences_empty(gpu):
    spec = synth.CaseSpec(batch=3, q_dtype="bf16", kv_dtype="fp8", lengths=[0, 0, 0], extra_pool_rows=4, seed=610)
    out = to64(DevCase(synth.make_case(spec), gpu).run())
    assert np.array_equal(out, np.zeros_like(out))


def test_single_row_returns_v_exactly(gpu):
    # bf16 KV: softmax over one row is exactly 1, so the output is V itself
    spec = synth.CaseSpec(batch=3, q_dtype="bf16", kv_dtype="bf16", lengths=[1, 1, 1], permuted=True,
                          extra_pool_rows=10, seed=700)
    case = synth.make_case(spec)
    out = DevCase(case, gpu).run().cpu()
    rows = case.kv_indices.long()
    expect = case.kv[rows, :512][:, None, :].expand(3, 16, 512)
    assert torch.equal(out.view(torch.int16), expect.contiguous().view(torch.int16))
    # fp8 KV: the output is the float32 product kv_scale * v rounded to bf16
    spec8 = synth.CaseSpec(batch=2, q_dtype="fp8", kv_dtype="fp8", lengths=[1, 1], seed=701)
    case8 = synth.make_case(spec8)
    out8 = DevCase(case8, gpu).run().cpu()
    v = case8.kv[case8.kv_indices.long(), :512].to(torch.float32) * case8.kv_scale
    assert torch.equal(out8.view(torch.int16), v[:, None, :].expand(2, 16, 512).to(torch.bfloat16).view(torch.int16))


def test_constant_v_returns_constant(gpu):
    spec = synth.CaseSpec(batch=2, q_dtype="bf16", kv_dtype="bf16", lengths=[700, 2000], seed=800)
    case = synth.make_case(spec)
    c = torch.randn(512, generator=torch.Generator().manual_seed(801)).to(torch.bfloat16)
    case.kv[:, :512] = c  # rope dims stay random, scores still differ
    out = DevCase(case, gpu).run(num_units=16, min_chunk=64).cpu().float()
    err = (out - c.float()).abs().max().item()
    log(f"  constant V: max err {err:.3e}")
    assert err <= float(c.float().abs().max()) * 2.0 ** -8


@pytest.mark.parametrize("qd,kd", PAIRS)
def test_zero_q_returns_mean_of_v(gpu, qd, kd):
    """q = 0 makes every score 0, so each output is the plain mean of its sequence's V rows.

    Every weight is exactly 1 (2^0), split or not, so the only rounding is the float32 sum, the
    merge's float32 weights and the bf16 output: the result must lie within 2^-8 max|v| of the
    float64 mean, for every split tried and with the fp8 cast of Q in the kernel too.
    """
    spec = synth.CaseSpec(batch=4, q_dtype=qd, kv_dtype=kd, lengths=[1, 37, 700, 2053], permuted=True,
                          extra_pool_rows=11, seed=1100 + PAIRS.index((qd, kd)))
    case = synth.make_case(spec)
    case.q_bf16.zero_()
    dc = DevCase(case, gpu)
    scale = float(case.kv_scale[0]) if case.kv_scale is not None else None
    vals = torch.from_numpy(oracle.decode_operand(case.kv_bits().numpy(), kd, scale))
    for units, chunk, flags in [(1, 32, 0), (16, 64, 0), (256, 32, 0), (256, 32, 1)]:
        out = to64(dc.run(num_units=units, min_chunk=chunk, flags=flags, q_cast=qd == "fp8"))
        for b in range(spec.batch):
            rows = case.kv_indices[case.kv_indptr[b]:case.kv_indptr[b + 1]].long()
            v = vals[rows, :512]
            mean = v.mean(dim=0).numpy()
            err = np.abs(out[b] - mean[None, :]).max()
            bound = 2.0 ** -8 * float(v.abs().max())
            assert err <= bound, (qd, kd, units, chunk, flags, b, err, bound)
        log(f"  zero q {qd}/{kd} units={units} chunk={chunk} flags={flags}: ok")


@pytest.mark.parametrize("qd,kd", PAIRS)
def test_dominant_last_row(gpu, qd, kd):
    """A row that outscores every other by ~90 (natural log) at the end of each sequence.

    Every head of a sequence's query is the same +-1 vector u, and the sequence's last row (in its
    logical order) holds c u with c = 4 (bf16 KV; for fp8 KV c = min(4, 400 kv_scale), inside the
    e4m3 range), so that row scores 24 c >= 48 against a few units for the random rows.  The walk meets it in its last tile, after the running max has settled, so the
    rescale of everything accumulated so far is taken, and a split sequence's last piece outweighs
    the others in the merge by ~2^130.  The result must match the oracle and equal that row's V up
    to the bf16 rounding, with nothing overflowing.
    """
    spec = synth.CaseSpec(batch=3, q_dtype=qd, kv_dtype=kd, lengths=[3000, 777, 1500], permuted=True,
                          extra_pool_rows=5, seed=1200 + PAIRS.index((qd, kd)))
    case = synth.make_case(spec)
    gen = torch.Generator().manual_seed(1210)
    scale = float(case.kv_scale[0]) if case.kv_scale is not None else None
    for b in range(spec.batch):
        u = (torch.randint(0, 2, (576,), generator=gen) * 2 - 1).float()
        case.q_bf16[b] = u.to(torch.bfloat16)  # all 16 heads
        last = int(case.kv_indices[int(case.kv_indptr[b + 1]) - 1])
        if kd == "bf16":
            case.kv[last] = (4 * u).to(torch.bfloat16)
        else:
            case.kv[last] = (min(4.0, 400 * scale) * u / scale).to(torch.float8_e4m3fn)
    dc = DevCase(case, gpu)
    ref = oracle_ref(case)
    vals = oracle.decode_operand(case.kv_bits().numpy(), kd, scale)
    for units, chunk in [(1, 32), (16, 64), (256, 32)]:
        out = dc.run(num_units=units, min_chunk=chunk, q_cast=qd == "fp8")
        torch.cuda.synchronize()
        got = to64(out)
        assert np.isfinite(got).all()
        assert_parity(ref, got, f"dominant row {qd}/{kd} units={units}")
        for b in range(spec.batch):
            v = vals[int(case.kv_indices[int(case.kv_indptr[b + 1]) - 1]), :512]
            assert np.abs(got[b] - v[None, :]).max() <= 2.0 ** -8 * np.abs(v).max(), (qd, kd, units, b)
        log(f"  dominant last row {qd}/{kd} units={units}: ok")


@pytest.mark.parametrize("sm_scale", [0.25 / 24, 3.0 / 24])
@pytest.mark.parametrize("qd,kd", PAIRS)
def test_scale_arguments(gpu, qd, kd, sm_scale):
    """sm_scale, q_scale and kv_scale away from their usual values: the scores are
    sm_scale * q_scale * kv_scale * (q . k) and the output is kv_scale times the softmax-weighted rows, so a
    scale applied in the wrong place, twice or not at all moves the result far outside the tolerance."""
    spec = synth.CaseSpec(batch=4, q_dtype=qd, kv_dtype=kd, lengths=[700, 1, 2100, 64], permuted=True, seed=2700)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    q_bits = case.q_bits().numpy()
    q_scale = kv_scale = None
    if qd == "fp8":
        q_bits = oracle.bf16_bits_to_fp8_bits(q_bits)
        q_scale = 0.5
        dc.q_scale = torch.tensor([q_scale], dtype=torch.float32, device=gpu)
    if kd == "fp8":
        kv_scale = float(case.kv_scale[0]) * 2.0
        dc.kv_scale = torch.tensor([kv_scale], dtype=torch.float32, device=gpu)
    ref = oracle.mla_decode(q_bits, case.kv_bits().numpy(), case.qo_indptr.numpy(), case.kv_indptr.numpy(),
                            case.kv_indices.numpy(), q_dtype=qd, kv_dtype=kd, q_scale=q_scale, kv_scale=kv_scale,
                            sm_scale=sm_scale)
    default = oracle.mla_decode(q_bits, case.kv_bits().numpy(), case.qo_indptr.numpy(), case.kv_indptr.numpy(),
                                case.kv_indices.numpy(), q_dtype=qd, kv_dtype=kd,
                                q_scale=1.0 if qd == "fp8" else None,
                                kv_scale=float(case.kv_scale[0]) if kd == "fp8" else None)
    assert not compare(default, ref, "scaled against default scales")["elem_ok"]  # the scales matter here
    for units in (1, 64):
        out = dc.run(num_units=units, min_chunk=32, sm_scale=sm_scale)
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"scales {qd}/{kd} sm={sm_scale:.4f} u{units}")


@pytest.mark.parametrize("qd,kd", PAIRS)
def test_wide_range_q(gpu, qd, kd):
    """Q values spread over 2^-12 .. 2^6 in magnitude in every head: the scores span thousands, so the running
    maximum jumps often and by far more than the speculative weights' slack (each such step is redone with
    the new maximum)."""
    spec = synth.CaseSpec(batch=3, q_dtype=qd, kv_dtype=kd, lengths=[1500, 300, 4100], permuted=True, seed=2800)
    case = synth.make_case(spec)
    g = torch.Generator().manual_seed(2801)
    mag = torch.pow(2.0, torch.empty(case.q_bf16.shape).uniform_(-12.0, 6.0, generator=g))
    case.q_bf16 = (case.q_bf16.float() * mag).to(torch.bfloat16)
    dc = DevCase(case, gpu)
    ref = oracle_ref(case)
    for units in (1, 32, 256):
        out = dc.run(num_units=units, min_chunk=32)
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"wide-range q {qd}/{kd} u{units}")


@pytest.mark.parametrize("qd,kd", [("bf16", "bf16"), ("fp8", "fp8")])
def test_pool_beyond_2gib(gpu, qd, kd):
    """The same rows at the end of a KV pool larger than 2 GiB (indices rebased) give the same bits as in a
    compact pool: row addresses are formed in 64 bits."""
    spec = synth.CaseSpec(batch=3, q_dtype=qd, kv_dtype=kd, lengths=[300, 1, 2000], permuted=True, seed=2900)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    small = dc.run(num_units=64, min_chunk=32).clone()
    rows = dc.kv.shape[0]
    row_bytes = dc.kv.shape[1] * dc.kv.element_size()
    total = (2 ** 31) // row_bytes + 2 * rows + 1024  # the case's rows start past byte 2^31
    base = total - rows
    assert base * row_bytes > 2 ** 31
    big = torch.empty((total, dc.kv.shape[1]), dtype=dc.kv.dtype, device=gpu)
    big[base:].copy_(dc.kv)
    dc.kv = big
    dc.kv_indices = dc.kv_indices + base
    moved = dc.run(num_units=64, min_chunk=32)
    torch.cuda.synchronize()
    assert torch.equal(small.view(torch.int16), moved.view(torch.int16))
    assert_parity(oracle_ref(case), to64(moved), f"pool beyond 2 GiB {qd}/{kd}")
    del big


@pytest.mark.parametrize("qd,kd", PAIRS)
def test_shared_and_repeated_pages(gpu, qd, kd):
    """Sequences that share pages (a common prefix, as with prefix caching) and a sequence that lists
    pages twice: kv_indices is only followed, so the result must match the oracle on the same indices
    under every split (a repeated row counts twice in its softmax)."""
    spec = synth.CaseSpec(batch=3, q_dtype=qd, kv_dtype=kd, lengths=[600, 900, 300], permuted=True,
                          extra_pool_rows=64, seed=1300 + PAIRS.index((qd, kd)))
    case = synth.make_case(spec)
    idx = case.kv_indices.clone()
    p = case.kv_indptr.tolist()
    idx[p[1]:p[1] + 400] = idx[p[0]:p[0] + 400]  # sequence 1 starts with sequence 0's first 400 rows
    idx[p[2] + 150:p[3]] = idx[p[2]:p[2] + 150]  # sequence 2 lists its first 150 rows twice
    case.kv_indices = idx
    dc = DevCase(case, gpu)
    ref = oracle_ref(case)
    for units, chunk in [(1, 32), (16, 64), (256, 32)]:
        out = dc.run(num_units=units, min_chunk=chunk, q_cast=qd == "fp8")
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"shared pages {qd}/{kd} units={units}")


def test_external_reduce_matches_merge(gpu):
    """The external reduce against the oracle's merge, output and final log-sum-exp.  Parts with lse = -inf
    hold NaN rows (an empty shard's 0/0): they carry no weight and must not reach the output."""
    rng = np.random.default_rng(900)
    counts = [0, 1, 2, 5, 64, 70, 3, 2]
    P = sum(counts)
    part_o = rng.standard_normal((P, 16, 512)).astype(np.float32)
    lse = (rng.standard_normal((P, 16)) * 3).astype(np.float32)
    lse[1, 3] = -np.inf
    lse[rng.random((P, 16)) < 0.05] = -np.inf
    lse[P - 2:, 5] = -np.inf  # the last sequence: head 5 has only empty parts
    part_o[np.isneginf(lse)] = np.nan
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    out = torch.full((len(counts), 16, 512), float("nan"), dtype=torch.bfloat16, device=gpu)
    lse_out = torch.full((len(counts), 16), float("nan"), dtype=torch.float32, device=gpu)
    binding.mla_decode_reduce(torch.from_numpy(part_o).to(gpu), torch.from_numpy(lse).to(gpu),
                              torch.from_numpy(indptr).to(gpu), out, lse_out)
    torch.cuda.synchronize()
    got = to64(out)
    got_lse = lse_out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    for b in range(len(counts)):
        p0, p1 = indptr[b], indptr[b + 1]
        if p1 == p0:
            assert np.array_equal(got[b], np.zeros((16, 512)))
            assert np.all(np.isneginf(got_lse[b]))
            continue
        po = np.where(np.isneginf(lse[p0:p1])[:, :, None], 0.0, part_o[p0:p1].astype(np.float64))
        ref = oracle.merge_partials(po, lse[p0:p1].astype(np.float64))
        assert np.max(np.abs(got[b] - ref)) <= 2.0 ** -8 * np.max(np.abs(ref)) + 1e-6, b
        ref_lse = oracle.merge_lse(lse[p0:p1].astype(np.float64))
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isneginf(got_lse[b]), ~fin), b
        assert np.max(np.abs(got_lse[b][fin] - ref_lse[fin]), initial=0.0) <= 1e-5 * (1 + np.max(np.abs(ref_lse[fin]), initial=0.0)), b
    # without lse_out the output is the same
    out2 = torch.empty_like(out)
    binding.mla_decode_reduce(torch.from_numpy(part_o).to(gpu), torch.from_numpy(lse).to(gpu),
                              torch.from_numpy(indptr).to(gpu), out2)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def _oracle_lse(case, sequences=None, causal=False, logit_cap=0.0):
    q_bits = case.q_bits().numpy()
    q_scale = None
    if case.spec.q_dtype == "fp8":
        q_bits, q_scale = oracle.bf16_bits_to_fp8_bits(q_bits), 1.0
    kv_scale = float(case.kv_scale[0]) if case.kv_scale is not None else None
    return oracle.mla_decode_lse(q_bits, case.kv_bits().numpy(), case.qo_indptr.numpy(), case.kv_indptr.numpy(),
                                 case.kv_indices.numpy(), q_dtype=case.spec.q_dtype, kv_dtype=case.spec.kv_dtype,
                                 q_scale=q_scale, kv_scale=kv_scale, sequences=sequences,
                                 page_size=case.spec.page_size, kv_last_page_len=case.kv_last_page_len.numpy(),
                                 causal=causal, logit_cap=logit_cap)


def _check_lse(ref, got, what):
    """Finite entries within 2e-3 absolute plus 1e-4 relative (the row sum uses bf16-rounded weights, each off by
    at most 2^-9 relative, so log of the sum is off by at most ~2^-9; the max and the log add float32 rounding);
    -inf exactly where the oracle has it."""
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{what}: -inf pattern differs"
    err = np.abs(got[fin] - ref[fin])
    bound = 2e-3 + 1e-4 * np.abs(ref[fin])
    log(f"  {what}: lse max_abs={err.max(initial=0.0):.3e}")
    assert np.all(err <= bound), f"{what}: lse error {err.max()}"


@pytest.mark.parametrize("qd,kd", PAIRS)
def test_final_lse_output(gpu, qd, kd):
    """lse_out of mla_decode_run_paged: the natural-log sum-exp of every token and head, for sequences one
    workgroup finishes, split ones (written by the merge), the fused merge and empty sequences."""
    lens = [0, 1, 2, 31, 33, 100, 513, 2053, 0, 7]
    spec = synth.CaseSpec(batch=len(lens), q_dtype=qd, kv_dtype=kd, lengths=lens, permuted=True,
                          extra_pool_rows=17, seed=950 + PAIRS.index((qd, kd)))
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    ref_o = oracle_ref(case)
    ref_l = _oracle_lse(case)
    for units, chunk, flags in ((1, 32, 0), (8, 32, 0), (256, 32, 0), (256, 32, 1)):
        dec = dc.decoder(num_units=units, min_chunk=chunk, flags=flags)
        out = torch.full((case.total_q, 16, 512), float("nan"), dtype=torch.bfloat16, device=gpu)
        lse = torch.full((case.total_q, 16), float("nan"), dtype=torch.float32, device=gpu)
        dec.run(dc.q, dc.kv, dc.qo_indptr, dc.kv_indptr, dc.kv_indices, dc.q_scale, dc.kv_scale,
                oracle.SM_SCALE, out, lse_out=lse)
        torch.cuda.synchronize()
        assert_parity(ref_o, to64(out), f"lse run {qd}/{kd} u{units} f{flags}")
        _check_lse(ref_l, lse.cpu().numpy().astype(np.float64), f"{qd}/{kd} u{units} f{flags}")


def test_final_lse_tokens_pages_and_cap(gpu):
    lens = [3, 17, 1000, 4100, 64, 0]
    q_lens = [2, 3, 1, 4, 2, 1]
    spec = synth.CaseSpec(batch=len(lens), q_dtype="bf16", kv_dtype="fp8", lengths=lens, q_lens=q_lens,
                          permuted=True, extra_pool_rows=40, page_size=16, seed=960)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    for causal, cap in ((True, 0.0), (False, 5.0), (True, 5.0)):
        ref_l = _oracle_lse(case, causal=causal, logit_cap=cap)
        for units in (8, 256):
            dec = dc.decoder(num_units=units, min_chunk=32, logit_cap=cap,
                             flags=binding.MLA_FLAG_CAUSAL if causal else 0)
            out = torch.empty((case.total_q, 16, 512), dtype=torch.bfloat16, device=gpu)
            lse = torch.full((case.total_q, 16), float("nan"), dtype=torch.float32, device=gpu)
            dec.run(dc.q, dc.kv, dc.qo_indptr, dc.kv_indptr, dc.kv_indices, dc.q_scale, dc.kv_scale,
                    oracle.SM_SCALE, out, kv_last_page_len=dc.kv_last_page_len, lse_out=lse)
            torch.cuda.synchronize()
            _check_lse(ref_l, lse.cpu().numpy().astype(np.float64), f"causal={causal} cap={cap} u{units}")


def test_lengths_change_without_replanning(gpu):
    # the split is recomputed from kv_indptr on every run: one plan serves growing lengths
    dec = binding.Decoder(3, "bf16", "fp8", gpu, num_units=32, min_chunk=32)
    for step, lens in enumerate(([10, 500, 33], [11, 501, 34], [900, 1, 4000])):
        case = synth.make_case(synth.CaseSpec(batch=3, q_dtype="bf16", kv_dtype="fp8", lengths=lens, seed=950 + step))
        dc = DevCase(case, gpu)
        assert_parity(oracle_ref(case), to64(dc.run(dec)), f"step{step}")


def _edge_q(case):
    """Put fp8 rounding ties, subnormal-range values and signed zeros into Q (the full code range is covered by
    the exhaustive cast test, which goes through the same eight-value conversion)."""
    q = case.q_bf16.clone()
    edge = torch.tensor([1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -11, -2.0 ** -10, 2.0 ** -7, 0.0, -0.0,
                         0.0156, 1.5, 2.25], dtype=torch.float32).to(torch.bfloat16)
    q.view(-1)[: edge.numel() * 97: 97] = edge  # scattered over heads and dims
    return q


@pytest.mark.parametrize("units", [1, 8, 256])
def test_fused_q_cast_matches_separate_cast(gpu, units):
    spec = synth.CaseSpec(batch=5, q_dtype="fp8", kv_dtype="fp8", lengths=[1, 70, 600, 2100, 33], permuted=True,
                          extra_pool_rows=11, seed=1100)
    case = synth.make_case(spec)
    case.q_bf16 = _edge_q(case)
    dc = DevCase(case, gpu)  # casts Q with mla_decode_quantize_q (step a0)
    sep = dc.run(num_units=units, min_chunk=32).cpu()
    fused = dc.run(num_units=units, min_chunk=32, q_cast=True).cpu()
    assert torch.equal(sep.view(torch.int16), fused.view(torch.int16))
    assert_parity(oracle_ref(case), to64(fused), f"fused cast u{units}")


def test_fused_q_cast_positive_nan_fallback(gpu):
    """A positive NaN in Q sends its lane through the exact conversion; the other lanes of the wave keep the
    hardware result, so every other head and sequence matches the separately cast Q bit for bit."""
    spec = synth.CaseSpec(batch=3, q_dtype="fp8", kv_dtype="fp8", lengths=[40, 300, 90], seed=1200)
    case = synth.make_case(spec)
    q = case.q_bf16.view(torch.int16).clone()
    q[1, 5, 17] = 0x7FC1  # positive NaN: the hardware cast gives the negative NaN code, the fallback fixes it
    q[2, 0, 3] = -0x7F7F  # bits 0x8081: a negative subnormal
    case.q_bf16 = q.view(torch.bfloat16)
    dc = DevCase(case, gpu)
    q8 = dc.q.cpu().numpy()
    assert q8[1, 5, 17] == 0x7F  # the standalone cast keeps the NaN's sign
    sep = dc.run(num_units=4, min_chunk=32).cpu()
    fused = dc.run(num_units=4, min_chunk=32, q_cast=True).cpu()
    assert torch.equal(sep.view(torch.int16), fused.view(torch.int16))
    ok = torch.isfinite(fused.float())
    assert not bool(ok[1, 5].any()) and bool(ok[0].all()) and bool(ok[2].all())


# ---------------------------------------------- many short sequences, big batches

def _token_rows(case, seqs):
    qo = case.qo_indptr.tolist()
    return [t for b in seqs for t in range(qo[b], qo[b + 1])]


@pytest.mark.parametrize("qd,kd", PAIRS)
def test_many_short_sequences(gpu, qd, kd):
    # average length far below 1024 rows: the split charges every sequence a fixed cost, so shares may
    # begin in the gaps between sequences
    rng = np.random.default_rng(3100)
    lens = rng.integers(0, 41, size=600).tolist()
    spec = synth.CaseSpec(batch=600, q_dtype=qd, kv_dtype=kd, lengths=lens, permuted=True, extra_pool_rows=9,
                          seed=3100 + PAIRS.index((qd, kd)))
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    ref = oracle_ref(case)
    for units, chunk, flags in ((1, 32, 0), (8, 32, 0), (256, 32, 0), (256, 256, 0), (4096, 32, 1)):
        out = dc.run(num_units=units, min_chunk=chunk, flags=flags)
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"short {qd}/{kd} u{units} c{chunk} f{flags}")


def test_one_row_sequences_spread_over_workgroups(gpu):
    spec = synth.CaseSpec(batch=256, q_dtype="bf16", kv_dtype="fp8", lengths=[1] * 256, permuted=True, seed=3200)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    dec = dc.decoder()
    out = dc.run(dec)
    torch.cuda.synchronize()
    assert_parity(oracle_ref(case), to64(out), "one-row sequences")
    for _ in range(3):
        dc.run(dec, out)
    torch.cuda.synchronize()
    with Timer("10 steps") as tm:
        for _ in range(10):
            dc.run(dec, out)
        torch.cuda.synchronize()
    per_step_us = (time.time() - tm.t) / 10 * 1e6
    log(f"  256 one-row sequences: {per_step_us:.1f} us per step (host-timed)")
    assert per_step_us < 300.0  # one workgroup walking all 256 took ~1300 us


@pytest.mark.parametrize("qd,kd", [("bf16", "fp8"), ("fp8", "fp8")])
def test_batch_beyond_lds_table(gpu, qd, kd):
    # more than 1024 sequences: the kernel reads the indptrs from memory in the piece loop
    rng = np.random.default_rng(3300)
    short = rng.integers(1, 200, size=1500).tolist()  # with the per-sequence cost
    spec = synth.CaseSpec(batch=1500, q_dtype=qd, kv_dtype=kd, lengths=short, permuted=True, seed=3300)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    ref = oracle_ref(case)
    for units in (64, 256):
        out = dc.run(num_units=units, min_chunk=32)
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"big batch short {qd}/{kd} u{units}")
    # equal lengths of 1024 rows and shares of 2048 (515 units): without the cost; then the same with one
    # length changed past the LDS table, which only the scan from memory sees: with it
    seqs = [0, 1, 513, 1023, 1024, 1025, 1027, 1029]
    for lens, cost in (([1024] * 1030, 0), ([1024] * 1027 + [1023] + [1024] * 2, PIECE_COST_ROWS)):
        spec = synth.CaseSpec(batch=1030, q_dtype=qd, kv_dtype=kd, lengths=lens, permuted=True, seed=3301)
        case = synth.make_case(spec)
        dc = DevCase(case, gpu)
        dec = dc.decoder(num_units=515, min_chunk=32)
        out = dc.run(dec)
        torch.cuda.synchronize()
        assert split_record(dec)[1] == cost
        assert split_record(dec) == expected_split(case, 515, 32)
        ref = oracle_ref(case, sequences=seqs)
        assert_parity(ref[seqs], to64(out)[seqs], f"big batch long {qd}/{kd} cost {cost}")
        del dc, case


@pytest.mark.parametrize("qd,kd,batch", [
    ("bf16", "fp8", 512), ("bf16", "fp8", 513), ("fp8", "fp8", 512), ("fp8", "fp8", 513),  # LDS ring: 512
    ("bf16", "bf16", 1024), ("bf16", "bf16", 1025),  # register ring: a table of 1024 sequences
])
def test_batch_at_lds_table_size(gpu, qd, kd, batch):
    """Batches at the LDS sequence table's size and one past it (the instantiation that reads the indptrs
    from memory), with one sequence whose length differs at the end of the batch so that the uniformity
    scan past the table decides the split."""
    rng = np.random.default_rng(3400 + batch)
    lens = rng.integers(1, 120, size=batch).tolist()
    spec = synth.CaseSpec(batch=batch, q_dtype=qd, kv_dtype=kd, lengths=lens, permuted=True, seed=3400 + batch)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    ref = oracle_ref(case)
    for units in (48, 256):
        out = dc.run(num_units=units, min_chunk=32)
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"table edge {qd}/{kd} b{batch} u{units}")
    # equal lengths but the last: only the scan reaches it past a full table
    lens = [1024] * (batch - 1) + [1000]
    spec = synth.CaseSpec(batch=batch, q_dtype=qd, kv_dtype=kd, lengths=lens, seed=3401 + batch)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    dec = dc.decoder(num_units=256, min_chunk=32)
    out = dc.run(dec)
    torch.cuda.synchronize()
    assert split_record(dec) == expected_split(case, 256, 32)
    seqs = [0, batch // 2, batch - 2, batch - 1]
    assert_parity(oracle_ref(case, sequences=seqs)[seqs], to64(out)[seqs], f"table edge long {qd}/{kd} b{batch}")


def split_record(dec: binding.Decoder) -> list:
    """The split (base, cost, total, chunk, shares) the last attention launch recorded in the workspace."""
    words = dec.workspace.view(torch.int32)
    at = dec.plan.off_counters // 4 + dec.params.batch
    return words[at:at + 5].cpu().tolist()


def expected_split(case, units: int, min_chunk: int) -> list:
    """The split rule restated on the host: positions are pages; every sequence costs PIECE_COST_ROWS of
    positions unless all have one length of at least 1024 rows that the share size divides or is
    divided by."""
    sh = case.spec.page_size.bit_length() - 1
    ind = case.kv_indptr.tolist()
    lens = [ind[i + 1] - ind[i] for i in range(len(ind) - 1)]
    pos = ind[-1] - ind[0]

    def share(total):
        c = -(-total // units)
        al = max(1, 32 >> sh)
        return max(-(-c // al) * al, max(1, min_chunk >> sh))

    c0 = share(pos)
    L = lens[0]
    if all(x == L for x in lens) and L >= max(1, 1024 >> sh) and (L % c0 == 0 or c0 % L == 0):
        cost, total, chunk = 0, pos, c0
    else:
        cost = max(1, PIECE_COST_ROWS >> sh)
        total = pos + cost * len(lens)
        chunk = share(total)
    return [ind[0], cost, total, chunk, max(1, -(-total // chunk))]


@pytest.mark.parametrize("lens,page,units,cost", [
    ([4096] * 8, 1, 256, 0),  # equal, long, shares of 128 divide the length
    ([5000] * 3, 1, 256, PIECE_COST_ROWS),  # equal and long, but shares of 64 neither divide nor are divided by 5000
    ([512] * 16, 1, 256, PIECE_COST_ROWS),  # equal but short
    ([8192, 8191, 8192, 8192], 1, 64, PIECE_COST_ROWS),  # one length differs
    ([8010] * 4, 16, 256, PIECE_COST_ROWS >> 4),  # pages of 16: 501 positions each, shares of 16 positions
    ([8192] * 64, 16, 256, 0),  # pages of 16, shares of 128 positions
])
def test_split_rule(gpu, lens, page, units, cost):
    spec = synth.CaseSpec(batch=len(lens), q_dtype="bf16", kv_dtype="fp8", lengths=lens, page_size=page,
                          seed=3350 + len(lens))
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    dec = dc.decoder(num_units=units)
    out = dc.run(dec)
    torch.cuda.synchronize()
    rec = split_record(dec)
    log(f"  split {rec} for {len(lens)} sequences, pages of {page}, {units} units")
    assert rec[1] == cost
    assert rec == expected_split(case, units, dec.plan.params.min_chunk)
    seqs = list(range(min(len(lens), 4)))
    ref = oracle_ref(case, sequences=seqs)
    assert_parity(ref[seqs], to64(out)[seqs], f"split rule {lens[:2]} p{page} u{units}")


@pytest.mark.parametrize("units,q_len,qd,kd", [(16, 1, "bf16", "fp8"), (32, 1, "bf16", "fp8"), (64, 1, "bf16", "fp8"),
                                             (32, 2, "bf16", "fp8"), (32, 2, "bf16", "bf16"), (64, 2, "fp8", "fp8")])
@pytest.mark.parametrize("flags", [0, binding.MLA_FLAG_FUSED_MERGE], ids=["merge_launch", "fused_merge"])
def test_per_sequence_partial_slots(gpu, units, q_len, qd, kd, flags):
    """The first units // batch pieces of each sequence (2 to 8 of them) sit in slots of their own, which the
    merge launch loads before it reads the split; further pieces stay in their shares' slots.  Lengths are
    mixed so that sequences have one piece (nothing to merge), fewer, as many and more pieces than those
    slots, with the per-sequence cost in the split (lengths differ)."""
    lens = [700, 64, 2500, 1, 1300, 4000, 333, 1800]
    spec = synth.CaseSpec(batch=len(lens), q_dtype=qd, kv_dtype=kd, lengths=lens, permuted=True,
                          q_lens=[q_len] * len(lens) if q_len > 1 else None, extra_pool_rows=11, seed=8800 + units)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    causal = q_len > 1
    ref = oracle_ref(case, causal=causal)
    for rep in range(2):  # the second run finds the first run's partials in the slots
        log(f"[per-sequence slots units={units} q_len={q_len} flags={flags} run {rep}]")
        out = dc.run(num_units=units, min_chunk=32, flags=flags, causal=causal, q_cast=qd == "fp8")
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"slots {qd}/{kd} u{units} q{q_len} f{flags} r{rep}")


def test_merge_before_any_attention_writes_nothing(gpu):
    spec = synth.CaseSpec(batch=4, q_dtype="bf16", kv_dtype="fp8", lengths=[3000, 10, 4000, 700], seed=3360)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    dec = dc.decoder(num_units=64)
    out = torch.full((4, 16, 512), float("nan"), dtype=torch.bfloat16, device=gpu)
    binding.mla_decode_merge(dec.plan, dc.qo_indptr, dc.kv_indptr, out)
    torch.cuda.synchronize()
    assert split_record(dec) == [0, 0, 0, 0, 0]
    assert bool(torch.isnan(out.float()).all())


def test_batch_beyond_lds_table_with_tokens(gpu):
    rng = np.random.default_rng(3400)
    lens = rng.integers(1, 120, size=1100).tolist()
    q_lens = rng.integers(1, 4, size=1100).tolist()
    spec = synth.CaseSpec(batch=1100, q_dtype="fp8", kv_dtype="fp8", lengths=lens, q_lens=q_lens, permuted=True,
                          page_size=8, seed=3400)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    seqs = [0, 5, 700, 1023, 1024, 1099]
    ref = oracle_ref(case, sequences=seqs, causal=True)
    rows = _token_rows(case, seqs)
    out = dc.run(num_units=256, min_chunk=32, causal=True)
    torch.cuda.synchronize()
    assert_parity(ref[rows], to64(out)[rows], "big batch tokens")


# ----------------------------------------------------------------- graph capture

@pytest.mark.parametrize("qd,flags", [("bf16", 0), ("bf16", 1), ("fp8", 2)])
def test_graph_capture_and_replay(gpu, qd, flags):
    """A captured decode step replays correctly, also after the sequence lengths change in place (the plan
    does not depend on them), with eager work between the replays; every replay is checked against an
    eager run on the same inputs."""
    lens_a = [300, 1, 2049, 700, 64, 1500]
    lens_b = [10, 900, 33, 2000, 64, 1]
    spec = synth.CaseSpec(batch=6, q_dtype=qd, kv_dtype="fp8", lengths=lens_a, permuted=True,
                          extra_pool_rows=3000, seed=3500)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    q = dc.q_bf16 if flags & binding.MLA_FLAG_FUSED_Q_CAST else dc.q
    dec = dc.decoder(num_units=64, min_chunk=32, flags=flags)
    indptr_a = dc.kv_indptr.clone()
    indptr_b = torch.tensor([0] + list(np.cumsum(lens_b)), dtype=torch.int32, device=gpu)
    out_g = torch.zeros((6, 16, 512), dtype=torch.bfloat16, device=gpu)

    def step(out, indptr):
        dec.run(q, dc.kv, dc.qo_indptr, indptr, dc.kv_indices, dc.q_scale, dc.kv_scale, oracle.SM_SCALE, out)

    live_indptr = dc.kv_indptr  # the buffer the graph reads
    step(out_g, live_indptr)  # warm up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out_g, live_indptr)
    torch.cuda.synchronize()
    for rep, src in enumerate([indptr_a, indptr_b, indptr_a, indptr_b]):
        live_indptr.copy_(src)
        eager = torch.empty_like(out_g)
        step(eager, src)  # eager work between replays, on the same workspace
        torch.cuda.synchronize()
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
    # the last replay ran lengths B: check it against the oracle too
    case_b = synth.Case(spec, case.q_bf16, case.kv, case.kv_scale, case.qo_indptr, indptr_b.cpu(), case.kv_indices,
                        torch.tensor(lens_b), case.kv_last_page_len)
    assert_parity(oracle_ref(case_b), to64(out_g), f"graph lengths B {qd} flags={flags}")


@pytest.mark.parametrize("qd,kd", [("bf16", "fp8"), ("fp8", "fp8")])
def test_one_sequence_over_every_workgroup(gpu, qd, kd):
    """A single sequence of 65,573 rows split over 256 shares: the merge folds 256 pieces in four chunks of 64
    (the per-sequence slots hold only the first 16)."""
    spec = synth.CaseSpec(batch=1, q_dtype=qd, kv_dtype=kd, lengths=[65573], permuted=True, extra_pool_rows=5,
                          seed=3800)
    case = synth.make_case(spec)
    dc = DevCase(case, gpu)
    ref = oracle_ref(case)
    for units, flags in ((256, 0), (256, binding.MLA_FLAG_FUSED_MERGE), (100, 0)):
        log(f"[one sequence {qd}/{kd} units={units} flags={flags}]")
        out = dc.run(num_units=units, min_chunk=32, flags=flags, q_cast=qd == "fp8")
        torch.cuda.synchronize()
        assert_parity(ref, to64(out), f"one sequence {qd}/{kd} u{units} f{flags}")
