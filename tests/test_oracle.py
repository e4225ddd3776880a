"""Pins for the float64 oracle (CPU only).

Each check ties the oracle to something other than itself: torch's CPU casts
(exhaustive over every code), float64 scaled-dot-product attention (the
multi-query special case of MLA decode), a pure-Python brute force, closed
forms, split/merge identities, and deliberately wrong variants that must be
rejected by the same gate the GPU parity tests use.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import formats, mla
from mla_decode_paged_split_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RTOL, ATOL, NORM_GATE = 2e-2, 1e-2, 1e-2


def gate(ref, got):
    """The parity gate: elementwise allclose AND normwise relative error."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    ok_elem = bool(np.all(np.abs(got - ref) <= ATOL + RTOL * np.abs(ref)))
    nrm = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    return ok_elem and nrm <= NORM_GATE


# ----------------------------------------------------------------- page constants


def test_constants_match_pages():
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        g = json.load(f)
    assert mla.NUM_HEADS == g["num_heads"]
    assert mla.QK_DIM == g["qk_head_dim"]
    assert mla.V_DIM == g["v_head_dim"]
    assert mla.SM_SCALE == 1.0 / math.sqrt(g["qk_head_dim"]) == 1.0 / 24.0
    finite = formats.FP8_TABLE[np.isfinite(formats.FP8_TABLE)]
    assert finite.max() == g["fp8_e4m3_range"][1] and finite.min() == g["fp8_e4m3_range"][0]


# ----------------------------------------------------------------- number formats


def test_bf16_decode_exhaustive_vs_torch():
    codes = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16)
    ref = codes.view(torch.bfloat16).to(torch.float64).numpy()
    got = formats.decode_bf16(codes.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    # signed zeros and infinities keep their sign
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_fp8_decode_exhaustive_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = formats.decode_fp8_e4m3fn(codes.numpy())
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    assert got[1] == 2.0 ** -9 and np.nanmax(got) == 448.0


def test_fp8_cast_exhaustive_over_bf16_vs_torch():
    codes = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16)
    ref = codes.view(torch.bfloat16).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = formats.bf16_bits_to_fp8_bits(codes.numpy())
    assert np.array_equal(ref, got)


def test_fp8_cast_float_edges_vs_torch():
    rng = np.random.default_rng(7)
    vals = np.concatenate(
        [
            rng.standard_normal(4000) * 3,
            rng.standard_normal(2000) * 200,
            rng.standard_normal(2000) * 1e-3,
            np.array([0.0, -0.0, 448, 456, 464, 464.0001, 465, -464, -465, 2**-9, 2**-10, 3 * 2**-11,
                      2**-6, 2**-6 - 2**-12, 1.0625, 1.1875, 1e30, -1e30]),
        ]
    ).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = formats.encode_fp8_e4m3fn(vals.astype(np.float64))
    assert np.array_equal(ref, got)


def test_bf16_rne_vs_torch():
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(3000), rng.standard_normal(500) * 1e-39,
                           np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 0.0, -0.0])])
    # float64 -> bf16 directly; compare with torch where float32 holds the value exactly
    v32 = vals.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = formats.encode_bf16_rne(v32)
    assert np.array_equal(ref, got)


# ------------------------------------------------------------ attention special cases


def _rand_case(rng, B, lens, dtype_q="bf16", dtype_kv="bf16", permute=False):
    total = int(sum(lens))
    q32 = torch.from_numpy(rng.standard_normal((B, 16, 576)).astype(np.float32))
    kv32 = torch.from_numpy(rng.standard_normal((total, 576)).astype(np.float32))
    q_bits = q32.to(torch.bfloat16).view(torch.int16).numpy()
    if dtype_kv == "bf16":
        kv_bits = kv32.to(torch.bfloat16).view(torch.int16).numpy()
        kv_scale = None
    else:
        kv_scale = float((kv32.abs().max() / 448.0).item())
        kv_bits = (kv32 / kv_scale).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    kv_indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    idx = rng.permutation(total) if permute else np.arange(total)
    # when permuting, physically move rows so that the logical sequence is unchanged
    if permute:
        moved = np.empty_like(kv_bits)
        moved[idx] = kv_bits
        kv_bits = moved
    return q_bits, kv_bits, np.arange(B + 1), kv_indptr, idx, kv_scale


def _sdpa_reference(q_bits, kv_bits, kv_indptr, kv_indices, kv_dtype, kv_scale, q_dtype="bf16", q_scale=None):
    """torch float64 scaled_dot_product_attention, K/V broadcast to 16 heads."""
    B = len(kv_indptr) - 1
    out = []
    for b in range(B):
        rows = np.asarray(kv_indices[kv_indptr[b]: kv_indptr[b + 1]])
        if q_dtype == "bf16":
            Q = torch.from_numpy(q_bits[b]).view(torch.bfloat16).to(torch.float64)
        else:
            Q = torch.from_numpy(q_bits[b]).view(torch.float8_e4m3fn).to(torch.float64) * q_scale
        if kv_dtype == "bf16":
            K = torch.from_numpy(kv_bits[rows]).view(torch.bfloat16).to(torch.float64)
        else:
            K = torch.from_numpy(kv_bits[rows]).view(torch.float8_e4m3fn).to(torch.float64) * kv_scale
        q4 = Q[None, :, None, :]  # [1, H, 1, 576]
        k4 = K[None, None].expand(1, 16, K.shape[0], 576)
        v4 = K[:, :512][None, None].expand(1, 16, K.shape[0], 512)
        o = torch.nn.functional.scaled_dot_product_attention(q4, k4, v4, scale=1.0 / 24.0)
        out.append(o[0, :, 0, :].numpy())
    return np.stack(out)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_oracle_vs_sdpa_float64(kv_dtype):
    rng = np.random.default_rng(11)
    lens = [1, 2, 17, 64, 300, 1000]
    q_bits, kv_bits, qo, kvp, idx, kvs = _rand_case(rng, len(lens), lens, dtype_kv=kv_dtype, permute=True)
    got = oracle.mla_decode(q_bits, kv_bits, qo, kvp, idx, q_dtype="bf16", kv_dtype=kv_dtype, kv_scale=kvs)
    ref = _sdpa_reference(q_bits, kv_bits, kvp, idx, kv_dtype, kvs)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_oracle_vs_sdpa_fp8_q():
    rng = np.random.default_rng(12)
    lens = [5, 129, 700]
    q_bits, kv_bits, qo, kvp, idx, kvs = _rand_case(rng, 3, lens, dtype_kv="fp8")
    q8 = formats.bf16_bits_to_fp8_bits(q_bits)
    q_scale = 1.0
    got = oracle.mla_decode(q8, kv_bits, qo, kvp, idx, q_dtype="fp8", kv_dtype="fp8", q_scale=q_scale, kv_scale=kvs)
    ref = _sdpa_reference(q8, kv_bits, kvp, idx, "fp8", kvs, q_dtype="fp8", q_scale=q_scale)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_oracle_vs_bruteforce_tiny():
    rng = np.random.default_rng(5)
    lens = [1, 3, 5]
    q_bits, kv_bits, qo, kvp, idx, _ = _rand_case(rng, 3, lens, permute=True)
    got = oracle.mla_decode(q_bits, kv_bits, qo, kvp, idx, q_dtype="bf16", kv_dtype="bf16")
    for b in range(3):
        Q = formats.decode_bf16(q_bits[b]).tolist()
        K = [formats.decode_bf16(kv_bits[idx[i]]).tolist() for i in range(kvp[b], kvp[b + 1])]
        bf = np.array(mla.mla_decode_bruteforce(Q, K, 1.0 / 24.0, 512))
        assert np.max(np.abs(bf - got[b])) <= 1e-12


# ------------------------------------------------------------------- closed forms


def _seq(rng, n, scale=1.0):
    Q = rng.standard_normal((16, 576)) * scale
    K = rng.standard_normal((n, 576))
    return Q, K


def test_single_row_returns_its_v():
    rng = np.random.default_rng(1)
    Q, K = _seq(rng, 1, 10.0)
    O = mla.mla_decode_sequence(Q, K, mla.SM_SCALE)
    assert np.array_equal(O, np.broadcast_to(K[0, :512], O.shape))


def test_zero_query_returns_mean_of_v():
    rng = np.random.default_rng(2)
    _, K = _seq(rng, 37)
    O = mla.mla_decode_sequence(np.zeros((16, 576)), K, mla.SM_SCALE)
    assert np.max(np.abs(O - K[:, :512].mean(axis=0))) <= 1e-13


def test_constant_v_returns_constant():
    rng = np.random.default_rng(3)
    Q, K = _seq(rng, 50, 3.0)
    c = rng.standard_normal(512)
    K[:, :512] = c  # rope dims stay random, so scores still differ
    O = mla.mla_decode_sequence(Q, K, mla.SM_SCALE)
    assert np.max(np.abs(O - c)) <= 1e-13


def test_two_rows_logistic():
    rng = np.random.default_rng(4)
    Q, K = _seq(rng, 2)
    s = mla.SM_SCALE * (Q @ K.T)
    w1 = 1.0 / (1.0 + np.exp(s[:, 1] - s[:, 0]))
    expect = w1[:, None] * K[0, :512] + (1 - w1)[:, None] * K[1, :512]
    O = mla.mla_decode_sequence(Q, K, mla.SM_SCALE)
    assert np.max(np.abs(O - expect)) <= 1e-13


def test_dominant_row_no_overflow():
    rng = np.random.default_rng(5)
    Q, K = _seq(rng, 64)
    # row 7 aligned with head 0's query and scaled so its score leads by > 40
    K[7] = Q[0] / np.linalg.norm(Q[0]) * 24.0 * 60.0 / np.linalg.norm(Q[0])
    O = mla.mla_decode_sequence(Q, K, mla.SM_SCALE)
    assert np.all(np.isfinite(O))
    assert np.max(np.abs(O[0] - K[7, :512])) <= 1e-12 * np.max(np.abs(K[7, :512])) + 1e-12


def test_duplicate_row_equals_ln2_bias():
    rng = np.random.default_rng(6)
    Q, K = _seq(rng, 20)
    dup = np.concatenate([K, K[3:4]], axis=0)
    O_dup = mla.mla_decode_sequence(Q, dup, mla.SM_SCALE)
    s = mla.SM_SCALE * (Q @ K.T)
    s[:, 3] += math.log(2.0)
    P = np.exp(s - s.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    assert np.max(np.abs(O_dup - P @ K[:, :512])) <= 1e-13


def test_empty_sequence_is_zero():
    O = mla.mla_decode_sequence(np.ones((16, 576)), np.zeros((0, 576)), mla.SM_SCALE)
    assert np.array_equal(O, np.zeros((16, 512)))


# ------------------------------------------------------------- split / merge


@pytest.mark.parametrize("nsplit", [1, 2, 3, 7, 40])
def test_split_merge_equals_unsplit(nsplit):
    rng = np.random.default_rng(100 + nsplit)
    Q, K = _seq(rng, 333, 2.0)
    cuts = np.sort(rng.choice(np.arange(1, 333), size=nsplit - 1, replace=False)) if nsplit > 1 else []
    bounds = [0, *cuts, 333]
    parts = [mla.attention_partial(Q, K[a:b], mla.SM_SCALE) for a, b in zip(bounds[:-1], bounds[1:])]
    O = mla.merge_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    assert np.max(np.abs(O - mla.mla_decode_sequence(Q, K, mla.SM_SCALE))) <= 1e-13


def test_merge_ignores_empty_parts_and_all_empty_is_zero():
    rng = np.random.default_rng(9)
    Q, K = _seq(rng, 10)
    p_full = mla.attention_partial(Q, K, mla.SM_SCALE)
    p_empty = mla.attention_partial(Q, K[:0], mla.SM_SCALE)
    assert np.all(np.isneginf(p_empty[1]))
    O = mla.merge_partials(np.stack([p_empty[0], p_full[0]]), np.stack([p_empty[1], p_full[1]]))
    assert np.max(np.abs(O - mla.mla_decode_sequence(Q, K, mla.SM_SCALE))) <= 1e-14
    Z = mla.merge_partials(np.stack([p_empty[0]] * 3), np.stack([p_empty[1]] * 3))
    assert np.array_equal(Z, np.zeros_like(Z))


def test_lse_is_log_sum_exp():
    rng = np.random.default_rng(10)
    Q, K = _seq(rng, 30)
    _, lse = mla.attention_partial(Q, K, mla.SM_SCALE)
    s = mla.SM_SCALE * (Q @ K.T)
    assert np.max(np.abs(lse - np.log(np.exp(s).sum(axis=1)))) <= 1e-12


# ------------------------------------------------------------ final log-sum-exp


def test_final_lse_zero_query_is_log_n():
    # every score is 0, so sum_j exp(0) = n
    rng = np.random.default_rng(31)
    _, K = _seq(rng, 37)
    lse = mla.mla_decode_sequence_lse(np.zeros((16, 576)), K, mla.SM_SCALE)
    assert np.max(np.abs(lse - math.log(37))) <= 1e-14


def test_final_lse_single_row_is_its_score():
    rng = np.random.default_rng(32)
    Q, K = _seq(rng, 1, 3.0)
    lse = mla.mla_decode_sequence_lse(Q, K, mla.SM_SCALE)
    s = [math.fsum(Q[h, d] * K[0, d] for d in range(576)) / 24.0 for h in range(16)]
    assert np.max(np.abs(lse - np.array(s))) <= 1e-12


def test_final_lse_duplicate_row_adds_its_weight():
    # duplicating every row doubles the sum: + log 2
    rng = np.random.default_rng(33)
    Q, K = _seq(rng, 25, 2.0)
    a = mla.mla_decode_sequence_lse(Q, K, mla.SM_SCALE)
    b = mla.mla_decode_sequence_lse(Q, np.concatenate([K, K]), mla.SM_SCALE)
    assert np.max(np.abs(b - a - math.log(2.0))) <= 1e-13


def test_final_lse_vs_scipy_logsumexp_of_bruteforce_scores():
    from scipy.special import logsumexp

    rng = np.random.default_rng(34)
    lens = [1, 3, 5]
    q_bits, kv_bits, qo, kvp, idx, _ = _rand_case(rng, 3, lens, permute=True)
    got = oracle.mla_decode_lse(q_bits, kv_bits, qo, kvp, idx, q_dtype="bf16", kv_dtype="bf16")
    for b in range(3):
        Q = formats.decode_bf16(q_bits[b]).tolist()
        K = [formats.decode_bf16(kv_bits[idx[i]]).tolist() for i in range(kvp[b], kvp[b + 1])]
        for h in range(16):
            s = [math.fsum(Q[h][d] * K[j][d] for d in range(576)) / 24.0 for j in range(len(K))]
            assert abs(logsumexp(s) - got[b, h]) <= 1e-12


def test_final_lse_equals_merge_of_part_lses():
    rng = np.random.default_rng(35)
    Q, K = _seq(rng, 301, 2.0)
    bounds = [0, 1, 90, 91, 250, 301]
    lses = np.stack([mla.attention_partial(Q, K[a:b], mla.SM_SCALE)[1] for a, b in zip(bounds[:-1], bounds[1:])])
    whole = mla.mla_decode_sequence_lse(Q, K, mla.SM_SCALE)
    assert np.max(np.abs(mla.merge_lse(lses) - whole)) <= 1e-12
    # empty parts add nothing; no parts or only empty ones give -inf
    empty = mla.attention_partial(Q, K[:0], mla.SM_SCALE)[1]
    assert np.max(np.abs(mla.merge_lse(np.stack([empty, *lses])) - whole)) <= 1e-12
    assert np.all(np.isneginf(mla.merge_lse(np.stack([empty, empty]))))
    assert np.all(np.isneginf(mla.merge_lse(np.zeros((0, 16)))))


def test_final_lse_soft_cap_limits():
    # a tiny cap flattens every score to ~0 (log n); a huge cap changes nothing
    rng = np.random.default_rng(36)
    Q, K = _seq(rng, 40, 3.0)
    assert np.max(np.abs(mla.mla_decode_sequence_lse(Q, K, mla.SM_SCALE, logit_cap=1e-9) - math.log(40))) <= 1e-8
    plain = mla.mla_decode_sequence_lse(Q, K, mla.SM_SCALE)
    assert np.max(np.abs(mla.mla_decode_sequence_lse(Q, K, mla.SM_SCALE, logit_cap=1e9) - plain)) <= 1e-9


def test_final_lse_tokens_and_empty_sequences():
    # causal token i sees a prefix (its lse is that prefix's); tokens of an empty sequence get -inf
    rng = np.random.default_rng(37)
    q_bits = torch.from_numpy(rng.standard_normal((4, 16, 576)).astype(np.float32)).to(torch.bfloat16)
    q_bits = q_bits.view(torch.int16).numpy()
    kv = torch.from_numpy(rng.standard_normal((9, 576)).astype(np.float32)).to(torch.bfloat16)
    kv_bits = kv.view(torch.int16).numpy()
    qo, kvp, idx = [0, 3, 4], [0, 9, 9], list(range(9))
    got = oracle.mla_decode_lse(q_bits, kv_bits, qo, kvp, idx, q_dtype="bf16", kv_dtype="bf16", causal=True)
    K = formats.decode_bf16(kv_bits)
    for i in range(3):
        ref = mla.mla_decode_sequence_lse(formats.decode_bf16(q_bits[i]), K[:9 - 2 + i], mla.SM_SCALE)
        assert np.array_equal(got[i], ref)
    assert np.all(np.isneginf(got[3]))


# -------------------------------------------------------------------- invariants


def test_pool_permutation_invariance():
    rng = np.random.default_rng(21)
    lens = [40, 1, 90]
    q_bits, kv_bits, qo, kvp, idx, _ = _rand_case(rng, 3, lens, permute=False)
    a = oracle.mla_decode(q_bits, kv_bits, qo, kvp, idx, q_dtype="bf16", kv_dtype="bf16")
    perm = rng.permutation(kv_bits.shape[0])
    moved = np.empty_like(kv_bits)
    moved[perm] = kv_bits
    b = oracle.mla_decode(q_bits, moved, qo, kvp, perm[idx], q_dtype="bf16", kv_dtype="bf16")
    assert np.array_equal(a, b)


def test_head_permutation_and_scale_trade():
    rng = np.random.default_rng(22)
    Q, K = _seq(rng, 70)
    perm = rng.permutation(16)
    O = mla.mla_decode_sequence(Q, K, mla.SM_SCALE)
    assert np.max(np.abs(mla.mla_decode_sequence(Q[perm], K, mla.SM_SCALE) - O[perm])) <= 1e-14
    assert np.max(np.abs(mla.mla_decode_sequence(Q / 4.0, K, mla.SM_SCALE * 4.0) - O)) <= 1e-13


def test_sequences_are_independent():
    rng = np.random.default_rng(23)
    lens = [50, 60]
    q_bits, kv_bits, qo, kvp, idx, _ = _rand_case(rng, 2, lens)
    a = oracle.mla_decode(q_bits, kv_bits, qo, kvp, idx, q_dtype="bf16", kv_dtype="bf16")
    kv2 = kv_bits.copy()
    kv2[60:] = kv2[60:][::-1]  # scramble sequence 1's rows only
    b = oracle.mla_decode(q_bits, kv2, qo, kvp, idx, q_dtype="bf16", kv_dtype="bf16")
    assert np.array_equal(a[0], b[0]) and not np.array_equal(a[1], b[1])


# ------------------------------------------------------------- mutation checks


def _mutants():
    """Plausible mistakes in an MLA-decode implementation, planted on the CPU."""

    def no_rope(Q, K):
        return mla.mla_decode_sequence(Q[:, :512], K[:, :512], mla.SM_SCALE)

    def wrong_scale(Q, K):
        return mla.mla_decode_sequence(Q, K, 1.0 / math.sqrt(512.0))

    def v_from_tail(Q, K):
        S = mla.SM_SCALE * Q @ K.T
        P = np.exp(S - S.max(1, keepdims=True))
        P /= P.sum(1, keepdims=True)
        return P @ K[:, 64:]

    def drop_last_row(Q, K):
        return mla.mla_decode_sequence(Q, K[:-1], mla.SM_SCALE)

    def no_max_subtract_but_wrong_sign(Q, K):
        return mla.mla_decode_sequence(-Q, K, mla.SM_SCALE)

    def head_swap(Q, K):
        return mla.mla_decode_sequence(Q[::-1].copy(), K, mla.SM_SCALE)[::-1]

    def first_head_only(Q, K):
        O = mla.mla_decode_sequence(Q, K, mla.SM_SCALE)
        return np.broadcast_to(O[0], O.shape)

    return [no_rope, wrong_scale, v_from_tail, drop_last_row, no_max_subtract_but_wrong_sign, first_head_only]


@pytest.mark.parametrize("n", [1024, 8192])
def test_mutants_fail_the_gate(n):
    rng = np.random.default_rng(31 + n)
    Q = formats.decode_bf16(torch.from_numpy(rng.standard_normal((16, 576)).astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy())
    K = formats.decode_bf16(torch.from_numpy(rng.standard_normal((n, 576)).astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy())
    ref = mla.mla_decode_sequence(Q, K, mla.SM_SCALE)
    # the true result rounded to bf16 passes
    rounded = formats.decode_bf16(formats.encode_bf16_rne(ref[:2]))
    assert gate(ref[:2], rounded)
    for mut in _mutants():
        if mut.__name__ == "drop_last_row" and n > 1024:
            continue  # one row in 8192 is below any bf16-level gate; checked at n=1024 only
        got = mut(Q, K)
        assert not gate(ref, got), mut.__name__


def test_mutant_missing_kv_scale_fails():
    rng = np.random.default_rng(41)
    lens = [256, 512]
    q_bits, kv_bits, qo, kvp, idx, kvs = _rand_case(rng, 2, lens, dtype_kv="fp8")
    ref = oracle.mla_decode(q_bits, kv_bits, qo, kvp, idx, q_dtype="bf16", kv_dtype="fp8", kv_scale=kvs)
    bad = oracle.mla_decode(q_bits, kv_bits, qo, kvp, idx, q_dtype="bf16", kv_dtype="fp8", kv_scale=1.0)
    assert not gate(ref, bad)


# -------------------------------------------------------------------- generator


def test_generator_is_seeded_and_shaped():
    spec = synth.CaseSpec(batch=5, q_dtype="bf16", kv_dtype="fp8", ragged_max=300, permuted=True, seed=77)
    a = synth.make_case(spec)
    b = synth.make_case(spec)
    assert torch.equal(a.kv.view(torch.uint8), b.kv.view(torch.uint8)) and torch.equal(a.kv_indices, b.kv_indices)
    assert a.q_bf16.shape == (5, 16, 576) and a.kv.shape == (int(a.lengths.sum()), 576)
    assert int(a.kv_indptr[-1]) == int(a.lengths.sum()) and a.lengths.min() >= 1
    assert sorted(a.kv_indices.tolist()) == list(range(a.kv.shape[0]))
    # per-tensor scale maps the largest magnitude onto the fp8 maximum
    assert a.kv.view(torch.uint8).numpy().view(np.uint8).max() in (0x7E, 0xFE) or \
        np.abs(formats.decode_fp8_e4m3fn(a.kv.view(torch.uint8).numpy())).max() == 448.0


# ------------------------------------------------------------ logit soft-cap


def test_soft_cap_zero_is_off_and_large_cap_is_plain():
    rng = np.random.default_rng(51)
    Q, K = _seq(rng, 200, 2.0)
    plain = mla.mla_decode_sequence(Q, K, mla.SM_SCALE)
    assert np.array_equal(mla.mla_decode_sequence(Q, K, mla.SM_SCALE, logit_cap=0.0), plain)
    # cap * tanh(s / cap) = s - s^3 / (3 cap^2) + ...: scores of size ~5 move by ~1e-11 at cap 1e6
    assert np.max(np.abs(mla.mla_decode_sequence(Q, K, mla.SM_SCALE, logit_cap=1e6) - plain)) <= 1e-9


def test_soft_cap_tiny_cap_flattens_to_mean_of_v():
    rng = np.random.default_rng(52)
    Q, K = _seq(rng, 33, 5.0)
    O = mla.mla_decode_sequence(Q, K, mla.SM_SCALE, logit_cap=1e-9)  # every capped score is within 1e-9 of 0
    assert np.max(np.abs(O - K[:, :512].mean(axis=0))) <= 1e-8


def test_soft_cap_three_to_one_closed_form():
    """Two rows whose scaled scores are cap*atanh(1/2) and 0: capped they are cap/2 and 0,
    and with cap = 2 ln 3 the softmax weights are exactly 3/4 and 1/4 for every head."""
    rng = np.random.default_rng(53)
    cap = 2.0 * math.log(3.0)
    Q = rng.standard_normal((16, 576))
    target = cap * math.atanh(0.5) / mla.SM_SCALE  # raw dot product wanted for row 0, all heads
    k0 = Q.T @ np.linalg.solve(Q @ Q.T, np.full(16, target))  # least-norm solution of Q k0 = target
    k1 = rng.standard_normal(576)
    k1 -= Q.T @ np.linalg.solve(Q @ Q.T, Q @ k1)  # orthogonal to every head's query: score 0
    K = np.stack([k0, k1])
    assert np.max(np.abs(Q @ k1)) <= 1e-9 and np.max(np.abs(Q @ k0 - target)) <= 1e-9
    O = mla.mla_decode_sequence(Q, K, mla.SM_SCALE, logit_cap=cap)
    assert np.max(np.abs(O - (0.75 * k0[:512] + 0.25 * k1[:512]))) <= 1e-9 * np.max(np.abs(K))
    # a cap applied before sm_scale, or tanh without the 1/cap inside, misses this value
    wrong = mla.soft_cap(Q @ K.T, cap) * mla.SM_SCALE
    assert not np.allclose(np.exp(wrong[:, 0] - wrong[:, 1]), 3.0, rtol=1e-3)
    assert not np.allclose(cap * np.tanh(mla.SM_SCALE * (Q @ k0)), cap / 2, rtol=1e-3)


def test_soft_cap_rejects_negative():
    with pytest.raises(ValueError):
        mla.soft_cap(np.zeros(3), -1.0)


# ------------------------------------------------------------------ pages


def test_paged_rows_worked_example():
    kv_indptr = [0, 2, 3, 3]
    kv_indices = [5, 2, 7]
    # page p of 4 rows holds pool rows 4p..4p+3; last pages hold 3, 4 and (empty sequence) - rows
    assert oracle.paged_rows(kv_indptr, kv_indices, 0, 4, [3, 4, 1]).tolist() == [20, 21, 22, 23, 8, 9, 10]
    assert oracle.paged_rows(kv_indptr, kv_indices, 1, 4, [3, 4, 1]).tolist() == [28, 29, 30, 31]
    assert oracle.paged_rows(kv_indptr, kv_indices, 2, 4, [3, 4, 1]).tolist() == []
    # lengths outside [1, page_size] clamp: 9 -> 4 (full), 0 -> 1
    assert oracle.paged_rows(kv_indptr, kv_indices, 0, 4, [9, 0, 1]).tolist() == [20, 21, 22, 23, 8, 9, 10, 11]
    assert oracle.paged_rows(kv_indptr, kv_indices, 1, 4, [9, 0, 1]).tolist() == [28]
    # no lengths: every page full; page size 1: the indices themselves
    assert oracle.paged_rows(kv_indptr, kv_indices, 0, 2).tolist() == [10, 11, 4, 5]
    assert oracle.paged_rows(kv_indptr, kv_indices, 0, 1).tolist() == [5, 2]


@pytest.mark.parametrize("ps", [2, 8, 16])
def test_paged_pool_equals_row_pool(ps):
    """The same logical rows laid into pages of ps rows (pages shuffled, the tail of each
    last page filled with junk) give the page-size-1 result."""
    rng = np.random.default_rng(60 + ps)
    lens = [1, ps, ps + 1, 3 * ps - 1, 100]
    B = len(lens)
    q_bits, kv_bits, qo, kvp, idx, _ = _rand_case(rng, B, lens)
    ref = oracle.mla_decode(q_bits, kv_bits, qo, kvp, idx, q_dtype="bf16", kv_dtype="bf16")
    pages_per = [(n + ps - 1) // ps for n in lens]
    n_pages = sum(pages_per) + 3
    order = rng.permutation(n_pages)
    pool = rng.integers(-30000, 30000, size=(n_pages * ps, 576)).astype(np.int16)  # junk everywhere
    kv_indices, last, nxt = [], [], 0
    for b, n in enumerate(lens):
        for pg in range(pages_per[b]):
            page = int(order[nxt])
            nxt += 1
            kv_indices.append(page)
            for s in range(ps):
                r = pg * ps + s
                if r < n:
                    pool[page * ps + s] = kv_bits[idx[kvp[b] + r]]
        last.append(n - (pages_per[b] - 1) * ps)
    page_indptr = np.concatenate([[0], np.cumsum(pages_per)])
    got = oracle.mla_decode(q_bits, pool, qo, page_indptr, kv_indices, q_dtype="bf16", kv_dtype="bf16",
                            page_size=ps, kv_last_page_len=last)
    assert np.array_equal(got, ref)


def test_page_size_one_with_sequence_length_as_last_len():
    # one page passes the sequence length as the last-page length with page size 1: every page full
    rng = np.random.default_rng(70)
    lens = [7, 40]
    q_bits, kv_bits, qo, kvp, idx, _ = _rand_case(rng, 2, lens, permute=True)
    ref = oracle.mla_decode(q_bits, kv_bits, qo, kvp, idx, q_dtype="bf16", kv_dtype="bf16")
    got = oracle.mla_decode(q_bits, kv_bits, qo, kvp, idx, q_dtype="bf16", kv_dtype="bf16", page_size=1,
                            kv_last_page_len=lens)
    assert np.array_equal(got, ref)


# --------------------------------------------------------- several query tokens


def _multi_token_case(rng, lens, q_lens):
    B = len(lens)
    total_q = int(sum(q_lens))
    q_bits = torch.from_numpy(rng.standard_normal((total_q, 16, 576)).astype(np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy()
    kv_bits = torch.from_numpy(rng.standard_normal((int(sum(lens)), 576)).astype(np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy()
    qo = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    kvp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q_bits, kv_bits, qo, kvp, np.arange(int(sum(lens)))


def _sdpa_tokens(q_bits, kv_bits, t0, q_len, r0, n, is_causal):
    Q = torch.from_numpy(q_bits[t0:t0 + q_len]).view(torch.bfloat16).to(torch.float64)  # [q, 16, 576]
    K = torch.from_numpy(kv_bits[r0:r0 + n]).view(torch.bfloat16).to(torch.float64)
    q4 = Q.permute(1, 0, 2)[None]  # [1, 16, q, 576]
    k4 = K[None, None].expand(1, 16, n, 576)
    v4 = K[:, :512][None, None].expand(1, 16, n, 512)
    o = torch.nn.functional.scaled_dot_product_attention(q4, k4, v4, scale=1.0 / 24.0, is_causal=is_causal)
    return o[0].permute(1, 0, 2).numpy()  # [q, 16, 512]


def test_causal_prefill_equals_sdpa_is_causal():
    # when every row of a sequence is also a query token (q_len = L), the causal rule is the
    # square lower-triangular mask of scaled_dot_product_attention(is_causal=True)
    rng = np.random.default_rng(80)
    lens = [1, 5, 12]
    q_bits, kv_bits, qo, kvp, idx = _multi_token_case(rng, lens, lens)
    got = oracle.mla_decode(q_bits, kv_bits, qo, kvp, idx, q_dtype="bf16", kv_dtype="bf16", causal=True)
    for b, n in enumerate(lens):
        ref = _sdpa_tokens(q_bits, kv_bits, qo[b], n, kvp[b], n, True)
        assert np.max(np.abs(got[qo[b]:qo[b + 1]] - ref)) <= 1e-12


def test_non_causal_tokens_equal_sdpa_without_mask():
    rng = np.random.default_rng(81)
    lens, q_lens = [9, 300], [3, 2]
    q_bits, kv_bits, qo, kvp, idx = _multi_token_case(rng, lens, q_lens)
    got = oracle.mla_decode(q_bits, kv_bits, qo, kvp, idx, q_dtype="bf16", kv_dtype="bf16", causal=False)
    for b in range(2):
        ref = _sdpa_tokens(q_bits, kv_bits, qo[b], q_lens[b], kvp[b], lens[b], False)
        assert np.max(np.abs(got[qo[b]:qo[b + 1]] - ref)) <= 1e-12


def test_causal_token_sees_its_prefix():
    # token i of q_len decodes over the first L - q_len + 1 + i rows; the last token sees all of them;
    # tokens whose prefix is empty (L < q_len) give zeros
    rng = np.random.default_rng(82)
    lens, q_lens = [50, 2, 1], [4, 4, 3]
    q_bits, kv_bits, qo, kvp, idx = _multi_token_case(rng, lens, q_lens)
    got = oracle.mla_decode(q_bits, kv_bits, qo, kvp, idx, q_dtype="bf16", kv_dtype="bf16", causal=True)
    for b, (L, ql) in enumerate(zip(lens, q_lens)):
        for i in range(ql):
            n = L - ql + 1 + i
            t = qo[b] + i
            if n <= 0:
                assert np.array_equal(got[t], np.zeros((16, 512)))
                continue
            one = oracle.mla_decode(q_bits[t:t + 1], kv_bits, [0, 1], [kvp[b], kvp[b] + n], idx, q_dtype="bf16",
                                    kv_dtype="bf16")
            assert np.array_equal(got[t], one[0])
    assert oracle.visible_rows(50, 4, 3, True) == 50 and oracle.visible_rows(50, 4, 0, True) == 47
    assert oracle.visible_rows(2, 4, 1, True) == 0 and oracle.visible_rows(2, 4, 0, False) == 2


# ------------------------------------------------------- amax-scaled Q cast


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy()


@pytest.mark.parametrize("mag", [1e-3, 1.0, 37.0, 3e4])
def test_dynamic_q_cast_vs_torch(mag):
    rng = np.random.default_rng(90)
    bits = _bf16_bits(rng.standard_normal((3, 16, 576)) * mag)
    codes, scale = oracle.quantize_q_dynamic(bits)
    x = torch.from_numpy(bits).view(torch.bfloat16).to(torch.float32)
    t_scale = x.abs().max() / torch.tensor(448.0, dtype=torch.float32)
    t_codes = (x / t_scale).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.float32(scale) == t_scale.item()
    assert np.array_equal(codes, t_codes)
    # the largest magnitude lands on +-448 and the dequantised values stay within half an fp8 step
    i = np.argmax(np.abs(x.numpy()))
    assert codes.reshape(-1)[i] & 0x7F == 0x7E
    deq = formats.decode_fp8_e4m3fn(codes) * scale
    xv = x.numpy().astype(np.float64)
    big = np.abs(xv) >= 2.0 ** -6 * scale
    assert np.all(np.abs(deq - xv)[big] <= 2.0 ** -4 * np.abs(xv)[big] * (1 + 1e-6))


def test_dynamic_q_cast_degenerate_inputs():
    codes, scale = oracle.quantize_q_dynamic(_bf16_bits([0.0, -0.0, 0.0]))
    assert scale == 1.0 and codes.tolist() == [0x00, 0x80, 0x00]
    codes, scale = oracle.quantize_q_dynamic(np.zeros(0, dtype=np.int16))
    assert scale == 1.0 and codes.size == 0
    # non-finite values become the NaN code with their sign and do not enter the amax
    bits = _bf16_bits([1.0, -2.0, 0.5]).copy()
    bits = np.concatenate([bits, np.array([0x7F80, 0xFF80, 0x7FC1], dtype=np.uint16).view(np.int16)])
    codes, scale = oracle.quantize_q_dynamic(bits)
    assert np.float32(scale) == np.float32(2.0) / np.float32(448.0)
    assert codes[3:].tolist() == [0x7F, 0xFF, 0x7F]
    assert codes[1] == 0xFE  # -2 -> -448
