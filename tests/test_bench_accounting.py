"""The bench's algorithmic byte count against the figures tabulated for each configuration.

The bench reports HBM throughput as algorithmic bytes per second: every KV row once (576 B fp8,
1152 B bf16), a 4-byte page index per row, Q (fp8 when cast before the launch), the bf16 output and
both indptr arrays.  The expected values below were worked out per configuration from the shapes
alone, independently of bench.py, and are the ones the roofline targets are stated against.  The
cases are light stand-ins carrying only what the count reads, so no KV pool is generated.
"""

from __future__ import annotations

import types

import pytest
import torch

import bench
from mla_decode_paged_split_amd import synth

# configuration -> algorithmic bytes with fp8 Q read as 1 byte per value (bf16 Q as 2)
EXPECTED = {
    "c1_bf16_b4_kv1024": 4_874_280,
    "c2_bf16q_fp8kv_b64_kv1024": 40_239_624,
    "c3_a8w8_b32_kv8192": 152_862_984,
    "c4_a8w8_b256_kv8192": 1_222_903_816,
    "m_bf16q_fp8kv_b64_kv8192": 306_315_784,
    "m_a8w8_b64_kv8192": 305_725_960,
}


def stand_in(spec):
    B, L = spec.batch, spec.kv_len
    return types.SimpleNamespace(total_q=B, total_kv=B * L, kv_indptr=torch.arange(B + 1, dtype=torch.int32) * L)


@pytest.mark.parametrize("name", list(EXPECTED))
def test_algorithmic_bytes(name):
    spec = synth.CONFIGS[name]
    q_elt = 1 if spec.q_dtype == "fp8" else 2
    assert bench.algorithmic_bytes(spec, stand_in(spec), q_elt) == EXPECTED[name]


def test_fused_cast_counts_bf16_q():
    # with the cast inside the attention launch, that launch reads Q as bf16: 1 more byte per value
    spec = synth.CONFIGS["m_a8w8_b64_kv8192"]
    extra = spec.batch * 16 * 576
    assert bench.algorithmic_bytes(spec, stand_in(spec), 2) == EXPECTED["m_a8w8_b64_kv8192"] + extra


def test_mfma_flops_of_the_headline_batch():
    # 2 flops per multiply-add, 16 heads, 576 (scores) + 512 (P.V) per visible row: 34,816 per row
    spec = synth.CONFIGS["m_bf16q_fp8kv_b64_kv8192"]
    case = types.SimpleNamespace(qo_indptr=torch.arange(spec.batch + 1), lengths=torch.full((spec.batch,), 8192))
    assert bench.mfma_flops(case, causal=False) == 64 * 8192 * 34_816 == 18_253_611_008


def test_causal_flops_count_each_tokens_prefix():
    # two tokens over 10 rows, causal: token 0 sees 9 rows, token 1 sees 10
    case = types.SimpleNamespace(qo_indptr=torch.tensor([0, 2]), lengths=torch.tensor([10]))
    assert bench.mfma_flops(case, causal=True) == (9 + 10) * 34_816
    assert bench.mfma_flops(case, causal=False) == 20 * 34_816
