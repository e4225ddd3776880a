"""Seeded synthetic MLA-decode inputs (shared by the tests, the smoke check and the bench).

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Everything is generated on the CPU with
``torch.Generator`` so the float64 oracle and the GPU read the very same bytes.

Recipe (the workload shapes of the kernelindex amd-mixed-mla submissions:
16 heads x 576 over one 576-wide latent KV head, page size 1 for the decode
configurations; the harness's own generator is not on the pages, so these
distributions stand in for it):

* Q: ``randn`` float32 -> bf16, shape [total_q, 16, 576] (one query token per
  sequence unless ``q_lens`` gives more).  fp8 Q is *not* made here: casting
  Q is step a0 of the path and is done by the library (or by the oracle's own
  encoder) from these bf16 bits.
* bf16 KV: ``randn`` float32 -> bf16, shape [rows, 576].
* fp8 KV: ``randn`` float32, per-tensor scale ``amax(|kv|) / 448`` in float32,
  then ``(kv / scale).to(float8_e4m3fn)`` (torch's cast); the scale is returned
  next to the codes, as the pages receive ``(kv_fp8, kv_scale)``.
* lengths: a fixed length per sequence, or ``randint(1, max_len + 1)`` per
  sequence for the ragged case.
* pages of ``page_size`` rows: sequence b of L rows takes ceil(L / page_size)
  pages, the last one holding ``kv_last_page_len[b]`` rows (the unused slots
  keep their random values, so a kernel that reads them is caught).
* ``kv_indptr`` = exclusive cumulative sum of the pages per sequence;
  ``qo_indptr`` = exclusive cumulative sum of the query tokens per sequence.
* ``kv_indices``: ``arange`` (contiguous pool) or a seeded ``randperm`` of the
  pool pages (ragged, paged case).
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import torch

__all__ = ["CaseSpec", "Case", "CONFIGS", "FEATURE_WORKLOADS", "make_case", "config_spec", "workload"]

NUM_HEADS = 16
QK_DIM = 576


@dataclasses.dataclass(frozen=True)
class CaseSpec:
    batch: int
    q_dtype: str  # "bf16" or "fp8" (fp8 means: cast from the bf16 Q by step a0)
    kv_dtype: str  # "bf16" or "fp8"
    kv_len: int = 0  # fixed per-sequence length (used when lengths is None and not ragged)
    lengths: Optional[Sequence[int]] = None  # explicit per-sequence lengths
    ragged_max: int = 0  # > 0: lengths ~ randint(1, ragged_max + 1)
    permuted: bool = False  # kv_indices = randperm(pool) instead of arange
    extra_pool_rows: int = 0  # pool rows not referenced by any sequence (permuted pools)
    seed: int = 0  # base seed; Q/KV/lengths/permutation use seed+1..seed+4
    page_size: int = 1  # rows per page
    q_lens: Optional[Sequence[int]] = None  # query tokens per sequence (None: one each)

    @property
    def name(self) -> str:
        kind = f"ragged{self.ragged_max}" if self.ragged_max else f"kv{self.kv_len}"
        return f"b{self.batch}_{kind}_{self.q_dtype}q_{self.kv_dtype}kv"


@dataclasses.dataclass
class Case:
    spec: CaseSpec
    q_bf16: torch.Tensor  # [total_q, 16, 576] bf16
    kv: torch.Tensor  # [pool_pages * page_size, 576] bf16 or float8_e4m3fn
    kv_scale: Optional[torch.Tensor]  # [1] float32 for fp8 KV, else None
    qo_indptr: torch.Tensor  # [batch + 1] int32
    kv_indptr: torch.Tensor  # [batch + 1] int32, in pages
    kv_indices: torch.Tensor  # [total pages] int32
    lengths: torch.Tensor  # [batch] int64, rows per sequence
    kv_last_page_len: Optional[torch.Tensor] = None  # [batch] int32, rows in each last page

    @property
    def total_kv(self) -> int:
        """KV rows over all sequences."""
        return int(self.lengths.sum())

    @property
    def total_q(self) -> int:
        return int(self.qo_indptr[-1])

    def q_bits(self) -> torch.Tensor:
        """bf16 Q as raw 16-bit patterns (int16 storage)."""
        return self.q_bf16.view(torch.int16)

    def kv_bits(self) -> torch.Tensor:
        """KV as raw patterns: int16 for bf16, uint8 for e4m3fn."""
        if self.kv.dtype == torch.bfloat16:
            return self.kv.view(torch.int16)
        return self.kv.view(torch.uint8)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def make_case(spec: CaseSpec) -> Case:
    B = spec.batch
    if spec.lengths is not None:
        lengths = torch.tensor(list(spec.lengths), dtype=torch.int64)
        assert lengths.numel() == B
    elif spec.ragged_max > 0:
        lengths = torch.randint(1, spec.ragged_max + 1, (B,), generator=_gen(spec.seed + 3), dtype=torch.int64)
    else:
        lengths = torch.full((B,), spec.kv_len, dtype=torch.int64)
    ps = spec.page_size
    pages = (lengths + ps - 1) // ps
    total_pages = int(pages.sum())
    pool_pages = total_pages + (spec.extra_pool_rows + ps - 1) // ps
    rows = pool_pages * ps
    q_lens = torch.ones(B, dtype=torch.int64) if spec.q_lens is None else torch.tensor(list(spec.q_lens))
    assert q_lens.numel() == B
    total_q = int(q_lens.sum())

    q = torch.randn((total_q, NUM_HEADS, QK_DIM), generator=_gen(spec.seed + 1), dtype=torch.float32).to(
        torch.bfloat16)

    kv32 = torch.randn((rows, QK_DIM), generator=_gen(spec.seed + 2), dtype=torch.float32)
    if spec.kv_dtype == "bf16":
        kv = kv32.to(torch.bfloat16)
        kv_scale = None
    elif spec.kv_dtype == "fp8":
        amax = kv32.abs().max() if rows > 0 else torch.tensor(1.0)
        scale = (amax / 448.0).to(torch.float32).reshape(1)
        kv = (kv32 / scale).to(torch.float8_e4m3fn)
        kv_scale = scale
    else:
        raise ValueError(spec.kv_dtype)
    del kv32

    kv_indptr = torch.zeros(B + 1, dtype=torch.int64)
    kv_indptr[1:] = torch.cumsum(pages, 0)
    qo_indptr = torch.zeros(B + 1, dtype=torch.int64)
    qo_indptr[1:] = torch.cumsum(q_lens, 0)
    if spec.permuted:
        kv_indices = torch.randperm(pool_pages, generator=_gen(spec.seed + 4))[:total_pages]
    else:
        kv_indices = torch.arange(total_pages, dtype=torch.int64)
    last = torch.where(pages > 0, lengths - (pages - 1) * ps, torch.full_like(lengths, ps))
    return Case(
        spec=spec,
        q_bf16=q,
        kv=kv,
        kv_scale=kv_scale,
        qo_indptr=qo_indptr.to(torch.int32),
        kv_indptr=kv_indptr.to(torch.int32),
        kv_indices=kv_indices.to(torch.int32),
        lengths=lengths,
        kv_last_page_len=last.to(torch.int32),
    )


# The five workloads the pages' leaderboard shapes reduce to, plus the
# bs=64 / kv=8192 fp8-KV case the headline throughput is quoted on (in its
# bf16-Q and its fp8-Q form).  Seeds follow 1000*c: Q +1, KV +2, lengths +3,
# permutation +4.
CONFIGS = {
    "c1_bf16_b4_kv1024": CaseSpec(batch=4, q_dtype="bf16", kv_dtype="bf16", kv_len=1024, seed=1000),
    "c2_bf16q_fp8kv_b64_kv1024": CaseSpec(batch=64, q_dtype="bf16", kv_dtype="fp8", kv_len=1024, seed=2000),
    "c3_a8w8_b32_kv8192": CaseSpec(batch=32, q_dtype="fp8", kv_dtype="fp8", kv_len=8192, seed=3000),
    "c4_a8w8_b256_kv8192": CaseSpec(batch=256, q_dtype="fp8", kv_dtype="fp8", kv_len=8192, seed=4000),
    "c5_ragged_bf16q_fp8kv_b128": CaseSpec(
        batch=128, q_dtype="bf16", kv_dtype="fp8", ragged_max=8192, permuted=True, seed=5000
    ),
    "m_bf16q_fp8kv_b64_kv8192": CaseSpec(batch=64, q_dtype="bf16", kv_dtype="fp8", kv_len=8192, seed=6000),
    "m_a8w8_b64_kv8192": CaseSpec(batch=64, q_dtype="fp8", kv_dtype="fp8", kv_len=8192, seed=6000),
}


# The widened forms at the headline shape (64 sequences of 8192 rows, fp8
# KV): pages of 16 rows, the amax-scaled Q cast, two causal query tokens per
# sequence, and a soft-cap of 30.  Each entry: the case and how to run it.
FEATURE_WORKLOADS = {
    "f1_paged16_bf16q_fp8kv_b64_kv8192": (
        CaseSpec(batch=64, q_dtype="bf16", kv_dtype="fp8", kv_len=8192, permuted=True, page_size=16, seed=7000),
        {}),
    "f2_dynq_a8w8_b64_kv8192": (
        CaseSpec(batch=64, q_dtype="fp8", kv_dtype="fp8", kv_len=8192, seed=6000), {"dynamic_q": True}),
    "f3_mtp2_causal_bf16q_fp8kv_b64_kv8192": (
        CaseSpec(batch=64, q_dtype="bf16", kv_dtype="fp8", kv_len=8192, q_lens=[2] * 64, seed=7100),
        {"causal": True}),
    "f3_mtp2_causal_a8w8_b64_kv8192": (
        CaseSpec(batch=64, q_dtype="fp8", kv_dtype="fp8", kv_len=8192, q_lens=[2] * 64, seed=7100),
        {"causal": True}),
    "f4_cap30_bf16q_fp8kv_b64_kv8192": (
        CaseSpec(batch=64, q_dtype="bf16", kv_dtype="fp8", kv_len=8192, seed=6000), {"logit_cap": 30.0}),
    "f3_mtp2_causal_bf16_b64_kv8192": (
        CaseSpec(batch=64, q_dtype="bf16", kv_dtype="bf16", kv_len=8192, q_lens=[2] * 64, seed=7100),
        {"causal": True}),
}


def config_spec(name: str) -> CaseSpec:
    return CONFIGS[name]


def workload(name: str):
    """(CaseSpec, run options) of a named workload: a decode configuration or a widened form."""
    if name in CONFIGS:
        return CONFIGS[name], {}
    return FEATURE_WORKLOADS[name]
