"""Helpers shared by the GPU tests: run a synthetic case through the C ABI and
through the float64 oracle, and compare them with the parity gate."""

from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
from mla_decode_paged_split_amd import binding, synth

RTOL, ATOL = 2e-2, 1e-2  # elementwise, torch.allclose rule
NORM_GATE = 1e-2  # normwise relative error


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class DevCase:
    """A synthetic case moved to the device, with fp8 Q made by the library's cast (step a0)."""

    def __init__(self, case: synth.Case, dev: torch.device):
        self.case = case
        self.dev = dev
        self.q_bf16 = case.q_bf16.to(dev)
        self.kv = case.kv.to(dev)
        self.kv_scale = case.kv_scale.to(dev) if case.kv_scale is not None else None
        self.qo_indptr = case.qo_indptr.to(dev)
        self.kv_indptr = case.kv_indptr.to(dev)
        self.kv_indices = case.kv_indices.to(dev)
        self.kv_last_page_len = case.kv_last_page_len.to(dev) if case.kv_last_page_len is not None else None
        self.page_size = case.spec.page_size
        self.total_q = case.total_q
        self.max_q_len = int((case.qo_indptr[1:] - case.qo_indptr[:-1]).max())
        self.q_dtype = case.spec.q_dtype
        self.kv_dtype = case.spec.kv_dtype
        if self.q_dtype == "fp8":
            self.q = torch.empty(self.q_bf16.shape, dtype=torch.uint8, device=dev)
            binding.mla_decode_quantize_q(self.q_bf16, self.q)
            self.q_scale = torch.ones(1, dtype=torch.float32, device=dev)
        else:
            self.q = self.q_bf16
            self.q_scale = None

    @property
    def batch(self) -> int:
        return self.case.spec.batch

    def decoder(self, **kw) -> binding.Decoder:
        kw.setdefault("page_size", self.page_size)
        kw.setdefault("max_q_len", self.max_q_len if self.max_q_len > 1 else 0)
        kw.setdefault("total_q", self.total_q)
        return binding.Decoder(self.batch, self.q_dtype, self.kv_dtype, self.dev, **kw)

    def run(self, dec: binding.Decoder | None = None, out: torch.Tensor | None = None, q_cast: bool = False,
            causal: bool = False, paged: bool | None = None, sm_scale: float = oracle.SM_SCALE,
            **kw) -> torch.Tensor:
        """One decode step; with q_cast the fp8 Q is cast inside the attention kernel from the bf16 Q.

        Pages of more than one row go through mla_decode_run_paged with the case's last-page lengths
        (``paged`` forces either entry point)."""
        if q_cast:
            kw["flags"] = kw.get("flags", 0) | binding.MLA_FLAG_FUSED_Q_CAST
        if causal:
            kw["flags"] = kw.get("flags", 0) | binding.MLA_FLAG_CAUSAL
        dec = dec or self.decoder(**kw)
        if out is None:
            out = torch.full((self.total_q, 16, 512), float("nan"), dtype=torch.bfloat16, device=self.dev)
        q = self.q_bf16 if q_cast else self.q
        use_paged = self.page_size > 1 if paged is None else paged
        dec.run(q, self.kv, self.qo_indptr, self.kv_indptr, self.kv_indices, self.q_scale, self.kv_scale,
                sm_scale, out, kv_last_page_len=self.kv_last_page_len if use_paged else None)
        return out


def oracle_ref(case: synth.Case, sequences=None, causal: bool = False, logit_cap: float = 0.0,
               q_fp8=None) -> np.ndarray:
    """float64 oracle on the same host bytes (fp8 Q from the oracle's own encoder with a unit scale,
    or the given (codes, q_scale))."""
    q_bits = case.q_bits().numpy()
    if case.spec.q_dtype == "fp8":
        if q_fp8 is not None:
            q_bits, q_scale = q_fp8
            q_bits = np.asarray(q_bits).reshape(case.q_bf16.shape)
        else:
            q_bits = oracle.bf16_bits_to_fp8_bits(q_bits)
            q_scale = 1.0
    else:
        q_scale = None
    kv_scale = float(case.kv_scale[0]) if case.kv_scale is not None else None
    return oracle.mla_decode(q_bits, case.kv_bits().numpy(), case.qo_indptr.numpy(), case.kv_indptr.numpy(),
                             case.kv_indices.numpy(), q_dtype=case.spec.q_dtype, kv_dtype=case.spec.kv_dtype,
                             q_scale=q_scale, kv_scale=kv_scale, sequences=sequences,
                             page_size=case.spec.page_size, kv_last_page_len=case.kv_last_page_len.numpy(),
                             causal=causal, logit_cap=logit_cap)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def compare(ref: np.ndarray, got: np.ndarray, what: str = "") -> dict:
    err = np.abs(got - ref)
    elem_ok = bool(np.all(err <= ATOL + RTOL * np.abs(ref)))
    nrm = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    finite = bool(np.all(np.isfinite(got)))
    res = dict(max_abs=float(err.max()) if err.size else 0.0, normwise=nrm, elem_ok=elem_ok, finite=finite,
               ok=elem_ok and finite and nrm <= NORM_GATE)
    log(f"  {what}: max_abs={res['max_abs']:.3e} normwise={nrm:.3e} ok={res['ok']}")
    return res


def assert_parity(ref: np.ndarray, got: np.ndarray, what: str = "") -> None:
    r = compare(ref, got, what)
    assert r["finite"], f"{what}: non-finite output"
    assert r["elem_ok"], f"{what}: allclose(rtol={RTOL}, atol={ATOL}) failed, max_abs={r['max_abs']}"
    assert r["normwise"] <= NORM_GATE, f"{what}: normwise error {r['normwise']} > {NORM_GATE}"


class Timer:
    def __init__(self, what):
        self.what = what

    def __enter__(self):
        self.t = time.time()
        return self

    def __exit__(self, *a):
        log(f"  [{self.what}: {time.time() - self.t:.1f}s]")
