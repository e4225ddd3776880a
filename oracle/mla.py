"""Plain float64 CPU reference for paged MLA decode (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It shares no code with the HIP path and
imports nothing from the product package.

What is computed (kernelindex amd-mixed-mla submission 689529, module
constants and ``custom_kernel``; submission 690201, the direct stage-1 call):

* 16 query heads of width 576 per query token; a single latent KV head of width
  576 stored one row per page (page size 1), rows addressed through
  ``kv_indptr`` / ``kv_indices`` (sequence b owns index positions
  ``kv_indptr[b] .. kv_indptr[b+1]-1``, each naming a row of the pool);
* the query token of sequence b is ``q[qo_indptr[b] .. qo_indptr[b+1]-1]``;
* scores ``s = sm_scale * (q . k)`` over all 576 dims, ``sm_scale = 1/sqrt(576)``;
* output ``O = softmax(s) . V`` where V is the first 512 dims of the same KV row
  (the latent part; dims 512..575 are the rope part and enter the scores only);
* fp8 operands are dequantised by one per-tensor float32 scale each
  (``q_scale``, ``kv_scale``, passed next to the fp8 tensors in the submission
  690201 stage-1 call).  bf16 operands take no scale.

Every value is decoded exactly from its bits (``oracle.formats``), all
arithmetic is float64 numpy, and sequences are processed one at a time.
"""

from __future__ import annotations

import math
from typing import Sequence

import numpy as np

from .formats import decode_bf16, decode_fp8_e4m3fn

__all__ = [
    "NUM_HEADS",
    "QK_DIM",
    "V_DIM",
    "SM_SCALE",
    "decode_operand",
    "mla_decode",
    "mla_decode_sequence",
    "mla_decode_bruteforce",
    "attention_partial",
    "merge_partials",
]

# kernelindex amd-mixed-mla submission 689529, module constants.
NUM_HEADS = 16
QK_DIM = 576
V_DIM = 512
SM_SCALE = 1.0 / math.sqrt(QK_DIM)  # = 1/24 exactly


def decode_operand(bits: np.ndarray, dtype: str, scale: float | None) -> np.ndarray:
    """Raw storage bits -> float64 values, dequantised by the per-tensor scale.

    ``dtype`` is "bf16" (uint16 bits, no scale) or "fp8" (uint8 e4m3fn bits,
    multiplied by ``scale``).
    """
    if dtype == "bf16":
        return decode_bf16(bits)
    if dtype == "fp8":
        s = 1.0 if scale is None else float(scale)
        return decode_fp8_e4m3fn(bits) * s
    raise ValueError(f"unknown dtype {dtype!r}")


def mla_decode_sequence(Q: np.ndarray, K: np.ndarray, sm_scale: float, v_dim: int = V_DIM) -> np.ndarray:
    """One sequence: Q [H, D] and K [n, D] float64 -> O [H, v_dim] float64.

    softmax over the n rows of sm_scale * Q K^T, then times the first v_dim
    columns of the same rows.  n == 0 gives zeros (an empty sequence attends
    to nothing; the pages never form one).
    """
    H = Q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((H, v_dim), dtype=np.float64)
    S = sm_scale * (Q @ K.T)  # [H, n]
    S = S - S.max(axis=1, keepdims=True)
    P = np.exp(S)
    P /= P.sum(axis=1, keepdims=True)
    return P @ K[:, :v_dim]


def mla_decode(
    q_bits: np.ndarray,
    kv_bits: np.ndarray,
    qo_indptr: Sequence[int],
    kv_indptr: Sequence[int],
    kv_indices: Sequence[int],
    *,
    q_dtype: str,
    kv_dtype: str,
    q_scale: float | None = None,
    kv_scale: float | None = None,
    sm_scale: float = SM_SCALE,
    v_dim: int = V_DIM,
    sequences: Sequence[int] | None = None,
) -> np.ndarray:
    """Full paged MLA decode in float64.

    q_bits  [total_q, H, D] (uint16 for bf16, uint8 for fp8)
    kv_bits [rows, D]       (uint16 for bf16, uint8 for fp8); the page-size-1
                            pool with its single KV head squeezed out.
    Returns O [total_q, H, v_dim] float64.  With ``sequences`` given, only the
    query rows of those sequences are computed (the rest stay zero), which lets
    a test sample a large batch.
    """
    q_bits = np.asarray(q_bits)
    kv_bits = np.asarray(kv_bits)
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    kv_indices = np.asarray(kv_indices, dtype=np.int64)
    total_q, H, D = q_bits.shape
    B = len(kv_indptr) - 1
    out = np.zeros((total_q, H, v_dim), dtype=np.float64)
    seqs = range(B) if sequences is None else sequences
    for b in seqs:
        rows = kv_indices[kv_indptr[b] : kv_indptr[b + 1]]
        K = decode_operand(kv_bits[rows], kv_dtype, kv_scale)
        for t in range(qo_indptr[b], qo_indptr[b + 1]):
            Q = decode_operand(q_bits[t], q_dtype, q_scale)
            out[t] = mla_decode_sequence(Q, K, sm_scale, v_dim)
    return out


def mla_decode_bruteforce(Q: list, K: list, sm_scale: float, v_dim: int) -> list:
    """Pure-Python triple loop on tiny inputs: Q [H][D], K [n][D] -> O [H][v_dim].

    Written independently of ``mla_decode_sequence`` (scalar math.exp and
    math.fsum, no numpy) so the two can check each other.
    """
    H = len(Q)
    n = len(K)
    out = []
    for h in range(H):
        if n == 0:
            out.append([0.0] * v_dim)
            continue
        s = [sm_scale * math.fsum(Q[h][d] * K[j][d] for d in range(len(Q[h]))) for j in range(n)]
        mx = max(s)
        e = [math.exp(v - mx) for v in s]
        z = math.fsum(e)
        out.append([math.fsum(e[j] * K[j][c] for j in range(n)) / z for c in range(v_dim)])
    return out


def attention_partial(Q: np.ndarray, K: np.ndarray, sm_scale: float, v_dim: int = V_DIM):
    """Split-KV partial over a subset of rows: (O_part [H, v_dim], lse [H]).

    O_part is the softmax-weighted mean of V over just these rows and
    ``lse = log(sum_j exp(s_j))`` (natural log).  An empty subset gives
    O_part = 0 and lse = -inf.  The split partial / log-sum-exp pair is the
    stage-1 output the pages pass to the reduce step (submission 690201:
    ``logits`` and ``attn_lse`` into ``mla_reduce_v1``).
    """
    H = Q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((H, v_dim)), np.full(H, -np.inf)
    S = sm_scale * (Q @ K.T)
    mx = S.max(axis=1, keepdims=True)
    E = np.exp(S - mx)
    z = E.sum(axis=1, keepdims=True)
    O = (E @ K[:, :v_dim]) / z
    lse = (mx + np.log(z))[:, 0]
    return O, lse


def merge_partials(O_parts: np.ndarray, lse_parts: np.ndarray) -> np.ndarray:
    """Merge split partials: O = sum_i w_i O_i / sum_i w_i, w_i = exp(lse_i - max lse).

    O_parts [S, H, v_dim], lse_parts [S, H] (natural log).  Parts with
    lse = -inf carry no weight; if every part is empty the result is 0.
    Softmax over a union of disjoint row sets is the lse-weighted mean of the
    per-set softmax means, which is why this reproduces the unsplit result.
    """
    O_parts = np.asarray(O_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)  # [H]
    out = np.zeros(O_parts.shape[1:], dtype=np.float64)
    finite = np.isfinite(M)
    if not finite.any():
        return out
    Msafe = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - Msafe[None, :]), 0.0)  # [S, H]
    z = w.sum(axis=0)  # [H]
    num = np.einsum("sh,shc->hc", w, O_parts)
    out[finite] = num[finite] / z[finite, None]
    return out
