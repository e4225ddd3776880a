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

Widened forms (arguments the pages pass to the decode and metadata calls:
pages of 2 and 8 rows with ``kv_last_page_lens`` in submission 598454's
a8w8 path and submission 641982's dispatch; ``q_seq_len``, ``is_causal`` and
``logit_cap`` in submission 689529's cache builder and ``custom_kernel``):

* pages of ``page_size`` rows: the pool is ``[num_pages * page_size, D]``,
  ``kv_indices`` names pages and the last page of sequence b holds
  ``kv_last_page_len[b]`` rows (read as clamped into ``[1, page_size]``:
  submission 689529 passes the sequence length there with page size 1,
  which this reading turns into "every page full");
* several query tokens per sequence (``qo_indptr``); with ``causal`` token i
  of a sequence with q_len tokens and L rows sees its first
  ``L - q_len + 1 + i`` rows (the tokens are the sequence's last rows), else
  all L rows;
* ``logit_cap > 0`` replaces every score s by ``logit_cap * tanh(s / logit_cap)``
  before the softmax (the pages pass 0, i.e. off, and do not print the
  formula; this is the usual soft-cap reading).

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
    "soft_cap",
    "paged_rows",
    "visible_rows",
    "mla_decode",
    "mla_decode_sequence",
    "mla_decode_sequence_lse",
    "mla_decode_lse",
    "mla_decode_bruteforce",
    "attention_partial",
    "merge_partials",
    "merge_lse",
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


def soft_cap(S: np.ndarray, logit_cap: float) -> np.ndarray:
    """Scores through the logit soft-cap: cap * tanh(S / cap) for cap > 0, S unchanged for cap == 0."""
    if logit_cap == 0:
        return S
    if not logit_cap > 0:
        raise ValueError("logit_cap must be >= 0")
    return logit_cap * np.tanh(S / logit_cap)


def paged_rows(kv_indptr, kv_indices, b: int, page_size: int = 1, kv_last_page_len=None) -> np.ndarray:
    """Pool rows of sequence b, in order: every slot of each page, the last page cut to its length.

    Page p holds pool rows ``p * page_size .. p * page_size + page_size - 1``.
    ``kv_last_page_len`` None means every page is full.
    """
    p0, p1 = int(kv_indptr[b]), int(kv_indptr[b + 1])
    if p1 <= p0:
        return np.zeros(0, dtype=np.int64)
    last = page_size if kv_last_page_len is None else min(max(int(kv_last_page_len[b]), 1), page_size)
    rows = []
    for i in range(p0, p1):
        page = int(kv_indices[i])
        n = page_size if i < p1 - 1 else last
        rows.extend(page * page_size + s for s in range(n))
    return np.asarray(rows, dtype=np.int64)


def visible_rows(n_rows: int, q_len: int, i: int, causal: bool) -> int:
    """How many of a sequence's n_rows rows its query token i (of q_len) sees."""
    if not causal:
        return n_rows
    return max(0, min(n_rows, n_rows - q_len + 1 + i))


def mla_decode_sequence(Q: np.ndarray, K: np.ndarray, sm_scale: float, v_dim: int = V_DIM,
                        logit_cap: float = 0.0) -> np.ndarray:
    """One sequence: Q [H, D] and K [n, D] float64 -> O [H, v_dim] float64.

    softmax over the n rows of the (optionally soft-capped) scores
    sm_scale * Q K^T, then times the first v_dim columns of the same rows.
    n == 0 gives zeros (an empty sequence attends to nothing; the pages never
    form one).
    """
    H = Q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((H, v_dim), dtype=np.float64)
    S = soft_cap(sm_scale * (Q @ K.T), logit_cap)  # [H, n]
    S = S - S.max(axis=1, keepdims=True)
    P = np.exp(S)
    P /= P.sum(axis=1, keepdims=True)
    return P @ K[:, :v_dim]


def mla_decode_sequence_lse(Q: np.ndarray, K: np.ndarray, sm_scale: float, logit_cap: float = 0.0) -> np.ndarray:
    """Log-sum-exp (natural log) of one sequence's scores: Q [H, D], K [n, D] -> [H].

    ``log sum_j exp(s_j)`` over the n rows, with s the (optionally
    soft-capped) scores ``sm_scale * Q K^T``: the normaliser of the softmax
    in ``mla_decode_sequence``.  It is the final-LSE output of the pages'
    reduce step (submission 690201, ``custom_kernel``: the last argument of
    ``mla_reduce_v1``, left as None there).  n == 0 gives -inf.
    """
    H = Q.shape[0]
    if K.shape[0] == 0:
        return np.full(H, -np.inf)
    S = soft_cap(sm_scale * (Q @ K.T), logit_cap)  # [H, n]
    mx = S.max(axis=1)
    return mx + np.log(np.exp(S - mx[:, None]).sum(axis=1))


def mla_decode_lse(
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
    sequences: Sequence[int] | None = None,
    page_size: int = 1,
    kv_last_page_len: Sequence[int] | None = None,
    causal: bool = False,
    logit_cap: float = 0.0,
) -> np.ndarray:
    """Log-sum-exp of every query token's scores over the rows it sees: [total_q, H] float64.

    Same inputs and row / token rules as ``mla_decode``; tokens that see no
    row (and the rows of sequences not in ``sequences``) get -inf.
    """
    q_bits = np.asarray(q_bits)
    kv_bits = np.asarray(kv_bits)
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    kv_indices = np.asarray(kv_indices, dtype=np.int64)
    total_q, H, _ = q_bits.shape
    out = np.full((total_q, H), -np.inf)
    seqs = range(len(kv_indptr) - 1) if sequences is None else sequences
    for b in seqs:
        rows = paged_rows(kv_indptr, kv_indices, b, page_size, kv_last_page_len)
        K = decode_operand(kv_bits[rows], kv_dtype, kv_scale)
        q_len = int(qo_indptr[b + 1] - qo_indptr[b])
        for i in range(q_len):
            t = int(qo_indptr[b]) + i
            n = visible_rows(len(rows), q_len, i, causal)
            out[t] = mla_decode_sequence_lse(decode_operand(q_bits[t], q_dtype, q_scale), K[:n], sm_scale, logit_cap)
    return out


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
    page_size: int = 1,
    kv_last_page_len: Sequence[int] | None = None,
    causal: bool = False,
    logit_cap: float = 0.0,
) -> np.ndarray:
    """Full paged MLA decode in float64.

    q_bits  [total_q, H, D] (uint16 for bf16, uint8 for fp8)
    kv_bits [pool_rows, D]  (uint16 for bf16, uint8 for fp8); the pool of
                            ``pool_rows / page_size`` pages with its single KV
                            head squeezed out.
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
        rows = paged_rows(kv_indptr, kv_indices, b, page_size, kv_last_page_len)
        K = decode_operand(kv_bits[rows], kv_dtype, kv_scale)
        q_len = int(qo_indptr[b + 1] - qo_indptr[b])
        for i in range(q_len):
            t = int(qo_indptr[b]) + i
            n = visible_rows(len(rows), q_len, i, causal)
            Q = decode_operand(q_bits[t], q_dtype, q_scale)
            out[t] = mla_decode_sequence(Q, K[:n], sm_scale, v_dim, logit_cap)
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


def merge_lse(lse_parts: np.ndarray) -> np.ndarray:
    """Log-sum-exp of the whole from the parts' log-sum-exps: [S, H] -> [H].

    ``log sum_i exp(lse_i)``: the rows of all parts together have
    ``sum_i exp(lse_i)`` as their softmax normaliser.  Parts with lse = -inf
    add nothing; no parts, or only empty ones, give -inf.
    """
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    if lse_parts.shape[0] == 0:
        return np.full(lse_parts.shape[1:], -np.inf)
    M = lse_parts.max(axis=0)
    finite = np.isfinite(M)
    Msafe = np.where(finite, M, 0.0)
    z = np.where(np.isfinite(lse_parts), np.exp(lse_parts - Msafe[None, :]), 0.0).sum(axis=0)
    return np.where(finite, Msafe + np.log(np.where(finite, z, 1.0)), -np.inf)
