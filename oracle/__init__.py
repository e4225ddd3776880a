"""CPU float64 oracle for paged MLA decode -- TEST INFRASTRUCTURE ONLY.

This package states, slowly and plainly, what the MLA-decode path computes,
so the HIP kernels can be checked against it.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it; the product library never calls into it and shares no code with
it (no common kernels, helpers, tables or constants).

Sources (the kernelindex amd-mixed-mla submission pages):

* ``formats``  -- exact bf16 / e4m3fn decoding from the field definitions and
  the round-to-nearest-even cast of bf16 Q to e4m3fn (submission 689529,
  docstring and ``custom_kernel``: Q cast straight to fp8 with unit scale),
  plus the per-tensor amax-scaled cast that docstring names as skipped.
* ``mla``      -- the decode itself (submission 689529 constants block and
  ``custom_kernel``; submission 690201 stage-1 and reduce calls), split
  partials and their log-sum-exp merge; pages of several rows, several
  causal query tokens per sequence and the logit soft-cap.

Pins (tests marked "not gpu" in ``tests/test_oracle.py``): exhaustive format
checks against torch's CPU casts, float64 scaled-dot-product attention as the
multi-query special case, a pure-Python brute force, closed forms (one row,
q = 0, constant V, two rows, dominant row, duplicated row), split/merge
invariance, and deliberately wrong variants that must fail.  The widened
forms: the soft-cap against its limits (cap -> 0 gives the mean of V, a huge
cap the plain result) and a 3:1 closed form through atanh(1/2); pages
against a hand-worked row expansion and against the same rows laid out one
per page; several query tokens against torch's scaled-dot-product attention
(no mask, and the square causal mask when every row is a query); the
amax-scaled cast against torch's float32 division and e4m3fn cast.  The
final log-sum-exp: q = 0 gives log n, one row gives its own score, a
duplicated row adds log 2, scipy's logsumexp over the brute-force scores,
and the whole equals the merge of its parts' log-sum-exps.  No function here
is "parity unpinned".
"""

from .formats import (  # noqa: F401
    BF16_TABLE,
    FP8_TABLE,
    bf16_bits_to_fp8_bits,
    decode_bf16,
    decode_fp8_e4m3fn,
    encode_bf16_rne,
    encode_fp8_e4m3fn,
    quantize_q_dynamic,
)
from .mla import (  # noqa: F401
    NUM_HEADS,
    QK_DIM,
    SM_SCALE,
    V_DIM,
    attention_partial,
    decode_operand,
    merge_lse,
    merge_partials,
    mla_decode,
    mla_decode_bruteforce,
    mla_decode_lse,
    mla_decode_sequence,
    mla_decode_sequence_lse,
    paged_rows,
    soft_cap,
    visible_rows,
)
