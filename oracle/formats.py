"""Exact number-format conversions for the oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the product path never does.

The MLA-decode pages feed the kernels two storage formats (kernelindex
amd-mixed-mla submission 689529, module constants and ``custom_kernel``;
submission 598454, ``custom_kernel``):

* bfloat16 -- 1 sign bit, 8 exponent bits (bias 127), 7 mantissa bits;
* float8 e4m3 "fn" (OCP) -- 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
  bits, no infinities, the two codes S.1111.111 are NaN, largest finite 448
  (the submission 689529 docstring gives the +-448 range, which singles out
  this variant and not the bias-8 "fnuz" one whose maximum is 240).

Decoding is written out from those field definitions and is exact in float64
(every bf16 and every e4m3 value is a float64).  Encoding to e4m3 follows the
same definition with round-to-nearest-even; a magnitude above 464 (half-way
between 448 and the first unrepresentable step 480), an infinity or a NaN
becomes the NaN code with the input's sign.  That is the convention of a
plain non-saturating cast, which is what the pages apply to Q
(``q.to(fp8)``, submission 689529 ``custom_kernel``).
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "decode_bf16",
    "decode_fp8_e4m3fn",
    "encode_fp8_e4m3fn",
    "encode_bf16_rne",
    "quantize_q_dynamic",
    "BF16_TABLE",
    "FP8_TABLE",
]


def _decode_bf16_code(code: int) -> float:
    sign = -1.0 if (code >> 15) & 1 else 1.0
    exp = (code >> 7) & 0xFF
    man = code & 0x7F
    if exp == 0xFF:
        return sign * math.inf if man == 0 else math.copysign(math.nan, sign)
    if exp == 0:
        # subnormal: 0.mmmmmmm * 2^(1-127)
        return sign * man * 2.0 ** (-126 - 7)
    return sign * (1.0 + man / 128.0) * 2.0 ** (exp - 127)


def _decode_fp8_code(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.copysign(math.nan, sign)
    if exp == 0:
        # subnormal: 0.mmm * 2^(1-7)
        return sign * man * 2.0 ** (-6 - 3)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


# Lookup tables built once from the field definitions above.
BF16_TABLE = np.array([_decode_bf16_code(c) for c in range(1 << 16)], dtype=np.float64)
FP8_TABLE = np.array([_decode_fp8_code(c) for c in range(1 << 8)], dtype=np.float64)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16 / int16 array) -> exact float64 values."""
    bits = np.asarray(bits)
    return BF16_TABLE[bits.astype(np.uint16, copy=False)]


def decode_fp8_e4m3fn(bits: np.ndarray) -> np.ndarray:
    """e4m3fn bit patterns (uint8 array) -> exact float64 values."""
    bits = np.asarray(bits)
    return FP8_TABLE[bits.astype(np.uint8, copy=False)]


def _encode_fp8_scalar(x: float) -> int:
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    if math.isnan(x) or math.isinf(x):
        return sign | 0x7F
    a = abs(x)
    if a > 464.0:
        return sign | 0x7F
    if a == 0.0:
        return sign
    # Candidate grid spacing: normal binade [2^e, 2^(e+1)) with e >= -6 has
    # spacing 2^(e-3); below 2^-6 the subnormal spacing is 2^-9.
    e = math.floor(math.log2(a))
    # guard against log2 rounding at exact powers of two
    if 2.0 ** e > a:
        e -= 1
    elif 2.0 ** (e + 1) <= a:
        e += 1
    e = max(e, -6)
    step = 2.0 ** (e - 3)
    q = a / step  # exact in float64: a has <= 53 significant bits, step a power of 2
    n = math.floor(q)
    frac = q - n
    if frac > 0.5 or (frac == 0.5 and (n & 1)):
        n += 1
    v = n * step
    if v == 0.0:
        return sign
    # re-derive the fields of v (v may have carried into the next binade)
    if v < 2.0 ** -6:
        return sign | int(round(v / 2.0 ** -9))
    ev = math.floor(math.log2(v))
    man = int(round((v / 2.0 ** ev - 1.0) * 8.0))
    code = ((ev + 7) << 3) | man
    if code >= 0x7F:  # only 464 -> 448 reaches here with code 0x7E; anything larger is NaN
        return sign | 0x7F
    return sign | code


def encode_fp8_e4m3fn(x: np.ndarray) -> np.ndarray:
    """float64 values -> e4m3fn codes, round-to-nearest-even, non-saturating.

    Element by element in plain Python: meant for small arrays and for the
    65,536 bf16 codes of the exhaustive cast check.
    """
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.fromiter((_encode_fp8_scalar(float(v)) for v in flat), dtype=np.uint8, count=flat.size)
    return out.reshape(x.shape)


# All 65,536 bf16 codes -> their e4m3fn codes.  Every bf16 value is exact in
# float64, so encoding the decoded value is the cast of the bf16 input itself.
_BF16_TO_FP8 = None


def bf16_bits_to_fp8_bits(bits: np.ndarray) -> np.ndarray:
    """Cast bf16 bit patterns to e4m3fn codes (round-to-nearest-even)."""
    global _BF16_TO_FP8
    if _BF16_TO_FP8 is None:
        _BF16_TO_FP8 = encode_fp8_e4m3fn(BF16_TABLE)
    return _BF16_TO_FP8[np.asarray(bits).astype(np.uint16, copy=False)]


def quantize_q_dynamic(bits: np.ndarray) -> tuple[np.ndarray, float]:
    """bf16 Q -> (e4m3fn codes, float32 per-tensor scale), the amax variant of the Q cast.

    The pages cast Q with a unit scale and name the per-tensor amax pass as
    the step they skipped (submission 689529 docstring).  Reading of that
    step, in the same form as the KV scale the pages pair with fp8 KV:

    * amax = the largest |q| over the finite values (bf16 is exact in float32);
    * q_scale = amax / 448 in float32 (1 when amax is 0: nothing to scale);
    * each finite q is divided by q_scale in float32 and cast to e4m3fn with
      round-to-nearest-even; +-inf and NaN inputs give the NaN code with the
      input's sign.

    The dequantised value is code * q_scale.  The float32 division is the
    precision the device kernel uses; it decides the codes, so both sides
    take it in float32.
    """
    bits = np.asarray(bits).astype(np.uint16, copy=False)
    x = decode_bf16(bits)
    finite = np.isfinite(x)
    amax = np.float32(np.max(np.abs(x[finite]))) if finite.any() else np.float32(0.0)
    scale = np.float32(amax) / np.float32(448.0) if amax > 0 else np.float32(1.0)
    y = np.where(finite, x, 0.0).astype(np.float32) / scale  # float32 division, correctly rounded
    codes = encode_fp8_e4m3fn(y.astype(np.float64))
    sign = ((bits >> 8) & 0x80).astype(np.uint8)
    codes = np.where(finite, codes, sign | np.uint8(0x7F)).astype(np.uint8)
    return codes, float(scale)


def encode_bf16_rne(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 codes with round-to-nearest-even (via exact float32 step).

    Used only to state what a correctly rounded bf16 result is (the GPU output
    is bf16).  float64 -> float32 is itself round-to-nearest-even; rounding the
    float32 to bf16 afterwards could double-round, so the float64 value is
    rounded directly on its bits instead.
    """
    x = np.asarray(x, dtype=np.float64)
    b = x.view(np.uint64)
    sign = (b >> np.uint64(63)).astype(np.uint16) << np.uint16(15)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    flat_s = sign.reshape(-1)
    for i, v in enumerate(flat_x):
        v = float(v)
        s = int(flat_s[i])
        if math.isnan(v):
            flat_o[i] = s | 0x7FC0
            continue
        a = abs(v)
        if a == 0.0:
            flat_o[i] = s
            continue
        e = math.frexp(a)[1] - 1  # a in [2^e, 2^(e+1))
        e = max(e, -126)
        step = 2.0 ** (e - 7)
        q = a / step
        n = math.floor(q)
        frac = q - n
        if frac > 0.5 or (frac == 0.5 and (n & 1)):
            n += 1
        r = n * step
        if r >= 2.0 ** 128:
            flat_o[i] = s | 0x7F80
            continue
        f32 = np.array([r], dtype=np.float32)  # exact: r has <= 8 significant bits
        flat_o[i] = s | int(f32.view(np.uint32)[0] >> 16) & 0x7FFF
    return out
