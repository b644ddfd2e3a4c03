"""OCP FP8 E4M3 codec and bf16 helpers (oracle; test infrastructure only).

The E4M3 format is the one the pages call e4m3 / float8_e4m3fn ([INTEG]
Summary; [AITER] Steps to Reproduce use ``dtypes.fp8`` on a ROCm part).  The
pages do not restate the format, so this follows the OCP OFP8 definition:
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
subnormal (value = m/8 * 2^-6); S.1111.111 is NaN; there is no infinity; the
largest finite magnitude is S.1111.110 = 448.

Everything here is exact in float64: E4M3 values have at most 4 significant
bits and exponents in [-9, 8].
"""

import numpy as np

E4M3_MAX = 448.0
EXP_BIAS = 7
MIN_NORMAL = 2.0 ** -6
MIN_SUBNORMAL = 2.0 ** -9


def _decode_formula(codes):
    """E4M3 codes -> exact float64 values by the OCP definition; NaN codes -> nan."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    neg = (c & 0x80) != 0
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0,
                   np.ldexp(m / 8.0, 1 - EXP_BIAS),
                   np.ldexp(1.0 + m / 8.0, (e - EXP_BIAS).astype(np.int64)))
    val = np.where(neg, -mag, mag)
    return np.where((e == 15) & ((c & 0x7) == 7), np.nan, val)


# All 256 code values, from the definition above.
DECODE_TABLE = _decode_formula(np.arange(256))


def decode(codes):
    """E4M3 codes (uint8) -> exact float64 values; NaN codes -> nan.  [OCP]
    (A lookup into DECODE_TABLE, the definition evaluated for every code.)"""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_rne(v):
    """Round float64 values to the nearest E4M3 code, ties to even.  [OCP]

    ``v`` must be finite with |v| <= 448 (the quantizer clamps first, so the
    saturating behaviour lives in ``quant.quantize_with_scale``).  The sign
    bit is kept for every input, so -0.0 and negative values that round to
    zero give 0x80.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("encode_rne: non-finite input")
    if np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("encode_rne: |v| > 448; clamp before encoding")
    sign = np.signbit(v).astype(np.int64) << 7
    a = np.abs(v)
    # Subnormal range (a < 2^-6): the quantum is 2^-9, so the code is the
    # integer round(a * 2^9); a result of 8 is exactly the min-normal code.
    q_sub = np.rint(np.ldexp(a, 9)).astype(np.int64)
    # Normal range: a = f * 2^E with f in [1, 2); keep 3 fraction bits.
    _, ex = np.frexp(a)             # a = mant * 2^ex, mant in [0.5, 1)
    big_e = ex.astype(np.int64) - 1
    frac = np.ldexp(a, -big_e)      # exact power-of-two rescale
    mq = np.rint((frac - 1.0) * 8.0).astype(np.int64)
    carry = mq == 8
    big_e = np.where(carry, big_e + 1, big_e)
    mq = np.where(carry, 0, mq)
    q_norm = ((big_e + EXP_BIAS) << 3) | mq
    code = np.where(a < MIN_NORMAL, q_sub, q_norm) | sign
    return code.astype(np.uint8)


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32 values (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns, IEEE round-to-nearest-even (finite x)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def rne_bf16(x):
    """float32 -> float32 holding the bf16-rounded value (RNE)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))
