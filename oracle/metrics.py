"""Error metrics (oracle; test infrastructure only)."""

import numpy as np


def sqnr_db(ref, out):
    """Signal-to-quantization-noise ratio in dB: 20 log10(|ref| / |ref - out|).

    [GENERIC] review thread asks for SQNR in the numerics tests; [REPRO]
    Findings So Far prints SQNR values next to the norms they come from
    (the printed collapse SQNRs follow from the printed norms under this
    formula; tests/golden pins that).  Frobenius norms, float64.
    """
    ref = np.asarray(ref, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    num = np.linalg.norm(ref)
    den = np.linalg.norm(ref - out)
    if den == 0:
        return float("inf")
    return float(20.0 * np.log10(num / den))


def rel_frobenius(ref, out):
    """|ref - out|_F / |ref|_F in float64."""
    ref = np.asarray(ref, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(ref - out) / n) if n else float(np.linalg.norm(out))


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (float64): the gap from |x| to the next
    larger bf16 value, 2^(floor(log2|x|) - 7) for normal |x| >= 2^-126; zero
    and subnormal |x| get the subnormal spacing 2^-133.  (bf16 keeps 8
    significant bits, 7 stored, and the fp32 exponent range.)"""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, ex = np.frexp(a)                      # a = f 2^ex with f in [0.5, 1)
    e = np.where(a >= 2.0 ** -126, ex.astype(np.int64) - 1, -126)
    return np.ldexp(1.0, e - 7)
