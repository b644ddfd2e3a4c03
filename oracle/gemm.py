"""Blockwise- and tensorwise-scaled FP8 GEMM (oracle; test infrastructure only).

Operand convention: out = A . B^T with A[M, K] and B[N, K] both K-contiguous,
"x @ weight.T, like F.linear" ([AITER] Steps to Reproduce).

Blockwise ([REPRO] What Changed / Findings So Far; [INTEG] Summary):

    out[m, n] = sum_kb  ra[m, kb] * rb[beta(n), kb] * P_kb[m, n],
    P_kb[m, n] = sum_{k in block kb} a[m, k] * b[n, k]

where a, b are the decoded E4M3 values, ra, rb the reciprocal scales, and
beta(n) = n // 128 for 128x128 B scales (fwd, dgrad) or beta(n) = n for 1x128
B scales (wgrad).  K must be a multiple of 128.

Exactness: E4M3 values are multiples of 2^-9 below 2^9 in magnitude, so each
product is a multiple of 2^-18 below 2^18 and any partial sum of 128 of them
is below 2^25: 43 significant bits, exact in float64 in any order.  P_kb is
therefore exact whatever order the BLAS call uses.  The scale product
ra * rb (two 24-bit significands) is exact in float64.  Only the final
sum over kb rounds, at float64 precision.
"""

import numpy as np

from . import e4m3

BLOCK = 128


def _expand_b_scales(rb, n_rows, b_block):
    rb = np.asarray(rb, dtype=np.float32)
    if b_block == "1x128":
        if rb.shape[0] != n_rows:
            raise ValueError("1x128 B scales need one row per B row")
        return rb.astype(np.float64)
    if b_block == "128x128":
        return np.repeat(rb.astype(np.float64), BLOCK, axis=0)[:n_rows]
    raise ValueError(f"unknown b_block {b_block!r}")


def blockwise_gemm(a_codes, ra, b_codes, rb, b_block="128x128", with_bound=False):
    """Block-rescaled accumulation in float64.  Returns ref64[M, N].

    With ``with_bound`` also returns S[m, n] = sum_kb |P|_kb[m, n] * ra * rb
    where |P|_kb uses |a| and |b|; S bounds the rounding error of any fp32
    evaluation order (used for the tolerance floor in the parity tests).
    """
    A = e4m3.decode(a_codes)
    B = e4m3.decode(b_codes)
    M, K = A.shape
    N, K2 = B.shape
    if K != K2 or K % BLOCK:
        raise ValueError("K mismatch or K not a multiple of 128")
    kbs = K // BLOCK
    ra64 = np.asarray(ra, dtype=np.float32).astype(np.float64)
    rbx = _expand_b_scales(rb, N, b_block)
    out = np.zeros((M, N), dtype=np.float64)
    bound = np.zeros((M, N), dtype=np.float64) if with_bound else None
    for kb in range(kbs):
        sl = slice(kb * BLOCK, (kb + 1) * BLOCK)
        p = A[:, sl] @ B[:, sl].T
        sc = ra64[:, kb][:, None] * rbx[:, kb][None, :]
        out += p * sc
        if with_bound:
            bound += (np.abs(A[:, sl]) @ np.abs(B[:, sl]).T) * np.abs(sc)
    return (out, bound) if with_bound else out


def block_partial(a_codes, b_codes, kb):
    """P_kb = A_kb . B_kb^T, exact in float64 (see module docstring)."""
    sl = slice(kb * BLOCK, (kb + 1) * BLOCK)
    return e4m3.decode(a_codes[:, sl]) @ e4m3.decode(b_codes[:, sl]).T


def dequant_gemm64(a_codes, ra, b_codes, rb, b_block="128x128"):
    """Explicit dequantize-then-matmul in float64 ([REPRO] What Changed:
    the "explicit dequantized matmul" result).  Dequantization is exact."""
    A = e4m3.decode(a_codes)
    B = e4m3.decode(b_codes)
    ra64 = np.asarray(ra, dtype=np.float32).astype(np.float64)
    rbx = _expand_b_scales(rb, B.shape[0], b_block)
    Ad = A * np.repeat(ra64, BLOCK, axis=1)[:, :A.shape[1]]
    Bd = B * np.repeat(rbx, BLOCK, axis=1)[:, :B.shape[1]]
    return Ad @ Bd.T


def dequant_gemm32(a_codes, ra, b_codes, rb, b_block="128x128"):
    """The same dequantized matmul done in float32 on the CPU (torch), as
    the pages' reference does in fp32 ([AITER]: dequantize with float(),
    then F.linear)."""
    import torch
    A = e4m3.decode(a_codes).astype(np.float32)
    B = e4m3.decode(b_codes).astype(np.float32)
    ra32 = np.asarray(ra, dtype=np.float32)
    rbx = _expand_b_scales(rb, B.shape[0], b_block).astype(np.float32)
    Ad = A * np.repeat(ra32, BLOCK, axis=1)[:, :A.shape[1]]
    Bd = B * np.repeat(rbx, BLOCK, axis=1)[:, :B.shape[1]]
    return torch.from_numpy(Ad).matmul(torch.from_numpy(Bd).T).numpy()


def tensorwise_gemm(a_codes, ra, b_codes, rb):
    """Per-tensor scaled GEMM: out = (A_q . B_q^T) * ra * rb ([AITER]).

    The code product is exact in float64 for K below about 171,000
    (|product| <= 448^2, multiples of 2^-18).  Returns float64; the parity
    target is its float32 rounding.  K need not be a multiple of 128.
    """
    A = e4m3.decode(a_codes)
    B = e4m3.decode(b_codes)
    if A.shape[1] >= 171000:
        raise ValueError("tensorwise oracle exact only for K < 171000")
    p = A @ B.T
    return p * (float(np.float32(ra)) * float(np.float32(rb)))


def tensorwise_bound(a_codes, ra, b_codes, rb):
    """|A| . |B|^T * |ra * rb|: scale of the fp32 rounding error of any order."""
    A = np.abs(e4m3.decode(a_codes))
    B = np.abs(e4m3.decode(b_codes))
    return (A @ B.T) * abs(float(np.float32(ra)) * float(np.float32(rb)))


def grouped_blockwise_gemm(a_codes, ra, b_codes, rb, group_end, with_bound=False):
    """Grouped blockwise GEMM (mixture-of-experts layout): rows
    [group_end[g-1], group_end[g]) of A are multiplied by B_g^T with B_g's
    128x128 scales rb[g]; rows past the last end are NaN (not written).
    Each group is exactly blockwise_gemm on its rows.  Returns ref64 [M, N]
    (and S with with_bound)."""
    a_codes = np.asarray(a_codes)
    M, N = a_codes.shape[0], b_codes.shape[1]
    ref = np.full((M, N), np.nan)
    S = np.full((M, N), np.nan)
    start = 0
    for g, end in enumerate(np.asarray(group_end, dtype=np.int64)):
        end = min(max(int(end), start), M)
        if end > start:
            r, s = blockwise_gemm(a_codes[start:end], np.asarray(ra)[start:end], b_codes[g],
                                  rb[g], "128x128", with_bound=True)
            ref[start:end], S[start:end] = r, s
        start = end
    return (ref, S) if with_bound else ref


def add_bias(ref, bias_bits):
    """Bias epilogue: out[m, n] = ref[m, n] + bias[n], the bf16 bias widened
    exactly, in float64.  Both GEMM interfaces on the pages take an optional
    bias ([AITER] Steps to Reproduce: gemm_a8w8 and torch._scaled_mm, passed
    as None; [INDUCT] Describe the bug: has_bias parametrizes the tests) and
    define no arithmetic for it; this is the plain reading: added per output
    column after scaling, before the output cast."""
    b = e4m3.bf16_bits_to_f32(bias_bits).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if b.shape != (ref.shape[1],):
        raise ValueError("bias needs one value per output column")
    return ref + b[None, :]


def fp32_reference(x_bits, w_bits):
    """The unquantized product X . W^T of the bf16 inputs, accumulated in
    float64 ([REPRO] What Changed: the "FP32 reference matmul").  Used as the
    SQNR denominator."""
    x = e4m3.bf16_bits_to_f32(x_bits).astype(np.float64)
    w = e4m3.bf16_bits_to_f32(w_bits).astype(np.float64)
    return x @ w.T
