"""Shared helpers for the GPU parity tests (host-side marshalling only)."""

import sys

import numpy as np
import torch

from synth import inputs


def say(*a):
    """Name the case before each GPU step (flushed), so a failing run shows it."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def host_u8(t):
    return t.detach().cpu().numpy()


def host_f32(t):
    return t.detach().float().cpu().numpy()


def host_bf16_as_f32(t):
    return t.detach().cpu().float().numpy()


def bits(t):
    return inputs.bf16_bits(t)


def bf16_from_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def assert_codes_equal(got, want, what):
    got = np.atleast_1d(np.asarray(got))
    want = np.atleast_1d(np.asarray(want))
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.nonzero(got != want)
    if bad[0].size:
        idx = tuple(b[0] for b in bad)
        raise AssertionError(f"{what}: {bad[0].size} code mismatches; first at {idx}: "
                             f"gpu={got[idx]:#04x} oracle={want[idx]:#04x}")


def assert_f32_equal(got, want, what):
    got = np.atleast_1d(np.asarray(got, dtype=np.float32))
    want = np.atleast_1d(np.asarray(want, dtype=np.float32))
    assert got.shape == want.shape, (what, got.shape, want.shape)
    gb, wb = got.view(np.uint32), want.view(np.uint32)
    bad = np.nonzero(gb != wb)
    if bad[0].size:
        idx = tuple(b[0] for b in bad)
        raise AssertionError(f"{what}: {bad[0].size} scale mismatches; first at {idx}: "
                             f"gpu={got[idx]!r} oracle={want[idx]!r}")


# The gfx950 FP8 matrix-core dot product of one K block is not "exact, then
# rounded once": it drops low-order bits of small products next to large
# ones (on the GPU: 448^2 + 127 * 2^-12 returns 448^2; uniformly random codes
# over the whole E4M3 range give errors up to 9.7e-5 * sum|products|, codes
# with exponents >= 2 up to 3.3e-5).  tests/test_gpu_mfma_numerics.py keeps
# that measurement honest: it asserts the per-block error stays below
# MFMA_BLOCK_REL * sum|products|.  The method's per-128 promotion to fp32
# bounds the damage to one K block's worth.
MFMA_BLOCK_REL = 2.0 ** -12


def gemm_gamma(kblocks):
    """Error factor, relative to S = sum_kb |P|_kb * |ra rb|, for the GPU's
    evaluation of the block-rescaled sum: the matrix-core error per K block
    (MFMA_BLOCK_REL) plus fp32 rounding of the scale product, the rescale
    multiply and the KB additions across blocks (unit roundoff 2^-24 each,
    doubled for second-order terms)."""
    return MFMA_BLOCK_REL + 2.0 * (2 + kblocks) * 2.0 ** -24


# Largest fraction of bf16 output elements allowed to fall outside 2 bf16
# ulp of the oracle and pass only by the cancellation floor.  Measured on
# every GPU parity case: at most 0.33% (random codes over the whole E4M3
# range, tiny outputs), at most 0.13% on the linear shapes with Gaussian
# data, K from 128 to 128256.
MAX_FLOOR_FRAC = 0.01


def check_gemm_output(got, ref64, bound, kblocks, out_dtype, what, rel_fro_max=1e-3,
                      max_floor_frac=MAX_FLOOR_FRAC):
    """Parity bar for GEMM outputs against the oracle's float64 result.

    fp32 out: relative Frobenius error <= 1e-3 against the oracle's fp32
    block-rescaled result, and elementwise |got - ref| <= gamma * S +
    2^-24 |ref|, where S is the oracle's sum of |block partial| * |scale| (a
    rigorous bound for any fp32 summation order).
    bf16 out: compared with the oracle's result rounded to bf16 (RNE): within
    2 bf16 ulp, or, where cancellation makes that unattainable, within
    gamma * S + 1 ulp; the relative Frobenius error against that bf16
    reference must also stay <= 1e-3.  (The bf16 cast alone moves the
    output ~1.6e-3 in relative Frobenius norm, so the 1e-3 bar is only
    meaningful before the cast.)  The number of bf16 elements that needed
    the floor is printed and must stay within max_floor_frac of the output.
    Returns (#elements that needed the floor, relative Frobenius error)."""
    from oracle import e4m3, metrics
    got = np.asarray(got, dtype=np.float64)
    ref64 = np.asarray(ref64, dtype=np.float64)
    gam = gemm_gamma(kblocks)
    err = np.abs(got - ref64)
    if out_dtype == "f32":
        rf = metrics.rel_frobenius(ref64, got)
        lim = gam * bound + 2.0 ** -24 * np.abs(ref64)
        bad = err > lim
        floor_used = 0
    else:
        ref_bf16 = e4m3.rne_bf16(ref64.astype(np.float32)).astype(np.float64)
        rf = metrics.rel_frobenius(ref_bf16, got)
        ulp = metrics.bf16_ulp(ref_bf16)
        within2 = np.abs(got - ref_bf16) <= 2 * ulp
        floor = err <= gam * bound + metrics.bf16_ulp(got)
        bad = ~(within2 | floor)
        floor_used = int(np.count_nonzero(~within2 & floor))
    n = int(got.size)
    print(f"[floor] {what}: {floor_used} of {n} elements outside 2 bf16 ulp, within the floor "
          f"({floor_used / max(n, 1):.3%}); rel. Frobenius {rf:.3e}", flush=True)
    assert rf <= rel_fro_max, f"{what}: relative Frobenius error {rf:.3e} > {rel_fro_max}"
    assert floor_used <= max_floor_frac * n, (
        f"{what}: {floor_used} of {n} elements needed the floor (> {max_floor_frac:.2%})")
    if bad.any():
        idx = tuple(b[0] for b in np.nonzero(bad))
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; first {idx}: "
                             f"gpu={got[idx]!r} oracle={ref64[idx]!r} S={bound[idx]!r}")
    return floor_used, rf
