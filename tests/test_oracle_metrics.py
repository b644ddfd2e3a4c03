"""Pins for the oracle's tolerance helpers (CPU only): the bf16 spacing used by
the "within 2 bf16 ulp" clause, the relative Frobenius error, and the error
scale S of the block-rescaled and per-tensor GEMMs.  Every expected value is
derived here independently of the oracle: bf16 spacing from neighbouring bit
patterns, S as an exact rational sum, the Frobenius ratio from closed-form
cases."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import gemm, metrics
from tests import exact


def _bf16_value(bits):
    """bf16 bit patterns (int array) -> float64 values, by placing the 16
    bits in the top half of an fp32 word."""
    w = (np.asarray(bits, dtype=np.uint32) << 16).astype(np.uint32)
    return w.view(np.float32).astype(np.float64)


def test_bf16_ulp_equals_next_pattern_spacing_for_every_bf16_value():
    """For every finite bf16 pattern but the largest, bf16_ulp(v) is the gap
    from |v| to the next larger bf16 value (next bit pattern minus this
    one), both signs, zeros and subnormals included."""
    mag = np.arange(0x7F7F, dtype=np.uint32)            # |v| below the largest finite
    spacing = _bf16_value(mag + 1) - _bf16_value(mag)
    for sign in (0, 0x8000):
        v = _bf16_value(mag | sign)
        got = metrics.bf16_ulp(v)
        bad = np.nonzero(got != spacing)[0]
        assert bad.size == 0, (hex(int(mag[bad[0]] | sign)), got[bad[0]], spacing[bad[0]])


def test_bf16_ulp_special_values():
    assert metrics.bf16_ulp(0.0) == 2.0 ** -133
    assert metrics.bf16_ulp(-0.0) == 2.0 ** -133
    assert metrics.bf16_ulp(2.0 ** -133) == 2.0 ** -133        # smallest subnormal
    assert metrics.bf16_ulp(2.0 ** -126) == 2.0 ** -133        # smallest normal
    assert metrics.bf16_ulp(1.0) == 2.0 ** -7
    assert metrics.bf16_ulp(1.9921875) == 2.0 ** -7            # largest below 2
    assert metrics.bf16_ulp(-2.0) == 2.0 ** -6
    assert metrics.bf16_ulp(448.0) == 2.0
    # vectorised and shape-preserving
    assert metrics.bf16_ulp(np.array([[1.0, 0.0]])).shape == (1, 2)


def test_rel_frobenius_closed_forms():
    # |(0, 1)| / |(3, 4)| = 1 / 5
    assert metrics.rel_frobenius([[3.0, 4.0]], [[3.0, 5.0]]) == pytest.approx(0.2, rel=1e-15)
    # the denominator is the reference's norm, not the output's
    assert metrics.rel_frobenius([3.0, 4.0], [6.0, 8.0]) == pytest.approx(1.0, rel=1e-15)
    assert metrics.rel_frobenius([6.0, 8.0], [3.0, 4.0]) == pytest.approx(0.5, rel=1e-15)
    # a whole-matrix (Frobenius) norm, not a per-row or max norm
    ref = np.ones((3, 4))
    out = ref.copy()
    out[1, 2] += 0.5
    out[2, 0] -= 1.0
    assert metrics.rel_frobenius(ref, out) == pytest.approx(np.sqrt(1.25 / 12), rel=1e-15)
    assert metrics.rel_frobenius(ref, ref) == 0.0
    # zero reference: the absolute norm of the output
    assert metrics.rel_frobenius(np.zeros(2), [3.0, 4.0]) == pytest.approx(5.0, rel=1e-15)


def _codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


def _exact_S(a, b, sa, sb, m, n, kblocks, sb_row):
    table = exact.e4m3_table()
    tot = Fraction(0)
    for kb in range(kblocks):
        p = sum(abs(table[int(a[m, k])]) * abs(table[int(b[n, k])])
                for k in range(kb * 128, (kb + 1) * 128))
        tot += p * abs(exact.f32_frac(sa[m, kb]) * exact.f32_frac(sb[sb_row(n), kb]))
    return tot


@pytest.mark.parametrize("b_block", ["128x128", "1x128"])
def test_blockwise_bound_is_the_exact_sum_of_abs_products(b_block):
    """S[m, n] = sum_kb sum_k |a[m,k]| |b[n,k]| |ra[m,kb] rb[beta(n),kb]|,
    checked against the exact rational sum with scales of both signs (a
    missing absolute value on a code or a scale, a wrong scale index, or a
    bound taken as |P| instead of the sum of |products| all fail)."""
    rng = np.random.default_rng(12)
    M, N, kb = 3, 260, 3
    a = _codes(rng, (M, 128 * kb))
    b = _codes(rng, (N, 128 * kb))
    sign = lambda shape: np.where(rng.random(shape) < 0.5, -1.0, 1.0)
    ra = (rng.uniform(0.5, 2, (M, kb)) * sign((M, kb))).astype(np.float32)
    nb = N if b_block == "1x128" else 3
    rb = (rng.uniform(0.5, 2, (nb, kb)) * sign((nb, kb))).astype(np.float32)
    ref, S = gemm.blockwise_gemm(a, ra, b, rb, b_block, with_bound=True)
    row = (lambda n: n) if b_block == "1x128" else (lambda n: n // 128)
    for m in range(M):
        for n in (0, 5, 127, 128, 200, 256, 259):
            want = _exact_S(a, b, ra, rb, m, n, kb, row)
            assert abs(Fraction(S[m, n]) - want) <= want * Fraction(2) ** -50, (m, n)
            assert S[m, n] >= abs(ref[m, n])


def test_tensorwise_bound_is_the_exact_sum_of_abs_products():
    rng = np.random.default_rng(13)
    a = _codes(rng, (2, 48))
    b = _codes(rng, (3, 48))
    ra, rb = np.float32(-0.37), np.float32(2.5)
    S = gemm.tensorwise_bound(a, ra, b, rb)
    table = exact.e4m3_table()
    for m in range(2):
        for n in range(3):
            want = sum(abs(table[int(a[m, k])]) * abs(table[int(b[n, k])]) for k in range(48))
            want *= abs(exact.f32_frac(ra) * exact.f32_frac(rb))
            assert abs(Fraction(S[m, n]) - want) <= want * Fraction(2) ** -50
            assert S[m, n] >= abs(gemm.tensorwise_gemm(a[[m]], ra, b[[n]], rb)[0, 0])
