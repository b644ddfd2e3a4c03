"""Pins for the oracle's quantizers (CPU only).

The quantizer recipe (amax -> s = 448/max(amax, eps) -> saturating RNE codes,
recip = 1/s) is recomputed here in exact rational arithmetic with an
independent float32 rounding, and checked against block invariants that any
correct implementation must satisfy.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, quant
from tests import exact

EPS_F = Fraction(float(np.float32(1e-12)))


def _bf16(x):
    return e4m3.f32_to_bf16_bits(np.asarray(x, np.float32))


def _brute_block(vals_bits, table):
    """Exact-rational quantization of one block of bf16 bit patterns."""
    xs = [Fraction(float(v)) for v in e4m3.bf16_bits_to_f32(vals_bits).ravel()]
    amax = max(abs(x) for x in xs) if xs else Fraction(0)
    a = max(amax, EPS_F)
    s = exact.round_to_f32(Fraction(448) / a)
    recip = exact.round_to_f32(1 / s)
    codes = []
    for x, xf in zip(xs, e4m3.bf16_bits_to_f32(vals_bits).ravel()):
        v = exact.round_to_f32(x * s)
        v = min(max(v, Fraction(-448)), Fraction(448))
        codes.append(exact.nearest_code_signed(v, bool(np.signbit(xf)), table))
    return np.array(codes, np.uint8).reshape(np.shape(vals_bits)), recip


@pytest.fixture(scope="module")
def table():
    return exact.e4m3_table()


def _adversarial_rows(rng, n):
    rows = []
    for i in range(n):
        kind = i % 6
        if kind == 0:
            r = rng.standard_normal(128)
        elif kind == 1:
            r = rng.standard_normal(128) * 1e-30      # tiny amax, subnormal codes
        elif kind == 2:
            r = np.zeros(128)                          # all-zero block
            r[rng.integers(128)] = -0.0
        elif kind == 3:
            r = rng.uniform(-1, 1, 128) * 3.0e38       # near float32 max
        elif kind == 4:
            r = np.full(128, 1.0)
            r[:64] = rng.standard_normal(64) * 1e-3    # one dominant value
        else:
            r = rng.standard_normal(128) * 2.0 ** rng.integers(-40, 40)
        rows.append(r)
    return _bf16(np.array(rows))


def test_quant_1x128_matches_exact_rational(table):
    rng = np.random.default_rng(0)
    x = _adversarial_rows(rng, 12).reshape(3, 512)       # 3 rows x 4 blocks
    codes, recip = quant.quant_1x128(x)
    for r in range(3):
        for kb in range(4):
            blk = x[r, kb * 128:(kb + 1) * 128]
            bc, br = _brute_block(blk, table)
            assert np.array_equal(codes[r, kb * 128:(kb + 1) * 128], bc), (r, kb)
            assert exact.f32_frac(recip[r, kb]) == br, (r, kb)


def test_quant_128x128_ragged_matches_exact_rational(table):
    rng = np.random.default_rng(1)
    x = _bf16(rng.standard_normal((130, 256)) * np.array([1.0, 1e-20])[np.arange(256) // 128])
    codes, recip = quant.quant_128x128(x)
    assert recip.shape == (2, 2)
    for i, (r0, r1) in enumerate([(0, 128), (128, 130)]):
        for j in range(2):
            blk = x[r0:r1, j * 128:(j + 1) * 128]
            bc, br = _brute_block(blk, table)
            assert np.array_equal(codes[r0:r1, j * 128:(j + 1) * 128], bc)
            assert exact.f32_frac(recip[i, j]) == br


def test_tensorwise_matches_exact_rational(table):
    rng = np.random.default_rng(2)
    x = _bf16(rng.standard_normal((16, 32)))
    codes, recip = quant.quant_tensorwise(x)
    bc, br = _brute_block(x, table)
    assert np.array_equal(codes, bc)
    assert exact.f32_frac(recip) == br


def test_every_nonzero_block_hits_448():
    """The block's amax element maps to +-448 (0x7E / 0xFE): s*amax rounds
    to within one float32 ulp of 448, which clamps/rounds to 448."""
    rng = np.random.default_rng(3)
    x = _adversarial_rows(rng, 60).reshape(15, 512)
    codes, _ = quant.quant_1x128(x)
    xf = e4m3.bf16_bits_to_f32(x).reshape(15, 4, 128)
    cb = codes.reshape(15, 4, 128)
    for r in range(15):
        for kb in range(4):
            if np.abs(xf[r, kb]).max() >= 1e-12:
                assert np.any((cb[r, kb] & 0x7F) == 0x7E)


def test_all_bf16_amax_values_hit_448():
    """Exhaustive over every positive finite bf16 value >= 1e-12 used as amax."""
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint16)
    a = e4m3.bf16_bits_to_f32(bits)
    a = a[a >= np.float32(1e-12)]
    s, _ = quant.scale_from_amax(a)
    codes = quant.quantize_with_scale(a, s)
    assert np.all(codes == 0x7E)


def test_power_of_two_rescale_invariance():
    """x -> x * 2^j leaves codes unchanged and multiplies recip by 2^j
    (exact while no value crosses the eps clamp or float32 range)."""
    rng = np.random.default_rng(4)
    x = _bf16(rng.standard_normal((8, 256)))
    c0, r0 = quant.quant_1x128(x)
    for j in (-20, -3, 5, 17):
        xj = _bf16(e4m3.bf16_bits_to_f32(x) * np.float32(2.0 ** j))
        cj, rj = quant.quant_1x128(xj)
        assert np.array_equal(c0, cj)
        assert np.array_equal(r0 * np.float32(2.0 ** j), rj)


def test_negation_flips_only_sign_bits():
    rng = np.random.default_rng(5)
    x = _bf16(rng.standard_normal((4, 384)))
    c0, r0 = quant.quant_1x128(x)
    c1, r1 = quant.quant_1x128(x ^ np.uint16(0x8000))
    assert np.array_equal(c0 ^ np.uint8(0x80), c1)
    assert np.array_equal(r0, r1)


def test_blocks_are_independent():
    rng = np.random.default_rng(6)
    x = _bf16(rng.standard_normal((3, 512)))
    c0, r0 = quant.quant_1x128(x)
    y = x.copy()
    y[1, 128:256] = _bf16(rng.standard_normal(128) * 1e5)
    c1, r1 = quant.quant_1x128(y)
    mask = np.ones_like(c0, bool)
    mask[1, 128:256] = False
    assert np.array_equal(c0[mask], c1[mask])
    rmask = np.ones_like(r0, bool)
    rmask[1, 1] = False
    assert np.array_equal(r0[rmask], r1[rmask])


def test_zero_block():
    x = np.zeros((2, 256), np.uint16)
    x[1, 5] = 0x8000   # -0.0
    codes, recip = quant.quant_1x128(x)
    assert np.all(codes[0] == 0)
    assert codes[1, 5] == 0x80 and np.all(np.delete(codes[1], 5) == 0)
    want = np.float32(1.0) / (np.float32(448.0) / np.float32(1e-12))
    assert np.all(recip == want)


def test_128x128_transposed_equals_transpose_of_codes():
    rng = np.random.default_rng(7)
    x = _bf16(rng.standard_normal((200, 384)))
    c, r = quant.quant_128x128(x)
    ct, rt = quant.quant_128x128_transposed(x)
    assert np.array_equal(ct, c.T)
    assert np.array_equal(rt, r.T)


def test_along_rows_matches_explicit_column_loop():
    """The transposed 1x128 quantizer, checked against an explicit loop over
    columns and 128-row segments."""
    rng = np.random.default_rng(8)
    x = _bf16(rng.standard_normal((256, 5)) * np.array([1, 1e-3, 1e3, 1e-25, 7])[None, :])
    ct, rt = quant.quant_1x128_along_rows(x)
    assert ct.shape == (5, 256) and rt.shape == (5, 2)
    xf = e4m3.bf16_bits_to_f32(x)
    for c in range(5):
        for mb in range(2):
            col = xf[mb * 128:(mb + 1) * 128, c]
            s, rc = quant.scale_from_amax(np.abs(col).max())
            assert rt[c, mb] == rc
            assert np.array_equal(ct[c, mb * 128:(mb + 1) * 128], quant.quantize_with_scale(col, s))


def test_recip_is_reciprocal_of_used_scale_not_amax_over_448():
    """The two fp32 recipes for the dequant multiplier, 1/(448/amax) and
    amax/448, differ in the last bit for some amax; the oracle hands out the
    reciprocal of the scale it quantized with."""
    bits = np.arange(0x3F80, 0x4000, dtype=np.uint16)   # amax in [1, 2)
    a = e4m3.bf16_bits_to_f32(bits)
    s, r = quant.scale_from_amax(a)
    assert np.array_equal(r, (np.float32(1) / s).astype(np.float32))
    differs = r != (a / np.float32(448)).astype(np.float32)
    assert differs.any()
