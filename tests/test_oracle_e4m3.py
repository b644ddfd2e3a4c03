"""Pins for the oracle's E4M3 codec (CPU only)."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_decode_matches_ocp_special_values():
    with open(os.path.join(GOLDEN, "ocp_e4m3_special.json")) as f:
        g = json.load(f)
    for item in g["values"]:
        code = int(item["code"], 16)
        want = float(eval(item["value"].replace("-0", "-0.0") if item["value"] == "-0"
                          else item["value"]))
        got = e4m3.decode(np.array([code], np.uint8))[0]
        assert got == want, item
        assert np.signbit(got) == np.signbit(want), item
    for c in g["nan_codes"]:
        assert np.isnan(e4m3.decode(np.array([int(c, 16)], np.uint8))[0])
    finite = np.isfinite(e4m3.decode(np.arange(256, dtype=np.uint8))).sum()
    assert finite == g["finite_codes"]


def test_decode_matches_torch_float8_e4m3fn_for_all_codes():
    table = exact.e4m3_table()
    ours = e4m3.decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        if table[c] is None:
            assert np.isnan(ours[c])
        else:
            assert Fraction(float(ours[c])) == table[c], hex(c)


def test_encode_decode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = e4m3.decode(codes)
    assert np.array_equal(e4m3.encode_rne(vals), codes)


def _probe_values():
    """All finite bf16 values with |x| <= 448, every midpoint between
    adjacent E4M3 values, and each midpoint +- 1 float32 ulp."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = e4m3.bf16_bits_to_f32(bits)
    f = f[np.isfinite(f) & (np.abs(f) <= 448)]
    pos = np.sort(np.unique(np.abs(e4m3.decode(np.arange(0x7F, dtype=np.uint8)))))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    extra = np.concatenate([mids, up, dn])
    extra = extra[np.abs(extra) <= 448]
    return np.concatenate([f, extra, -extra]).astype(np.float32)


def test_encode_matches_brute_force_nearest_code():
    table = exact.e4m3_table()
    v = _probe_values()
    rng = np.random.default_rng(0)
    # every midpoint case plus a random slice of the bf16 grid
    pick = np.concatenate([np.arange(v.size - 6 * 126, v.size),
                           rng.choice(v.size, 4000, replace=False)])
    ours = e4m3.encode_rne(v[pick].astype(np.float64))
    for i, x in zip(pick, ours):
        val = v[i]
        want = exact.nearest_code_signed(Fraction(float(val)), bool(np.signbit(val)), table)
        assert int(x) == want, (float(val), hex(int(x)), hex(want))


def test_encode_matches_torch_cast_on_clamped_range():
    """torch's CPU float32 -> float8_e4m3fn cast is RNE (not saturating);
    inside [-448, 448] it must agree with the oracle everywhere."""
    v = _probe_values()
    ours = e4m3.encode_rne(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("scale", [1.0, 0.37, 3.1e-3, 17.125, 2.0 ** -20, 6.02e4])
def test_encode_matches_torch_cast_on_scaled_bf16_grid(scale):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = e4m3.bf16_bits_to_f32(bits)
    f = f[np.isfinite(f)]
    with np.errstate(over="ignore"):
        v = np.clip((f * np.float32(scale)).astype(np.float32), -448, 448).astype(np.float32)
    v = v[np.isfinite(v)]
    ours = e4m3.encode_rne(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_specific_cases():
    cases = {
        1.0625: 0x38,        # tie between 1.0 and 1.125 -> even (1.0)
        1.1875: 0x3A,        # tie between 1.125 and 1.25 -> even (1.25)
        1.5 * 2.0 ** -9: 0x02,
        2.0 ** -10: 0x00,    # tie between 0 and min subnormal -> 0
        -1e-6: 0x80,         # negative underflow keeps the sign
        448.0: 0x7E,
        -448.0: 0xFE,
        15.0 * 2.0 ** -10: 0x08,  # rounds up into the min normal
    }
    for v, c in cases.items():
        assert int(e4m3.encode_rne(np.array([v]))[0]) == c, v


def test_encode_rejects_unclamped():
    with pytest.raises(ValueError):
        e4m3.encode_rne(np.array([449.0]))


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    ours = e4m3.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
