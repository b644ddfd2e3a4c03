"""Measured accuracy of the gfx950 FP8 matrix-core dot product, through the
blockwise GEMM with one K block and unit scales (so the output is exactly
one MFMA partial).  These tests pin the error model the parity bar uses."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_amd as fp8
from oracle import gemm
from tests.gpu_util import MFMA_BLOCK_REL, host_f32, say

pytestmark = pytest.mark.gpu


def _one_block(dev, aq, bq):
    M, N = aq.shape[0], bq.shape[0]
    nb = -(-N // 128)
    ones_a = torch.ones((1, M), dtype=torch.float32, device=dev).t()
    ones_b = torch.ones((1, nb), dtype=torch.float32, device=dev).t()
    out = fp8.fp8_scaled_gemm_blockwise(torch.from_numpy(aq).to(dev), ones_a,
                                        torch.from_numpy(bq).to(dev), ones_b,
                                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, S = gemm.blockwise_gemm(aq, np.ones((M, 1), np.float32), bq,
                                 np.ones((nb, 1), np.float32), "128x128", with_bound=True)
    return host_f32(out).astype(np.float64), ref, S


def _codes(rng, shape, min_exp=0):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    bad = ((c & 0x7F) == 0x7F) | (((c >> 3) & 0xF) < min_exp)
    while bad.any():
        c[bad] = rng.integers(0, 256, size=int(bad.sum())).astype(np.uint8)
        bad = ((c & 0x7F) == 0x7F) | (((c >> 3) & 0xF) < min_exp)
    return c


def test_subnormal_codes_are_exact(gpu):
    """E4M3 subnormals are not flushed: 128 x (2^-9 * 1.0) = 0.25 exactly,
    and one 7*2^-9 times 448 = 6.125 exactly."""
    a = np.full((16, 128), 0x01, np.uint8)
    b = np.full((16, 128), 0x38, np.uint8)
    say("mfma subnormal")
    got, ref, _ = _one_block(gpu, a, b)
    assert np.all(got == 0.25) and np.all(ref == 0.25)
    a = np.zeros((16, 128), np.uint8)
    a[:, 5] = 0x07
    b = np.full((16, 128), 0x7E, np.uint8)
    got, ref, _ = _one_block(gpu, a, b)
    assert np.all(got == 6.125)


@pytest.mark.parametrize("min_exp", [0, 9])
def test_block_dot_error_within_model(gpu, min_exp):
    """Per-K-block error relative to sum|products| stays below the bound
    the parity tests assume; report the measured maximum."""
    rng = np.random.default_rng(100 + min_exp)
    a = _codes(rng, (256, 128), min_exp)
    b = _codes(rng, (256, 128), min_exp)
    say("mfma error model", min_exp)
    got, ref, S = _one_block(gpu, a, b)
    rel = np.max(np.abs(got - ref) / S)
    say("max |gpu - exact| / sum|p| =", rel)
    assert rel <= MFMA_BLOCK_REL


def test_small_terms_next_to_a_large_product(gpu):
    """Documents the truncation: 448^2 + 127 * (2^-6)^2 comes back as 448^2."""
    a = np.full((16, 128), 0x08, np.uint8)
    b = np.full((16, 128), 0x08, np.uint8)
    a[:, 0] = 0x7E
    b[:, 0] = 0x7E
    say("mfma large + small")
    got, ref, S = _one_block(gpu, a, b)
    assert np.all(np.abs(got - ref) <= MFMA_BLOCK_REL * S)
    assert np.all(got == 200704.0)
