"""Dynamic E4M3 quantization with amax scales (oracle; test infrastructure only).

What is computed, per block (a 1x128 row segment, a 128x128 tile, a
128-long column segment, or the whole tensor):

  1. amax = max |x| over the block's bf16 values (exact in float32).
  2. a = max(amax, EPS) with EPS = float32(1e-12).  The pages never say what
     happens for an all-zero block; this guard keeps one formula (reading
     recorded in the design notes).
  3. s = float32(448) / a, IEEE float32 division.
  4. codes = RNE_e4m3(clamp(float32(x) * s, -448, 448)), float32 multiply:
     saturating round-to-nearest-even.
  5. recip = float32(1) / s, IEEE float32 division.  The quantizer hands out
     the reciprocal of the scale it used rather than the scale itself
     ([INTEG] Summary: the kernels write reciprocal scales directly instead of
     a later ``1.0/scales``), which is also the dequantization multiplier:
     x ~= decode(code) * recip ([AITER] Steps to Reproduce dequantizes with
     ``x_q.float() * x_scale``).

Block shapes: 1x128 for activations and gradients, 128x128 for weights
([REPRO] Findings So Far names the (BlockWise1x128, BlockWise128x128) regime;
[GENERIC] Performance table quantizes with block_shape (1,128) and (128,128));
one scale for the whole tensor in the per-tensor case ([AITER]
``per_tensor_quant``).

Scales are returned in their *logical* layout (block row index first, block
column index second).  The column-major storage the GEMM consumes ([INTEG]
Summary) is a storage detail the tests apply when reading device buffers.
"""

import numpy as np

from . import e4m3

EPS = np.float32(1e-12)
FP8_MAX = np.float32(448.0)


def scale_from_amax(amax):
    """amax (float32 array) -> (s, recip), both float32, per steps 2, 3, 5."""
    amax = np.asarray(amax, dtype=np.float32)
    a = np.maximum(amax, EPS)
    s = (FP8_MAX / a).astype(np.float32)
    recip = (np.float32(1.0) / s).astype(np.float32)
    return s, recip


def quantize_with_scale(x_f32, s_f32):
    """Step 4: float32 multiply, clamp to +-448, round to nearest E4M3 (even)."""
    v = (np.asarray(x_f32, dtype=np.float32) * np.asarray(s_f32, dtype=np.float32))
    v = v.astype(np.float32)
    v = np.clip(v, np.float32(-448.0), np.float32(448.0))
    return e4m3.encode_rne(v.astype(np.float64))


def _blocks_2d(x_bits, br, bc):
    """Quantize with br x bc blocks; ragged last blocks use only valid elements."""
    x = e4m3.bf16_bits_to_f32(x_bits)
    rows, cols = x.shape
    nrb = -(-rows // br)
    ncb = -(-cols // bc)
    codes = np.zeros((rows, cols), dtype=np.uint8)
    recip = np.zeros((nrb, ncb), dtype=np.float32)
    for i in range(nrb):
        r0, r1 = i * br, min(rows, (i + 1) * br)
        for j in range(ncb):
            c0, c1 = j * bc, min(cols, (j + 1) * bc)
            blk = x[r0:r1, c0:c1]
            amax = np.abs(blk).max() if blk.size else np.float32(0)
            s, rcp = scale_from_amax(amax)
            codes[r0:r1, c0:c1] = quantize_with_scale(blk, s)
            recip[i, j] = rcp
    return codes, recip


def quant_1x128(x_bits):
    """1x128 (per row, per 128 columns) quantization of bf16 x[R, C].

    Returns codes[R, C] (uint8) and recip[R, ceil(C/128)] (float32).  Vectorised
    over rows; a ragged last column block uses its valid elements only.
    """
    x = e4m3.bf16_bits_to_f32(x_bits)
    rows, cols = x.shape
    ncb = -(-cols // 128)
    pad = ncb * 128 - cols
    xp = np.pad(x, ((0, 0), (0, pad))) if pad else x
    xb = xp.reshape(rows, ncb, 128)
    amax = np.abs(xb).max(axis=2) if rows else np.zeros((0, ncb), np.float32)
    s, recip = scale_from_amax(amax)
    codes = quantize_with_scale(xb, s[:, :, None]).reshape(rows, ncb * 128)
    return codes[:, :cols].copy(), recip


def quant_128x128(x_bits):
    """128x128 (weight) quantization of bf16 x[R, C].

    Returns codes[R, C] and recip[ceil(R/128), ceil(C/128)].  Ragged edge
    tiles take their amax over the valid elements.
    """
    return _blocks_2d(np.asarray(x_bits, dtype=np.uint16), 128, 128)


def quant_1x128_along_rows(x_bits):
    """1x128 blocks that run down the rows of x[R, C], output transposed.

    Each block is 128 consecutive rows of one column.  This is the same
    definition as ``quant_1x128`` applied to x^T, which is how the wgrad
    operands dY^T and X^T are produced (the 1x128 x 1x128 recipe of [REPRO]
    review comments).  Returns codes_t[C, R] and recip[C, ceil(R/128)].
    """
    xt = np.ascontiguousarray(np.asarray(x_bits, dtype=np.uint16).T)
    return quant_1x128(xt)


def quant_128x128_transposed(x_bits):
    """128x128 quantization of x^T: codes_t[C, R], recip[ceil(C/128), ceil(R/128)].

    Used for the dgrad operand W^T.  Computed from the definition on x^T, not
    by transposing ``quant_128x128``'s output (the tests check that the two
    agree, since a block's amax does not depend on orientation).
    """
    xt = np.ascontiguousarray(np.asarray(x_bits, dtype=np.uint16).T)
    return _blocks_2d(xt, 128, 128)


def quant_tensorwise(x_bits):
    """One scale for the whole tensor ([AITER] ``per_tensor_quant``).

    Returns codes (same shape) and a float32 scalar recip, the dequant
    multiplier: x ~= decode(codes) * recip.
    """
    x = e4m3.bf16_bits_to_f32(x_bits)
    amax = np.abs(x).max() if x.size else np.float32(0)
    s, recip = scale_from_amax(amax)
    return quantize_with_scale(x, s), np.float32(recip)
