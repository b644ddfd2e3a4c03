"""GPU parity of fp8_scaled_gemm_blockwise_kn: the blockwise GEMM with its
second operand given in [K, N] layout (the transposed view of an [N, K]
matrix, as torch._scaled_mm takes the weight: [AITER] Steps to Reproduce),
read into LDS row by row and turned into matrix-core operands with
transposing LDS reads.  Checked against the oracle and bit for bit against
fp8_scaled_gemm_blockwise on the [N, K] copy of the same codes."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_amd as fp8
from oracle import gemm, linear, quant
from synth import inputs
from tests.gpu_util import bits, check_gemm_output, host_f32, say

pytestmark = pytest.mark.gpu


def _random_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


def _colmajor(r, dev):
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(r, np.float32).T)).to(dev)
    return t.t()


@pytest.mark.parametrize("M,N,K,b_block,ldb_pad,ldo_pad", [
    (300, 448, 1024, "128x128", 48, 0),     # ragged M and N, padded B rows
    (1000, 1040, 1152, "1x128", 0, 8),      # per-row B scales, 9 K blocks, padded output
    (256, 256, 128, "1x128", 16, 0),        # one tile, one K block
    (4352, 4096, 2048, "128x128", 0, 0),    # 272 tiles: the leftover tiles split over K
])
def test_kn_layout_matches_oracle_and_nk(gpu, M, N, K, b_block, ldb_pad, ldo_pad):
    rng = np.random.default_rng(M + N + K)
    kb = K // 128
    aq = _random_codes(rng, (M, K))
    bkn = _random_codes(rng, (K, N))
    ar = rng.uniform(0.01, 0.02, (M, kb)).astype(np.float32)
    nrb = N if b_block == "1x128" else -(-N // 128)
    br = rng.uniform(0.01, 0.02, (nrb, kb)).astype(np.float32)
    a_d = torch.from_numpy(aq).to(gpu)
    bbuf = torch.zeros((K, N + ldb_pad), dtype=torch.uint8, device=gpu)
    bbuf[:, :N] = torch.from_numpy(bkn).to(gpu)
    ra_d, rb_d = _colmajor(ar, gpu), _colmajor(br, gpu)
    # Large problems: the oracle on the first and last 64 rows (the last row
    # tiles are the leftover tiles that run split over K); every element is
    # compared bit for bit with the [N, K] path.
    rows = np.arange(M) if M * N <= (1 << 22) else np.r_[0:64, M - 64:M]
    ref, S = gemm.blockwise_gemm(aq[rows], ar[rows], np.ascontiguousarray(bkn.T), br, b_block,
                                 with_bound=True)
    for od, name in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        say("gemm kn", M, N, K, b_block, name, ldb_pad, ldo_pad)
        obuf = torch.full((M, N + ldo_pad), float("nan"), dtype=od, device=gpu)
        out = fp8.fp8_scaled_gemm_blockwise_kn(a_d, ra_d, bbuf[:, :N], rb_d, b_block=b_block,
                                               out=obuf[:, :N])
        nk = fp8.fp8_scaled_gemm_blockwise(a_d, ra_d, bbuf[:, :N].t().contiguous(), rb_d,
                                           b_block=b_block, out_dtype=od)
        torch.cuda.synchronize()
        if ldo_pad:
            assert torch.isnan(obuf[:, N:].float()).all(), "wrote past N"
        assert torch.equal(out.view(torch.int16 if name == "bf16" else torch.int32),
                           nk.view(torch.int16 if name == "bf16" else torch.int32)), \
            "[K, N] and [N, K] layouts give different bits"
        check_gemm_output(host_f32(out)[rows], ref, S, kb, name,
                          f"kn M{M} N{N} K{K} {b_block} {name}")


def test_kn_dgrad_from_weight_codes(gpu):
    """dX = dY . W straight from W's own 128x128 codes and scales (the
    scales' transposed view), against the oracle's dgrad, which quantizes
    W^T: 128x128 block amax does not depend on orientation."""
    M, N, K = 384, 256, 512            # tokens, W rows (contraction), W columns (dX columns)
    dy = bits(inputs.randn_bf16((M, N), seed=inputs.tensor_seed(3, "dy")))
    w = bits(inputs.linear_weight_bf16(N, K, seed=inputs.tensor_seed(3, "w")))
    dq, dr = quant.quant_1x128(dy)
    wq, wr = quant.quant_128x128(w)         # codes [N, K], scales [N/128, K/128]
    say("gemm kn dgrad", M, N, K)
    out = fp8.fp8_scaled_gemm_blockwise_kn(
        torch.from_numpy(dq).to(gpu), _colmajor(dr, gpu), torch.from_numpy(wq).to(gpu),
        _colmajor(np.ascontiguousarray(wr.T), gpu), b_block="128x128")
    torch.cuda.synchronize()
    ref, S = linear.dgrad(dy, w, with_bound=True)
    check_gemm_output(host_f32(out), ref, S, N // 128, "bf16", "kn dgrad from W codes")


def test_kn_refuses_unsupported(gpu):
    rng = np.random.default_rng(5)
    for M, N in ((128, 512), (512, 208), (512, 336)):   # M < 256, N < 256, N % 64 != 0
        a = torch.from_numpy(_random_codes(rng, (M, 256))).to(gpu)
        b = torch.from_numpy(_random_codes(rng, (256, N))).to(gpu)
        ra = _colmajor(np.ones((M, 2), np.float32), gpu)
        rb = _colmajor(np.ones((-(-N // 128), 2), np.float32), gpu)
        with pytest.raises(fp8.FP8BWError, match="UNSUPPORTED"):
            fp8.fp8_scaled_gemm_blockwise_kn(a, ra, b, rb, b_block="128x128")
