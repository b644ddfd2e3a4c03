"""GPU parity of the quantizers against the oracle: bit-exact E4M3 codes and
bit-exact fp32 reciprocal scales, called through the C ABI."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_amd as fp8
from oracle import e4m3, quant
from synth import inputs
from tests.gpu_util import assert_codes_equal, assert_f32_equal, bits, host_f32, host_u8, say

pytestmark = pytest.mark.gpu


def _check_1x128(x_cpu, dev, what):
    say("quant 1x128", what, tuple(x_cpu.shape))
    q, r = fp8.fp8_blockwise_quant(x_cpu.to(dev), "1x128")
    torch.cuda.synchronize()
    oq, orc = quant.quant_1x128(bits(x_cpu))
    assert_codes_equal(host_u8(q), oq, what)
    assert_f32_equal(host_f32(r), orc, what)


def _check_128(x_cpu, dev, what, transpose=False):
    say("quant 128x128", what, tuple(x_cpu.shape), "T" if transpose else "")
    q, r = fp8.fp8_blockwise_quant(x_cpu.to(dev), "128x128", transpose=transpose)
    torch.cuda.synchronize()
    if transpose:
        oq, orc = quant.quant_128x128_transposed(bits(x_cpu))
    else:
        oq, orc = quant.quant_128x128(bits(x_cpu))
    assert_codes_equal(host_u8(q), oq, what)
    assert_f32_equal(host_f32(r), orc, what)


def _check_cols_t(x_cpu, dev, what):
    say("quant 1x128 along rows (T)", what, tuple(x_cpu.shape))
    q, r = fp8.fp8_blockwise_quant(x_cpu.to(dev), "1x128", transpose=True)
    torch.cuda.synchronize()
    oq, orc = quant.quant_1x128_along_rows(bits(x_cpu))
    assert_codes_equal(host_u8(q), oq, what)
    assert_f32_equal(host_f32(r), orc, what)


def _adversarial(rows, cols, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, cols, generator=g)
    kind = torch.arange(rows * ((cols + 127) // 128)).reshape(rows, -1) % 7
    xb = torch.nn.functional.pad(x, (0, (-cols) % 128)).reshape(rows, -1, 128)
    mult = torch.tensor([1.0, 1e-30, 0.0, 5e37, 1e-3, 2.0 ** 60, 1.0])[kind]
    xb = xb * mult[..., None]
    xb[kind == 6] = torch.where(xb[kind == 6].abs() < 1.5, torch.zeros(()), xb[kind == 6])
    return xb.reshape(rows, -1)[:, :cols].to(torch.bfloat16)


@pytest.mark.parametrize("shape", [(128, 512), (77, 384), (1, 128), (300, 400), (64, 16), (2, 4096)])
def test_quant_1x128_small(gpu, shape):
    x = inputs.randn_bf16(shape, seed=inputs.tensor_seed(1, "x"))
    _check_1x128(x, gpu, f"randn {shape}")
    _check_1x128(_adversarial(*shape, seed=5), gpu, f"adversarial {shape}")


@pytest.mark.parametrize("shape", [(16400, 1152), (8200, 1664)])
def test_quant_1x128_several_tiles_per_workgroup_sampled(gpu, shape):
    """Shapes where one workgroup walks several column tiles (odd and even
    counts, a partial last tile, a partial last band of rows): bit-exact on
    sampled rows, which the oracle quantizes independently."""
    rows = np.unique(np.r_[0, 1, 15, 16, shape[0] - 1, shape[0] - 9, shape[0] - 17,
                           np.random.default_rng(shape[0]).integers(0, shape[0], 40)])
    for what, x in (("randn", inputs.randn_bf16(shape, seed=inputs.tensor_seed(1, "x"))),
                    ("adversarial", _adversarial(*shape, seed=5))):
        say("quant 1x128 sampled", what, shape)
        q, r = fp8.fp8_blockwise_quant(x.to(gpu), "1x128")
        torch.cuda.synchronize()
        oq, orc = quant.quant_1x128(bits(x[torch.from_numpy(rows)]))
        assert_codes_equal(host_u8(q)[rows], oq, f"{what} {shape}")
        assert_f32_equal(host_f32(r)[rows], orc, f"{what} {shape}")


def _sweep_rows(amax):
    """Rows of 128 bf16 values: each row holds +amax (fixing the block scale
    at 448/amax) followed by 127 consecutive bf16 patterns of magnitude <=
    amax, both signs: every representable input of that range is quantized."""
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = e4m3.bf16_bits_to_f32(allb)
    keep = np.isfinite(f) & (np.abs(f) <= np.float32(amax))
    vals = allb[keep]
    n = -(-vals.size // 127)
    vals = np.concatenate([vals, np.zeros(n * 127 - vals.size, np.uint16)]).reshape(n, 127)
    head = np.full((n, 1), e4m3.f32_to_bf16_bits(np.float32(amax)), np.uint16)
    rows = np.concatenate([head, vals], axis=1)
    return torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("amax", [448.0, 1.0, 3.0, 0.0078125, 1.7e-5, 2.5e30, 5.9e-39])
def test_quant_codec_sweep_every_bf16_value(gpu, amax):
    """Exhaustive over every bf16 input with |x| <= amax, for scales that are
    exact (amax 448 -> s = 1), powers of two, and inexact (amax 3 -> s =
    149.33..), including subnormal and near-overflow amax."""
    x = _sweep_rows(amax)
    _check_1x128(x, gpu, f"codec sweep amax={amax}")


@pytest.mark.parametrize("n", [1024, 4096])
def test_quant_1x128_square_full(gpu, n):
    x = inputs.randn_bf16((n, n), seed=inputs.tensor_seed(3, "a"))
    _check_1x128(x, gpu, f"square {n}")


@pytest.mark.parametrize("shape", [(256, 512), (130, 384), (1, 128), (1024, 1024), (4096, 4096),
                                   (2600, 8320)])
def test_quant_128x128(gpu, shape):
    x = inputs.randn_bf16(shape, seed=inputs.tensor_seed(4, "w"))
    _check_128(x, gpu, f"randn {shape}")
    if shape[0] <= 1024:
        _check_128(_adversarial(*shape, seed=6), gpu, f"adversarial {shape}")


@pytest.mark.parametrize("shape", [(256, 512), (144, 384), (16, 128), (384, 272), (1024, 2048),
                                   (2608, 8320)])
def test_quant_128x128_transposed(gpu, shape):
    x = inputs.linear_weight_bf16(*shape, seed=inputs.tensor_seed(5, "w"))
    _check_128(x, gpu, f"linear-init {shape}", transpose=True)
    _check_128(_adversarial(*shape, seed=7), gpu, f"adversarial {shape}", transpose=True)


@pytest.mark.parametrize("shape", [(256, 64), (128, 80), (272, 48), (384, 208), (1024, 1024),
                                   (2048, 640), (16640, 1040), (8320, 2000)])
def test_quant_1x128_along_rows_transposed(gpu, shape):
    x = inputs.randn_bf16(shape, seed=inputs.tensor_seed(6, "dy"))
    _check_cols_t(x, gpu, f"randn {shape}")
    xt = _adversarial(shape[1], shape[0], seed=8).t().contiguous()
    _check_cols_t(xt, gpu, f"adversarial {shape}")


@pytest.mark.parametrize("block,shape", [("1x128", (256, 512)), ("1x128", (144, 384)),
                                         ("1x128", (272, 48)), ("1x128", (1040, 2000)),
                                         ("128x128", (256, 512)), ("128x128", (144, 384)),
                                         ("128x128", (2608, 1040))])
def test_quant_dual_layouts(gpu, block, shape):
    """One read, both layouts: each output bit-exact against the oracle's
    quantizer for that layout, and equal to the single-layout kernels."""
    for what, x in (("randn", inputs.randn_bf16(shape, seed=inputs.tensor_seed(12, "x"))),
                    ("adversarial", _adversarial(*shape, seed=13))):
        say("quant dual", block, what, shape)
        xd = x.to(gpu)
        q, r, qt, rt = fp8.fp8_blockwise_quant_dual(xd, block)
        q1, r1 = fp8.fp8_blockwise_quant(xd, block)
        q2, r2 = fp8.fp8_blockwise_quant(xd, block, transpose=True)
        # nontemporal stores of the transposed codes: the same bits
        streamed = fp8.fp8_blockwise_quant_dual(xd, block, stream_t=True)
        torch.cuda.synchronize()
        for a, b in zip(streamed, (q, r, qt, rt)):   # codes, and positive finite scales
            assert torch.equal(a, b), f"dual {block} {what} {shape}: stream_t changed the result"
        if block == "1x128":
            oq, orc = quant.quant_1x128(bits(x))
            oqt, ort = quant.quant_1x128_along_rows(bits(x))
        else:
            oq, orc = quant.quant_128x128(bits(x))
            oqt, ort = quant.quant_128x128_transposed(bits(x))
        assert_codes_equal(host_u8(q), oq, f"dual {block} {what} {shape} codes")
        assert_f32_equal(host_f32(r), orc, f"dual {block} {what} {shape} recip")
        assert_codes_equal(host_u8(qt), oqt, f"dual {block} {what} {shape} codes^T")
        assert_f32_equal(host_f32(rt), ort, f"dual {block} {what} {shape} recip^T")
        assert torch.equal(q, q1) and torch.equal(qt, q2)
        assert torch.equal(r.view(torch.int32), r1.view(torch.int32))
        assert torch.equal(rt.view(torch.int32), r2.view(torch.int32))


@pytest.mark.parametrize("shape", [(16, 32), (32, 32), (256, 1024), (4096, 1024), (3, 48)])
def test_quant_tensorwise(gpu, shape):
    x = inputs.randn_bf16(shape, seed=inputs.tensor_seed(7, "x"))
    say("quant tensorwise", shape)
    q, r = fp8.fp8_tensorwise_quant(x.to(gpu))
    torch.cuda.synchronize()
    oq, orc = quant.quant_tensorwise(bits(x))
    assert_codes_equal(host_u8(q), oq, f"tensorwise {shape}")
    assert_f32_equal(host_f32(r)[0], orc, f"tensorwise {shape}")


@pytest.mark.parametrize("shape,ldx,ldq", [((1000, 208), 208, 208), ((300, 1024), 1040, 1056),
                                           ((4099, 512), 520, 512)])
def test_quant_tensorwise_strides_and_partial_blocks(gpu, shape, ldx, ldq):
    """Per-tensor quantization of strided views (input row stride ldx, codes
    written into a canary-filled [rows, ldq] buffer) and of chunk counts
    that leave a partial 16 KB block after the whole ones."""
    rows, cols = shape
    xb = inputs.randn_bf16((rows, ldx), seed=inputs.tensor_seed(8, "x"))
    x = xb[:, :cols]
    buf = torch.full((rows, ldq), 0xA5, dtype=torch.uint8, device=gpu)
    r = torch.empty(1, dtype=torch.float32, device=gpu)
    say("quant tensorwise strided", shape, ldx, ldq)
    fp8.fp8_tensorwise_quant(xb.to(gpu)[:, :cols], q=buf[:, :cols], recip=r)
    torch.cuda.synchronize()
    oq, orc = quant.quant_tensorwise(bits(x.contiguous()))
    assert_codes_equal(host_u8(buf[:, :cols]), oq, f"tensorwise strided {shape}")
    assert_f32_equal(host_f32(r)[0], orc, f"tensorwise strided {shape}")
    assert bool((buf[:, cols:] == 0xA5).all())


def test_quant_outputs_stay_in_bounds_and_honour_strides(gpu):
    """Canary-padded outputs: codes written with ld_q > cols, scales written
    row-major into a NaN-filled buffer with padding; nothing outside the
    logical region may change."""
    rows, cols = 200, 384
    x = inputs.randn_bf16((rows, cols), seed=9)
    xd = x.to(gpu)
    qbuf = torch.full((rows, cols + 32), 0xA5, dtype=torch.uint8, device=gpu)
    rbuf = torch.full((rows, 5), float("nan"), dtype=torch.float32, device=gpu)
    recip = rbuf[:, :3]                       # row-major view, strides (5, 1)
    say("quant canary 1x128")
    fp8.fp8_blockwise_quant(xd, "1x128", q=qbuf[:, :cols], recip=recip)
    torch.cuda.synchronize()
    oq, orc = quant.quant_1x128(bits(x))
    assert_codes_equal(host_u8(qbuf[:, :cols]), oq, "canary codes")
    assert np.all(host_u8(qbuf[:, cols:]) == 0xA5)
    assert_f32_equal(host_f32(recip), orc, "canary recip")
    assert np.all(np.isnan(host_f32(rbuf[:, 3:])))
    # 128x128 transposed into a padded buffer
    qt = torch.full((cols, 192 + 48), 0x5A, dtype=torch.uint8, device=gpu)
    say("quant canary 128x128 T")
    _, rt = fp8.fp8_blockwise_quant(xd[:192], "128x128", transpose=True, q=qt[:, :192])
    torch.cuda.synchronize()
    oq, orc = quant.quant_128x128_transposed(bits(x[:192]))
    assert_codes_equal(host_u8(qt[:, :192]), oq, "canary T codes")
    assert np.all(host_u8(qt[:, 192:]) == 0x5A)
    assert_f32_equal(host_f32(rt), orc, "canary T recip")


@pytest.mark.parametrize("stream_t", [False, True])
@pytest.mark.parametrize("block", ["1x128", "128x128"])
def test_quant_dual_outputs_stay_in_bounds(gpu, block, stream_t):
    """Both layouts of the dual quantizer (transposed codes with plain or
    nontemporal stores) written into canary-padded code
    buffers (ld > width) and strided views of NaN-filled scale buffers, from
    a 208 x 384 input (a partly filled last row block): bit-exact against
    the oracle, and nothing outside the logical regions changes."""
    rows, cols = 208, 384
    x = inputs.randn_bf16((rows, cols), seed=inputs.tensor_seed(14, "x"))
    xd = x.to(gpu)
    ni, nj = fp8.ops.scale_grid(rows, cols, block, False)
    ti, tj = fp8.ops.scale_grid(rows, cols, block, True)
    qbuf = torch.full((rows, cols + 32), 0xA5, dtype=torch.uint8, device=gpu)
    qtbuf = torch.full((cols, rows + 48), 0x5A, dtype=torch.uint8, device=gpu)
    rbuf = torch.full((ni, nj + 2), float("nan"), dtype=torch.float32, device=gpu)
    rtbuf = torch.full((ti, tj + 3), float("nan"), dtype=torch.float32, device=gpu)
    say("quant dual canary", block, "stream_t" if stream_t else "")
    fp8.fp8_blockwise_quant_dual(xd, block, q=qbuf[:, :cols], recip=rbuf[:, :nj],
                                 qt=qtbuf[:, :rows], recip_t=rtbuf[:, :tj], stream_t=stream_t)
    torch.cuda.synchronize()
    if block == "1x128":
        oq, orc = quant.quant_1x128(bits(x))
        oqt, ort = quant.quant_1x128_along_rows(bits(x))
    else:
        oq, orc = quant.quant_128x128(bits(x))
        oqt, ort = quant.quant_128x128_transposed(bits(x))
    assert_codes_equal(host_u8(qbuf[:, :cols]), oq, f"dual canary {block} codes")
    assert_codes_equal(host_u8(qtbuf[:, :rows]), oqt, f"dual canary {block} codes^T")
    assert_f32_equal(host_f32(rbuf[:, :nj]), orc, f"dual canary {block} recip")
    assert_f32_equal(host_f32(rtbuf[:, :tj]), ort, f"dual canary {block} recip^T")
    assert np.all(host_u8(qbuf[:, cols:]) == 0xA5) and np.all(host_u8(qtbuf[:, rows:]) == 0x5A)
    assert np.all(np.isnan(host_f32(rbuf[:, nj:]))) and np.all(np.isnan(host_f32(rtbuf[:, tj:])))


def test_quant_deterministic(gpu):
    x = inputs.randn_bf16((512, 1024), seed=10).to(gpu)
    say("quant determinism")
    a = [fp8.fp8_blockwise_quant(x, b, transpose=t) for b in ("1x128", "128x128") for t in (False, True)]
    b = [fp8.fp8_blockwise_quant(x, b, transpose=t) for b in ("1x128", "128x128") for t in (False, True)]
    torch.cuda.synchronize()
    for (q1, r1), (q2, r2) in zip(a, b):
        assert torch.equal(q1, q2) and torch.equal(r1.view(torch.int32), r2.view(torch.int32))


def test_quant_large_sampled(gpu):
    """Square 8192^2 and 32768^2 bf16 inputs: bit-exact on sampled rows / row
    blocks; at full size every block with a nonzero amax holds a +-448 code."""
    for n in (8192, 32768):
        say("quant large", n, "generate")
        x = inputs.randn_bf16((n, n), seed=inputs.tensor_seed(11, "a"), device="cuda")
        for block in ("1x128", "128x128"):
            say("quant large", n, block)
            q, r = fp8.fp8_blockwise_quant(x, block)
            torch.cuda.synchronize()
            if block == "1x128":
                hit = ((q.view(n, n // 128, 128) & 0x7F) == 0x7E).any(dim=2)
                assert bool(hit.all())
                rows = np.unique(np.r_[0, n - 1, np.random.default_rng(n).integers(0, n, 14)])
                xs = bits(x[rows])
                oq, orc = quant.quant_1x128(xs)
                assert_codes_equal(host_u8(q[rows]), oq, f"1x128 {n} sampled rows")
                assert_f32_equal(host_f32(r[rows]), orc, f"1x128 {n} sampled rows")
            else:
                hit = ((q.view(n // 128, 128, n // 128, 128) & 0x7F) == 0x7E).any(dim=3).any(dim=1)
                assert bool(hit.all())
                for rb in (0, n // 128 - 1):
                    sl = slice(rb * 128, rb * 128 + 128)
                    oq, orc = quant.quant_128x128(bits(x[sl]))
                    assert_codes_equal(host_u8(q[sl]), oq, f"128x128 {n} row block {rb}")
                    assert_f32_equal(host_f32(r[rb:rb + 1]), orc, f"128x128 {n} row block {rb}")
            del q, r
        del x
        torch.cuda.empty_cache()
