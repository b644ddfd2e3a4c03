"""GPU parity of the blockwise and tensorwise GEMMs against the oracle,
called through the C ABI.  The GEMM inputs (codes and reciprocal scales) are
produced by the oracle on the host and uploaded, so these tests isolate the
GEMM; the linear tests run the whole GPU pipeline."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_amd as fp8
from oracle import e4m3, gemm, metrics, quant
from synth import inputs
from tests.gpu_util import bits, check_gemm_output, host_f32, say

pytestmark = pytest.mark.gpu


def _up_codes(c, dev):
    return torch.from_numpy(np.ascontiguousarray(c)).to(dev)


def _up_scales_colmajor(r, dev):
    """Logical [ni, nj] float32 -> device tensor with column-major strides."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(r, np.float32).T)).to(dev)
    return t.t()


def _random_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


def _run_blockwise(dev, aq, ar, bq, br, b_block, out_dtype, what, config=None, splits=None,
                   ldo_pad=0):
    """One GEMM call against the oracle; with ldo_pad the output is a view
    of a NaN-filled [M, N + ldo_pad] buffer whose padding must stay NaN."""
    say("gemm blockwise", what, aq.shape, bq.shape, b_block, out_dtype, config, splits, ldo_pad)
    od = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    M, N = aq.shape[0], bq.shape[0]
    buf = torch.full((M, N + ldo_pad), float("nan"), dtype=od, device=dev)
    out = fp8.fp8_scaled_gemm_blockwise(_up_codes(aq, dev), _up_scales_colmajor(ar, dev),
                                        _up_codes(bq, dev), _up_scales_colmajor(br, dev),
                                        b_block=b_block, out_dtype=od, config=config,
                                        splits=splits, out=buf[:, :N])
    torch.cuda.synchronize()
    if ldo_pad:
        assert torch.isnan(buf[:, N:].float()).all(), f"{what}: wrote past N"
    ref, S = gemm.blockwise_gemm(aq, ar, bq, br, b_block, with_bound=True)
    return check_gemm_output(host_f32(out), ref, S, aq.shape[1] // 128, out_dtype, what)


def test_tiny_linear_shapes(gpu):
    """X[128,512] N(0,1) x W[256,512] nn.Linear init, X 1x128 and W 128x128."""
    x = bits(inputs.randn_bf16((128, 512), seed=inputs.tensor_seed(0, "x")))
    w = bits(inputs.linear_weight_bf16(256, 512, seed=inputs.tensor_seed(0, "w")))
    xq, xr = quant.quant_1x128(x)
    wq, wr = quant.quant_128x128(w)
    for od in ("bf16", "f32"):
        _run_blockwise(gpu, xq, xr, wq, wr, "128x128", od, "tiny linear")


@pytest.mark.parametrize("kb", [1, 2, 3, 5, 7])
@pytest.mark.parametrize("mn", [(1, 16), (16, 96), (77, 130), (128, 256), (200, 300)])
def test_blockwise_ragged_and_k_blocks(gpu, kb, mn):
    rng = np.random.default_rng(kb * 1000 + mn[0])
    M, N = mn
    K = 128 * kb
    aq = _random_codes(rng, (M, K))
    bq = _random_codes(rng, (N, K))
    ar = rng.uniform(0.5, 2.0, (M, kb)).astype(np.float32) * np.float32(2.0 ** -8)
    for b_block in ("128x128", "1x128"):
        nbr = N if b_block == "1x128" else -(-N // 128)
        br = rng.uniform(0.5, 2.0, (nbr, kb)).astype(np.float32) * np.float32(2.0 ** -9)
        _run_blockwise(gpu, aq, ar, bq, br, b_block, "bf16", f"M{M} N{N} kb{kb} {b_block}")
        _run_blockwise(gpu, aq, ar, bq, br, b_block, "f32", f"M{M} N{N} kb{kb} {b_block}")


def test_power_of_two_scale_probe(gpu):
    """Distinct power-of-two scales per (row, kb) and per (block, kb): any
    scale-indexing error shows up as an exact power-of-two discrepancy."""
    rng = np.random.default_rng(3)
    M, N, kb = 96, 272, 6
    aq = _random_codes(rng, (M, 128 * kb))
    bq = _random_codes(rng, (N, 128 * kb))
    ar = np.array([[2.0 ** ((m % 13) - 6 + 2 * k) for k in range(kb)] for m in range(M)], np.float32)
    for b_block in ("128x128", "1x128"):
        nbr = N if b_block == "1x128" else 3
        br = np.array([[2.0 ** (-(r % 11) - k) for k in range(kb)] for r in range(nbr)], np.float32)
        _run_blockwise(gpu, aq, ar, bq, br, b_block, "f32", f"pow2 probe {b_block}")


# Large-tile configurations and their tile sizes (BM, BN): they need M >= BM
# and N >= BN (an edge tile's operand window moves back inside the matrix).
LARGE_TILES = {2: (256, 128), 3: (256, 256)}


def _config_accepts(cfg, M, N, b_block):
    bm, bn = LARGE_TILES.get(cfg, (1, 1))
    if cfg in LARGE_TILES and b_block == "128x128" and N % 64:
        return False      # a wave's 64 columns must keep one B scale block
    return M >= bm and N >= bn


@pytest.mark.parametrize("mn,pad", [((200, 300), 0), ((300, 448), 0), ((300, 401), 3)])
def test_every_config_and_split(gpu, mn, pad):
    """Force every tile configuration and several split-K counts (a kernel
    variant can be wrong where the others are right).  300 x 448 and
    300 x 401 give the large-tile kernels ragged edge tiles in both
    dimensions (at 401 columns, per-row B scales, an output row stride of
    404 and column quads that do not start on a multiple of 4); a large
    configuration forced on a problem it does not take is refused."""
    rng = np.random.default_rng(4 + mn[0] + mn[1])
    M, N = mn
    kb = 8
    aq = _random_codes(rng, (M, 128 * kb))
    bq = _random_codes(rng, (N, 128 * kb))
    ar = rng.uniform(0.01, 0.02, (M, kb)).astype(np.float32)
    for b_block in ("128x128", "1x128"):
        nbr = N if b_block == "1x128" else -(-N // 128)
        br = rng.uniform(0.01, 0.02, (nbr, kb)).astype(np.float32)
        for cfg in range(fp8.fp8bw_gemm_num_configs()):
            if not _config_accepts(cfg, M, N, b_block):
                with pytest.raises(fp8.FP8BWError, match="UNSUPPORTED"):
                    _run_blockwise(gpu, aq, ar, bq, br, b_block, "f32", f"cfg{cfg} refused",
                                   config=cfg, splits=1)
                continue
            for splits in (1, 2, 3, 8):
                for od in ("bf16", "f32"):
                    _run_blockwise(gpu, aq, ar, bq, br, b_block, od,
                                   f"M{M} N{N} {b_block} cfg{cfg} split{splits}", config=cfg,
                                   splits=splits, ldo_pad=pad)


@pytest.mark.parametrize("pad", [16, 4, 2])
def test_large_tile_staged_epilogue_canary(gpu, pad):
    """The 256x256 kernel stages interior tiles through LDS and stores whole
    rows of the tile (bf16 when the output row stride is a multiple of 8
    elements, fp32 outputs and K-split partials when it is a multiple of 4;
    otherwise the direct quad stores).  M = 520, N = 576 gives four interior
    tiles and five edge tiles; the output is a view 8 columns into a
    NaN-filled buffer of row stride N + 8 + pad, and every column on either
    side of it must keep its canary.  pad 16: all staged; 4: fp32 staged,
    bf16 direct; 2: all direct."""
    rng = np.random.default_rng(41 + pad)
    M, N, kb = 520, 576, 3
    aq = _random_codes(rng, (M, 128 * kb))
    bq = _random_codes(rng, (N, 128 * kb))
    ar = rng.uniform(0.01, 0.02, (M, kb)).astype(np.float32)
    for b_block in ("128x128", "1x128"):
        nbr = N if b_block == "1x128" else -(-N // 128)
        br = rng.uniform(0.01, 0.02, (nbr, kb)).astype(np.float32)
        ref, S = gemm.blockwise_gemm(aq, ar, bq, br, b_block, with_bound=True)
        for od_name, od in (("bf16", torch.bfloat16), ("f32", torch.float32)):
            for splits in (1, 2):
                what = f"staged epilogue {b_block} {od_name} split{splits} pad{pad}"
                say("gemm", what)
                buf = torch.full((M, N + 8 + pad), float("nan"), dtype=od, device=gpu)
                out = buf[:, 8:8 + N]
                fp8.fp8_scaled_gemm_blockwise(_up_codes(aq, gpu), _up_scales_colmajor(ar, gpu),
                                              _up_codes(bq, gpu), _up_scales_colmajor(br, gpu),
                                              b_block=b_block, out_dtype=od, config=3,
                                              splits=splits, out=out)
                torch.cuda.synchronize()
                assert torch.isnan(buf[:, :8].float()).all(), f"{what}: wrote before column 0"
                assert torch.isnan(buf[:, 8 + N:].float()).all(), f"{what}: wrote past N"
                check_gemm_output(host_f32(out), ref, S, kb, od_name, what)


@pytest.mark.parametrize("mode,leftover", [("128x128", False), ("1x128", False),
                                           ("tensorwise", False), ("128x128", True),
                                           ("1x128", True)])
def test_persistent_main_launch(gpu, mode, leftover):
    """Two full rounds of interior 256x256 tiles (one tile per CU each) run as
    a persistent launch: one workgroup per CU takes its tile of every round
    in turn, and the waves that issue no operand loads store each tile's
    output while the next tile's K loop runs; with leftover tiles (a 17th
    row of tiles, cus / 8 of them), the workgroups then run those tiles' K
    pieces before the reduce.  The same GEMM into an output whose row stride
    is not a multiple of 8 elements runs one tile per workgroup with the
    direct quad stores and a separate launch for the pieces: the two must
    agree bit for bit, and with the oracle on sampled rows (first, middle
    and last 64; the last are the leftover tiles' rows)."""
    cus = torch.cuda.get_device_properties(gpu).multi_processor_count
    if cus % 8:
        pytest.skip(f"{cus} CUs: the shape below assumes a multiple of 8")
    # 16 (17) x (cus / 8) tiles = two rounds (+ cus / 8 leftover tiles, split
    # in 4 K pieces of 4 K blocks)
    M, N, K = (4352, 32 * cus, 2048) if leftover else (4096, 32 * cus, 384)
    kb = K // 128
    pl = fp8.gemm_plan(M, N, K, "1x128" if mode == "1x128" else "128x128")
    assert pl["config"] == 3 and pl["tiles_full"] == 2 * cus, pl
    assert pl["tail_splits"] == (4 if leftover else 1), pl
    rng = np.random.default_rng(61 + len(mode) + leftover)
    aq = _random_codes(rng, (M, K))
    bq = _random_codes(rng, (N, K))
    rows = np.r_[0:64, M // 2 - 32:M // 2 + 32, M - 64:M]
    a_d, b_d = _up_codes(aq, gpu), _up_codes(bq, gpu)
    if mode == "tensorwise":
        ra, rb = np.float32(0.0123), np.float32(0.0456)
        ref = gemm.tensorwise_gemm(aq[rows], ra, bq, rb)
        S = gemm.tensorwise_bound(aq[rows], ra, bq, rb)
        ra_d, rb_d = torch.tensor([ra], device=gpu), torch.tensor([rb], device=gpu)
        call = lambda out: fp8.fp8_scaled_gemm_tensorwise(a_d, ra_d, b_d, rb_d, out=out)
    else:
        ar = rng.uniform(0.01, 0.02, (M, kb)).astype(np.float32)
        nbr = N if mode == "1x128" else N // 128
        br = rng.uniform(0.01, 0.02, (nbr, kb)).astype(np.float32)
        ref, S = gemm.blockwise_gemm(aq[rows], ar[rows], bq, br, mode, with_bound=True)
        ra_d, rb_d = _up_scales_colmajor(ar, gpu), _up_scales_colmajor(br, gpu)
        call = lambda out: fp8.fp8_scaled_gemm_blockwise(a_d, ra_d, b_d, rb_d, b_block=mode,
                                                         out=out)
    outs = []
    for pad in (0, 4):    # row stride N: persistent; N + 4: one tile per workgroup
        say("gemm persistent", mode, M, N, K, "ldo pad", pad, "leftover", leftover)
        buf = torch.full((M, N + pad), float("nan"), dtype=torch.bfloat16, device=gpu)
        call(buf[:, :N])   # (the binding allocates the workspace the plan asks for)
        torch.cuda.synchronize()
        if pad:
            assert torch.isnan(buf[:, N:].float()).all(), "wrote past N"
        outs.append(buf[:, :N])
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), \
        "persistent and one-tile-per-workgroup launches differ"
    check_gemm_output(host_f32(outs[0])[rows], ref, S, kb, "bf16", f"persistent {mode}")


def _scale_view(r, layout, dev):
    """Logical fp32 [ni, nj] on the device in a given memory layout."""
    r = np.asarray(r, np.float32)
    ni, nj = r.shape
    if layout == "colmajor":
        return _up_scales_colmajor(r, dev)
    if layout == "rowmajor":
        return torch.from_numpy(np.ascontiguousarray(r)).to(dev)
    if layout == "rowmajor_padded":
        buf = torch.full((ni, nj + 3), float("nan"), dtype=torch.float32, device=dev)
        buf[:, :nj] = torch.from_numpy(r).to(dev)
        return buf[:, :nj]
    if layout == "colmajor_padded":
        buf = torch.full((nj, ni + 5), float("nan"), dtype=torch.float32, device=dev)
        buf[:, :ni] = torch.from_numpy(np.ascontiguousarray(r.T)).to(dev)
        return buf[:, :ni].t()
    raise ValueError(layout)


@pytest.mark.parametrize("layout", ["rowmajor", "rowmajor_padded", "colmajor_padded"])
def test_scale_strides_any_nested_layout(gpu, layout):
    """A and B scales given as row-major, padded row-major and padded
    column-major views (no copies), for both B recipes, on the small-tile
    and the large-tile kernels (ragged 300 x 448), against the oracle on
    the logical scale grids."""
    rng = np.random.default_rng(17)
    M, N, kb = 300, 448, 6
    aq = _random_codes(rng, (M, 128 * kb))
    bq = _random_codes(rng, (N, 128 * kb))
    ar = (rng.uniform(0.5, 2.0, (M, kb)) * 2.0 ** -8).astype(np.float32)
    for b_block in ("128x128", "1x128"):
        nbr = N if b_block == "1x128" else -(-N // 128)
        br = (rng.uniform(0.5, 2.0, (nbr, kb)) * 2.0 ** -9).astype(np.float32)
        ref, S = gemm.blockwise_gemm(aq, ar, bq, br, b_block, with_bound=True)
        for cfg in (None, 0, 1, 2, 3):
            say("gemm scale strides", layout, b_block, cfg)
            out = fp8.fp8_scaled_gemm_blockwise(_up_codes(aq, gpu), _scale_view(ar, layout, gpu),
                                                _up_codes(bq, gpu), _scale_view(br, layout, gpu),
                                                b_block=b_block, out_dtype=torch.float32,
                                                config=cfg, splits=None if cfg is None else 1)
            torch.cuda.synchronize()
            check_gemm_output(host_f32(out), ref, S, kb, "f32", f"strides {layout} {b_block} cfg{cfg}")


def test_canary_output_and_strided_b_scales(gpu):
    """Output written with ldo > N into a canary-filled buffer; B scales given
    row-major (strides (kb, 1)) instead of column-major."""
    rng = np.random.default_rng(5)
    M, N, kb = 130, 200, 3
    aq = _random_codes(rng, (M, 128 * kb))
    bq = _random_codes(rng, (N, 128 * kb))
    ar = rng.uniform(0.01, 0.02, (M, kb)).astype(np.float32)
    br = rng.uniform(0.01, 0.02, (2, kb)).astype(np.float32)
    buf = torch.full((M, N + 24), float("nan"), dtype=torch.float32, device=gpu)
    rb_rowmajor = torch.from_numpy(br).to(gpu)            # strides (kb, 1)
    say("gemm canary")
    fp8.fp8_scaled_gemm_blockwise(_up_codes(aq, gpu), _up_scales_colmajor(ar, gpu),
                                  _up_codes(bq, gpu), rb_rowmajor, out=buf[:, :N])
    torch.cuda.synchronize()
    ref, S = gemm.blockwise_gemm(aq, ar, bq, br, "128x128", with_bound=True)
    check_gemm_output(host_f32(buf[:, :N]), ref, S, kb, "f32", "canary")
    assert np.all(np.isnan(host_f32(buf[:, N:])))


def test_long_k_1000_1001_1002_blocks(gpu):
    """M = N = 1024, K in {128000, 128128, 128256}: A N(0,1) 1x128, B nn.Linear
    init 128x128, bf16 out, whole pipeline on the GPU.  Sampled outputs match
    the oracle; SQNR vs the fp32 product stays in the band for all three
    (the pages report a collapse of another library at 1001 / 1002)."""
    M = N = 1024
    results = {}
    for K in (128000, 128128, 128256):
        say("long-K", K, "generate")
        a = inputs.randn_bf16((M, K), seed=inputs.tensor_seed(20, "a"), device="cuda")
        b = inputs.linear_weight_bf16(N, K, seed=inputs.tensor_seed(20, "b"), device="cuda")
        say("long-K", K, "gpu quant + gemm")
        aq, ar = fp8.fp8_blockwise_quant(a, "1x128")
        bq, br = fp8.fp8_blockwise_quant(b, "128x128")
        out = fp8.fp8_scaled_gemm_blockwise(aq, ar, bq, br, "128x128")
        torch.cuda.synchronize()
        rows = np.sort(np.random.default_rng(K).choice(M, 24, replace=False))
        nblk = (0, 5)
        cols = np.concatenate([np.arange(n * 128, n * 128 + 128) for n in nblk])
        say("long-K", K, "oracle on sample")
        a_s = bits(a[torch.from_numpy(rows).to(a.device)])
        oaq, oar = quant.quant_1x128(a_s)
        b_s = bits(b[torch.from_numpy(cols).to(b.device)])
        obq, obr = quant.quant_128x128(b_s)
        ref, S = gemm.blockwise_gemm(oaq, oar, obq, obr, "128x128", with_bound=True)
        got = host_f32(out)[np.ix_(rows, cols)]
        check_gemm_output(got, ref, S, K // 128, "bf16", f"long-K {K}")
        fp32ref = gemm.fp32_reference(a_s, b_s)
        s_gpu = metrics.sqnr_db(fp32ref, got)
        s_orc = metrics.sqnr_db(fp32ref, e4m3.rne_bf16(ref.astype(np.float32)))
        assert 28.0 <= s_gpu <= 32.5, (K, s_gpu)
        assert abs(s_gpu - s_orc) <= 0.05, (K, s_gpu, s_orc)
        # no collapse anywhere in the full output: |out| ~ sqrt(M N / 3)
        nrm = float(torch.linalg.vector_norm(out.float()))
        assert 0.9 * np.sqrt(M * N / 3) < nrm < 1.1 * np.sqrt(M * N / 3), (K, nrm)
        results[K] = s_gpu
        del a, b, aq, bq, out
    say("long-K SQNR dB", results)


@pytest.mark.parametrize("splits", [1, 7, 13, 64])
def test_long_k_forced_splits(gpu, splits):
    """K = 128128 (1001 blocks, 7 x 11 x 13) with forced split counts that do
    and do not divide the block count, on every tile configuration (M = 320:
    the 256-row kernels get a ragged second row tile)."""
    rng = np.random.default_rng(splits)
    M, N, K = 320, 256, 128128
    aq = _random_codes(rng, (M, K))
    bq = _random_codes(rng, (N, K))
    ar = rng.uniform(1e-3, 2e-3, (M, K // 128)).astype(np.float32)
    br = rng.uniform(1e-3, 2e-3, (2, K // 128)).astype(np.float32)
    ref, S = gemm.blockwise_gemm(aq, ar, bq, br, "128x128", with_bound=True)
    args = (_up_codes(aq, gpu), _up_scales_colmajor(ar, gpu), _up_codes(bq, gpu),
            _up_scales_colmajor(br, gpu))
    for cfg in range(fp8.fp8bw_gemm_num_configs()):
        say("gemm long-K forced", splits, cfg)
        out = fp8.fp8_scaled_gemm_blockwise(*args, out_dtype=torch.float32, config=cfg,
                                            splits=splits)
        torch.cuda.synchronize()
        check_gemm_output(host_f32(out), ref, S, K // 128, "f32",
                          f"long-K splits={splits} cfg{cfg}")


def _tensorwise_case(dev, M, N, K, out_dtype, seed):
    x = bits(inputs.randn_bf16((M, K), seed=inputs.tensor_seed(seed, "x")))
    w = bits(inputs.randn_bf16((N, K), seed=inputs.tensor_seed(seed, "w")))
    xq, xr = quant.quant_tensorwise(x)
    wq, wr = quant.quant_tensorwise(w)
    od = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    say("gemm tensorwise", M, N, K, out_dtype)
    out = fp8.fp8_scaled_gemm_tensorwise(_up_codes(xq, dev), torch.tensor([xr], device=dev),
                                         _up_codes(wq, dev), torch.tensor([wr], device=dev),
                                         out_dtype=od)
    torch.cuda.synchronize()
    ref = gemm.tensorwise_gemm(xq, xr, wq, wr)
    S = gemm.tensorwise_bound(xq, xr, wq, wr)
    got = host_f32(out)
    check_gemm_output(got, ref, S, -(-K // 128), out_dtype, f"tensorwise {M}x{N}x{K}")
    return got, ref


def test_tensorwise_256x4096x1024(gpu):
    got, ref = _tensorwise_case(gpu, 256, 4096, 1024, "bf16", seed=30)
    # the checks the per-tensor issue applies, against the dequant reference
    refb = torch.from_numpy(e4m3.rne_bf16(ref.astype(np.float32)))
    g = torch.from_numpy(got)
    for rtol, atol in ((1e-2, 1e-2), (5e-2, 5e-2)):
        assert torch.allclose(g, refb, rtol=rtol, atol=atol)


def test_tensorwise_edge_16x32x32_fp32(gpu):
    got, ref = _tensorwise_case(gpu, 16, 32, 32, "f32", seed=31)
    assert np.allclose(got, ref, rtol=0.01, atol=0.05)


@pytest.mark.parametrize("mnk", [(1, 16, 16), (33, 17, 48), (130, 70, 400), (64, 64, 128)])
def test_tensorwise_ragged(gpu, mnk):
    _tensorwise_case(gpu, *mnk, "f32", seed=32 + mnk[0])


def test_gemm_deterministic(gpu):
    rng = np.random.default_rng(6)
    aq = _up_codes(_random_codes(rng, (300, 1024)), gpu)
    bq = _up_codes(_random_codes(rng, (260, 1024)), gpu)
    ar = _up_scales_colmajor(rng.uniform(0.5, 1, (300, 8)).astype(np.float32), gpu)
    br = _up_scales_colmajor(rng.uniform(0.5, 1, (3, 8)).astype(np.float32), gpu)
    say("gemm determinism")
    o1 = fp8.fp8_scaled_gemm_blockwise(aq, ar, bq, br, splits=4, config=0, out_dtype=torch.float32)
    o2 = fp8.fp8_scaled_gemm_blockwise(aq, ar, bq, br, splits=4, config=0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))


@pytest.mark.parametrize("mode,od", [("128x128", "f32"), ("128x128", "bf16"), ("1x128", "f32"),
                                     ("1x128", "bf16"), ("tensorwise", "f32"),
                                     ("tensorwise", "bf16")])
def test_tail_split_of_last_round(mode, od):
    """272 tiles of 256x256 on 256 CUs: the leftover 16 tiles (the last
    row-block of tiles in the grouped order) run split over K into
    tile-local partials after the 256 whole tiles, then an ordered reduce.
    Rows of that block and random others match the oracle for every scale
    mode and output type, and so does the plan forced to one unsplit
    launch; rows of whole tiles are identical in both runs."""
    import torch as _t
    dev = _t.device("cuda", 0)
    rng = np.random.default_rng(40)
    M, N, K = 4352, 4096, 2048
    aq = _random_codes(rng, (M, K))
    bq = _random_codes(rng, (N, K))
    dt = _t.bfloat16 if od == "bf16" else _t.float32
    rows = np.unique(np.r_[np.arange(M - 256, M, 3), rng.choice(M - 256, 32, replace=False)])
    if mode == "tensorwise":
        ar, br = np.float32(1.5e-3), np.float32(1.25e-3)
        say("gemm tail split tensorwise", od)
        auto = fp8.fp8_scaled_gemm_tensorwise(_up_codes(aq, dev), _t.tensor([ar], device=dev),
                                              _up_codes(bq, dev), _t.tensor([br], device=dev),
                                              out_dtype=dt)
        _t.cuda.synchronize()
        ref = gemm.tensorwise_gemm(aq[rows], ar, bq, br)
        S = gemm.tensorwise_bound(aq[rows], ar, bq, br)
        check_gemm_output(host_f32(auto)[rows], ref, S, K // 128, od, f"tail split tensorwise {od}")
        return
    ar = rng.uniform(1e-3, 2e-3, (M, K // 128)).astype(np.float32)
    nb = N if mode == "1x128" else N // 128
    br = rng.uniform(1e-3, 2e-3, (nb, K // 128)).astype(np.float32)
    args = (_up_codes(aq, dev), _up_scales_colmajor(ar, dev), _up_codes(bq, dev),
            _up_scales_colmajor(br, dev))
    say("gemm tail split auto", mode, od)
    auto = fp8.fp8_scaled_gemm_blockwise(*args, b_block=mode, out_dtype=dt)
    say("gemm tail split forced off", mode, od)
    plain = fp8.fp8_scaled_gemm_blockwise(*args, b_block=mode, out_dtype=dt, config=3, splits=1)
    _t.cuda.synchronize()
    ref, S = gemm.blockwise_gemm(aq[rows], ar[rows], bq, br, mode, with_bound=True)
    for name, out in (("auto", auto), ("plain", plain)):
        check_gemm_output(host_f32(out)[rows], ref, S, K // 128, od, f"tail split {name} {mode}")
    # rows outside the leftover block come from whole tiles in both runs
    whole = host_f32(auto)[: M - 256]
    assert np.array_equal(whole, host_f32(plain)[: M - 256])


@pytest.mark.parametrize("mnk,b_block,od", [
    ((128, 256, 512), "128x128", "bf16"),      # small-tile kernel
    ((77, 130, 384), "1x128", "f32"),          # ragged edges
    ((256, 256, 16384), "128x128", "f32"),     # whole-problem split-K: bias in the reduce
    ((2048, 2048, 1024), "128x128", "bf16"),   # large-tile kernel
    ((4352, 4096, 2048), "128x128", "f32"),    # full rounds + tail split (tiled reduce)
    ((4352, 8192, 2048), "1x128", "bf16"),     # 256 CUs: persistent launch + leftover pieces
])
def test_blockwise_bias_epilogue(gpu, mnk, b_block, od):
    """out = acc + bias[n] before the cast, on every store path the built-in
    plan takes (direct stores, whole-problem split-K, tail split); sampled
    rows against oracle add_bias(ref64, bias) with S + |bias| as the bound."""
    M, N, K = mnk
    rng = np.random.default_rng(M + N + K)
    aq, bq = _random_codes(rng, (M, K)), _random_codes(rng, (N, K))
    ar = rng.uniform(1e-3, 2e-3, (M, K // 128)).astype(np.float32)
    nb = N if b_block == "1x128" else -(-N // 128)
    br = rng.uniform(1e-3, 2e-3, (nb, K // 128)).astype(np.float32)
    bias = e4m3.f32_to_bf16_bits(rng.normal(0, 4, N).astype(np.float32))
    dt = torch.bfloat16 if od == "bf16" else torch.float32
    say("gemm blockwise bias", mnk, b_block, od)
    bias_d = torch.from_numpy(bias.view(np.int16)).view(torch.bfloat16).to(gpu)
    out = fp8.fp8_scaled_gemm_blockwise(_up_codes(aq, gpu), _up_scales_colmajor(ar, gpu),
                                        _up_codes(bq, gpu), _up_scales_colmajor(br, gpu),
                                        b_block=b_block, out_dtype=dt, bias=bias_d)
    nob = fp8.fp8_scaled_gemm_blockwise(_up_codes(aq, gpu), _up_scales_colmajor(ar, gpu),
                                        _up_codes(bq, gpu), _up_scales_colmajor(br, gpu),
                                        b_block=b_block, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, M - 1, rng.integers(0, M, 24)])
    ref, S = gemm.blockwise_gemm(aq[rows], ar[rows], bq, br, b_block, with_bound=True)
    refb = gemm.add_bias(ref, bias)
    Sb = S + np.abs(e4m3.bf16_bits_to_f32(bias).astype(np.float64))[None, :]
    check_gemm_output(host_f32(out)[rows], refb, Sb, K // 128, od, f"bias {mnk}")
    if od == "f32":
        # the bias is one fp32 add on the unbiased fp32 result
        expect = host_f32(nob) + e4m3.bf16_bits_to_f32(bias)[None, :]
        assert np.array_equal(host_f32(out), expect.astype(np.float32))


@pytest.mark.parametrize("mnk,od", [((256, 4096, 1024), "bf16"), ((16, 32, 32), "f32")])
def test_tensorwise_bias_epilogue(gpu, mnk, od):
    M, N, K = mnk
    x = bits(inputs.randn_bf16((M, K), seed=inputs.tensor_seed(33, "x")))
    w = bits(inputs.randn_bf16((N, K), seed=inputs.tensor_seed(33, "w")))
    xq, xr = quant.quant_tensorwise(x)
    wq, wr = quant.quant_tensorwise(w)
    bias = e4m3.f32_to_bf16_bits(np.random.default_rng(N).normal(0, 8, N).astype(np.float32))
    dt = torch.bfloat16 if od == "bf16" else torch.float32
    say("gemm tensorwise bias", mnk, od)
    out = fp8.fp8_scaled_gemm_tensorwise(
        _up_codes(xq, gpu), torch.tensor([xr], device=gpu), _up_codes(wq, gpu),
        torch.tensor([wr], device=gpu), out_dtype=dt,
        bias=torch.from_numpy(bias.view(np.int16)).view(torch.bfloat16).to(gpu))
    torch.cuda.synchronize()
    ref = gemm.add_bias(gemm.tensorwise_gemm(xq, xr, wq, wr), bias)
    S = gemm.tensorwise_bound(xq, xr, wq, wr) + np.abs(e4m3.bf16_bits_to_f32(bias))[None, :]
    check_gemm_output(host_f32(out), ref, S, -(-K // 128), od, f"tensorwise bias {mnk}")


@pytest.mark.parametrize("shape", ["persistent_leftover", "ragged_small_tiles", "whole_split"])
def test_bf16_output_is_rne_of_the_fp32_output(gpu, shape):
    """Every bf16 store path rounds its fp32 value to nearest even: the bf16
    output of a GEMM equals, bit for bit on every element, the host's RNE of
    the fp32 output of the same GEMM (same plan, same accumulation order):
    the persistent launch's staged epilogue and its leftover tiles' reduce,
    the small-tile kernel's direct stores at ragged edges, and the
    whole-problem split-K reduce."""
    cus = torch.cuda.get_device_properties(gpu).multi_processor_count
    M, N, K = {"persistent_leftover": (4352, 32 * cus, 2048),
               "ragged_small_tiles": (300, 200, 512),
               "whole_split": (512, 512, 16384)}[shape]
    kb = K // 128
    rng = np.random.default_rng(70 + len(shape))
    aq, bq = _random_codes(rng, (M, K)), _random_codes(rng, (N, K))
    ar = rng.uniform(0.01, 0.02, (M, kb)).astype(np.float32)
    br = rng.uniform(0.01, 0.02, (-(-N // 128), kb)).astype(np.float32)
    a_d, b_d = _up_codes(aq, gpu), _up_codes(bq, gpu)
    ra_d, rb_d = _up_scales_colmajor(ar, gpu), _up_scales_colmajor(br, gpu)
    say("bf16 = RNE(fp32)", shape, M, N, K, fp8.gemm_plan(M, N, K))
    outs = {}
    for od in (torch.float32, torch.bfloat16):
        outs[od] = fp8.fp8_scaled_gemm_blockwise(a_d, ra_d, b_d, rb_d, "128x128", out_dtype=od)
    torch.cuda.synchronize()
    want = e4m3.f32_to_bf16_bits(outs[torch.float32].cpu().numpy())
    got = outs[torch.bfloat16].cpu().view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, (f"{shape}: {bad[0].size} bf16 outputs differ from RNE of the fp32 "
                              f"output, first at {tuple(b[0] for b in bad)}")
