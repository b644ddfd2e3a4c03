"""GPU parity of the FP8 linear wrapper (quantize + blockwise GEMM, all on the
GPU, through the C ABI) against the oracle's composition."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_amd as fp8
from oracle import e4m3, gemm, linear, metrics, quant
from synth import inputs
from tests.gpu_util import bits, check_gemm_output, host_f32, say

pytestmark = pytest.mark.gpu


def _inputs(M, N, K, seed, device):
    x = inputs.randn_bf16((M, K), seed=inputs.tensor_seed(seed, "x"), device=device)
    w = inputs.linear_weight_bf16(N, K, seed=inputs.tensor_seed(seed, "w"), device=device)
    dy = inputs.randn_bf16((M, N), seed=inputs.tensor_seed(seed, "dy"), device=device)
    return x, w, dy


@pytest.mark.parametrize("mnk", [(128, 256, 512), (256, 384, 640), (384, 128, 256), (128, 128, 128)])
def test_linear_full_compare(gpu, mnk):
    M, N, K = mnk
    x, w, dy = _inputs(M, N, K, seed=1, device="cpu")
    xb, wb, dyb = bits(x), bits(w), bits(dy)
    xd, wd, dyd = x.to(gpu), w.to(gpu), dy.to(gpu)
    say("linear fwd", mnk)
    y = fp8.fp8_linear_fwd(xd, wd)
    torch.cuda.synchronize()
    ref, S = linear.fwd(xb, wb, with_bound=True)
    check_gemm_output(host_f32(y), ref, S, K // 128, "bf16", f"fwd {mnk}")
    say("linear dgrad", mnk)
    dx = fp8.fp8_linear_dgrad(dyd, wd)
    torch.cuda.synchronize()
    ref, S = linear.dgrad(dyb, wb, with_bound=True)
    check_gemm_output(host_f32(dx), ref, S, N // 128, "bf16", f"dgrad {mnk}")
    say("linear wgrad", mnk)
    dw = fp8.fp8_linear_wgrad(dyd, xd)
    torch.cuda.synchronize()
    ref, S = linear.wgrad(dyb, xb, with_bound=True)
    check_gemm_output(host_f32(dw), ref, S, M // 128, "bf16", f"wgrad {mnk}")


def _idx(t, rows=None, cols=None):
    if rows is not None:
        t = t[torch.from_numpy(rows).to(t.device)]
    if cols is not None:
        t = t[:, torch.from_numpy(cols).to(t.device)]
    return bits(t)


@pytest.mark.parametrize("mnk", [(16640, 5120, 8192), (16640, 8192, 5120)])
def test_linear_llama4_shapes_sampled(gpu, mnk):
    """Full-size fwd, dgrad and wgrad at the llama4 shapes; outputs checked
    on sampled rows x two 128-column blocks, which the oracle computes from
    the same bf16 inputs; SQNR of the sample vs the fp32 product in band."""
    M, N, K = mnk
    say("llama4 generate", mnk)
    x, w, dy = _inputs(M, N, K, seed=2, device="cuda")
    rng = np.random.default_rng(M + N)
    # random rows plus rows of the last row-block of tiles (where leftover
    # tiles of a partial last round are computed split-K)
    rows = np.unique(np.r_[rng.choice(M, 12, replace=False), M - 1, M - 77, M - 200, M - 256])
    say("llama4 fwd", mnk)
    y = fp8.fp8_linear_fwd(x, w)
    torch.cuda.synchronize()
    ncols = np.r_[np.arange(0, 128), np.arange(N - 128, N)]
    xs, ws = _idx(x, rows=rows), _idx(w, rows=ncols)
    ref, S = gemm.blockwise_gemm(*quant.quant_1x128(xs), *quant.quant_128x128(ws), "128x128",
                                 with_bound=True)
    got = host_f32(y)[np.ix_(rows, ncols)]
    check_gemm_output(got, ref, S, K // 128, "bf16", f"fwd {mnk}")
    assert 27.5 < metrics.sqnr_db(gemm.fp32_reference(xs, ws), got) < 32.5
    del y
    say("llama4 dgrad", mnk)
    dx = fp8.fp8_linear_dgrad(dy, w)
    torch.cuda.synchronize()
    kcols = np.r_[np.arange(128, 256), np.arange(K - 128, K)]
    dys = _idx(dy, rows=rows)
    wcols = _idx(w, cols=kcols)                    # W[:, kcols] -> [N, 256]
    ref, S = gemm.blockwise_gemm(*quant.quant_1x128(dys), *quant.quant_128x128_transposed(wcols),
                                 "128x128", with_bound=True)
    got = host_f32(dx)[np.ix_(rows, kcols)]
    check_gemm_output(got, ref, S, N // 128, "bf16", f"dgrad {mnk}")
    del dx
    say("llama4 wgrad", mnk)
    dw = fp8.fp8_linear_wgrad(dy, x)
    torch.cuda.synchronize()
    nrows = np.unique(np.r_[rng.choice(N, 12, replace=False), N - 1, N - 100, N - 255])
    dycols = _idx(dy, cols=nrows)                  # dY[:, n] -> [M, 16]
    xcols = _idx(x, cols=kcols)                    # X[:, k]  -> [M, 256]
    ref, S = gemm.blockwise_gemm(*quant.quant_1x128_along_rows(dycols),
                                 *quant.quant_1x128_along_rows(xcols), "1x128", with_bound=True)
    got = host_f32(dw)[np.ix_(nrows, kcols)]
    check_gemm_output(got, ref, S, M // 128, "bf16", f"wgrad {mnk}")
    fp32 = (e4m3.bf16_bits_to_f32(dycols).astype(np.float64).T
            @ e4m3.bf16_bits_to_f32(xcols).astype(np.float64))
    assert 27.5 < metrics.sqnr_db(fp32, got) < 32.5


def test_linear_shared_workspace_reuse(gpu):
    """One workspace reused across fwd, dgrad and wgrad calls in a row."""
    M, N, K = 256, 256, 384
    x, w, dy = _inputs(M, N, K, seed=3, device="cpu")
    need = max(fp8.load_library().fp8bw_linear_ws_bytes(M, N, K, i) for i in range(3))
    ws = torch.empty(need, dtype=torch.uint8, device=gpu)
    say("linear workspace reuse")
    y = fp8.fp8_linear_fwd(x.to(gpu), w.to(gpu), ws=ws)
    dx = fp8.fp8_linear_dgrad(dy.to(gpu), w.to(gpu), ws=ws)
    dw = fp8.fp8_linear_wgrad(dy.to(gpu), x.to(gpu), ws=ws)
    torch.cuda.synchronize()
    for got, (ref, S), kb, name in (
            (y, linear.fwd(bits(x), bits(w), True), K // 128, "fwd"),
            (dx, linear.dgrad(bits(dy), bits(w), True), N // 128, "dgrad"),
            (dw, linear.wgrad(bits(dy), bits(x), True), M // 128, "wgrad")):
        check_gemm_output(host_f32(got), ref, S, kb, "bf16", name)


@pytest.mark.parametrize("mnk", [(384, 256, 640), (16640, 5120, 8192), (16640, 8192, 5120)])
def test_fused_quant_linear_matches_separate(gpu, mnk):
    """fp8_linear_fwd_save + fp8_linear_bwd (X and dY each quantized once
    into both layouts, W^T quantized by the backward) give bit-identical Y, dX and dW to the three separate
    entry points, whose results the tests above check against the oracle;
    a skipped gradient leaves the other unchanged."""
    M, N, K = mnk
    say("fused linear", mnk)
    x, w, dy = _inputs(M, N, K, seed=5, device=gpu)
    y_ref = fp8.fp8_linear_fwd(x, w)
    dx_ref = fp8.fp8_linear_dgrad(dy, w)
    dw_ref = fp8.fp8_linear_wgrad(dy, x)
    y, saved = fp8.fp8_linear_fwd_save(x, w)
    dx, dw = fp8.fp8_linear_bwd(dy, w, saved)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref), "fused fwd differs from fp8_linear_fwd"
    assert torch.equal(dx, dx_ref), "fused dgrad differs from fp8_linear_dgrad"
    assert torch.equal(dw, dw_ref), "fused wgrad differs from fp8_linear_wgrad"
    dx2, none_dw = fp8.fp8_linear_bwd(dy, w, saved, need_dx=True, need_dw=False)
    none_dx, dw2 = fp8.fp8_linear_bwd(dy, w, saved, need_dx=False, need_dw=True)
    torch.cuda.synchronize()
    assert none_dw is None and none_dx is None
    assert torch.equal(dx2, dx_ref) and torch.equal(dw2, dw_ref)


def test_fused_linear_canaries(gpu):
    """fp8_linear_fwd_save / fp8_linear_bwd through the C ABI with the saved
    buffer, the workspaces and the outputs placed in canary-filled buffers
    larger than the sizes passed: nothing past the stated sizes is written,
    and the results equal the binding's bit for bit."""
    from blockwise_scaled_fp8_amd._lib import check
    lib = fp8.load_library()
    M, N, K = 384, 256, 640
    x, w, dy = (t.to(gpu) for t in _inputs(M, N, K, seed=9, device="cpu"))
    pad = 4096
    saved_bytes = lib.fp8bw_linear_saved_bytes(M, N, K)
    ws_f, ws_b = lib.fp8bw_linear_ws_bytes(M, N, K, 3), lib.fp8bw_linear_ws_bytes(M, N, K, 4)
    canary = 0xA5

    def u8(n):
        return torch.full((n + pad,), canary, dtype=torch.uint8, device=gpu)

    saved, wsf, wsb = u8(saved_bytes), u8(ws_f), u8(ws_b)
    yb, dxb, dwb = u8(2 * M * N), u8(2 * M * K), u8(2 * N * K)
    stream = torch.cuda.current_stream().cuda_stream
    say("fused linear canaries")
    check(lib.fp8_linear_fwd_save(x.data_ptr(), w.data_ptr(), yb.data_ptr(), M, N, K,
                                  saved.data_ptr(), saved_bytes, wsf.data_ptr(), ws_f, stream))
    check(lib.fp8_linear_bwd(dy.data_ptr(), w.data_ptr(), saved.data_ptr(), saved_bytes,
                             dxb.data_ptr(), dwb.data_ptr(), M, N, K, wsb.data_ptr(), ws_b, stream))
    y_ref, saved_ref = fp8.fp8_linear_fwd_save(x, w)
    dx_ref, dw_ref = fp8.fp8_linear_bwd(dy, w, saved_ref)
    torch.cuda.synchronize()
    for buf, n, name in ((saved, saved_bytes, "saved"), (wsf, ws_f, "fwd workspace"),
                         (wsb, ws_b, "bwd workspace"), (yb, 2 * M * N, "y"),
                         (dxb, 2 * M * K, "dx"), (dwb, 2 * N * K, "dw")):
        assert bool((buf[n:] == canary).all()), f"{name}: bytes past its size were written"
    for buf, ref, name in ((yb, y_ref, "y"), (dxb, dx_ref, "dx"), (dwb, dw_ref, "dw")):
        got = buf[: ref.numel() * 2].view(torch.int16).view(ref.shape)
        assert torch.equal(got, ref.view(torch.int16)), f"{name} differs from the binding's"


@pytest.mark.parametrize("mnk", [(208, 256, 384), (16, 128, 128)])
def test_fused_forward_ragged_tokens(gpu, mnk):
    """fp8_linear_fwd_save takes a token count that is not a multiple of 128
    (its saved X^T codes end in a partial 1x128 block along M): Y equals
    fp8_linear_fwd's bit for bit, and the backward, whose weight gradient
    contracts over tokens in 128-blocks, refuses the shape before launching."""
    M, N, K = mnk
    x, w, dy = (t.to(gpu) for t in _inputs(M, N, K, seed=11, device="cpu"))
    say("fused forward ragged", mnk)
    y, saved = fp8.fp8_linear_fwd_save(x, w)
    y_ref = fp8.fp8_linear_fwd(x, w)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    with pytest.raises(fp8.FP8BWError, match="multiples of 128"):
        fp8.fp8_linear_bwd(dy, w, saved)


@pytest.mark.parametrize("mnk", [(384, 256, 640), (16640, 5120, 8192)])
def test_bench_step_is_the_training_pair(gpu, mnk):
    """The launches bench.py times one by one as the step (its step plan)
    produce exactly what fp8_linear_fwd_save + fp8_linear_bwd produce: the
    timed sequence is the training pair, call for call."""
    import bench
    M, N, K = mnk
    say("bench step plan vs training pair", mnk)
    wl = bench.Workload(3, gpu, shape=(M, N, K))
    for _, fn, _, _ in bench.step_plan_dual(wl):
        fn()
    y, saved = fp8.fp8_linear_fwd_save(wl.x, wl.w)
    dx, dw = fp8.fp8_linear_bwd(wl.dy, wl.w, saved)
    torch.cuda.synchronize()
    for got, ref, name in ((wl.y, y, "Y"), (wl.dx, dx, "dX"), (wl.dw, dw, "dW")):
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{name} {mnk} differs"
