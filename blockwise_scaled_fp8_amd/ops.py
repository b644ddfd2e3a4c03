"""Thin torch-facing binding of the C ABI: the same entry-point names as
include/fp8bw.h.  Each function only checks tensor placement, allocates its
outputs with torch (device memory is plumbing), passes raw pointers, sizes and
the current HIP stream, and raises FP8BWError on a non-OK status.  Every step
of the computation runs in the HIP kernels of libfp8bw.so."""

import functools

import torch

from ._lib import check, load_library

BLOCKS = {"1x128": 0, "128x128": 1}
OUT_DTYPES = {torch.bfloat16: 0, torch.float32: 1}


def _stream(t):
    # the raw handle of torch's current stream on t's device (the direct C
    # accessor: torch.cuda.current_stream(device) costs microseconds per call)
    return torch._C._cuda_getCurrentRawStream(t.device.index)


def _need_cuda(*ts):
    for t in ts:
        if not (isinstance(t, torch.Tensor) and t.is_cuda):
            raise ValueError("fp8bw ops take CUDA (HIP) tensors")


def _on_tensor_device(fn):
    """Every tensor argument (inputs and caller-provided outputs or
    workspace) must be a HIP tensor on one device; that device is made
    current for the call, so the library's launches, its per-device queries
    and the stream all refer to the device that holds the data."""
    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        dev = None
        for t in list(args) + list(kwargs.values()):
            if not isinstance(t, torch.Tensor):
                continue
            if not t.is_cuda:
                raise ValueError("fp8bw ops take CUDA (HIP) tensors")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"fp8bw ops take tensors on one device ({dev} and {t.device} given)")
        if dev is None or dev.index == torch._C._cuda_getDevice():
            return fn(*args, **kwargs)
        with torch.cuda.device(dev):
            return fn(*args, **kwargs)
    return wrapper


def _rowmajor(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")


def _cdiv(a, b):
    return (a + b - 1) // b


def scale_grid(rows, cols, block, transpose):
    """Logical shape (ni, nj) of the reciprocal-scale tensor."""
    if block == "1x128":
        return (cols, _cdiv(rows, 128)) if transpose else (rows, _cdiv(cols, 128))
    return (_cdiv(cols, 128), _cdiv(rows, 128)) if transpose else (_cdiv(rows, 128), _cdiv(cols, 128))


def colmajor_empty(ni, nj, device):
    """fp32 [ni, nj] with column-major strides (1, ni)."""
    return torch.empty((nj, max(ni, 1)), dtype=torch.float32, device=device)[:, :ni].t()


def _check_codes(a, b, K):
    for t in (a, b):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise ValueError("GEMM operands are E4M3 codes (uint8 or float8_e4m3fn)")
    if b.shape[1] != K:
        raise ValueError(f"b has K={b.shape[1]}, a has K={K}")


def _check_shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


CODE_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def _check_codes_out(t, shape, name):
    """A caller-provided code buffer: E4M3 bytes, row-major rows."""
    _check_shape(t, shape, name)
    if t.dtype not in CODE_DTYPES:
        raise ValueError(f"{name} must be uint8 or float8_e4m3fn, got {t.dtype}")
    _rowmajor(t, name)


def _check_scales(t, shape, name):
    """fp32 reciprocal scales of a given logical shape (any strides; the
    library checks that they do not overlap)."""
    _check_shape(t, shape, name)
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32, got {t.dtype}")


def _check_out(t, shape, name="out"):
    _check_shape(t, shape, name)
    if t.dtype not in OUT_DTYPES:
        raise ValueError(f"{name} must be bfloat16 or float32, got {t.dtype}")
    _rowmajor(t, name)


@_on_tensor_device
def fp8_blockwise_quant(x, block="1x128", transpose=False, q=None, recip=None):
    """Quantize bf16 x[rows, cols] to E4M3 codes with per-block reciprocal scales.

    Returns (q, recip): q uint8 [rows, cols] (or [cols, rows] with transpose),
    recip fp32 [ni, nj] (column-major unless a tensor is passed in)."""
    lib = load_library()
    _need_cuda(x)
    _rowmajor(x, "x")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16")
    rows, cols = x.shape
    qshape = (cols, rows) if transpose else (rows, cols)
    if q is None:
        q = torch.empty(qshape, dtype=torch.uint8, device=x.device)
    _check_codes_out(q, qshape, "q")
    ni, nj = scale_grid(rows, cols, block, transpose)
    if recip is None:
        recip = colmajor_empty(ni, nj, x.device)
    _check_scales(recip, (ni, nj), "recip")
    check(lib.fp8_blockwise_quant(x.data_ptr(), rows, cols, x.stride(0), BLOCKS[block],
                                  int(bool(transpose)), q.data_ptr(), q.stride(0),
                                  recip.data_ptr(), recip.stride(0), recip.stride(1), _stream(x)))
    return q, recip


@_on_tensor_device
def fp8_blockwise_quant_dual(x, block="1x128", q=None, recip=None, qt=None, recip_t=None,
                             stream_t=False):
    """Both layouts from one read of x: returns (q, recip, qt, recip_t), equal
    to fp8_blockwise_quant(x, block) and fp8_blockwise_quant(x, block,
    transpose=True).  stream_t writes qt with nontemporal stores (codes read
    only much later; the same bits)."""
    lib = load_library()
    _need_cuda(x)
    _rowmajor(x, "x")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16")
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if qt is None:
        qt = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    _check_codes_out(q, (rows, cols), "q")
    _check_codes_out(qt, (cols, rows), "qt")
    ni, nj = scale_grid(rows, cols, block, False)
    ti, tj = scale_grid(rows, cols, block, True)
    if recip is None:
        recip = colmajor_empty(ni, nj, x.device)
    if recip_t is None:
        recip_t = colmajor_empty(ti, tj, x.device)
    _check_scales(recip, (ni, nj), "recip")
    _check_scales(recip_t, (ti, tj), "recip_t")
    check(lib.fp8_blockwise_quant_dual(x.data_ptr(), rows, cols, x.stride(0), BLOCKS[block],
                                       q.data_ptr(), q.stride(0), recip.data_ptr(), recip.stride(0),
                                       recip.stride(1), qt.data_ptr(), qt.stride(0),
                                       recip_t.data_ptr(), recip_t.stride(0), recip_t.stride(1),
                                       1 if stream_t else 0, _stream(x)))
    return q, recip, qt, recip_t


@_on_tensor_device
def fp8_tensorwise_quant(x, q=None, recip=None):
    """Per-tensor quantization: (q uint8 like x, recip fp32 [1] on device)."""
    lib = load_library()
    _need_cuda(x)
    _rowmajor(x, "x")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16")
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    _check_codes_out(q, (rows, cols), "q")
    if recip is None:
        recip = torch.empty(1, dtype=torch.float32, device=x.device)
    if recip.numel() != 1 or recip.dtype != torch.float32:
        raise ValueError("recip must be a one-element float32 tensor")
    nws = lib.fp8bw_tensorwise_quant_ws_bytes(rows, cols)
    ws = torch.empty(nws, dtype=torch.uint8, device=x.device)
    check(lib.fp8_tensorwise_quant(x.data_ptr(), rows, cols, x.stride(0), q.data_ptr(), q.stride(0),
                                   recip.data_ptr(), ws.data_ptr(), nws, _stream(x)))
    return q, recip


@_on_tensor_device
def fp8_tensorwise_quant_noalloc(x, q, recip):
    """fp8_tensorwise_quant with no workspace: the library keeps the partial
    amaxes in its own per-device array.  q (uint8 like x) and recip (fp32
    [1]) are the caller's; nothing is allocated here or in the library."""
    lib = load_library()
    _need_cuda(x)
    _rowmajor(x, "x")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16")
    rows, cols = x.shape
    _check_codes_out(q, (rows, cols), "q")
    if recip.numel() != 1 or recip.dtype != torch.float32:
        raise ValueError("recip must be a one-element float32 tensor")
    check(lib.fp8_tensorwise_quant_noalloc(x.data_ptr(), rows, cols, x.stride(0), q.data_ptr(),
                                           q.stride(0), recip.data_ptr(), _stream(x)))
    return q, recip


def _check_bias(bias, N, device):
    if bias is None:
        return
    if bias.dtype != torch.bfloat16 or bias.dim() != 1 or bias.shape[0] != N or bias.stride(0) != 1:
        raise ValueError(f"bias must be a contiguous bf16 [{N}] tensor")
    if bias.device != device:
        raise ValueError("bias must be on the GEMM's device")


@_on_tensor_device
def fp8_scaled_gemm_blockwise(a, ra, b, rb, b_block="128x128", out_dtype=torch.bfloat16,
                              out=None, config=None, splits=None, bias=None):
    """out[M, N] = blockwise-scaled A . B^T (see include/fp8bw.h).

    a uint8 [M, K], ra fp32 [M, K/128] (column-major), b uint8 [N, K], rb fp32
    [N/128 or N, K/128].  config/splits force a tile configuration / split-K
    count (None = built-in choice)."""
    lib = load_library()
    _need_cuda(a, b, ra, rb)
    _rowmajor(a, "a")
    _rowmajor(b, "b")
    M, K = a.shape
    N = b.shape[0]
    _check_codes(a, b, K)
    kb = _cdiv(K, 128)
    if b_block not in BLOCKS:
        raise ValueError(f"b_block must be one of {sorted(BLOCKS)}")
    _check_scales(ra, (M, kb), "ra")
    _check_scales(rb, (N if b_block == "1x128" else _cdiv(N, 128), kb), "rb")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _check_out(out, (M, N))
    args = (a.data_ptr(), a.stride(0), ra.data_ptr(), ra.stride(0), ra.stride(1),
            b.data_ptr(), b.stride(0), rb.data_ptr(), rb.stride(0), rb.stride(1),
            BLOCKS[b_block], M, N, K, out.data_ptr(), out.stride(0), OUT_DTYPES[out.dtype])
    _check_bias(bias, N, a.device)
    if bias is not None:
        if config is not None or splits is not None:
            raise ValueError("bias is not combined with a forced config/splits")
        nws = lib.fp8bw_gemm_blockwise_ws_bytes(M, N, K)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=a.device)
        check(lib.fp8_scaled_gemm_blockwise_bias(*args[:14], bias.data_ptr(), *args[14:],
                                                 ws.data_ptr(), nws, _stream(a)))
        return out
    if config is None and splits is None:
        nws = lib.fp8bw_gemm_blockwise_ws_bytes(M, N, K)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=a.device)
        check(lib.fp8_scaled_gemm_blockwise(*args, ws.data_ptr(), nws, _stream(a)))
    else:
        s = 0 if splits is None else int(splits)
        if s > 0:
            nws = lib.fp8bw_gemm_ws_bytes_for_split(M, N, s)
        else:
            nws = lib.fp8bw_gemm_blockwise_ws_bytes(M, N, K)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=a.device)
        check(lib.fp8_scaled_gemm_blockwise_cfg(*args, -1 if config is None else int(config), s,
                                                ws.data_ptr(), nws, _stream(a)))
    return out


@_on_tensor_device
def fp8_scaled_gemm_blockwise_kn(a, ra, b_kn, rb, b_block="128x128", out_dtype=torch.bfloat16,
                                 out=None):
    """out[M, N] = blockwise-scaled A . B with B given in [K, N] layout
    (N contiguous), e.g. a weight's codes W [N_w, K_w] used as the B of
    dX = dY . W without a transposed copy (see include/fp8bw.h).

    a uint8 [M, K], ra fp32 [M, K/128], b_kn uint8 [K, N], rb fp32
    [N/128 or N, K/128] indexed by (output column block, K block)."""
    lib = load_library()
    _need_cuda(a, b_kn, ra, rb)
    _rowmajor(a, "a")
    _rowmajor(b_kn, "b_kn")
    M, K = a.shape
    if b_kn.dim() != 2 or b_kn.shape[0] != K:
        raise ValueError(f"b_kn must be [K={K}, N]")
    N = b_kn.shape[1]
    _check_codes(a, b_kn.t(), K)
    kb = _cdiv(K, 128)
    if b_block not in BLOCKS:
        raise ValueError(f"b_block must be one of {sorted(BLOCKS)}")
    _check_scales(ra, (M, kb), "ra")
    _check_scales(rb, (N if b_block == "1x128" else _cdiv(N, 128), kb), "rb")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _check_out(out, (M, N))
    nws = lib.fp8bw_gemm_blockwise_ws_bytes(M, N, K)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=a.device)
    check(lib.fp8_scaled_gemm_blockwise_kn(
        a.data_ptr(), a.stride(0), ra.data_ptr(), ra.stride(0), ra.stride(1), b_kn.data_ptr(),
        b_kn.stride(0), rb.data_ptr(), rb.stride(0), rb.stride(1), BLOCKS[b_block], M, N, K,
        out.data_ptr(), out.stride(0), OUT_DTYPES[out.dtype], ws.data_ptr(), nws, _stream(a)))
    return out


def fp8bw_gemm_num_configs():
    return load_library().fp8bw_gemm_num_configs()


def gemm_plan(M, N, K, b_block="128x128"):
    """How the library runs an M x N x K blockwise GEMM (contiguous operands,
    column-major scales) on the current device: tile configuration,
    whole-problem split count, leftover-tile split count, tiles, tiles run
    unsplit and workspace bytes."""
    import ctypes
    info = (ctypes.c_int64 * 6)()
    check(load_library().fp8bw_gemm_blockwise_plan(M, N, K, BLOCKS[b_block], info))
    keys = ("config", "splits", "tail_splits", "tiles", "tiles_full", "ws_bytes")
    return dict(zip(keys, (int(v) for v in info)))


@_on_tensor_device
def fp8_scaled_gemm_tensorwise(a, ra, b, rb, out_dtype=torch.bfloat16, out=None, bias=None):
    """out[M, N] = (A . B^T) * ra * rb with one-element device scales."""
    lib = load_library()
    _need_cuda(a, b, ra, rb)
    _rowmajor(a, "a")
    _rowmajor(b, "b")
    M, K = a.shape
    N = b.shape[0]
    _check_codes(a, b, K)
    if ra.numel() != 1 or rb.numel() != 1:
        raise ValueError("tensorwise scales are one-element tensors")
    if ra.dtype != torch.float32 or rb.dtype != torch.float32:
        raise ValueError("tensorwise scales are float32")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _check_out(out, (M, N))
    _check_bias(bias, N, a.device)
    if bias is not None:
        check(lib.fp8_scaled_gemm_tensorwise_bias(a.data_ptr(), a.stride(0), ra.data_ptr(),
                                                  b.data_ptr(), b.stride(0), rb.data_ptr(), M, N, K,
                                                  bias.data_ptr(), out.data_ptr(), out.stride(0),
                                                  OUT_DTYPES[out.dtype], _stream(a)))
        return out
    check(lib.fp8_scaled_gemm_tensorwise(a.data_ptr(), a.stride(0), ra.data_ptr(), b.data_ptr(),
                                         b.stride(0), rb.data_ptr(), M, N, K, out.data_ptr(),
                                         out.stride(0), OUT_DTYPES[out.dtype], _stream(a)))
    return out


@_on_tensor_device
def fp8_scaled_grouped_gemm_blockwise(a, ra, b, rb, group_end, out_dtype=torch.bfloat16, out=None):
    """Grouped blockwise GEMM: rows [group_end[g-1], group_end[g]) of a
    (uint8 [M, K], ra fp32 [M, K/128] column-major) times b[g]^T (uint8
    [G, N, K], rb fp32 [G, N/128, K/128], any strides) -> out [M, N].
    group_end: device int32 [G], cumulative."""
    lib = load_library()
    _need_cuda(a, b, ra, rb, group_end)
    _rowmajor(a, "a")
    M, K = a.shape
    if b.dim() != 3 or b.shape[2] != K or b.stride(2) != 1:
        raise ValueError("b must be uint8 [G, N, K] with contiguous rows")
    G, N = b.shape[0], b.shape[1]
    if a.dtype != torch.uint8 or b.dtype != torch.uint8:
        raise ValueError("codes are uint8 tensors")
    kb = _cdiv(K, 128)
    _check_scales(ra, (M, kb), "ra")
    if ra.stride(0) != 1 and M > 1:
        raise ValueError("ra of the grouped GEMM must be column-major (unit row stride)")
    _check_scales(rb, (G, _cdiv(N, 128), kb), "rb")
    if group_end.dtype != torch.int32 or group_end.shape != (G,) or group_end.stride(0) != 1:
        raise ValueError("group_end must be a contiguous int32 [G] tensor")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _check_out(out, (M, N))
    check(lib.fp8_scaled_grouped_gemm_blockwise(
        a.data_ptr(), a.stride(0), ra.data_ptr(), ra.stride(1), b.data_ptr(), b.stride(1),
        b.stride(0), rb.data_ptr(), rb.stride(1), rb.stride(2), rb.stride(0), G,
        group_end.data_ptr(), M, N, K, out.data_ptr(), out.stride(0), OUT_DTYPES[out.dtype],
        _stream(a)))
    return out


def linear_saved_bytes(M, N, K):
    """Bytes of the buffer fp8_linear_fwd_save fills for fp8_linear_bwd."""
    return load_library().fp8bw_linear_saved_bytes(M, N, K)


def linear_workspace(M, N, K, which, device):
    n = load_library().fp8bw_linear_ws_bytes(M, N, K, which)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _linear(name, which, p0, p1, out_shape, M, N, K, ws):
    lib = load_library()
    _need_cuda(p0, p1)
    if not (p0.is_contiguous() and p1.is_contiguous()):
        raise ValueError("linear inputs must be contiguous")
    out = torch.empty(out_shape, dtype=torch.bfloat16, device=p0.device)
    if ws is None:
        ws = linear_workspace(M, N, K, which, p0.device)
    check(getattr(lib, name)(p0.data_ptr(), p1.data_ptr(), out.data_ptr(), M, N, K,
                             ws.data_ptr(), ws.numel(), _stream(p0)))
    return out


def _bf16_2d(*ts):
    for t in ts:
        if t.dim() != 2 or t.dtype != torch.bfloat16:
            raise ValueError("linear inputs are 2-D bf16 tensors")


@_on_tensor_device
def fp8_linear_fwd(x, w, ws=None):
    """Y[M, N] = X . W^T (X 1x128, W 128x128), bf16."""
    _bf16_2d(x, w)
    M, K = x.shape
    N = w.shape[0]
    _check_shape(w, (N, K), "w")
    return _linear("fp8_linear_fwd", 0, x, w, (M, N), M, N, K, ws)


@_on_tensor_device
def fp8_linear_dgrad(dy, w, ws=None):
    """dX[M, K] = dY . W (dY 1x128, W^T 128x128), bf16."""
    _bf16_2d(dy, w)
    M, N = dy.shape
    K = w.shape[1]
    _check_shape(w, (N, K), "w")
    return _linear("fp8_linear_dgrad", 1, dy, w, (M, K), M, N, K, ws)


@_on_tensor_device
def fp8_linear_fwd_save(x, w, ws=None):
    """Y[M, N] = X . W^T with fused quantization: returns (Y, saved), where
    saved (uint8, device) holds the X^T codes and scales that fp8_linear_bwd
    needs (see include/fp8bw.h)."""
    _bf16_2d(x, w)
    M, K = x.shape
    N = w.shape[0]
    _check_shape(w, (N, K), "w")
    lib = load_library()
    _need_cuda(x, w)
    if not (x.is_contiguous() and w.is_contiguous()):
        raise ValueError("linear inputs must be contiguous")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    saved = torch.empty(max(linear_saved_bytes(M, N, K), 1), dtype=torch.uint8, device=x.device)
    if ws is None:
        ws = linear_workspace(M, N, K, 3, x.device)
    check(lib.fp8_linear_fwd_save(x.data_ptr(), w.data_ptr(), y.data_ptr(), M, N, K,
                                  saved.data_ptr(), saved.numel(), ws.data_ptr(), ws.numel(),
                                  _stream(x)))
    return y, saved


@_on_tensor_device
def fp8_linear_bwd(dy, w, saved, need_dx=True, need_dw=True, ws=None):
    """(dX[M, K], dW[N, K]) from dY[M, N], the forward's bf16 W[N, K] and
    the saved buffer of fp8_linear_fwd_save (dY quantized once, W^T right
    before the dgrad GEMM); a gradient not needed is None."""
    _bf16_2d(dy, w)
    M, N = dy.shape
    K = w.shape[1]
    _check_shape(w, (N, K), "w")
    lib = load_library()
    _need_cuda(dy, w, saved)
    if not (dy.is_contiguous() and w.is_contiguous()):
        raise ValueError("dy and w must be contiguous")
    if saved.dtype != torch.uint8 or saved.dim() != 1:
        raise ValueError("saved must be the 1-D uint8 buffer from fp8_linear_fwd_save")
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dy.device) if need_dx else None
    dw = torch.empty((N, K), dtype=torch.bfloat16, device=dy.device) if need_dw else None
    if ws is None:
        ws = linear_workspace(M, N, K, 4, dy.device)
    check(lib.fp8_linear_bwd(dy.data_ptr(), w.data_ptr(), saved.data_ptr(), saved.numel(),
                             dx.data_ptr() if dx is not None else None,
                             dw.data_ptr() if dw is not None else None, M, N, K, ws.data_ptr(),
                             ws.numel(), _stream(dy)))
    return dx, dw


@_on_tensor_device
def fp8_linear_wgrad(dy, x, ws=None):
    """dW[N, K] = dY^T . X (1x128 x 1x128 along M), bf16."""
    _bf16_2d(dy, x)
    M, N = dy.shape
    K = x.shape[1]
    _check_shape(x, (M, K), "x")
    return _linear("fp8_linear_wgrad", 2, dy, x, (N, K), M, N, K, ws)
