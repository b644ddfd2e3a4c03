"""C-ABI checks that need no GPU: the library loads, exports every function
include/fp8bw.h declares, and rejects invalid arguments on the host before
any HIP call.  No compute call is made here."""

import ctypes
import os
import re

import pytest

import blockwise_scaled_fp8_amd as fp8
from blockwise_scaled_fp8_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bw.h")

OK, NULL, SHAPE, LAYOUT, ALIGN, UNSUP, WS = 0, 1, 2, 3, 4, 5, 6
P = 0x10000  # a 256-byte aligned fake device address; never dereferenced here


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z0-9_]+)\s*\(", text)) - {"defined"})


@pytest.fixture(scope="module")
def lib():
    return fp8.load_library()


def test_library_exports_every_header_function(lib):
    names = header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.PROTOTYPES), "binding prototypes must mirror the header"


def test_abi_version_and_status_strings(lib):
    assert lib.fp8bw_abi_version() == 2
    for s, name in _lib.STATUS.items():
        assert lib.fp8bw_status_str(s).decode() == name
    assert lib.fp8bw_gemm_num_configs() >= 1


def _quant(lib, **kw):
    a = dict(x=P, rows=128, cols=256, ld_x=256, block=0, transpose=0, q=P, ld_q=256,
             recip=P, rs_row=1, rs_kb=128, stream=None)
    a.update(kw)
    return lib.fp8_blockwise_quant(a["x"], a["rows"], a["cols"], a["ld_x"], a["block"],
                                   a["transpose"], a["q"], a["ld_q"], a["recip"], a["rs_row"],
                                   a["rs_kb"], a["stream"])


def test_quant_validation(lib):
    assert _quant(lib, block=2) == UNSUP
    assert _quant(lib, transpose=2) == UNSUP
    assert _quant(lib, rows=-1) == SHAPE
    assert _quant(lib, cols=200) == SHAPE                 # not a multiple of 16
    assert _quant(lib, transpose=1, rows=100) == SHAPE    # transposed rows % 16
    assert _quant(lib, x=None) == NULL
    assert _quant(lib, recip=None) == NULL
    assert _quant(lib, x=P + 8) == ALIGN
    assert _quant(lib, ld_x=200) == LAYOUT
    assert _quant(lib, ld_x=260) == LAYOUT                # not a multiple of 8
    assert _quant(lib, ld_q=264) == LAYOUT                # not a multiple of 16
    assert _quant(lib, rs_row=1, rs_kb=64) == LAYOUT      # aliases rows
    assert _quant(lib, rs_row=-1) == LAYOUT
    assert "recip strides" in lib.fp8bw_last_error().decode()
    # zero-sized problems are accepted and enqueue nothing (no HIP call)
    assert _quant(lib, rows=0, x=None, q=None, recip=None) == OK
    assert _quant(lib, cols=0, x=None, q=None, recip=None) == OK


def _dual(lib, **kw):
    a = dict(x=P, rows=64, cols=256, ld_x=256, block=0, q=P, ld_q=256, recip=P, rs_row=1,
             rs_kb=64, qt=P + (1 << 20), ld_qt=64, recip_t=P, rst_row=1, rst_kb=256, stream_t=0,
             stream=None)
    a.update(kw)
    return lib.fp8_blockwise_quant_dual(*[a[k] for k in (
        "x", "rows", "cols", "ld_x", "block", "q", "ld_q", "recip", "rs_row", "rs_kb", "qt",
        "ld_qt", "recip_t", "rst_row", "rst_kb", "stream_t", "stream")])


def test_dual_quant_validation(lib):
    """Both outputs are validated as fp8_blockwise_quant validates each
    orientation; the two code buffers may not overlap."""
    assert _dual(lib, block=2) == UNSUP
    assert _dual(lib, rows=100, rs_kb=128) == SHAPE      # transposed output needs rows % 16
    assert _dual(lib, cols=200) == SHAPE
    assert _dual(lib, qt=None) == NULL
    assert _dual(lib, recip_t=None) == NULL
    assert _dual(lib, ld_qt=32) == LAYOUT                # qt rows hold `rows` codes
    assert _dual(lib, rows=256, rs_kb=256, ld_qt=256, rst_kb=8) == LAYOUT  # transposed scales alias
    assert _dual(lib, qt=P + 4096) == LAYOUT             # overlaps q
    assert "overlap" in lib.fp8bw_last_error().decode()
    assert _dual(lib, rows=0, x=None, q=None, qt=None, recip=None, recip_t=None) == OK


def _gemm(lib, fn="fp8_scaled_gemm_blockwise", **kw):
    a = dict(a=P, lda=256, ra=P, ra_s_row=1, ra_s_kb=64, b=P, ldb=256, rb=P, rb_s_row=1,
             rb_s_kb=1, b_block=1, M=64, N=128, K=256, out=P, ldo=128, out_dtype=0, ws=P,
             ws_bytes=1 << 20, stream=None)
    a.update(kw)
    args = [a[k] for k in ("a", "lda", "ra", "ra_s_row", "ra_s_kb", "b", "ldb", "rb", "rb_s_row",
                           "rb_s_kb", "b_block", "M", "N", "K", "out", "ldo", "out_dtype")]
    if fn == "fp8_scaled_gemm_blockwise_cfg":
        args += [a.get("config", -1), a.get("splits", 0)]
    args += [a["ws"], a["ws_bytes"], a["stream"]]
    return getattr(lib, fn)(*args)


def test_gemm_validation(lib):
    assert _gemm(lib, K=200) == SHAPE                    # K % 128
    assert _gemm(lib, M=-1) == SHAPE
    assert _gemm(lib, b_block=3) == UNSUP
    assert _gemm(lib, out_dtype=5) == UNSUP
    assert _gemm(lib, a=None) == NULL
    assert _gemm(lib, rb=None) == NULL
    assert _gemm(lib, b=P + 1) == ALIGN
    assert _gemm(lib, lda=128) == LAYOUT                 # lda < K
    assert _gemm(lib, ldb=264) == LAYOUT                 # not a multiple of 16
    assert _gemm(lib, ldo=100) == LAYOUT                 # ldo < N
    assert _gemm(lib, ra_s_row=2) == LAYOUT              # row 32 meets (row 0, kb 1)
    assert _gemm(lib, ra_s_kb=32) == LAYOUT              # aliases rows of ra
    assert _gemm(lib, b_block=0, rb_s_row=2, rb_s_kb=200) == LAYOUT   # 1x128 rb: row 100 aliases
    assert _gemm(lib, b_block=0, rb_s_row=-2, rb_s_kb=256) == LAYOUT  # negative stride
    assert _gemm(lib, rb_s_row=1, rb_s_kb=0) == LAYOUT   # 128x128 rb: aliases
    assert _gemm(lib, M=0, a=None, b=None, out=None) == OK
    assert _gemm(lib, "fp8_scaled_gemm_blockwise_cfg", config=99) == UNSUP
    assert _gemm(lib, "fp8_scaled_gemm_blockwise_cfg", splits=-2) == SHAPE
    assert _gemm(lib, "fp8_scaled_gemm_blockwise_cfg", splits=3) == SHAPE   # > 2 K blocks
    need = lib.fp8bw_gemm_ws_bytes_for_split(64, 128, 2)
    assert need == 2 * 64 * 128 * 4
    assert _gemm(lib, "fp8_scaled_gemm_blockwise_cfg", splits=2, ws_bytes=need - 1) == WS
    assert _gemm(lib, "fp8_scaled_gemm_blockwise_cfg", splits=2, ws=None) == WS


def test_gemm_kn_validation(lib):
    """fp8_scaled_gemm_blockwise_kn: B is [K, N] (ldb >= N); it runs on the
    256x256 tiles only and refuses smaller or unaligned problems before any
    launch."""
    kn = dict(fn="fp8_scaled_gemm_blockwise_kn", M=512, N=512, K=256, lda=256, ldb=512,
              ldo=512, ra_s_kb=512, rb_s_kb=4)
    assert _gemm(lib, **{**kn, "ldb": 256}) == LAYOUT      # ldb < N
    assert _gemm(lib, **{**kn, "ldb": 520}) == LAYOUT      # not a multiple of 16
    assert _gemm(lib, **{**kn, "b": None}) == NULL
    assert _gemm(lib, **{**kn, "K": 200}) == SHAPE         # K % 128
    assert _gemm(lib, **{**kn, "M": 128}) == UNSUP         # M < 256
    assert _gemm(lib, **{**kn, "N": 200, "ldo": 200, "ldb": 208, "rb_s_kb": 2}) == UNSUP  # N < 256
    assert _gemm(lib, **{**kn, "N": 264, "ldo": 264, "ldb": 272, "rb_s_kb": 3}) == UNSUP  # N % 16
    assert _gemm(lib, **{**kn, "N": 336, "ldo": 336, "ldb": 336, "rb_s_kb": 3}) == UNSUP  # N % 64, 128x128
    assert "[K, N]" in lib.fp8bw_last_error().decode()
    assert _gemm(lib, **{**kn, "M": 0, "a": None, "b": None, "out": None}) == OK


def test_bias_entry_points_validate(lib):
    """The _bias entry points share the GEMMs' validation and add a 2-byte
    alignment check on the bias pointer."""
    a = dict(a=P, lda=256, ra=P, ra_s_row=1, ra_s_kb=64, b=P, ldb=256, rb=P, rb_s_row=1,
             rb_s_kb=1, b_block=1, M=64, N=128, K=256)
    args = [a[k] for k in ("a", "lda", "ra", "ra_s_row", "ra_s_kb", "b", "ldb", "rb", "rb_s_row",
                           "rb_s_kb", "b_block", "M", "N", "K")]
    assert lib.fp8_scaled_gemm_blockwise_bias(*args, P + 1, P, 128, 0, P, 1 << 20, None) == ALIGN
    assert lib.fp8_scaled_gemm_blockwise_bias(*args[:13], 200, P, P, 128, 0, P, 1 << 20,
                                              None) == SHAPE       # K % 128
    assert lib.fp8_scaled_gemm_tensorwise_bias(P, 256, P, P, 256, P, 64, 128, 256, P + 1, P, 128,
                                               0, None) == ALIGN
    assert lib.fp8_scaled_gemm_tensorwise_bias(P, 256, P, P, 256, P, 64, 128, 200, P, P, 128,
                                               0, None) == SHAPE   # K % 16


def _grouped(lib, **kw):
    a = dict(a=P, lda=256, ra=P, ra_s_kb=64, b=P, ldb=256, b_s_group=128 * 256, rb=P, rb_s_row=1,
             rb_s_kb=1, rb_s_group=2, groups=4, group_end=P, M=64, N=128, K=256, out=P, ldo=128,
             out_dtype=0, stream=None)
    a.update(kw)
    return lib.fp8_scaled_grouped_gemm_blockwise(*[a[k] for k in (
        "a", "lda", "ra", "ra_s_kb", "b", "ldb", "b_s_group", "rb", "rb_s_row", "rb_s_kb",
        "rb_s_group", "groups", "group_end", "M", "N", "K", "out", "ldo", "out_dtype", "stream")])


def test_grouped_gemm_validation(lib):
    assert _grouped(lib, groups=0) == SHAPE
    assert _grouped(lib, K=200) == SHAPE
    assert _grouped(lib, group_end=None) == NULL
    assert _grouped(lib, group_end=P + 2) == ALIGN
    assert _grouped(lib, b_s_group=100) == LAYOUT           # groups' weights overlap
    assert _grouped(lib, ra_s_kb=8) == LAYOUT               # ra not column-major
    assert _grouped(lib, rb_s_group=1) == LAYOUT            # groups' scales overlap
    assert _grouped(lib, M=0, a=None, out=None, group_end=None) == OK


def test_tensorwise_validation(lib):
    f = lib.fp8_scaled_gemm_tensorwise
    assert f(P, 32, P, P, 32, P, 16, 32, 24, P, 32, 1, None) == SHAPE        # K % 16
    assert f(P, 32, None, P, 32, P, 16, 32, 32, P, 32, 1, None) == NULL
    assert f(P, 32, P, P, 32, P, 16, 32, 32, P, 30, 1, None) == LAYOUT       # ldo < N
    q = lib.fp8_tensorwise_quant
    assert q(P, 16, 32, 32, P, 32, P, P, 0, None) == WS
    assert q(P, 16, 30, 32, P, 32, P, P, 4096, None) == SHAPE
    assert lib.fp8bw_tensorwise_quant_ws_bytes(16, 32) >= 4
    n = lib.fp8_tensorwise_quant_noalloc
    assert n(P, 16, 30, 32, P, 32, P, None) == SHAPE                         # cols % 16
    assert n(P, 16, 32, 32, P, 32, None, None) == NULL
    assert n(P, 16, 32, 32, P + 1, 32, P, None) == ALIGN
    assert n(P, 16, 32, 24, P, 32, P, None) == LAYOUT                        # ld_x < cols


def test_linear_validation_and_workspace(lib):
    for which, fn in enumerate(("fp8_linear_fwd", "fp8_linear_dgrad", "fp8_linear_wgrad")):
        f = getattr(lib, fn)
        need = lib.fp8bw_linear_ws_bytes(256, 256, 256, which)
        assert need >= 2 * 256 * 256
        assert f(P, P, P, 256, 256, 256, P, need - 1, None) == WS
        assert f(P, P, P, 256, 256, 256, None, need, None) == WS
        assert f(None, P, P, 256, 256, 256, P, need, None) == NULL
        assert f(P, P, P, 256, 256, 200, P, need, None) == SHAPE
        assert f(P, P, P, 256, 256, 256, P + 16, need, None) == ALIGN    # ws 256-aligned
    # contraction axis must be a multiple of 128
    assert lib.fp8_linear_fwd(P, P, P, 256, 256, 144, P, 1 << 24, None) == SHAPE
    assert lib.fp8_linear_dgrad(P, P, P, 256, 144, 256, P, 1 << 24, None) == SHAPE
    assert lib.fp8_linear_wgrad(P, P, P, 144, 256, 256, P, 1 << 24, None) == SHAPE


def test_fused_linear_validation_and_buffers(lib):
    """fp8_linear_fwd_save / fp8_linear_bwd reject bad shapes, buffers and
    alignment before launching anything."""
    M = N = K = 256
    saved = lib.fp8bw_linear_saved_bytes(M, N, K)
    assert saved >= 256 * 256                          # X^T codes at least
    assert lib.fp8bw_linear_saved_bytes(0, N, K) == 0
    need_f = lib.fp8bw_linear_ws_bytes(M, N, K, 3)
    need_b = lib.fp8bw_linear_ws_bytes(M, N, K, 4)
    assert need_f >= 2 * 256 * 256 and need_b >= 3 * 256 * 256   # dY, dY^T and W^T codes
    assert lib.fp8bw_linear_ws_bytes(M, N, K, 5) == 0
    f, b = lib.fp8_linear_fwd_save, lib.fp8_linear_bwd
    assert f(P, P, P, M, N, K, P, saved - 1, P, need_f, None) == WS           # saved too small
    assert f(P, P, P, M, N, K, P, saved, P, need_f - 1, None) == WS           # ws too small
    assert f(P, P, P, M, N, K, None, saved, P, need_f, None) == NULL
    assert f(None, P, P, M, N, K, P, saved, P, need_f, None) == NULL
    assert f(P, P, P, M, N, 144, P, 1 << 24, P, 1 << 26, None) == SHAPE       # K % 128
    assert f(P, P, P, M, N, K, P + 16, saved, P, need_f, None) == ALIGN       # saved 256-aligned
    assert b(P, P, P, saved, P, P, M, N, K, P, need_b - 1, None) == WS
    assert b(P, P, P, saved - 1, P, P, M, N, K, P, need_b, None) == WS
    assert b(P, P, None, saved, P, P, M, N, K, P, need_b, None) == NULL       # saved
    assert b(P, None, P, saved, P, P, M, N, K, P, need_b, None) == NULL       # w
    assert b(P, P, P, 1 << 24, P, P, 144, N, K, P, 1 << 26, None) == SHAPE    # M % 128
    assert b(P, P, P, 1 << 24, P, P, M, 144, K, P, 1 << 26, None) == SHAPE    # N % 128
    assert b(P, P, P, saved, P + 4, P, M, N, K, P, need_b, None) == ALIGN     # dx 16-aligned
    assert b(P, P + 4, P, saved, P, P, M, N, K, P, need_b, None) == ALIGN     # w 16-aligned


def test_binding_raises_with_message(lib):
    st = _gemm(lib, K=200)
    with pytest.raises(fp8.FP8BWError, match="K % 128"):
        _lib.check(st)


def test_no_host_fallback_in_binding():
    """The binding has no CPU path: ops refuse non-CUDA tensors."""
    import torch
    x = torch.zeros(16, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fp8.fp8_blockwise_quant(x)
    assert ctypes.sizeof(ctypes.c_void_p) == 8


def test_binding_refuses_a_library_of_another_abi_version(monkeypatch):
    """The ctypes prototypes describe one ABI version: a library reporting
    another one is refused at load, instead of being called with the wrong
    arguments."""
    from blockwise_scaled_fp8_amd import _lib as lib_mod
    monkeypatch.setattr(lib_mod, "_LIB", None)
    monkeypatch.setattr(lib_mod, "ABI_VERSION", lib_mod.ABI_VERSION + 1)
    with pytest.raises(RuntimeError, match="ABI version"):
        lib_mod.load_library()
    monkeypatch.undo()
    assert lib_mod.load_library().fp8bw_abi_version() == lib_mod.ABI_VERSION
