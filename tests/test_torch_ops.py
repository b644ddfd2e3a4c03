"""The PyTorch integration layer without a GPU: op registration, fake (meta)
shape propagation through forward, autograd and torch.compile tracing, the
module's interface, and that real CPU tensors are refused (no fallback)."""

import pytest
import torch

import blockwise_scaled_fp8_amd as fp8


def _meta(*shape, grad=False):
    return torch.empty(*shape, dtype=torch.bfloat16, device="meta", requires_grad=grad)


def test_ops_registered():
    for name in ("linear", "linear_fwd", "linear_dgrad", "linear_wgrad", "linear_fwd_save",
                 "linear_bwd"):
        assert hasattr(torch.ops.fp8bw, name)


def test_fake_shapes():
    x, w, dy = _meta(256, 512), _meta(384, 512), _meta(256, 384)
    assert torch.ops.fp8bw.linear_fwd(x, w).shape == (256, 384)
    assert torch.ops.fp8bw.linear(x, w).shape == (256, 384)
    assert torch.ops.fp8bw.linear_dgrad(dy, w).shape == (256, 512)
    assert torch.ops.fp8bw.linear_wgrad(dy, x).shape == (384, 512)
    with pytest.raises(ValueError):
        torch.ops.fp8bw.linear_fwd(x.float(), w)


def test_fused_fake_shapes():
    x, w, dy = _meta(256, 512), _meta(384, 512), _meta(256, 384)
    y, saved = torch.ops.fp8bw.linear_fwd_save(x, w)
    assert y.shape == (256, 384) and saved.dtype == torch.uint8 and saved.dim() == 1
    assert saved.numel() == fp8.linear_saved_bytes(256, 384, 512)
    dx, dw = torch.ops.fp8bw.linear_bwd(dy, w, saved, True, True)
    assert dx.shape == (256, 512) and dw.shape == (384, 512)
    dx, dw = torch.ops.fp8bw.linear_bwd(dy, w, saved, False, True)
    assert dx.numel() == 0 and dw.shape == (384, 512)


def test_module_autograd_shapes_on_meta():
    m = fp8.Float8BlockwiseLinear(512, 384, device="meta")
    assert m.weight.shape == (384, 512) and m.weight.dtype == torch.bfloat16
    x = _meta(2, 128, 512, grad=True)
    y = m(x)
    assert y.shape == (2, 128, 384)
    y.sum().backward()
    assert x.grad.shape == x.shape and m.weight.grad.shape == m.weight.shape


def test_compile_traces_the_custom_ops():
    """AOT autograd (no code generation) traces forward and backward through
    the fake implementations in one graph."""
    m = fp8.Float8BlockwiseLinear(256, 128, device="meta")
    cm = torch.compile(m, backend="aot_eager", fullgraph=True)
    x = _meta(128, 256, grad=True)
    y = cm(x)
    y.sum().backward()
    assert y.shape == (128, 128) and x.grad.shape == (128, 256)


def test_module_interface():
    with pytest.raises(NotImplementedError):
        fp8.Float8BlockwiseLinear(128, 128, bias=True)
    with pytest.raises(ValueError):
        fp8.Float8BlockwiseLinear(100, 128)
    lin = torch.nn.Linear(256, 128, bias=False)
    m = fp8.Float8BlockwiseLinear.from_linear(lin)
    assert torch.equal(m.weight, lin.weight.detach().to(torch.bfloat16))
    bound = 1 / 256 ** 0.5
    assert float(fp8.Float8BlockwiseLinear(256, 128).weight.detach().abs().max()) <= bound


def test_cpu_tensors_are_refused():
    m = fp8.Float8BlockwiseLinear(128, 128)
    with pytest.raises(ValueError, match="CUDA"):
        m(torch.zeros(128, 128, dtype=torch.bfloat16))


def test_training_token_count_checked_in_forward():
    """The weight gradient contracts over tokens in 1x128 blocks: a training
    forward with a token count that is not a multiple of 128 is refused at
    once, while inference (no gradient) takes any count."""
    m = fp8.Float8BlockwiseLinear(256, 128, device="meta")
    with pytest.raises(ValueError, match="multiple of 128"):
        m(_meta(2, 50, 256, grad=True))
    with torch.no_grad():
        y = m(_meta(2, 50, 256, grad=False))
    assert y.shape == (2, 50, 128)


def test_binding_rejects_wrong_dtypes_and_strides():
    """Caller-provided codes, scales and outputs are checked for dtype and
    layout before any pointer reaches the library (a bf16 scale tensor read
    as fp32, or a column-strided output, would address the wrong memory)."""
    from blockwise_scaled_fp8_amd import ops
    codes = torch.zeros((4, 32), dtype=torch.uint8)
    ops._check_codes_out(codes, (4, 32), "q")
    ops._check_codes_out(codes.view(torch.float8_e4m3fn), (4, 32), "q")
    with pytest.raises(ValueError, match="uint8 or float8"):
        ops._check_codes_out(codes.to(torch.int8), (4, 32), "q")
    with pytest.raises(ValueError, match="unit column stride"):
        ops._check_codes_out(torch.zeros((32, 4), dtype=torch.uint8).t(), (4, 32), "q")
    with pytest.raises(ValueError, match="shape"):
        ops._check_codes_out(codes, (4, 16), "q")
    sc = torch.zeros((4, 2), dtype=torch.float32)
    ops._check_scales(sc, (4, 2), "ra")
    ops._check_scales(sc.t().contiguous().t(), (4, 2), "ra")      # any strides
    with pytest.raises(ValueError, match="float32"):
        ops._check_scales(sc.to(torch.bfloat16), (4, 2), "ra")
    out = torch.zeros((4, 8), dtype=torch.bfloat16)
    ops._check_out(out, (4, 8))
    ops._check_out(out.float(), (4, 8))
    with pytest.raises(ValueError, match="bfloat16 or float32"):
        ops._check_out(out.half(), (4, 8))
    with pytest.raises(ValueError, match="unit column stride"):
        ops._check_out(torch.zeros((8, 4), dtype=torch.float32).t(), (4, 8))
