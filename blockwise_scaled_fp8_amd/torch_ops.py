"""PyTorch integration of the FP8 blockwise linear: custom ops, autograd and
an nn.Linear counterpart.

The layer above the hot path in the pages' design is a linear module whose
forward and backward quantize and run the blockwise-scaled GEMM
(pytorch/ao PR "integrate torch._scaled_mm into Float8BlockwiseLinear and
add bench script", Summary).  Here that is:

  * three custom ops, ``torch.ops.fp8bw.linear_fwd`` / ``linear_dgrad`` /
    ``linear_wgrad``, each one call of the C ABI (quantizers + GEMM all run
    in libfp8bw.so) with a fake (meta) implementation, so ``torch.compile``
    can trace through them without running them;
  * ``torch.ops.fp8bw.linear``, the forward op with autograd registered:
    its backward calls the dgrad and wgrad ops, each with the recipe the
    pages use for that GEMM (dY 1x128 x W^T 128x128; dY^T 1x128 x X^T 1x128
    along the token axis);
  * ``torch.ops.fp8bw.linear_fwd_save`` / ``linear_bwd``: the same
    computation with X and dY each quantized once per step into both code
    layouts (the forward keeps the X^T codes, the backward quantizes dY
    once and W^T right before the dgrad GEMM), bit-identical to the ops
    above;
  * ``Float8BlockwiseLinear``, a module with ``nn.Linear``'s interface
    (bias-free) that flattens leading dimensions into the token axis and
    trains through the fused-quantization ops.

Shapes follow the ABI's rules: in_features and out_features multiples of
128 (they are contraction axes in fwd and dgrad) and a token count that is a
multiple of 128 when the weight gradient is needed (its contraction axis).
Everything is bf16.  There is no fallback: without libfp8bw.so the ops raise.
"""

import math

import torch

from . import ops


def _check_2d_bf16(*ts):
    for t in ts:
        if t.dim() != 2 or t.dtype != torch.bfloat16:
            raise ValueError("fp8bw linear ops take 2-D bf16 tensors")


@torch.library.custom_op("fp8bw::linear_fwd", mutates_args=())
def linear_fwd(x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """Y[M, N] = X[M, K] . W[N, K]^T, X 1x128 and W 128x128 blocks."""
    _check_2d_bf16(x, w)
    return ops.fp8_linear_fwd(x.contiguous(), w.contiguous())


@linear_fwd.register_fake
def _linear_fwd_fake(x, w):
    _check_2d_bf16(x, w)
    return x.new_empty((x.shape[0], w.shape[0]))


@torch.library.custom_op("fp8bw::linear_dgrad", mutates_args=())
def linear_dgrad(dy: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """dX[M, K] = dY[M, N] . W[N, K], dY 1x128 and W^T 128x128 blocks."""
    _check_2d_bf16(dy, w)
    return ops.fp8_linear_dgrad(dy.contiguous(), w.contiguous())


@linear_dgrad.register_fake
def _linear_dgrad_fake(dy, w):
    _check_2d_bf16(dy, w)
    return dy.new_empty((dy.shape[0], w.shape[1]))


@torch.library.custom_op("fp8bw::linear_wgrad", mutates_args=())
def linear_wgrad(dy: torch.Tensor, x: torch.Tensor) -> torch.Tensor:
    """dW[N, K] = dY[M, N]^T . X[M, K], both 1x128 blocks along M."""
    _check_2d_bf16(dy, x)
    return ops.fp8_linear_wgrad(dy.contiguous(), x.contiguous())


@linear_wgrad.register_fake
def _linear_wgrad_fake(dy, x):
    _check_2d_bf16(dy, x)
    return dy.new_empty((dy.shape[1], x.shape[1]))


@torch.library.custom_op("fp8bw::linear", mutates_args=())
def linear(x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """Differentiable FP8 blockwise linear: Y = X . W^T (see linear_fwd)."""
    _check_2d_bf16(x, w)
    return ops.fp8_linear_fwd(x.contiguous(), w.contiguous())


@linear.register_fake
def _linear_fake(x, w):
    _check_2d_bf16(x, w)
    return x.new_empty((x.shape[0], w.shape[0]))


def _linear_setup_context(ctx, inputs, output):
    x, w = inputs
    ctx.save_for_backward(x, w)


def _linear_backward(ctx, dy):
    x, w = ctx.saved_tensors
    dy = dy.contiguous()
    dx = torch.ops.fp8bw.linear_dgrad(dy, w) if ctx.needs_input_grad[0] else None
    dw = torch.ops.fp8bw.linear_wgrad(dy, x) if ctx.needs_input_grad[1] else None
    return dx, dw


torch.library.register_autograd("fp8bw::linear", _linear_backward,
                                setup_context=_linear_setup_context)


@torch.library.custom_op("fp8bw::linear_fwd_save", mutates_args=())
def linear_fwd_save(x: torch.Tensor, w: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """(Y, saved): Y = X . W^T with X quantized once into both code layouts;
    saved holds the X^T codes and scales for linear_bwd (one C-ABI call,
    fp8_linear_fwd_save)."""
    _check_2d_bf16(x, w)
    return ops.fp8_linear_fwd_save(x.contiguous(), w.contiguous())


@linear_fwd_save.register_fake
def _linear_fwd_save_fake(x, w):
    _check_2d_bf16(x, w)
    M, K = x.shape
    N = w.shape[0]
    n = max(ops.linear_saved_bytes(M, N, K), 1)
    return x.new_empty((M, N)), x.new_empty((n,), dtype=torch.uint8)


@torch.library.custom_op("fp8bw::linear_bwd", mutates_args=())
def linear_bwd(dy: torch.Tensor, w: torch.Tensor, saved: torch.Tensor, need_dx: bool,
               need_dw: bool) -> tuple[torch.Tensor, torch.Tensor]:
    """(dX, dW) from dY (quantized once into both layouts), the forward's W
    and the saved buffer of linear_fwd_save; a gradient not asked for comes
    back empty."""
    _check_2d_bf16(dy, w)
    dx, dw = ops.fp8_linear_bwd(dy.contiguous(), w.contiguous(), saved, need_dx, need_dw)
    return (dx if dx is not None else dy.new_empty((0,)),
            dw if dw is not None else dy.new_empty((0,)))


@linear_bwd.register_fake
def _linear_bwd_fake(dy, w, saved, need_dx, need_dw):
    _check_2d_bf16(dy, w)
    M, N = dy.shape
    k = w.shape[1]
    return (dy.new_empty((M, k)) if need_dx else dy.new_empty((0,)),
            dy.new_empty((N, k)) if need_dw else dy.new_empty((0,)))


class _FusedQuantLinear(torch.autograd.Function):
    """Y = X . W^T whose backward uses the X^T codes its forward wrote (X and
    dY each read once per training step)."""

    @staticmethod
    def forward(ctx, x, w):
        y, saved = torch.ops.fp8bw.linear_fwd_save(x, w)
        ctx.save_for_backward(w, saved)
        return y

    @staticmethod
    def backward(ctx, dy):
        w, saved = ctx.saved_tensors
        need_dx, need_dw = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        dx, dw = torch.ops.fp8bw.linear_bwd(dy.contiguous(), w, saved, need_dx, need_dw)
        return (dx if need_dx else None), (dw if need_dw else None)


class Float8BlockwiseLinear(torch.nn.Module):
    """Bias-free ``nn.Linear`` counterpart whose forward and backward run the
    FP8 blockwise recipe: y = x W^T with x quantized per 1x128 and W per
    128x128 block; dX and dW as in ``torch.ops.fp8bw.linear``.

    The weight is a bf16 parameter [out_features, in_features] initialized
    as ``nn.Linear`` does (U(+-1/sqrt(in_features))).  Inputs [..., in_features]
    are flattened to [tokens, in_features]."""

    def __init__(self, in_features, out_features, bias=False, device=None, dtype=torch.bfloat16):
        super().__init__()
        if bias:
            raise NotImplementedError("Float8BlockwiseLinear is bias-free")
        if dtype != torch.bfloat16:
            raise ValueError("Float8BlockwiseLinear keeps a bf16 weight")
        if in_features % 128 or out_features % 128:
            raise ValueError("in_features and out_features must be multiples of 128")
        self.in_features = in_features
        self.out_features = out_features
        self.weight = torch.nn.Parameter(
            torch.empty(out_features, in_features, device=device, dtype=dtype))
        self.reset_parameters()

    def reset_parameters(self):
        bound = 1.0 / math.sqrt(self.in_features)
        with torch.no_grad():
            self.weight.uniform_(-bound, bound)

    @classmethod
    def from_linear(cls, lin):
        """The same layer from a bias-free ``nn.Linear`` (weight cast to bf16)."""
        if lin.bias is not None:
            raise NotImplementedError("Float8BlockwiseLinear is bias-free")
        m = cls(lin.in_features, lin.out_features, device=lin.weight.device)
        with torch.no_grad():
            m.weight.copy_(lin.weight.to(torch.bfloat16))
        return m

    def forward(self, x):
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features)
        if torch.is_grad_enabled() and (x.requires_grad or self.weight.requires_grad):
            # Training: quantize X once into both layouts and keep the
            # transposed fp8 codes (half the bytes of the bf16 X) for backward.
            # The weight gradient contracts over the tokens in 1x128 blocks,
            # so their count must be a multiple of 128; say so here rather
            # than in the backward.
            if x2.shape[0] % 128:
                raise ValueError(f"training needs the token count ({x2.shape[0]}) to be a multiple "
                                 "of 128: the weight gradient contracts over tokens in blocks of 128")
            y = _FusedQuantLinear.apply(x2, self.weight)
        else:
            y = torch.ops.fp8bw.linear_fwd(x2, self.weight)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self):
        return f"in_features={self.in_features}, out_features={self.out_features}, bias=False"
