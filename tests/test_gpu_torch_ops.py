"""GPU parity of the PyTorch integration: the module's forward and the
gradients autograd produces equal the C-ABI linear calls bit for bit, and
match the oracle's composition to the GEMM bar; torch.compile (AOT autograd,
no code generation) gives the same bits as eager."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_amd as fp8
from oracle import linear
from synth import inputs
from tests.gpu_util import bits, check_gemm_output, host_f32, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mnk", [(256, 384, 512), (384, 128, 256)])
def test_module_forward_backward(gpu, mnk):
    M, N, K = mnk
    x = inputs.randn_bf16((M, K), seed=inputs.tensor_seed(21, "x"))
    w = inputs.linear_weight_bf16(N, K, seed=inputs.tensor_seed(21, "w"))
    dy = inputs.randn_bf16((M, N), seed=inputs.tensor_seed(21, "dy"))
    m = fp8.Float8BlockwiseLinear(K, N, device=gpu)
    with torch.no_grad():
        m.weight.copy_(w.to(gpu))
    xd = x.to(gpu).requires_grad_(True)
    say("module fwd/bwd", mnk)
    y = m(xd)
    y.backward(dy.to(gpu))
    torch.cuda.synchronize()
    # bit-equal to the C-ABI calls
    assert torch.equal(y, fp8.fp8_linear_fwd(x.to(gpu), w.to(gpu)))
    assert torch.equal(xd.grad, fp8.fp8_linear_dgrad(dy.to(gpu), w.to(gpu)))
    assert torch.equal(m.weight.grad, fp8.fp8_linear_wgrad(dy.to(gpu), x.to(gpu)))
    # and within the GEMM bar of the oracle
    ref, S = linear.fwd(bits(x), bits(w), with_bound=True)
    check_gemm_output(host_f32(y.detach()), ref, S, K // 128, "bf16", f"module fwd {mnk}")
    ref, S = linear.dgrad(bits(dy), bits(w), with_bound=True)
    check_gemm_output(host_f32(xd.grad), ref, S, N // 128, "bf16", f"module dgrad {mnk}")
    ref, S = linear.wgrad(bits(dy), bits(x), with_bound=True)
    check_gemm_output(host_f32(m.weight.grad), ref, S, M // 128, "bf16", f"module wgrad {mnk}")


def test_compiled_module_matches_eager(gpu):
    M, N, K = 256, 256, 384
    x = inputs.randn_bf16((2, M // 2, K), seed=inputs.tensor_seed(22, "x"), device=gpu)
    m = fp8.Float8BlockwiseLinear(K, N, device=gpu)
    say("module compile aot_eager")
    cm = torch.compile(m, backend="aot_eager", fullgraph=True)
    xe = x.clone().requires_grad_(True)
    xc = x.clone().requires_grad_(True)
    ye = m(xe)
    ye.sum().backward()
    ge = m.weight.grad.clone()
    m.weight.grad = None
    yc = cm(xc)
    yc.sum().backward()
    torch.cuda.synchronize()
    assert torch.equal(ye, yc)
    assert torch.equal(xe.grad, xc.grad)
    assert torch.equal(ge, m.weight.grad)
    assert np.isfinite(host_f32(yc.detach())).all()
