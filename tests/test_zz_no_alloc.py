"""The allocation-free per-tensor quantizer (fp8_tensorwise_quant_noalloc,
partials in the library's own per-device array) against the workspace entry
point and the oracle, through the C ABI: bit-identical codes and reciprocal
scale on consecutive calls, each later call smaller than the one before and
with a smaller amax (a call that read the previous call's partials left in
the shared array would get a different scale)."""

import numpy as np
import pytest
import torch

import blockwise_scaled_fp8_amd as fp8
from oracle import quant
from synth import inputs
from tests.gpu_util import assert_codes_equal, assert_f32_equal, bits, say

pytestmark = pytest.mark.gpu


def test_noalloc_tensorwise_matches_workspace_entry_point(gpu):
    shapes = [((4096, 4096), 64.0, 0), ((1000, 208), 4.0, 1), ((48, 64), 1.0, 2)]
    for (rows, cols), gain, seed in shapes:
        x = inputs.randn_bf16((rows, cols), seed=inputs.tensor_seed(60 + seed, "x"))
        x = (x.float() * gain).to(torch.bfloat16)
        xd = x.to(gpu)
        q_new = torch.empty((rows, cols), dtype=torch.uint8, device=gpu)
        r_new = torch.empty(1, dtype=torch.float32, device=gpu)
        say("noalloc tensorwise quant", rows, cols, gain)
        fp8.fp8_tensorwise_quant_noalloc(xd, q_new, r_new)
        say("workspace tensorwise quant", rows, cols, gain)
        q_ref, r_ref = fp8.fp8_tensorwise_quant(xd)
        torch.cuda.synchronize()
        assert torch.equal(q_new, q_ref), f"codes differ at {rows}x{cols}"
        assert torch.equal(r_new.view(torch.int32), r_ref.view(torch.int32)), (rows, cols)
        if rows * cols <= 1 << 20:
            oq, orc = quant.quant_tensorwise(bits(x))
            assert_codes_equal(q_new.cpu().numpy(), oq, f"noalloc codes {rows}x{cols}")
            assert_f32_equal(r_new.cpu().numpy(), np.float32(orc), f"noalloc recip {rows}x{cols}")
