"""blockwise_scaled_fp8_amd: blockwise- and tensorwise-scaled FP8 (OCP E4M3)
quantization and GEMM for AMD MI355X (gfx950).

The computation lives in libfp8bw.so (hand-written HIP for gfx950 behind the
C ABI in include/fp8bw.h); this package is its ctypes binding.  PyTorch is
used for device memory and streams only.
"""

from ._lib import FP8BWError, PROTOTYPES, load_library, lib_path  # noqa: F401
from .ops import (  # noqa: F401
    colmajor_empty,
    fp8_blockwise_quant,
    fp8_blockwise_quant_dual,
    fp8_linear_bwd,
    fp8_linear_dgrad,
    fp8_linear_fwd,
    fp8_linear_fwd_save,
    fp8_linear_wgrad,
    fp8_scaled_gemm_blockwise,
    fp8_scaled_gemm_blockwise_kn,
    fp8_scaled_gemm_tensorwise,
    fp8_scaled_grouped_gemm_blockwise,
    fp8_tensorwise_quant,
    fp8_tensorwise_quant_noalloc,
    fp8bw_gemm_num_configs,
    gemm_plan,
    linear_saved_bytes,
    linear_workspace,
    scale_grid,
)
from .torch_ops import Float8BlockwiseLinear  # noqa: E402,F401  (registers torch.ops.fp8bw.*)
