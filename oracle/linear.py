"""FP8 blockwise linear forward / dgrad / wgrad (oracle; test infrastructure only).

The composition follows [INTEG] Summary (Float8BlockwiseLinear: quantize,
then the scaled GEMM) and [REPRO] review comments (the backward uses the
1x128 x 128x128 recipe for the grad path and 1x128 x 1x128 for the weight
gradient):

  fwd    Y  = X . W^T     A = X 1x128,          B = W 128x128
  dgrad  dX = dY . W      A = dY 1x128,         B = W^T 128x128
  wgrad  dW = dY^T . X    A = dY^T 1x128 along M, B = X^T 1x128 along M

Each returns the float64 block-rescaled result (before any output rounding).
Shapes: X[M, K], W[N, K], dY[M, N]; K, N, M multiples of 128 as each
contraction needs.
"""

from . import quant, gemm


def fwd(x_bits, w_bits, with_bound=False):
    xq, xr = quant.quant_1x128(x_bits)
    wq, wr = quant.quant_128x128(w_bits)
    return gemm.blockwise_gemm(xq, xr, wq, wr, "128x128", with_bound)


def dgrad(dy_bits, w_bits, with_bound=False):
    dq, dr = quant.quant_1x128(dy_bits)
    wtq, wtr = quant.quant_128x128_transposed(w_bits)
    return gemm.blockwise_gemm(dq, dr, wtq, wtr, "128x128", with_bound)


def wgrad(dy_bits, x_bits, with_bound=False):
    dtq, dtr = quant.quant_1x128_along_rows(dy_bits)
    xtq, xtr = quant.quant_1x128_along_rows(x_bits)
    return gemm.blockwise_gemm(dtq, dtr, xtq, xtr, "1x128", with_bound)
