/*
 * fp8bw.h -- C ABI of libfp8bw.so: blockwise- and tensorwise-scaled FP8
 * (OCP E4M3) quantization and GEMM for AMD MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [REPRO]   pytorch/ao PR "add repro for blockwise _scaled_mm
 *             investigation" -- What Changed; Findings So Far; review
 *             comments (the 1x128 x 128x128 and 1x128 x 1x128 recipes).
 *   [INTEG]   pytorch/ao PR "integrate torch._scaled_mm into
 *             Float8BlockwiseLinear and add bench script" -- Summary
 *             (reciprocal scales, column-major scale layout); Benchmarks
 *             (linear forward + backward at M16640 N5120 K8192).
 *   [GENERIC] pytorch/ao PR "add more generic kernel for fp8 blockwise
 *             scaling" -- Performance table (1x128 and 128x128 blocks).
 *   [AITER]   ROCm/aiter issue "Does gemm_a8w8 support per-tensor quant?"
 *             -- Steps to Reproduce (per-tensor quant, out = x @ w.T,
 *             dequant reference x_q.float() * x_scale).
 *   [INDUCT]  pytorch/pytorch inductor FP8 tensorwise issue -- Describe the
 *             bug (16x32x32 fp32-out tensorwise case).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers marked "device" are HIP device pointers; the library never
 *    allocates, frees or copies device memory and never synchronizes the
 *    host.  Scratch comes from a caller-owned workspace sized by the
 *    matching *_ws_bytes query.  The caller owns every buffer.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  All work
 *    is enqueued on it in order; the call returns after enqueueing.
 *  - bf16 tensors are raw 16-bit bf16 bit patterns; FP8 tensors are OCP
 *    E4M3 ("e4m3fn") codes, one byte each; scales are fp32.
 *  - Matrices are row-major with a leading dimension `ld*` in elements.
 *    Every matrix pointer must be 16-byte aligned, bf16 input leading
 *    dimensions a multiple of 8 and FP8 leading dimensions a multiple of 16
 *    (GEMM output leading dimensions only need ldo >= N).  The stride of a
 *    dimension of size 1 is ignored.  Every element offset a call can form
 *    ((rows - 1) * ld + cols of each matrix, the last scale of a strided
 *    scale grid, the last group of a grouped operand) must be below 2^48;
 *    larger ones give FP8BW_ERR_LAYOUT.
 *  - Dimensions are at most 2^30 (quantizer rows 2^32).  The GEMM and
 *    linear size queries return 0 for larger ones (the calls reject them),
 *    and fp8bw_gemm_ws_bytes_for_split returns SIZE_MAX when the size does
 *    not fit a size_t.
 *  - A *reciprocal scale* ("recip") is the dequantization multiplier: the
 *    quantizer computes s = 448 / max(amax, 1e-12) per block, stores
 *    codes = satRNE_e4m3(x * s) and recip = 1 / s (both fp32 IEEE ops),
 *    so x ~= e4m3_value(code) * recip ([INTEG] Summary; [AITER]).
 *  - Validation runs on the host before any HIP call.  A rejected call
 *    enqueues nothing and returns a status != FP8BW_OK;
 *    fp8bw_last_error() gives a message for the calling thread.  A launch
 *    failure returns FP8BW_ERR_HIP.  No exception crosses the ABI and the
 *    library prints nothing.
 *  - Zero-sized problems (rows == 0, cols == 0, M == 0 or N == 0) succeed
 *    and enqueue nothing (the tensorwise quantizer still writes its recip).
 *  - Inputs must be finite; outputs must not alias inputs.  Results for
 *    non-finite inputs are unspecified.
 */
#ifndef FP8BW_H
#define FP8BW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8BW_OK = 0,
  FP8BW_ERR_NULL = 1,        /* a required pointer is NULL */
  FP8BW_ERR_SHAPE = 2,       /* negative or unsupported dimension */
  FP8BW_ERR_LAYOUT = 3,      /* leading dimension / scale stride not allowed */
  FP8BW_ERR_ALIGN = 4,       /* pointer or leading dimension misaligned */
  FP8BW_ERR_UNSUPPORTED = 5, /* unknown enum value or config */
  FP8BW_ERR_WORKSPACE = 6,   /* workspace NULL or too small */
  FP8BW_ERR_HIP = 7          /* a HIP launch failed */
} fp8bw_status;

typedef enum { FP8BW_BLOCK_1x128 = 0, FP8BW_BLOCK_128x128 = 1 } fp8bw_block;
typedef enum { FP8BW_OUT_BF16 = 0, FP8BW_OUT_F32 = 1 } fp8bw_out;

/* Version of this ABI (incremented on incompatible change). */
int fp8bw_abi_version(void);
/* Static string for a status code. */
const char* fp8bw_status_str(int status);
/* Message for the last rejected call on this thread ("" if none). */
const char* fp8bw_last_error(void);

/*
 * fp8_blockwise_quant -- dynamic E4M3 quantization with per-block amax
 * scales ([GENERIC] Performance table: block_shape (1,128) and (128,128);
 * [INTEG] Summary: reciprocal scales written by the quantizer itself).
 *
 *   x      device bf16 [rows, cols], leading dim ld_x.
 *   block  FP8BW_BLOCK_1x128: one scale per row per 128 columns
 *          (transpose=0), or per column per 128 rows (transpose=1: the
 *          wgrad operands dY^T, X^T).
 *          FP8BW_BLOCK_128x128: one scale per 128x128 tile (weights);
 *          transpose=1 writes W^T codes for the dgrad GEMM.  A tile's amax
 *          is orientation-independent, so these codes are exactly the
 *          transpose of the transpose=0 codes.
 *   q      device E4M3 output.  transpose=0: q[rows, cols] (ld_q >= cols).
 *          transpose=1: q = x^T [cols, rows] (ld_q >= rows).
 *   recip  device fp32 reciprocal scales, indexed by (output row or output
 *          row block i, output column block j) at recip[i*rs_row + j*rs_kb]:
 *            1x128,   transpose=0: i = row r, j = r's 128-column block
 *            1x128,   transpose=1: i = column c (output row), j = 128-row block
 *            128x128, transpose=0: i = 128-row block, j = 128-column block
 *            128x128, transpose=1: i = 128-column block, j = 128-row block
 *          Column-major ([INTEG] Summary) is rs_row = 1, rs_kb = number of
 *          i indices; any non-negative strides are accepted.
 *   Blocks at a ragged edge take their amax over the valid elements only.
 *   Requires cols % 16 == 0, and rows % 16 == 0 when transpose=1.
 */
int fp8_blockwise_quant(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int block,
                        int transpose, void* q, int64_t ld_q, float* recip, int64_t rs_row,
                        int64_t rs_kb, void* stream);

/*
 * fp8_blockwise_quant_dual -- both layouts from one read of x: the same
 * codes and scales as fp8_blockwise_quant with transpose=0 into (q, recip)
 * and with transpose=1 into (qt, recip_t), for a training step that needs
 * X and X^T (or dY and dY^T, or W and W^T) and would otherwise read the
 * bf16 tensor twice; the quantizers are the part of the fp8 linear step
 * the pages single out as slow ([INTEG] Benchmarks).
 *
 *   block    FP8BW_BLOCK_1x128: q = 1x128 blocks along the columns with
 *            recip[r*rs_row + kb*rs_kb]; qt = x^T with 1x128 blocks along
 *            the rows, recip_t[c*rst_row + mb*rst_kb].
 *            FP8BW_BLOCK_128x128: q = tile-scaled codes, recip[rb*rs_row +
 *            cb*rs_kb]; qt = their transpose, recip_t[cb*rst_row +
 *            rb*rst_kb] (the same values in the other index order).
 *   q, qt    device E4M3 [rows, cols] (ld_q >= cols) and [cols, rows]
 *            (ld_qt >= rows); the two must not overlap (checked).
 *   stream_t nonzero: qt is written with nontemporal stores, which keep the
 *            transposed codes from evicting the caches' contents (for codes
 *            read only much later, such as the X^T a training forward keeps
 *            for its backward, while q feeds the GEMM that runs next).  The
 *            same bits either way.
 *   Requires cols % 16 == 0 and rows % 16 == 0; each output is validated as
 *   in fp8_blockwise_quant, and results are bit-identical to two calls of it.
 */
int fp8_blockwise_quant_dual(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int block,
                             void* q, int64_t ld_q, float* recip, int64_t rs_row, int64_t rs_kb,
                             void* qt, int64_t ld_qt, float* recip_t, int64_t rst_row,
                             int64_t rst_kb, int stream_t, void* stream);

/*
 * fp8_tensorwise_quant -- one scale for the whole tensor ([AITER]
 * per_tensor_quant: the scale returned is the dequant multiplier).
 *   x [rows, cols] bf16 (ld_x), q [rows, cols] E4M3 (ld_q), recip: one
 *   device fp32.  ws: device scratch of fp8bw_tensorwise_quant_ws_bytes().
 *   Two launches (partial amax, then quantize); deterministic.
 *   Requires cols % 16 == 0.
 */
size_t fp8bw_tensorwise_quant_ws_bytes(int64_t rows, int64_t cols);
int fp8_tensorwise_quant(const void* x, int64_t rows, int64_t cols, int64_t ld_x, void* q,
                         int64_t ld_q, float* recip, void* ws, size_t ws_bytes, void* stream);

/*
 * fp8_tensorwise_quant_noalloc -- fp8_tensorwise_quant without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * The partial amaxes go to a 4 KiB array the library holds on every GPU it
 * runs on until the process ends (at most 1024 partials, enough for any
 * input, so no size is refused for scratch; FP8BW_ERR_WORKSPACE guards the
 * invariant).  The call allocates nothing; its first call on a device looks
 * up that device's copy of the array (the device current at the call).
 * Results are bit-identical to fp8_tensorwise_quant.  All calls on one GPU
 * share the array: calls that overlap in time on one GPU (different
 * streams) race and give undefined results; calls ordered on one stream are
 * safe.  Arguments, layout and errors otherwise as fp8_tensorwise_quant.
 */
int fp8_tensorwise_quant_noalloc(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                 void* q, int64_t ld_q, float* recip, void* stream);

/*
 * fp8_scaled_gemm_blockwise -- out[M, N] = sum_kb ra[m, kb] * rb[beta(n), kb]
 *                              * sum_{k in block kb} a[m, k] * b[n, k]
 * ([REPRO] What Changed: the blockwise GEMM on the same codes and
 * reciprocal scales as the dequantized matmul; out = A . B^T as F.linear).
 *
 *   a   device E4M3 [M, K], lda; ra: 1x128 scales of A,
 *       ra[m*ra_s_row + kb*ra_s_kb].
 *   b   device E4M3 [N, K], ldb.  b_block selects rb's meaning:
 *         FP8BW_BLOCK_128x128: rb[(n/128)*rb_s_row + kb*rb_s_kb]  (fwd, dgrad)
 *         FP8BW_BLOCK_1x128:   rb[n*rb_s_row + kb*rb_s_kb]        (wgrad)
 *       Scale strides: the column-major layout the quantizers write
 *       (s_row = 1, s_kb >= rows: [INTEG] Summary) is the fast one; any
 *       other non-overlapping nested strides (row-major, transposed or
 *       padded views) are accepted as they are, without a copy.  Strides
 *       that alias (one stride does not span the other dimension's whole
 *       extent) or are negative give FP8BW_ERR_LAYOUT.
 *   out device [M, N] bf16 (RNE from the fp32 accumulator) or fp32, ldo.
 *   K % 128 == 0 (K blocks may number anything, e.g. 1001 or 1002).
 *   Each K block is accumulated in fp32 by the matrix cores and rescaled in
 *   fp32 before it is added to the running sum.
 *   ws: device scratch for split-K partials; size from
 *   fp8bw_gemm_blockwise_ws_bytes(M, N, K) (may be 0 -> ws may be NULL).
 */
size_t fp8bw_gemm_blockwise_ws_bytes(int64_t M, int64_t N, int64_t K);
int fp8_scaled_gemm_blockwise(const void* a, int64_t lda, const float* ra, int64_t ra_s_row,
                              int64_t ra_s_kb, const void* b, int64_t ldb, const float* rb,
                              int64_t rb_s_row, int64_t rb_s_kb, int b_block, int64_t M,
                              int64_t N, int64_t K, void* out, int64_t ldo, int out_dtype,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * fp8_scaled_gemm_blockwise_kn -- the same GEMM with B given in [K, N]
 * layout: out[M, N] = sum_kb ra[m, kb] * rb[beta(n), kb]
 *                     * sum_{k in block kb} a[m, k] * b_kn[k, n].
 * The second operand arrives as the transposed (column-major) view of an
 * [N, K] matrix, the way torch._scaled_mm takes the weight ([AITER] Steps to
 * Reproduce: the weight passed as its .t() view); e.g. dX = dY . W from W's
 * own codes, whose 128x128 blocks and scales serve W^T unchanged (block amax
 * does not depend on orientation), with no transposed copy of the codes.
 *   b_kn device E4M3 [K, N], row stride ldb >= N (N contiguous).
 *   rb   indexed by (output column n, K block) exactly as in
 *        fp8_scaled_gemm_blockwise (for W's scales sw[nb_w][kb_w]: the view
 *        with strides swapped).
 * The kernel reads B's [K block, 256 columns] tiles into LDS row by row and
 * forms the matrix-core operands with transposing LDS reads; outputs are
 * bit-identical to fp8_scaled_gemm_blockwise on b = b_kn^T.
 * Needs M >= 256, N >= 256, N % 16 == 0 (and N % 64 == 0 for 128x128 B
 * scales), 256 * ldb + K < 2^31 and K % 128 == 0; other problems give
 * FP8BW_ERR_UNSUPPORTED (use fp8_scaled_gemm_blockwise on a [N, K] copy).
 * Workspace: fp8bw_gemm_blockwise_ws_bytes(M, N, K).  Other arguments and
 * errors as fp8_scaled_gemm_blockwise.
 */
int fp8_scaled_gemm_blockwise_kn(const void* a, int64_t lda, const float* ra, int64_t ra_s_row,
                                 int64_t ra_s_kb, const void* b_kn, int64_t ldb, const float* rb,
                                 int64_t rb_s_row, int64_t rb_s_kb, int b_block, int64_t M,
                                 int64_t N, int64_t K, void* out, int64_t ldo, int out_dtype,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * Same as fp8_scaled_gemm_blockwise with an explicit tile configuration
 * (0 .. fp8bw_gemm_num_configs()-1, or -1 for the built-in choice) and
 * split-K count (>= 1, or 0 for the built-in choice).  Every configuration
 * computes the same result up to fp32 rounding order; this entry point
 * lets tests force each one (a kernel variant can be wrong where the
 * others are right: [INDUCT] Describe the bug).  Workspace for an explicit
 * split s is fp8bw_gemm_ws_bytes_for_split(M, N, s).
 */
int fp8bw_gemm_num_configs(void);

/*
 * fp8bw_gemm_blockwise_plan -- how fp8_scaled_gemm_blockwise runs an
 * M x N x K problem with contiguous operands and column-major scales on
 * the current device (host query, launches nothing; for profiling and
 * reporting).  Fills info[6] (caller-owned host array): tile
 * configuration, whole-problem split-K count, split count of the leftover
 * tiles of a partial last round, total tiles, tiles run unsplit, workspace
 * bytes.  Requires 0 < M, N, K and K % 128 == 0.
 */
int fp8bw_gemm_blockwise_plan(int64_t M, int64_t N, int64_t K, int b_block, int64_t* info);
size_t fp8bw_gemm_ws_bytes_for_split(int64_t M, int64_t N, int splits);
int fp8_scaled_gemm_blockwise_cfg(const void* a, int64_t lda, const float* ra, int64_t ra_s_row,
                                  int64_t ra_s_kb, const void* b, int64_t ldb, const float* rb,
                                  int64_t rb_s_row, int64_t rb_s_kb, int b_block, int64_t M,
                                  int64_t N, int64_t K, void* out, int64_t ldo, int out_dtype,
                                  int config, int splits, void* ws, size_t ws_bytes,
                                  void* stream);

/*
 * fp8_scaled_gemm_tensorwise -- out[M, N] = (sum_k a[m, k] * b[n, k]) * ra * rb
 * ([AITER]: per-tensor scales, out = x @ w.T; [INDUCT]: fp32 output).
 *   ra, rb: one device fp32 each (dequant multipliers).
 *   K % 16 == 0 (K need not be a multiple of 128).  No workspace.
 */
int fp8_scaled_gemm_tensorwise(const void* a, int64_t lda, const float* ra, const void* b,
                               int64_t ldb, const float* rb, int64_t M, int64_t N, int64_t K,
                               void* out, int64_t ldo, int out_dtype, void* stream);

/*
 * fp8_scaled_gemm_blockwise_bias / fp8_scaled_gemm_tensorwise_bias -- the
 * same GEMMs with a bias epilogue.  Both GEMM interfaces on the pages take
 * an optional bias (aiter gemm_a8w8 and torch._scaled_mm, [AITER] Steps to
 * Reproduce; the inductor tests parametrize has_bias, [INDUCT] Describe the
 * bug); the pages pass None and do not define its arithmetic.  Here:
 *
 *   out[m, n] = cast(acc[m, n] + bias[n])
 *
 * where acc is the fp32 result the call without bias would cast (after the
 * per-tensor scaling for the tensorwise GEMM), the bias value is widened
 * from bf16 exactly, the add is one fp32 add, and cast is RNE to bf16 or
 * none for fp32 out.  With split-K the add happens once, in the reduce.
 *
 *   bias   device bf16 [N], contiguous, 2-byte aligned; NULL = no bias
 *          (then identical to the call without _bias).
 *   Every other argument, status and workspace rule is that of the call
 *   without _bias.
 */
int fp8_scaled_gemm_blockwise_bias(const void* a, int64_t lda, const float* ra, int64_t ra_s_row,
                                   int64_t ra_s_kb, const void* b, int64_t ldb, const float* rb,
                                   int64_t rb_s_row, int64_t rb_s_kb, int b_block, int64_t M,
                                   int64_t N, int64_t K, const void* bias, void* out, int64_t ldo,
                                   int out_dtype, void* ws, size_t ws_bytes, void* stream);
int fp8_scaled_gemm_tensorwise_bias(const void* a, int64_t lda, const float* ra, const void* b,
                                    int64_t ldb, const float* rb, int64_t M, int64_t N, int64_t K,
                                    const void* bias, void* out, int64_t ldo, int out_dtype,
                                    void* stream);

/*
 * fp8_scaled_grouped_gemm_blockwise -- one call for G GEMMs that share N
 * and K and split the rows of A and out into consecutive groups, each with
 * its own B (the mixture-of-experts layout: tokens sorted by expert, one
 * weight per expert; the pages mention the grouped scaled matmul of MoE
 * training in [INTEG]'s review discussion).  For every group g and row m of
 * it, out[m, :] is what fp8_scaled_gemm_blockwise gives for that row with B_g
 * (1x128 A scales, 128x128 B scales):
 *
 *   rows of group g: [group_end[g-1], group_end[g])   (group_end[-1] = 0)
 *   B_g  = b  + g * b_s_group   [N, K] codes, leading dim ldb
 *   rb_g = rb + g * rb_s_group  scales of B_g, rb_g[(n/128)*rb_s_row + kb*rb_s_kb]
 *
 *   a, ra       device [M, K] codes and their column-major 1x128 scales
 *               ra[m + kb*ra_s_kb] (ra_s_kb >= M) for all groups' rows.
 *   group_end   DEVICE int32 [groups], cumulative row ends, read by the
 *               kernel (no host synchronization).  Values are clamped to
 *               [previous end, M]: a malformed table cannot make the kernel
 *               read or write outside A, ra and out.  Rows past the last end
 *               are not written.
 *   b_s_group   >= (N-1)*ldb + K, a multiple of 16 (distinct weights).
 *   rb_s_group  large enough that groups' scale grids do not overlap.
 *   Requires K % 128 == 0; no split-K, no workspace.  Problems with
 *   M >= 256 and N >= 128 (and 256*lda + K, 256*ldb + K < 2^31) run on the
 *   large-tile kernels, others on the small-tile kernel.  With up to 64
 *   groups on the large tiles the call enqueues two launches: the second
 *   takes the groups' last partial row tiles of at most 128 rows as 64-row
 *   tiles when the table (read on the device) shows that this saves a round
 *   of the GPU's compute units; otherwise it returns at once.  Every row is
 *   written by exactly one launch.  The grids must fit in 2^31 - 1
 *   workgroups (else FP8BW_ERR_UNSUPPORTED).
 */
int fp8_scaled_grouped_gemm_blockwise(const void* a, int64_t lda, const float* ra,
                                      int64_t ra_s_kb, const void* b, int64_t ldb,
                                      int64_t b_s_group, const float* rb, int64_t rb_s_row,
                                      int64_t rb_s_kb, int64_t rb_s_group, int groups,
                                      const int* group_end, int64_t M, int64_t N, int64_t K,
                                      void* out, int64_t ldo, int out_dtype, void* stream);

/*
 * FP8 blockwise linear layer, fwd / dgrad / wgrad ([INTEG] Summary:
 * Float8BlockwiseLinear; [REPRO] review comments: 1x128 x 128x128 on the
 * grad path, 1x128 x 1x128 for the weight gradient).  All tensors are
 * contiguous row-major bf16: X[M, K], W[N, K], dY[M, N].
 *   fwd:   Y[M, N]  = X . W^T   (X 1x128, W 128x128)        K % 128 == 0
 *   dgrad: dX[M, K] = dY . W    (dY 1x128, W^T 128x128)     N % 128 == 0
 *   wgrad: dW[N, K] = dY^T . X  (dY^T, X^T 1x128 along M)   M % 128 == 0
 * Each quantizes its inputs into the caller's workspace (codes and
 * reciprocal scales) and runs the blockwise GEMM; bf16 output.
 * which = 0 fwd, 1 dgrad, 2 wgrad for the workspace query (3 and 4: the
 * fused entry points below).  All dims must also be multiples of 16.
 */
size_t fp8bw_linear_ws_bytes(int64_t M, int64_t N, int64_t K, int which);
int fp8_linear_fwd(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                   void* ws, size_t ws_bytes, void* stream);
int fp8_linear_dgrad(const void* dy, const void* w, void* dx, int64_t M, int64_t N, int64_t K,
                     void* ws, size_t ws_bytes, void* stream);
int fp8_linear_wgrad(const void* dy, const void* x, void* dw, int64_t M, int64_t N, int64_t K,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * FP8 blockwise linear with each large bf16 tensor read once per step: the
 * same three GEMMs and the same codes and scales as fp8_linear_fwd / _dgrad
 * / _wgrad (bit-identical outputs), with fused quantization
 * (fp8_blockwise_quant_dual): the forward quantizes X once into X (1x128
 * along K) and X^T (1x128 along M), keeping X^T's codes and scales for the
 * backward (written with nontemporal stores, so that X's codes stay cached
 * for the forward GEMM), and W into W (128x128); the backward quantizes dY
 * once into dY
 * and dY^T, and W into W^T right before the dgrad GEMM.  The quantizers are
 * the part of the fp8 linear step the pages single out as slow ([INTEG]
 * Benchmarks); fp8 X^T codes are also half the size of the bf16 X a
 * backward would otherwise keep.  W^T is written by the backward rather
 * than kept from the forward because the dgrad GEMM then reads it from the
 * memory-side cache it was just written to (one more read of W, 2 bytes per
 * weight, against a faster dgrad GEMM).
 *
 *   fp8_linear_fwd_save: Y[M, N] = X . W^T; writes `saved`.
 *     Requires K % 128 == 0 (and M, N, K multiples of 16).
 *   fp8_linear_bwd: dX[M, K] = dY . W and dW[N, K] = dY^T . X from dY, the
 *     same bf16 W [N, K] and the `saved` of the forward with the same X, W,
 *     M, N, K.  dx or dw may be null to skip that gradient.  Requires
 *     M % 128 == 0 and N % 128 == 0.
 *   saved   caller device memory of fp8bw_linear_saved_bytes(M, N, K)
 *           bytes, 256-byte aligned, owned by the caller between the two
 *           calls; its layout is internal to the library.
 *   ws      workspace of fp8bw_linear_ws_bytes(M, N, K, which) bytes with
 *           which = 3 (fwd_save) or 4 (bwd), 256-byte aligned.
 * Errors as for fp8_linear_fwd; nothing is launched on an error.
 */
size_t fp8bw_linear_saved_bytes(int64_t M, int64_t N, int64_t K);
int fp8_linear_fwd_save(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                        void* saved, size_t saved_bytes, void* ws, size_t ws_bytes, void* stream);
int fp8_linear_bwd(const void* dy, const void* w, const void* saved, size_t saved_bytes, void* dx,
                   void* dw, int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8BW_H */
