// C ABI of libfp8bw.so: argument validation, workspace layout and kernel
// dispatch.  Declarations and the contract of every entry point are in
// include/fp8bw.h.  Validation is pure host code and runs before any HIP
// call, so a rejected call enqueues nothing.

#include "../../include/fp8bw.h"

#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "launch.h"

#define FP8BW_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int ok() {
  g_err.clear();
  return FP8BW_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(FP8BW_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;   // int32 indexing inside the kernels
constexpr int64_t kMaxGridY = 65535;

// Every element offset a call can form stays below 2^48: no allocation is
// larger, and the bound keeps each product the host and the kernels form on
// offsets (tile and byte offsets) far from int64 overflow.
constexpr int64_t kMaxExtent = (int64_t)1 << 48;

// (rows - 1) * ld + cols < kMaxExtent for a [rows, cols] matrix with
// leading dimension ld (1 <= rows, cols <= 2^32; the product is not formed).
bool extent_ok(int64_t rows, int64_t ld, int64_t cols) {
  if (ld < 0) return false;
  if (rows <= 1) return cols < kMaxExtent;
  return cols < kMaxExtent && ld <= (kMaxExtent - 1 - cols) / (rows - 1);
}

// A strided 2-D scale grid [ni, nj] with strides (si, sj) must map distinct
// index pairs to distinct addresses, and its last element must lie below
// kMaxExtent.  The stride of a dimension of size 1 is never used.
bool strides_injective(int64_t ni, int64_t nj, int64_t si, int64_t sj) {
  if (si < 0 || sj < 0) return false;
  if (ni <= 1 && nj <= 1) return true;
  if (ni <= 1) return sj >= 1 && extent_ok(nj, sj, 1);
  if (nj <= 1) return si >= 1 && extent_ok(ni, si, 1);
  // sj >= si * ni (or si >= sj * nj) without forming the product
  const bool nested = (si >= 1 && sj / ni >= si) || (sj >= 1 && si / nj >= sj);
  if (!nested) return false;
  // (ni - 1) * si + (nj - 1) * sj < kMaxExtent
  if (!extent_ok(ni, si, 1)) return false;
  const int64_t rest = kMaxExtent - 1 - (ni - 1) * si;
  return sj <= rest / (nj - 1);
}

// The stride of a size-1 dimension is never used; pass 0 for it so that
// no later arithmetic sees an arbitrary value.
int64_t used_stride(int64_t n, int64_t s) { return n > 1 ? s : 0; }

// a * b * c in size_t, SIZE_MAX when it does not fit.
size_t mul_sat(size_t a, size_t b, size_t c) {
  size_t ab, abc;
  if (__builtin_mul_overflow(a, b, &ab) || __builtin_mul_overflow(ab, c, &abc)) return SIZE_MAX;
  return abc;
}

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

FP8BW_API int fp8bw_abi_version(void) { return 2; }

FP8BW_API const char* fp8bw_status_str(int s) {
  switch (s) {
    case FP8BW_OK: return "FP8BW_OK";
    case FP8BW_ERR_NULL: return "FP8BW_ERR_NULL";
    case FP8BW_ERR_SHAPE: return "FP8BW_ERR_SHAPE";
    case FP8BW_ERR_LAYOUT: return "FP8BW_ERR_LAYOUT";
    case FP8BW_ERR_ALIGN: return "FP8BW_ERR_ALIGN";
    case FP8BW_ERR_UNSUPPORTED: return "FP8BW_ERR_UNSUPPORTED";
    case FP8BW_ERR_WORKSPACE: return "FP8BW_ERR_WORKSPACE";
    case FP8BW_ERR_HIP: return "FP8BW_ERR_HIP";
    default: return "FP8BW_ERR_UNKNOWN";
  }
}

FP8BW_API const char* fp8bw_last_error(void) { return g_err.c_str(); }

// ---------------------------------------------------------------------------
// Quantization.

static int check_quant_common(const void* x, int64_t rows, int64_t cols, int64_t ld_x, void* q,
                              int64_t ld_q, int64_t q_rows, int64_t q_row_len) {
  if (rows < 0 || cols < 0) return fail(FP8BW_ERR_SHAPE, "negative rows/cols (%lld, %lld)",
                                        (long long)rows, (long long)cols);
  if (rows > kMaxDim * 4 || cols > kMaxDim) return fail(FP8BW_ERR_SHAPE, "dimension too large");
  if (cols % 16) return fail(FP8BW_ERR_SHAPE, "cols=%lld must be a multiple of 16", (long long)cols);
  if (rows == 0 || cols == 0) return FP8BW_OK;
  if (!x || !q) return fail(FP8BW_ERR_NULL, "x and q must be non-null");
  if (!aligned(x, 16) || !aligned(q, 16)) return fail(FP8BW_ERR_ALIGN, "x and q must be 16-byte aligned");
  if (ld_x < cols || ld_x % 8) return fail(FP8BW_ERR_LAYOUT, "ld_x=%lld must be >= cols and a multiple of 8", (long long)ld_x);
  if (ld_q < q_row_len || ld_q % 16)
    return fail(FP8BW_ERR_LAYOUT, "ld_q=%lld must be >= %lld and a multiple of 16", (long long)ld_q, (long long)q_row_len);
  if (!extent_ok(rows, ld_x, cols) || !extent_ok(q_rows, ld_q, q_row_len))
    return fail(FP8BW_ERR_LAYOUT, "ld_x=%lld / ld_q=%lld reach past 2^48 elements", (long long)ld_x, (long long)ld_q);
  return FP8BW_OK;
}

// Validation of one quantizer output (codes q and scales recip) for a block
// kind and orientation.
static int check_quant_output(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int block,
                              int transpose, void* q, int64_t ld_q, float* recip, int64_t rs_row,
                              int64_t rs_kb) {
  if (block != FP8BW_BLOCK_1x128 && block != FP8BW_BLOCK_128x128)
    return fail(FP8BW_ERR_UNSUPPORTED, "unknown block kind %d", block);
  if (transpose != 0 && transpose != 1) return fail(FP8BW_ERR_UNSUPPORTED, "transpose must be 0 or 1");
  if (transpose && rows % 16) return fail(FP8BW_ERR_SHAPE, "transpose=1 needs rows %% 16 == 0 (rows=%lld)", (long long)rows);
  int st = check_quant_common(x, rows, cols, ld_x, q, ld_q, transpose ? cols : rows, transpose ? rows : cols);
  if (st != FP8BW_OK) return st;
  if (rows == 0 || cols == 0) return FP8BW_OK;
  if (!recip) return fail(FP8BW_ERR_NULL, "recip must be non-null");
  if (!aligned(recip, 4)) return fail(FP8BW_ERR_ALIGN, "recip must be 4-byte aligned");
  // Scale grid [ni, nj] in (output row or row block, output column block).
  int64_t ni, nj;
  if (block == FP8BW_BLOCK_1x128) {
    ni = transpose ? cols : rows;
    nj = transpose ? cdiv(rows, 128) : cdiv(cols, 128);
  } else {
    ni = transpose ? cdiv(cols, 128) : cdiv(rows, 128);
    nj = transpose ? cdiv(rows, 128) : cdiv(cols, 128);
  }
  if (!strides_injective(ni, nj, rs_row, rs_kb))
    return fail(FP8BW_ERR_LAYOUT, "recip strides (%lld, %lld) alias or are negative for a %lldx%lld scale grid",
                (long long)rs_row, (long long)rs_kb, (long long)ni, (long long)nj);
  if ((transpose || block == FP8BW_BLOCK_128x128) && cdiv(rows, 128) > kMaxGridY)
    return fail(FP8BW_ERR_SHAPE, "too many row blocks");
  return FP8BW_OK;
}

FP8BW_API int fp8_blockwise_quant(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                  int block, int transpose, void* q, int64_t ld_q, float* recip,
                                  int64_t rs_row, int64_t rs_kb, void* stream) {
  int st = check_quant_output(x, rows, cols, ld_x, block, transpose, q, ld_q, recip, rs_row, rs_kb);
  if (st != FP8BW_OK) return st;
  if (rows == 0 || cols == 0) return ok();
  hipStream_t s = (hipStream_t)stream;
  if (block == FP8BW_BLOCK_1x128 && !transpose)
    return hip_status(fp8bw::launch_quant_1x128_rows(x, rows, cols, ld_x, q, ld_q, recip, rs_row, rs_kb, s),
                      "fp8_blockwise_quant");
  if (block == FP8BW_BLOCK_1x128)
    return hip_status(fp8bw::launch_quant_1x128_cols_t(x, rows, cols, ld_x, q, ld_q, recip, rs_row, rs_kb, s),
                      "fp8_blockwise_quant");
  return hip_status(fp8bw::launch_quant_128x128(x, rows, cols, ld_x, transpose, q, ld_q, recip, rs_row, rs_kb, s),
                    "fp8_blockwise_quant");
}

// fp8_blockwise_quant_dual; stream_t writes the transposed codes with
// nontemporal stores (the training forward's X^T, read only by its backward).
static int quant_dual_impl(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int block,
                           void* q, int64_t ld_q, float* recip, int64_t rs_row, int64_t rs_kb,
                           void* qt, int64_t ld_qt, float* recip_t, int64_t rst_row,
                           int64_t rst_kb, bool stream_t, void* stream) {
  int st = check_quant_output(x, rows, cols, ld_x, block, 0, q, ld_q, recip, rs_row, rs_kb);
  if (st != FP8BW_OK) return st;
  st = check_quant_output(x, rows, cols, ld_x, block, 1, qt, ld_qt, recip_t, rst_row, rst_kb);
  if (st != FP8BW_OK) return st;
  if (rows == 0 || cols == 0) return ok();
  // The two code buffers must not overlap (scales are the caller's to keep apart).
  const uintptr_t q0 = (uintptr_t)q, q1 = q0 + (uintptr_t)((rows - 1) * ld_q + cols);
  const uintptr_t t0 = (uintptr_t)qt, t1 = t0 + (uintptr_t)((cols - 1) * ld_qt + rows);
  if (q0 < t1 && t0 < q1) return fail(FP8BW_ERR_LAYOUT, "q and qt overlap");
  return hip_status(fp8bw::launch_quant_dual(x, rows, cols, ld_x, block == FP8BW_BLOCK_128x128, q, ld_q,
                                             recip, rs_row, rs_kb, qt, ld_qt, recip_t, rst_row, rst_kb,
                                             stream_t, (hipStream_t)stream),
                    "fp8_blockwise_quant_dual");
}

FP8BW_API int fp8_blockwise_quant_dual(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                       int block, void* q, int64_t ld_q, float* recip,
                                       int64_t rs_row, int64_t rs_kb, void* qt, int64_t ld_qt,
                                       float* recip_t, int64_t rst_row, int64_t rst_kb,
                                       int stream_t, void* stream) {
  return quant_dual_impl(x, rows, cols, ld_x, block, q, ld_q, recip, rs_row, rs_kb, qt, ld_qt,
                         recip_t, rst_row, rst_kb, stream_t != 0, stream);
}

FP8BW_API size_t fp8bw_tensorwise_quant_ws_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 256;
  if (rows > kMaxDim * 4 || cols > kMaxDim)   // rejected by the quantizer; the cap
    return align_up((size_t)fp8bw::kMaxTensorwisePartials * sizeof(float));
  return align_up((size_t)fp8bw::tensorwise_partials(rows, cols) * sizeof(float));
}

FP8BW_API int fp8_tensorwise_quant(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                   void* q, int64_t ld_q, float* recip, void* ws,
                                   size_t ws_bytes, void* stream) {
  int st = check_quant_common(x, rows, cols, ld_x, q, ld_q, rows, cols);
  if (st != FP8BW_OK) return st;
  if (!recip) return fail(FP8BW_ERR_NULL, "recip must be non-null");
  if (!aligned(recip, 4)) return fail(FP8BW_ERR_ALIGN, "recip must be 4-byte aligned");
  if (!ws || ws_bytes < fp8bw_tensorwise_quant_ws_bytes(rows, cols))
    return fail(FP8BW_ERR_WORKSPACE, "workspace needs %zu bytes", fp8bw_tensorwise_quant_ws_bytes(rows, cols));
  if (!aligned(ws, 4)) return fail(FP8BW_ERR_ALIGN, "ws must be 4-byte aligned");
  const int64_t r = (rows == 0 || cols == 0) ? 0 : rows;
  const int64_t c = (rows == 0 || cols == 0) ? 0 : cols;
  return hip_status(fp8bw::launch_quant_tensorwise(x, r, c, ld_x, q, ld_q, recip, (float*)ws,
                                                   (hipStream_t)stream),
                    "fp8_tensorwise_quant");
}

FP8BW_API int fp8_tensorwise_quant_noalloc(const void* x, int64_t rows, int64_t cols,
                                           int64_t ld_x, void* q, int64_t ld_q, float* recip,
                                           void* stream) {
  int st = check_quant_common(x, rows, cols, ld_x, q, ld_q, rows, cols);
  if (st != FP8BW_OK) return st;
  if (!recip) return fail(FP8BW_ERR_NULL, "recip must be non-null");
  if (!aligned(recip, 4)) return fail(FP8BW_ERR_ALIGN, "recip must be 4-byte aligned");
  // The partials always fit the library's array (their count is capped);
  // the check guards the invariant.
  const int64_t r = (rows == 0 || cols == 0) ? 0 : rows;
  const int64_t c = (rows == 0 || cols == 0) ? 0 : cols;
  if (fp8bw::tensorwise_partials(r, c) > fp8bw::kMaxTensorwisePartials)
    return fail(FP8BW_ERR_WORKSPACE, "needs more than the %d partials of the library's scratch",
                fp8bw::kMaxTensorwisePartials);
  return hip_status(fp8bw::launch_quant_tensorwise_noalloc(x, r, c, ld_x, q, ld_q, recip,
                                                           (hipStream_t)stream),
                    "fp8_tensorwise_quant_noalloc");
}

// ---------------------------------------------------------------------------
// GEMM.

static int check_gemm_operands(const void* a, int64_t lda, const void* b, int64_t ldb,
                               int64_t M, int64_t N, int64_t K, void* out, int64_t ldo,
                               int out_dtype, bool b_kn = false) {
  if (out_dtype != FP8BW_OUT_BF16 && out_dtype != FP8BW_OUT_F32)
    return fail(FP8BW_ERR_UNSUPPORTED, "unknown out_dtype %d", out_dtype);
  if (M < 0 || N < 0 || K < 0)
    return fail(FP8BW_ERR_SHAPE, "negative dimension (M=%lld N=%lld K=%lld)", (long long)M, (long long)N, (long long)K);
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(FP8BW_ERR_SHAPE, "dimension too large");
  if (M == 0 || N == 0) return FP8BW_OK;
  if (!a || !b || !out) return fail(FP8BW_ERR_NULL, "a, b and out must be non-null");
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(out, 16))
    return fail(FP8BW_ERR_ALIGN, "a, b and out must be 16-byte aligned");
  if (lda < K || ldb < (b_kn ? N : K) || lda % 16 || ldb % 16)
    return fail(FP8BW_ERR_LAYOUT, "lda/ldb (%lld/%lld) must be >= K/%s and multiples of 16",
                (long long)lda, (long long)ldb, b_kn ? "N" : "K");
  if (ldo < N) return fail(FP8BW_ERR_LAYOUT, "ldo=%lld must be >= N", (long long)ldo);
  if (!extent_ok(M, lda, K) || !(b_kn ? extent_ok(K, ldb, N) : extent_ok(N, ldb, K)) ||
      !extent_ok(M, ldo, N))
    return fail(FP8BW_ERR_LAYOUT, "lda/ldb/ldo (%lld/%lld/%lld) reach past 2^48 elements",
                (long long)lda, (long long)ldb, (long long)ldo);
  return FP8BW_OK;
}

static int gemm_blockwise_impl(const void* a, int64_t lda, const float* ra, int64_t ra_s_row,
                               int64_t ra_s_kb, const void* b, int64_t ldb, const float* rb,
                               int64_t rb_s_row, int64_t rb_s_kb, int b_block, int64_t M,
                               int64_t N, int64_t K, void* out, int64_t ldo, int out_dtype,
                               int config, int splits, void* ws, size_t ws_bytes, void* stream,
                               const void* bias = nullptr, bool b_kn = false) {
  if (b_block != FP8BW_BLOCK_1x128 && b_block != FP8BW_BLOCK_128x128)
    return fail(FP8BW_ERR_UNSUPPORTED, "unknown b_block %d", b_block);
  int st = check_gemm_operands(a, lda, b, ldb, M, N, K, out, ldo, out_dtype, b_kn);
  if (st != FP8BW_OK) return st;
  if (K % 128) return fail(FP8BW_ERR_SHAPE, "blockwise GEMM needs K %% 128 == 0 (K=%lld)", (long long)K);
  if (M == 0 || N == 0) return ok();
  const int64_t kb = K / 128;
  if (kb > 0) {
    if (!ra || !rb) return fail(FP8BW_ERR_NULL, "ra and rb must be non-null");
    if (!aligned(ra, 4) || !aligned(rb, 4)) return fail(FP8BW_ERR_ALIGN, "ra/rb must be 4-byte aligned");
    // Any non-overlapping strides (column-major, row-major, views with
    // padding); strides of size-1 dimensions are never used.
    if (!strides_injective(M, kb, ra_s_row, ra_s_kb))
      return fail(FP8BW_ERR_LAYOUT, "ra strides (%lld, %lld) alias or are negative", (long long)ra_s_row, (long long)ra_s_kb);
    const int64_t nrb = b_block == FP8BW_BLOCK_1x128 ? N : cdiv(N, 128);
    if (!strides_injective(nrb, kb, rb_s_row, rb_s_kb))
      return fail(FP8BW_ERR_LAYOUT, "rb strides (%lld, %lld) alias or are negative", (long long)rb_s_row, (long long)rb_s_kb);
  }
  const int64_t nrb = b_block == FP8BW_BLOCK_1x128 ? N : cdiv(N, 128);
  fp8bw::GemmProblem p;
  p.a = a; p.lda = lda; p.b = b; p.ldb = ldb;
  p.ra = ra; p.ra_s_row = used_stride(M, ra_s_row); p.ra_s_kb = used_stride(kb, ra_s_kb);
  p.rb = rb; p.rb_s_row = used_stride(nrb, rb_s_row); p.rb_s_kb = used_stride(kb, rb_s_kb);
  p.out = out; p.ldo = ldo; p.M = M; p.N = N; p.K = K;
  p.mode = b_block == FP8BW_BLOCK_128x128 ? fp8bw::kBlockB128 : fp8bw::kBlockB1x128;
  p.out_kind = out_dtype == FP8BW_OUT_BF16 ? fp8bw::kOutBf16 : fp8bw::kOutF32;
  p.bias = bias;
  p.b_kn = b_kn ? 1 : 0;
  if (b_kn && !fp8bw::gemm_config_ok(p, 3))
    return fail(FP8BW_ERR_UNSUPPORTED,
                "B in [K, N] layout needs M, N >= 256, N %% 16 == 0 (%% 64 with 128x128 B "
                "scales) and 256 * ldb + K < 2^31");
  if (config >= 0 && !fp8bw::gemm_config_ok(p, config))
    return fail(FP8BW_ERR_UNSUPPORTED, "config %d does not support this problem", config);
  if (splits > kMaxGridY || (kb > 0 && splits > kb) || (kb == 0 && splits > 1))
    return fail(FP8BW_ERR_SHAPE, "splits=%d must be <= the number of K blocks (%lld)", splits, (long long)kb);
  fp8bw::GemmPlan plan = fp8bw::gemm_plan(p, config, splits, true);
  if (splits == 0 && plan.ws_bytes > 0 && (!ws || ws_bytes < plan.ws_bytes)) {
    // The built-in plan wanted scratch the caller did not provide: run
    // without splitting (same result up to rounding order, no workspace).
    plan = fp8bw::gemm_plan(p, config, 0, false);
  }
  if (plan.ws_bytes > 0) {
    if (!ws || ws_bytes < plan.ws_bytes)
      return fail(FP8BW_ERR_WORKSPACE, "workspace needs %zu bytes", plan.ws_bytes);
    if (!aligned(ws, 16)) return fail(FP8BW_ERR_ALIGN, "ws must be 16-byte aligned");
  }
  return hip_status(fp8bw::launch_gemm(p, plan, ws, (hipStream_t)stream), "fp8_scaled_gemm_blockwise");
}

FP8BW_API size_t fp8bw_gemm_blockwise_ws_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
  // Upper bound over every configuration's built-in plan (the configuration
  // chosen for a call also depends on its leading dimensions).
  fp8bw::GemmProblem p = {};
  p.M = M; p.N = N; p.K = K; p.lda = K; p.ldb = K;
  size_t need = 0;
  for (int mode : {fp8bw::kBlockB128, fp8bw::kBlockB1x128}) {
    p.mode = mode;
    for (int c = 0; c < fp8bw::gemm_num_configs(); ++c) {
      if (!fp8bw::gemm_config_ok(p, c)) continue;
      const size_t b = fp8bw::gemm_plan(p, c, 0, true).ws_bytes;
      if (b > need) need = b;
    }
  }
  return need;
}

FP8BW_API int fp8bw_gemm_num_configs(void) { return fp8bw::gemm_num_configs(); }

FP8BW_API int fp8bw_gemm_blockwise_plan(int64_t M, int64_t N, int64_t K, int b_block,
                                        int64_t* info) {
  if (!info) return fail(FP8BW_ERR_NULL, "info must be non-null");
  if (b_block != FP8BW_BLOCK_1x128 && b_block != FP8BW_BLOCK_128x128)
    return fail(FP8BW_ERR_UNSUPPORTED, "unknown b_block %d", b_block);
  if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim || K % 128)
    return fail(FP8BW_ERR_SHAPE, "plan needs 0 < M, N, K <= 2^30 and K %% 128 == 0");
  // The plan of a call with contiguous operands, column-major scales and the
  // workspace fp8bw_gemm_blockwise_ws_bytes(M, N, K) gives.
  fp8bw::GemmProblem p = {};
  p.M = M; p.N = N; p.K = K; p.lda = K; p.ldb = K;
  p.ra_s_row = 1; p.ra_s_kb = M;
  p.rb_s_row = 1; p.rb_s_kb = b_block == FP8BW_BLOCK_1x128 ? N : cdiv(N, 128);
  p.mode = b_block == FP8BW_BLOCK_128x128 ? fp8bw::kBlockB128 : fp8bw::kBlockB1x128;
  const fp8bw::GemmPlan pl = fp8bw::gemm_plan(p, -1, 0, true);
  info[0] = pl.cfg;
  info[1] = pl.splits;
  info[2] = pl.tail_splits;
  info[3] = pl.tiles;
  info[4] = pl.tiles_full;
  info[5] = (int64_t)pl.ws_bytes;
  return ok();
}

FP8BW_API size_t fp8bw_gemm_ws_bytes_for_split(int64_t M, int64_t N, int splits) {
  if (M <= 0 || N <= 0 || splits <= 1) return 0;
  return mul_sat((size_t)splits, mul_sat((size_t)M, (size_t)N, 1), sizeof(float));
}

FP8BW_API int fp8_scaled_gemm_blockwise(const void* a, int64_t lda, const float* ra,
                                        int64_t ra_s_row, int64_t ra_s_kb, const void* b,
                                        int64_t ldb, const float* rb, int64_t rb_s_row,
                                        int64_t rb_s_kb, int b_block, int64_t M, int64_t N,
                                        int64_t K, void* out, int64_t ldo, int out_dtype,
                                        void* ws, size_t ws_bytes, void* stream) {
  return gemm_blockwise_impl(a, lda, ra, ra_s_row, ra_s_kb, b, ldb, rb, rb_s_row, rb_s_kb, b_block,
                             M, N, K, out, ldo, out_dtype, -1, 0, ws, ws_bytes, stream);
}

FP8BW_API int fp8_scaled_gemm_blockwise_cfg(const void* a, int64_t lda, const float* ra,
                                            int64_t ra_s_row, int64_t ra_s_kb, const void* b,
                                            int64_t ldb, const float* rb, int64_t rb_s_row,
                                            int64_t rb_s_kb, int b_block, int64_t M, int64_t N,
                                            int64_t K, void* out, int64_t ldo, int out_dtype,
                                            int config, int splits, void* ws, size_t ws_bytes,
                                            void* stream) {
  if (config < -1 || config >= fp8bw::gemm_num_configs())
    return fail(FP8BW_ERR_UNSUPPORTED, "config %d out of range", config);
  if (splits < 0) return fail(FP8BW_ERR_SHAPE, "splits must be >= 0");
  return gemm_blockwise_impl(a, lda, ra, ra_s_row, ra_s_kb, b, ldb, rb, rb_s_row, rb_s_kb, b_block,
                             M, N, K, out, ldo, out_dtype, config, splits, ws, ws_bytes, stream);
}

FP8BW_API int fp8_scaled_gemm_blockwise_kn(const void* a, int64_t lda, const float* ra,
                                           int64_t ra_s_row, int64_t ra_s_kb, const void* b_kn,
                                           int64_t ldb, const float* rb, int64_t rb_s_row,
                                           int64_t rb_s_kb, int b_block, int64_t M, int64_t N,
                                           int64_t K, void* out, int64_t ldo, int out_dtype,
                                           void* ws, size_t ws_bytes, void* stream) {
  return gemm_blockwise_impl(a, lda, ra, ra_s_row, ra_s_kb, b_kn, ldb, rb, rb_s_row, rb_s_kb,
                             b_block, M, N, K, out, ldo, out_dtype, -1, 0, ws, ws_bytes, stream,
                             nullptr, true);
}

static int check_bias(const void* bias) {
  if (bias && !aligned(bias, 2)) return fail(FP8BW_ERR_ALIGN, "bias must be 2-byte aligned");
  return FP8BW_OK;
}

FP8BW_API int fp8_scaled_gemm_blockwise_bias(const void* a, int64_t lda, const float* ra,
                                             int64_t ra_s_row, int64_t ra_s_kb, const void* b,
                                             int64_t ldb, const float* rb, int64_t rb_s_row,
                                             int64_t rb_s_kb, int b_block, int64_t M, int64_t N,
                                             int64_t K, const void* bias, void* out, int64_t ldo,
                                             int out_dtype, void* ws, size_t ws_bytes,
                                             void* stream) {
  int st = check_bias(bias);
  if (st != FP8BW_OK) return st;
  return gemm_blockwise_impl(a, lda, ra, ra_s_row, ra_s_kb, b, ldb, rb, rb_s_row, rb_s_kb, b_block,
                             M, N, K, out, ldo, out_dtype, -1, 0, ws, ws_bytes, stream, bias);
}

FP8BW_API int fp8_scaled_grouped_gemm_blockwise(
    const void* a, int64_t lda, const float* ra, int64_t ra_s_kb, const void* b, int64_t ldb,
    int64_t b_s_group, const float* rb, int64_t rb_s_row, int64_t rb_s_kb, int64_t rb_s_group,
    int groups, const int* group_end, int64_t M, int64_t N, int64_t K, void* out, int64_t ldo,
    int out_dtype, void* stream) {
  if (groups < 1 || groups > (1 << 20)) return fail(FP8BW_ERR_SHAPE, "groups=%d must be in [1, 2^20]", groups);
  int st = check_gemm_operands(a, lda, b, ldb, M, N, K, out, ldo, out_dtype);
  if (st != FP8BW_OK) return st;
  if (K % 128) return fail(FP8BW_ERR_SHAPE, "blockwise GEMM needs K %% 128 == 0 (K=%lld)", (long long)K);
  if (M == 0 || N == 0) return ok();
  if (!group_end) return fail(FP8BW_ERR_NULL, "group_end must be non-null");
  if (!aligned(group_end, 4)) return fail(FP8BW_ERR_ALIGN, "group_end must be 4-byte aligned");
  const int64_t kb = K / 128, nb = cdiv(N, 128);
  // B groups: each group's [N, K] block lies inside its stride, and the
  // last group's end below 2^48 elements.
  const int64_t b_extent = (N - 1) * ldb + K;
  if (b_s_group < b_extent || b_s_group % 16)
    return fail(FP8BW_ERR_LAYOUT, "b_s_group=%lld must be >= (N-1)*ldb + K and a multiple of 16", (long long)b_s_group);
  if (groups > 1 && b_s_group > (kMaxExtent - b_extent) / (groups - 1))
    return fail(FP8BW_ERR_LAYOUT, "b_s_group=%lld: %d groups reach past 2^48 elements", (long long)b_s_group, groups);
  if (kb > 0) {
    if (!ra || !rb) return fail(FP8BW_ERR_NULL, "ra and rb must be non-null");
    if (!aligned(ra, 4) || !aligned(rb, 4)) return fail(FP8BW_ERR_ALIGN, "ra/rb must be 4-byte aligned");
    if (kb > 1 && ra_s_kb < M) return fail(FP8BW_ERR_LAYOUT, "ra must be column-major: ra_s_kb >= M");
    if (!strides_injective(M, kb, 1, ra_s_kb))
      return fail(FP8BW_ERR_LAYOUT, "ra_s_kb=%lld reaches past 2^48 elements", (long long)ra_s_kb);
    if (!strides_injective(nb, kb, rb_s_row, rb_s_kb))
      return fail(FP8BW_ERR_LAYOUT, "rb strides (%lld, %lld) alias or are negative", (long long)rb_s_row, (long long)rb_s_kb);
    const int64_t rb_extent = (nb - 1) * used_stride(nb, rb_s_row) + (kb - 1) * used_stride(kb, rb_s_kb) + 1;
    if (groups > 1 && rb_s_group < rb_extent)
      return fail(FP8BW_ERR_LAYOUT, "rb_s_group=%lld overlaps a group's %lld scales", (long long)rb_s_group, (long long)rb_extent);
    if (groups > 1 && rb_s_group > (kMaxExtent - rb_extent) / (groups - 1))
      return fail(FP8BW_ERR_LAYOUT, "rb_s_group=%lld: %d groups reach past 2^48 elements", (long long)rb_s_group, groups);
  }
  fp8bw::GemmProblem p;
  p.a = a; p.lda = lda; p.b = b; p.ldb = ldb;
  p.ra = ra; p.ra_s_row = 1; p.ra_s_kb = used_stride(kb, ra_s_kb);
  p.rb = rb; p.rb_s_row = used_stride(nb, rb_s_row); p.rb_s_kb = used_stride(kb, rb_s_kb);
  p.out = out; p.ldo = ldo; p.M = M; p.N = N; p.K = K;
  p.mode = fp8bw::kBlockB128;
  p.out_kind = out_dtype == FP8BW_OUT_BF16 ? fp8bw::kOutBf16 : fp8bw::kOutF32;
  if (!fp8bw::grouped_gemm_ok(p, groups))
    return fail(FP8BW_ERR_UNSUPPORTED, "grouped GEMM problem not supported");
  return hip_status(fp8bw::launch_grouped_gemm(p, groups, group_end, b_s_group, rb_s_group,
                                               (hipStream_t)stream),
                    "fp8_scaled_grouped_gemm_blockwise");
}

static int gemm_tensorwise_impl(const void* a, int64_t lda, const float* ra, const void* b,
                                int64_t ldb, const float* rb, int64_t M, int64_t N, int64_t K,
                                void* out, int64_t ldo, int out_dtype, void* stream,
                                const void* bias) {
  int st = check_gemm_operands(a, lda, b, ldb, M, N, K, out, ldo, out_dtype);
  if (st != FP8BW_OK) return st;
  if (K % 16) return fail(FP8BW_ERR_SHAPE, "tensorwise GEMM needs K %% 16 == 0 (K=%lld)", (long long)K);
  if (M == 0 || N == 0) return ok();
  if (!ra || !rb) return fail(FP8BW_ERR_NULL, "ra and rb must be non-null");
  if (!aligned(ra, 4) || !aligned(rb, 4)) return fail(FP8BW_ERR_ALIGN, "ra/rb must be 4-byte aligned");
  fp8bw::GemmProblem p = {};
  p.a = a; p.lda = lda; p.b = b; p.ldb = ldb;
  p.ra = ra; p.rb = rb;
  p.out = out; p.ldo = ldo; p.M = M; p.N = N; p.K = K;
  p.mode = fp8bw::kTensorwise;
  p.out_kind = out_dtype == FP8BW_OUT_BF16 ? fp8bw::kOutBf16 : fp8bw::kOutF32;
  p.bias = bias;
  // No workspace argument: never split.
  const fp8bw::GemmPlan plan = fp8bw::gemm_plan(p, -1, 0, false);
  return hip_status(fp8bw::launch_gemm(p, plan, nullptr, (hipStream_t)stream), "fp8_scaled_gemm_tensorwise");
}

FP8BW_API int fp8_scaled_gemm_tensorwise(const void* a, int64_t lda, const float* ra,
                                         const void* b, int64_t ldb, const float* rb, int64_t M,
                                         int64_t N, int64_t K, void* out, int64_t ldo,
                                         int out_dtype, void* stream) {
  return gemm_tensorwise_impl(a, lda, ra, b, ldb, rb, M, N, K, out, ldo, out_dtype, stream, nullptr);
}

FP8BW_API int fp8_scaled_gemm_tensorwise_bias(const void* a, int64_t lda, const float* ra,
                                              const void* b, int64_t ldb, const float* rb,
                                              int64_t M, int64_t N, int64_t K, const void* bias,
                                              void* out, int64_t ldo, int out_dtype,
                                              void* stream) {
  int st = check_bias(bias);
  if (st != FP8BW_OK) return st;
  return gemm_tensorwise_impl(a, lda, ra, b, ldb, rb, M, N, K, out, ldo, out_dtype, stream, bias);
}

// ---------------------------------------------------------------------------
// Linear wrapper.  Workspace layout (each region 256-byte aligned):
//   [A codes][B codes][A recip][B recip][GEMM split-K partials]

namespace {

struct LinearLayout {
  int64_t gm, gn, gk;          // GEMM shape
  size_t a_codes, b_codes, a_recip, b_recip, gemm_ws, total;
};

// Fused-quantization wrapper (fp8_linear_fwd_save / fp8_linear_bwd).
// Saved buffer: [X^T codes K x M][X^T recip K x cdiv(M,128)]
// fwd_save ws:  [X codes][W codes][X recip][W recip][fwd GEMM partials]
// bwd ws:       [dY codes][dY^T codes][dY recip][dY^T recip]
//               [W^T codes][W^T recip][GEMM partials]
// W^T is quantized by the backward, right before the dgrad GEMM, rather than
// kept from the forward: the GEMM then finds its freshly written B operand
// in the chip's 256 MB memory-side cache (on the 16640 x 5120 x 8192 linear
// step, dgrad 585 against 660 us, for 27 us of quantizer), and the saved
// buffer holds only what the backward cannot recompute from its inputs.
struct SavedLayout {
  size_t xt_codes, xt_recip, total;
};

SavedLayout saved_layout(int64_t M, int64_t N, int64_t K) {
  SavedLayout S = {};
  size_t off = 0;
  (void)N;
  S.xt_codes = off; off += align_up((size_t)(K * M));
  S.xt_recip = off; off += align_up((size_t)(K * cdiv(M, 128)) * 4);
  S.total = off;
  return S;
}

struct FusedLayout {
  size_t a_codes, a_codes_t, a_recip, a_recip_t, b_codes, b_recip, gemm_ws, total;
};   // bwd: b_codes / b_recip hold W^T

FusedLayout fused_layout(int64_t M, int64_t N, int64_t K, int which) {
  FusedLayout F = {};
  size_t off = 0;
  if (which == 3) {   // fwd_save: X and W codes for the forward GEMM
    F.a_codes = off; off += align_up((size_t)(M * K));
    F.b_codes = off; off += align_up((size_t)(N * K));
    F.a_recip = off; off += align_up((size_t)(M * cdiv(K, 128)) * 4);
    F.b_recip = off; off += align_up((size_t)(cdiv(N, 128) * cdiv(K, 128)) * 4);
    F.gemm_ws = off; off += align_up(fp8bw_gemm_blockwise_ws_bytes(M, N, K));
  } else {            // bwd: dY and dY^T codes for dgrad and wgrad, W^T for dgrad
    F.a_codes = off; off += align_up((size_t)(M * N));
    F.a_codes_t = off; off += align_up((size_t)(N * M));
    F.a_recip = off; off += align_up((size_t)(M * cdiv(N, 128)) * 4);
    F.a_recip_t = off; off += align_up((size_t)(N * cdiv(M, 128)) * 4);
    F.b_codes = off; off += align_up((size_t)(K * N));
    F.b_recip = off; off += align_up((size_t)(cdiv(K, 128) * cdiv(N, 128)) * 4);
    F.gemm_ws = off;
    const size_t g1 = fp8bw_gemm_blockwise_ws_bytes(M, K, N), g2 = fp8bw_gemm_blockwise_ws_bytes(N, K, M);
    off += align_up(g1 > g2 ? g1 : g2);
  }
  F.total = off;
  return F;
}

LinearLayout linear_layout(int64_t M, int64_t N, int64_t K, int which) {
  LinearLayout L = {};
  if (which == 0) { L.gm = M; L.gn = N; L.gk = K; }
  else if (which == 1) { L.gm = M; L.gn = K; L.gk = N; }
  else { L.gm = N; L.gn = K; L.gk = M; }
  const int64_t kb = cdiv(L.gk, 128);
  size_t off = 0;
  L.a_codes = off; off += align_up((size_t)(L.gm * L.gk));
  L.b_codes = off; off += align_up((size_t)(L.gn * L.gk));
  L.a_recip = off; off += align_up((size_t)(L.gm * kb) * 4);
  // 128x128 B scales need cdiv(gn,128)*kb; 1x128 (wgrad) need gn*kb.
  L.b_recip = off; off += align_up((size_t)((which == 2 ? L.gn : cdiv(L.gn, 128)) * kb) * 4);
  L.gemm_ws = off; off += align_up(fp8bw_gemm_blockwise_ws_bytes(L.gm, L.gn, L.gk));
  L.total = off;
  return L;
}

int check_linear(const void* p0, const void* p1, void* out, int64_t M, int64_t N, int64_t K,
                 void* ws, size_t ws_bytes, int which) {
  if (M < 0 || N < 0 || K < 0) return fail(FP8BW_ERR_SHAPE, "negative dimension");
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(FP8BW_ERR_SHAPE, "dimension too large");
  if (M % 16 || N % 16 || K % 16) return fail(FP8BW_ERR_SHAPE, "M, N, K must be multiples of 16");
  const int64_t contraction = which == 0 ? K : which == 1 ? N : M;
  if (contraction % 128)
    return fail(FP8BW_ERR_SHAPE, "the contraction dimension (%lld) must be a multiple of 128", (long long)contraction);
  if (M == 0 || N == 0 || K == 0) return FP8BW_OK;
  if (!p0 || !p1 || !out) return fail(FP8BW_ERR_NULL, "inputs and output must be non-null");
  if (!aligned(p0, 16) || !aligned(p1, 16) || !aligned(out, 16))
    return fail(FP8BW_ERR_ALIGN, "tensors must be 16-byte aligned");
  const LinearLayout L = linear_layout(M, N, K, which);
  if (!ws || ws_bytes < L.total) return fail(FP8BW_ERR_WORKSPACE, "workspace needs %zu bytes", L.total);
  if (!aligned(ws, 256)) return fail(FP8BW_ERR_ALIGN, "ws must be 256-byte aligned");
  return FP8BW_OK;
}

}  // namespace

FP8BW_API size_t fp8bw_linear_ws_bytes(int64_t M, int64_t N, int64_t K, int which) {
  if (which < 0 || which > 4 || M <= 0 || N <= 0 || K <= 0) return 0;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
  if (which >= 3) return fused_layout(M, N, K, which).total;
  return linear_layout(M, N, K, which).total;
}

FP8BW_API size_t fp8bw_linear_saved_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
  return saved_layout(M, N, K).total;
}

static int zero_output(void* out, int64_t rows, int64_t cols, void* stream) {
  // Empty contraction: the product is all zeros (a fill kernel, not a memset
  // node, so the call stays safe to capture into a graph).
  return hip_status(fp8bw::launch_zero_bf16(out, rows, cols, (hipStream_t)stream), "zero output");
}

FP8BW_API int fp8_linear_fwd(const void* x, const void* w, void* y, int64_t M, int64_t N,
                             int64_t K, void* ws, size_t ws_bytes, void* stream) {
  int st = check_linear(x, w, y, M, N, K, ws, ws_bytes, 0);
  if (st != FP8BW_OK) return st;
  if (M == 0 || N == 0) return ok();
  if (K == 0) return zero_output(y, M, N, stream);
  const LinearLayout L = linear_layout(M, N, K, 0);
  uint8_t* base = (uint8_t*)ws;
  const int64_t kb = K / 128, nb = cdiv(N, 128);
  uint8_t* xq = base + L.a_codes;
  uint8_t* wq = base + L.b_codes;
  float* xr = (float*)(base + L.a_recip);
  float* wr = (float*)(base + L.b_recip);
  if ((st = fp8_blockwise_quant(x, M, K, K, FP8BW_BLOCK_1x128, 0, xq, K, xr, 1, M, stream))) return st;
  if ((st = fp8_blockwise_quant(w, N, K, K, FP8BW_BLOCK_128x128, 0, wq, K, wr, 1, nb, stream))) return st;
  (void)kb;
  return fp8_scaled_gemm_blockwise(xq, K, xr, 1, M, wq, K, wr, 1, nb, FP8BW_BLOCK_128x128, M, N, K,
                                   y, N, FP8BW_OUT_BF16, base + L.gemm_ws, ws_bytes - L.gemm_ws, stream);
}

FP8BW_API int fp8_linear_dgrad(const void* dy, const void* w, void* dx, int64_t M, int64_t N,
                               int64_t K, void* ws, size_t ws_bytes, void* stream) {
  int st = check_linear(dy, w, dx, M, N, K, ws, ws_bytes, 1);
  if (st != FP8BW_OK) return st;
  if (M == 0 || K == 0) return ok();
  if (N == 0) return zero_output(dx, M, K, stream);
  const LinearLayout L = linear_layout(M, N, K, 1);
  uint8_t* base = (uint8_t*)ws;
  const int64_t kbo = cdiv(K, 128);
  uint8_t* dyq = base + L.a_codes;
  uint8_t* wtq = base + L.b_codes;
  float* dyr = (float*)(base + L.a_recip);
  float* wtr = (float*)(base + L.b_recip);
  // dY: 1x128 along N, column-major scales dyr[m + nb*M].
  if ((st = fp8_blockwise_quant(dy, M, N, N, FP8BW_BLOCK_1x128, 0, dyq, N, dyr, 1, M, stream))) return st;
  // W^T [K, N] codes; scales indexed (K block, N block): wtr[kbo_i + nb*kbo].
  if ((st = fp8_blockwise_quant(w, N, K, K, FP8BW_BLOCK_128x128, 1, wtq, N, wtr, 1, kbo, stream))) return st;
  return fp8_scaled_gemm_blockwise(dyq, N, dyr, 1, M, wtq, N, wtr, 1, kbo, FP8BW_BLOCK_128x128, M, K, N,
                                   dx, K, FP8BW_OUT_BF16, base + L.gemm_ws, ws_bytes - L.gemm_ws, stream);
}

FP8BW_API int fp8_linear_wgrad(const void* dy, const void* x, void* dw, int64_t M, int64_t N,
                               int64_t K, void* ws, size_t ws_bytes, void* stream) {
  int st = check_linear(dy, x, dw, M, N, K, ws, ws_bytes, 2);
  if (st != FP8BW_OK) return st;
  if (N == 0 || K == 0) return ok();
  if (M == 0) return zero_output(dw, N, K, stream);
  const LinearLayout L = linear_layout(M, N, K, 2);
  uint8_t* base = (uint8_t*)ws;
  uint8_t* dytq = base + L.a_codes;
  uint8_t* xtq = base + L.b_codes;
  float* dytr = (float*)(base + L.a_recip);
  float* xtr = (float*)(base + L.b_recip);
  // dY^T [N, M] with 1x128 blocks along M: dytr[n + mb*N].
  if ((st = fp8_blockwise_quant(dy, M, N, N, FP8BW_BLOCK_1x128, 1, dytq, M, dytr, 1, N, stream))) return st;
  // X^T [K, M]: xtr[k + mb*K].
  if ((st = fp8_blockwise_quant(x, M, K, K, FP8BW_BLOCK_1x128, 1, xtq, M, xtr, 1, K, stream))) return st;
  return fp8_scaled_gemm_blockwise(dytq, M, dytr, 1, N, xtq, M, xtr, 1, K, FP8BW_BLOCK_1x128, N, K, M,
                                   dw, K, FP8BW_OUT_BF16, base + L.gemm_ws, ws_bytes - L.gemm_ws, stream);
}

namespace {

int check_fused(const void* p0, const void* p1, int64_t M, int64_t N, int64_t K, const void* saved,
                size_t saved_bytes, void* ws, size_t ws_bytes, int which) {
  if (M < 0 || N < 0 || K < 0) return fail(FP8BW_ERR_SHAPE, "negative dimension");
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return fail(FP8BW_ERR_SHAPE, "dimension too large");
  if (M % 16 || N % 16 || K % 16) return fail(FP8BW_ERR_SHAPE, "M, N, K must be multiples of 16");
  if (which == 3 && K % 128) return fail(FP8BW_ERR_SHAPE, "K (%lld) must be a multiple of 128", (long long)K);
  if (which == 4 && (M % 128 || N % 128))
    return fail(FP8BW_ERR_SHAPE, "M (%lld) and N (%lld) must be multiples of 128", (long long)M, (long long)N);
  if (M == 0 || N == 0 || K == 0) return FP8BW_OK;
  if (!p0 || !p1 || !saved) return fail(FP8BW_ERR_NULL, "inputs and the saved buffer must be non-null");
  if (!aligned(p0, 16) || !aligned(p1, 16)) return fail(FP8BW_ERR_ALIGN, "tensors must be 16-byte aligned");
  const SavedLayout S = saved_layout(M, N, K);
  if (saved_bytes < S.total) return fail(FP8BW_ERR_WORKSPACE, "saved buffer needs %zu bytes", S.total);
  if (!aligned(saved, 256)) return fail(FP8BW_ERR_ALIGN, "saved must be 256-byte aligned");
  const FusedLayout F = fused_layout(M, N, K, which);
  if (!ws || ws_bytes < F.total) return fail(FP8BW_ERR_WORKSPACE, "workspace needs %zu bytes", F.total);
  if (!aligned(ws, 256)) return fail(FP8BW_ERR_ALIGN, "ws must be 256-byte aligned");
  return FP8BW_OK;
}

}  // namespace

FP8BW_API int fp8_linear_fwd_save(const void* x, const void* w, void* y, int64_t M, int64_t N,
                                  int64_t K, void* saved, size_t saved_bytes, void* ws,
                                  size_t ws_bytes, void* stream) {
  int st = check_fused(x, w, M, N, K, saved, saved_bytes, ws, ws_bytes, 3);
  if (st != FP8BW_OK) return st;
  if (M == 0 || N == 0 || K == 0) return ok();
  if (!y) return fail(FP8BW_ERR_NULL, "y must be non-null");
  if (!aligned(y, 16)) return fail(FP8BW_ERR_ALIGN, "y must be 16-byte aligned");
  const SavedLayout S = saved_layout(M, N, K);
  const FusedLayout F = fused_layout(M, N, K, 3);
  uint8_t* base = (uint8_t*)ws;
  uint8_t* sv = (uint8_t*)saved;
  const int64_t nb = cdiv(N, 128);
  uint8_t* xq = base + F.a_codes;
  uint8_t* wq = base + F.b_codes;
  float* xr = (float*)(base + F.a_recip);
  float* wr = (float*)(base + F.b_recip);
  // X: codes for the forward (1x128 along K, xr[m + kb*M]) and X^T for the
  // weight gradient (1x128 along M, xtr[k + mb*K]) from one read.  X^T is
  // not read until the backward: its codes are streamed out with
  // nontemporal stores, so that X's codes stay in the memory-side cache for
  // the forward GEMM.
  if ((st = quant_dual_impl(x, M, K, K, FP8BW_BLOCK_1x128, xq, K, xr, 1, M, sv + S.xt_codes, M,
                            (float*)(sv + S.xt_recip), 1, K, true, stream)))
    return st;
  // W: 128x128 codes, wr[nb_i + kb*nb] (W^T is quantized by the backward).
  if ((st = fp8_blockwise_quant(w, N, K, K, FP8BW_BLOCK_128x128, 0, wq, K, wr, 1, nb, stream)))
    return st;
  return fp8_scaled_gemm_blockwise(xq, K, xr, 1, M, wq, K, wr, 1, nb, FP8BW_BLOCK_128x128, M, N, K,
                                   y, N, FP8BW_OUT_BF16, base + F.gemm_ws, ws_bytes - F.gemm_ws, stream);
}

FP8BW_API int fp8_linear_bwd(const void* dy, const void* w, const void* saved, size_t saved_bytes,
                             void* dx, void* dw, int64_t M, int64_t N, int64_t K, void* ws,
                             size_t ws_bytes, void* stream) {
  int st = check_fused(dy, w, M, N, K, saved, saved_bytes, ws, ws_bytes, 4);
  if (st != FP8BW_OK) return st;
  if (K == 0) return ok();
  if (M == 0) return dw ? zero_output(dw, N, K, stream) : ok();
  if (N == 0) return dx ? zero_output(dx, M, K, stream) : ok();
  if ((dx && !aligned(dx, 16)) || (dw && !aligned(dw, 16)))
    return fail(FP8BW_ERR_ALIGN, "dx and dw must be 16-byte aligned");
  if (!dx && !dw) return ok();
  const SavedLayout S = saved_layout(M, N, K);
  const FusedLayout F = fused_layout(M, N, K, 4);
  uint8_t* base = (uint8_t*)ws;
  const uint8_t* sv = (const uint8_t*)saved;
  const int64_t kbo = cdiv(K, 128);
  uint8_t* dyq = base + F.a_codes;
  uint8_t* dytq = base + F.a_codes_t;
  float* dyr = (float*)(base + F.a_recip);
  float* dytr = (float*)(base + F.a_recip_t);
  uint8_t* wtq = base + F.b_codes;
  float* wtr = (float*)(base + F.b_recip);
  // dY: 1x128 along N (dyr[m + nb*M]) for dgrad and 1x128 along M
  // (dytr[n + mb*N]) for wgrad, from one read.  Plain stores for dY^T:
  // nontemporal ones measured slower here (dgrad 590-599 against 585-588
  // us on the 16640 x 5120 x 8192 step).
  if ((st = quant_dual_impl(dy, M, N, N, FP8BW_BLOCK_1x128, dyq, N, dyr, 1, M, dytq, M, dytr, 1, N,
                            false, stream)))
    return st;
  if (dx) {
    // W^T [K, N] codes, wtr[kb_i + nb_i*kbo], written just before their GEMM.
    if ((st = fp8_blockwise_quant(w, N, K, K, FP8BW_BLOCK_128x128, 1, wtq, N, wtr, 1, kbo, stream)))
      return st;
    if ((st = fp8_scaled_gemm_blockwise(dyq, N, dyr, 1, M, wtq, N, wtr, 1, kbo, FP8BW_BLOCK_128x128,
                                        M, K, N, dx, K, FP8BW_OUT_BF16, base + F.gemm_ws,
                                        ws_bytes - F.gemm_ws, stream)))
      return st;
  }
  if (dw)
    return fp8_scaled_gemm_blockwise(dytq, M, dytr, 1, N, sv + S.xt_codes, M,
                                     (const float*)(sv + S.xt_recip), 1, K, FP8BW_BLOCK_1x128, N, K,
                                     M, dw, K, FP8BW_OUT_BF16, base + F.gemm_ws,
                                     ws_bytes - F.gemm_ws, stream);
  return ok();
}
