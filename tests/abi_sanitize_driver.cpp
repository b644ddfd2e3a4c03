// Host-side driver for the sanitizer build of the C ABI (see
// tests/test_abi_sanitizers.py).  It is linked against the library's
// sources with the host code compiled under AddressSanitizer and
// UndefinedBehaviorSanitizer, and makes only calls that are answered on the
// host: argument
// validation (including extreme sizes, strides and leading dimensions whose
// products overflow int64), zero-sized calls, workspace and plan queries,
// and per-thread error messages.  A call that passes validation reaches a
// kernel launch, which fails on a host without a GPU, so it reports
// FP8BW_ERR_HIP and touches no memory; where a GPU is visible the driver
// runs nothing and exits with status 77 (its host pointers would reach the
// kernels).  Exit status 0 when every check holds; a sanitizer report
// aborts the process.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "fp8bw.h"

namespace {

int failures = 0;
int checks = 0;

#define CHECK(cond)                                                          \
  do {                                                                       \
    ++checks;                                                                \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      ++failures;                                                            \
    }                                                                        \
  } while (0)

// Status of a call, with the per-thread message checked for consistency: a
// rejected call leaves a non-empty message, an accepted one an empty one.
#define EXPECT_STATUS(call, want)                                                          \
  do {                                                                                     \
    const int st_ = (call);                                                                \
    ++checks;                                                                              \
    if (st_ != (want)) {                                                                   \
      std::fprintf(stderr, "line %d: %s -> %s (%s), want %s\n", __LINE__, #call,           \
                   fp8bw_status_str(st_), fp8bw_last_error(), fp8bw_status_str(want));     \
      ++failures;                                                                          \
    }                                                                                      \
    CHECK((st_ == FP8BW_OK) == (std::strlen(fp8bw_last_error()) == 0));                    \
  } while (0)

constexpr int64_t kI64Max = INT64_MAX;
constexpr int64_t kI64Min = INT64_MIN;
constexpr int64_t k2p48 = (int64_t)1 << 48;

// Host buffers standing in for device pointers; never dereferenced by the
// library (every call below is rejected, zero-sized or fails at launch).
alignas(256) unsigned char buf_a[4096];
alignas(256) unsigned char buf_b[4096];
alignas(256) unsigned char buf_out[4096];
alignas(256) float buf_s[1024];
alignas(256) unsigned char buf_ws[4096];

const int64_t kDims[] = {kI64Min, -1, 0, 1, 15, 16, 127, 128, 129, 256, 4096,
                         ((int64_t)1 << 30), ((int64_t)1 << 30) + 128, ((int64_t)1 << 32),
                         k2p48, kI64Max};
const int64_t kStrides[] = {kI64Min, -1, 0, 1, 16, 128, 4096, ((int64_t)1 << 31),
                            k2p48 - 16, k2p48, ((int64_t)1 << 62), kI64Max - 15, kI64Max};

bool known_status(int st) { return st >= FP8BW_OK && st <= FP8BW_ERR_HIP; }

void quant_validation() {
  // Exact statuses.
  EXPECT_STATUS(fp8_blockwise_quant(nullptr, 128, 128, 128, FP8BW_BLOCK_1x128, 0, buf_out, 128,
                                    buf_s, 1, 128, nullptr), FP8BW_ERR_NULL);
  EXPECT_STATUS(fp8_blockwise_quant(buf_a, -1, 128, 128, FP8BW_BLOCK_1x128, 0, buf_out, 128,
                                    buf_s, 1, 128, nullptr), FP8BW_ERR_SHAPE);
  EXPECT_STATUS(fp8_blockwise_quant(buf_a, 128, 120, 128, FP8BW_BLOCK_1x128, 0, buf_out, 128,
                                    buf_s, 1, 128, nullptr), FP8BW_ERR_SHAPE);
  EXPECT_STATUS(fp8_blockwise_quant(buf_a, 128, 128, 128, 7, 0, buf_out, 128, buf_s, 1, 128,
                                    nullptr), FP8BW_ERR_UNSUPPORTED);
  EXPECT_STATUS(fp8_blockwise_quant(buf_a + 2, 128, 128, 128, FP8BW_BLOCK_1x128, 0, buf_out, 128,
                                    buf_s, 1, 128, nullptr), FP8BW_ERR_ALIGN);
  EXPECT_STATUS(fp8_blockwise_quant(buf_a, 0, 128, 128, FP8BW_BLOCK_1x128, 0, nullptr, 128,
                                    nullptr, 1, 1, nullptr), FP8BW_OK);
  // Scale strides that alias, and strides whose products overflow int64.
  EXPECT_STATUS(fp8_blockwise_quant(buf_a, 256, 256, 256, FP8BW_BLOCK_1x128, 0, buf_out, 256,
                                    buf_s, 1, 255, nullptr), FP8BW_ERR_LAYOUT);
  EXPECT_STATUS(fp8_blockwise_quant(buf_a, 256, 256, 256, FP8BW_BLOCK_1x128, 0, buf_out, 256,
                                    buf_s, kI64Max, 1, nullptr), FP8BW_ERR_LAYOUT);
  EXPECT_STATUS(fp8_blockwise_quant(buf_a, 256, 256, 256, FP8BW_BLOCK_1x128, 0, buf_out, 256,
                                    buf_s, 1, kI64Max, nullptr), FP8BW_ERR_LAYOUT);
  EXPECT_STATUS(fp8_blockwise_quant(buf_a, 256, 256, 256, FP8BW_BLOCK_1x128, 0, buf_out, 256,
                                    buf_s, (int64_t)1 << 41, 1, nullptr), FP8BW_ERR_LAYOUT);
  // Leading dimensions: the last element's offset must stay below 2^48.
  EXPECT_STATUS(fp8_blockwise_quant(buf_a, 2, 128, k2p48 - 256, FP8BW_BLOCK_1x128, 0, buf_out,
                                    128, buf_s, 1, 2, nullptr), FP8BW_ERR_HIP);
  EXPECT_STATUS(fp8_blockwise_quant(buf_a, 2, 128, k2p48, FP8BW_BLOCK_1x128, 0, buf_out, 128,
                                    buf_s, 1, 2, nullptr), FP8BW_ERR_LAYOUT);
  EXPECT_STATUS(fp8_blockwise_quant(buf_a, 3, 128, kI64Max - 7, FP8BW_BLOCK_1x128, 0, buf_out,
                                    128, buf_s, 1, 3, nullptr), FP8BW_ERR_LAYOUT);
  EXPECT_STATUS(fp8_blockwise_quant(buf_a, 16, 128, 128, FP8BW_BLOCK_128x128, 1, buf_out,
                                    kI64Max - 15, buf_s, 1, 1, nullptr), FP8BW_ERR_LAYOUT);
  // One row: its leading dimension is never used.
  EXPECT_STATUS(fp8_blockwise_quant(buf_a, 1, 128, kI64Max - 7, FP8BW_BLOCK_1x128, 0, buf_out,
                                    kI64Max - 15, buf_s, 1, 1, nullptr), FP8BW_ERR_HIP);
  // Dual: overlapping code buffers; and extreme strides on the second output.
  EXPECT_STATUS(fp8_blockwise_quant_dual(buf_a, 128, 128, 128, FP8BW_BLOCK_1x128, buf_out, 128,
                                         buf_s, 1, 128, buf_out + 64, 128, buf_s + 512, 1, 128, 0,
                                         nullptr), FP8BW_ERR_LAYOUT);
  EXPECT_STATUS(fp8_blockwise_quant_dual(buf_a, 128, 128, 128, FP8BW_BLOCK_1x128, buf_out, 128,
                                         buf_s, 1, 128, buf_b, kI64Max - 15, buf_s + 512, 1, 128,
                                         1, nullptr), FP8BW_ERR_LAYOUT);

  // Sweep: every combination of extreme sizes and strides returns a known
  // status without undefined behaviour.
  for (int block : {FP8BW_BLOCK_1x128, FP8BW_BLOCK_128x128}) {
    for (int tr : {0, 1}) {
      for (int64_t rows : kDims) {
        for (int64_t cols : kDims) {
          for (int64_t ld : kStrides) {
            for (int64_t rs : kStrides) {
              // ld < cols (or rows) is rejected as a layout error; a call
              // that passes validation fails at launch.
              const int st = fp8_blockwise_quant(buf_a, rows, cols, ld, block, tr, buf_out, ld,
                                                 buf_s, 1, rs, nullptr);
              CHECK(known_status(st));
              const int st2 = fp8_blockwise_quant(buf_a, rows, cols, ld, block, tr, buf_out, ld,
                                                  buf_s, rs, 1, nullptr);
              CHECK(known_status(st2));
            }
          }
        }
      }
    }
  }
  for (int64_t rows : kDims)
    for (int64_t cols : kDims)
      for (int64_t ld : kStrides) {
        CHECK(known_status(fp8_blockwise_quant_dual(buf_a, rows, cols, ld, FP8BW_BLOCK_1x128,
                                                    buf_out, ld, buf_s, 1, ld, buf_b, ld,
                                                    buf_s + 512, 1, ld, (int)(ld & 1),
                                                    nullptr)));
      }
}

void tensorwise_validation() {
  for (int64_t rows : kDims)
    for (int64_t cols : kDims) {
      const size_t ws = fp8bw_tensorwise_quant_ws_bytes(rows, cols);
      CHECK(ws >= 4 && ws <= 4096 && ws % 256 == 0);
      for (int64_t ld : kStrides) {
        CHECK(known_status(fp8_tensorwise_quant(buf_a, rows, cols, ld, buf_out, ld, buf_s,
                                                buf_ws, sizeof(buf_ws), nullptr)));
        CHECK(known_status(fp8_tensorwise_quant_noalloc(buf_a, rows, cols, ld, buf_out, ld,
                                                        buf_s, nullptr)));
      }
    }
  EXPECT_STATUS(fp8_tensorwise_quant(buf_a, 256, 1024, 1024, buf_out, 1024, buf_s, buf_ws, 4,
                                     nullptr), FP8BW_ERR_WORKSPACE);
  EXPECT_STATUS(fp8_tensorwise_quant(buf_a, 256, 1024, 1024, buf_out, 1024, buf_s, nullptr,
                                     4096, nullptr), FP8BW_ERR_WORKSPACE);
  EXPECT_STATUS(fp8_tensorwise_quant_noalloc(buf_a, 256, 1024, 1024, buf_out, 1024, nullptr,
                                             nullptr), FP8BW_ERR_NULL);
  EXPECT_STATUS(fp8_tensorwise_quant_noalloc(buf_a, 2, 1024, kI64Max - 7, buf_out, 1024, buf_s,
                                             nullptr), FP8BW_ERR_LAYOUT);
}

void gemm_validation() {
  const float* s = buf_s;
  // Exact statuses.
  EXPECT_STATUS(fp8_scaled_gemm_blockwise(buf_a, 112, s, 1, 64, buf_b, 112, s, 1, 1,
                                          FP8BW_BLOCK_128x128, 64, 64, 112, buf_out, 64,
                                          FP8BW_OUT_BF16, nullptr, 0, nullptr), FP8BW_ERR_SHAPE);
  EXPECT_STATUS(fp8_scaled_gemm_blockwise(buf_a, 128, s, 1, 64, buf_b, 128, s, 1, 1, 9, 64, 64,
                                          128, buf_out, 64, FP8BW_OUT_BF16, nullptr, 0, nullptr),
                FP8BW_ERR_UNSUPPORTED);
  EXPECT_STATUS(fp8_scaled_gemm_blockwise(buf_a, 128, s, 1, 64, buf_b, 128, s, 1, 1,
                                          FP8BW_BLOCK_128x128, 64, 64, 128, buf_out, 64, 5,
                                          nullptr, 0, nullptr), FP8BW_ERR_UNSUPPORTED);
  EXPECT_STATUS(fp8_scaled_gemm_blockwise(buf_a, 128, s, 1, 64, buf_b, 128, s, 1, 1,
                                          FP8BW_BLOCK_128x128, 0, 64, 128, nullptr, 64,
                                          FP8BW_OUT_BF16, nullptr, 0, nullptr), FP8BW_OK);
  // Leading dimensions at and past the 2^48-element bound.
  EXPECT_STATUS(fp8_scaled_gemm_blockwise(buf_a, k2p48 - 256, s, 1, 2, buf_b, 128, s, 1, 1,
                                          FP8BW_BLOCK_128x128, 2, 64, 128, buf_out, 64,
                                          FP8BW_OUT_BF16, nullptr, 0, nullptr), FP8BW_ERR_HIP);
  EXPECT_STATUS(fp8_scaled_gemm_blockwise(buf_a, k2p48, s, 1, 2, buf_b, 128, s, 1, 1,
                                          FP8BW_BLOCK_128x128, 2, 64, 128, buf_out, 64,
                                          FP8BW_OUT_BF16, nullptr, 0, nullptr), FP8BW_ERR_LAYOUT);
  EXPECT_STATUS(fp8_scaled_gemm_blockwise(buf_a, 128, s, 1, 2, buf_b, kI64Max - 15, s, 1, 1,
                                          FP8BW_BLOCK_128x128, 2, 64, 128, buf_out, 64,
                                          FP8BW_OUT_BF16, nullptr, 0, nullptr), FP8BW_ERR_LAYOUT);
  EXPECT_STATUS(fp8_scaled_gemm_blockwise(buf_a, 128, s, 1, 2, buf_b, 128, s, 1, 1,
                                          FP8BW_BLOCK_128x128, 2, 64, 128, buf_out, kI64Max,
                                          FP8BW_OUT_F32, nullptr, 0, nullptr), FP8BW_ERR_LAYOUT);
  // Scale strides whose products overflow, and the unused stride of a
  // size-1 scale dimension (any value: one 128-column block of B, one K
  // block) on a problem the large tiles accept.
  EXPECT_STATUS(fp8_scaled_gemm_blockwise(buf_a, 128, s, 1, kI64Max, buf_b, 128, s, 1, 1,
                                          FP8BW_BLOCK_128x128, 2, 64, 256, buf_out, 64,
                                          FP8BW_OUT_BF16, nullptr, 0, nullptr), FP8BW_ERR_LAYOUT);
  EXPECT_STATUS(fp8_scaled_gemm_blockwise(buf_a, 128, s, kI64Max, 1, buf_b, 128, s, 1, 1,
                                          FP8BW_BLOCK_128x128, 2, 64, 256, buf_out, 64,
                                          FP8BW_OUT_BF16, nullptr, 0, nullptr), FP8BW_ERR_LAYOUT);
  EXPECT_STATUS(fp8_scaled_gemm_blockwise(buf_a, 128, s, 1, 256, buf_b, 128, s, kI64Max, kI64Max,
                                          FP8BW_BLOCK_128x128, 256, 128, 128, buf_out, 128,
                                          FP8BW_OUT_BF16, nullptr, 0, nullptr), FP8BW_ERR_HIP);
  EXPECT_STATUS(fp8_scaled_gemm_blockwise_cfg(buf_a, 128, s, 1, 256, buf_b, 128, s, kI64Max,
                                              kI64Max, FP8BW_BLOCK_128x128, 256, 128, 128,
                                              buf_out, 128, FP8BW_OUT_BF16, 2, 1, nullptr, 0,
                                              nullptr), FP8BW_ERR_HIP);
  // Forced splits beyond the K blocks, and a split whose workspace is absent.
  EXPECT_STATUS(fp8_scaled_gemm_blockwise_cfg(buf_a, 256, s, 1, 64, buf_b, 256, s, 1, 1,
                                              FP8BW_BLOCK_128x128, 64, 64, 256, buf_out, 64,
                                              FP8BW_OUT_BF16, -1, 3, nullptr, 0, nullptr),
                FP8BW_ERR_SHAPE);
  EXPECT_STATUS(fp8_scaled_gemm_blockwise_cfg(buf_a, 256, s, 1, 64, buf_b, 256, s, 1, 1,
                                              FP8BW_BLOCK_128x128, 64, 64, 256, buf_out, 64,
                                              FP8BW_OUT_BF16, -1, 2, nullptr, 0, nullptr),
                FP8BW_ERR_WORKSPACE);
  EXPECT_STATUS(fp8_scaled_gemm_blockwise_cfg(buf_a, 256, s, 1, 64, buf_b, 256, s, 1, 1,
                                              FP8BW_BLOCK_128x128, 64, 64, 256, buf_out, 64,
                                              FP8BW_OUT_BF16, 99, 0, nullptr, 0, nullptr),
                FP8BW_ERR_UNSUPPORTED);
  EXPECT_STATUS(fp8_scaled_gemm_blockwise_bias(buf_a, 128, s, 1, 64, buf_b, 128, s, 1, 1,
                                               FP8BW_BLOCK_128x128, 64, 64, 128, buf_a + 1,
                                               buf_out, 64, FP8BW_OUT_BF16, nullptr, 0, nullptr),
                FP8BW_ERR_ALIGN);
  EXPECT_STATUS(fp8_scaled_gemm_tensorwise(buf_a, 16, s, buf_b, 16, s, 0, 32, 32, buf_out, 32,
                                           FP8BW_OUT_F32, nullptr), FP8BW_OK);
  EXPECT_STATUS(fp8_scaled_gemm_tensorwise(buf_a, 32, s, buf_b, 32, s, 32, 32, 24, buf_out, 32,
                                           FP8BW_OUT_F32, nullptr), FP8BW_ERR_SHAPE);

  // Sweep over extreme sizes and strides, every configuration and split.
  const int ncfg = fp8bw_gemm_num_configs();
  CHECK(ncfg >= 1);
  for (int64_t M : kDims)
    for (int64_t N : kDims)
      for (int64_t K : {(int64_t)-128, (int64_t)0, (int64_t)128, (int64_t)4096,
                        ((int64_t)1 << 30), kI64Max - 127}) {
        for (int64_t ld : kStrides) {
          for (int b_block : {FP8BW_BLOCK_128x128, FP8BW_BLOCK_1x128}) {
            CHECK(known_status(fp8_scaled_gemm_blockwise(buf_a, ld, s, 1, ld, buf_b, ld, s, ld, 1,
                                                         b_block, M, N, K, buf_out, ld,
                                                         FP8BW_OUT_F32, buf_ws, sizeof(buf_ws),
                                                         nullptr)));
            for (int cfg = -1; cfg < ncfg; ++cfg)
              for (int sp : {0, 1, 2, 65535, 1 << 30})
                CHECK(known_status(fp8_scaled_gemm_blockwise_cfg(
                    buf_a, ld, s, ld, 1, buf_b, ld, s, 1, ld, b_block, M, N, K, buf_out, ld,
                    FP8BW_OUT_BF16, cfg, sp, buf_ws, sizeof(buf_ws), nullptr)));
          }
          CHECK(known_status(fp8_scaled_gemm_tensorwise(buf_a, ld, s, buf_b, ld, s, M, N, K,
                                                        buf_out, ld, FP8BW_OUT_BF16, nullptr)));
          for (int b_block : {FP8BW_BLOCK_128x128, FP8BW_BLOCK_1x128})
            CHECK(known_status(fp8_scaled_gemm_blockwise_kn(
                buf_a, ld, s, 1, ld, buf_b, ld, s, 1, ld, b_block, M, N, K, buf_out, ld,
                FP8BW_OUT_BF16, buf_ws, sizeof(buf_ws), nullptr)));
        }
      }
}

// B in [K, N] layout: ldb >= N, and the large tiles' limits.
void gemm_kn_validation() {
  const float* s = buf_s;
  auto kn = [&](int64_t M, int64_t N, int64_t K, int64_t ldb) {
    return fp8_scaled_gemm_blockwise_kn(buf_a, 256, s, 1, 512, buf_b, ldb, s, 1, 4,
                                        FP8BW_BLOCK_128x128, M, N, K, buf_out, 512,
                                        FP8BW_OUT_BF16, nullptr, 0, nullptr);
  };
  EXPECT_STATUS(kn(512, 512, 256, 256), FP8BW_ERR_LAYOUT);          // ldb < N
  EXPECT_STATUS(kn(512, 512, 256, kI64Max - 15), FP8BW_ERR_LAYOUT);  // past 2^48
  EXPECT_STATUS(kn(128, 512, 256, 512), FP8BW_ERR_UNSUPPORTED);      // M < 256
  EXPECT_STATUS(kn(512, 336, 256, 512), FP8BW_ERR_UNSUPPORTED);      // N % 64, 128x128 scales
  EXPECT_STATUS(kn(512, 512, 256, (int64_t)1 << 23), FP8BW_ERR_UNSUPPORTED);  // 256 ldb >= 2^31
  EXPECT_STATUS(kn(512, 512, 256, 512), FP8BW_ERR_HIP);              // valid; no GPU here
}

void grouped_validation() {
  const float* s = buf_s;
  const int* ends = (const int*)buf_ws;
  EXPECT_STATUS(fp8_scaled_grouped_gemm_blockwise(buf_a, 128, s, 256, buf_b, 128, 128 * 128, s,
                                                  1, 1, 1, 0, ends, 256, 128, 128, buf_out, 128,
                                                  FP8BW_OUT_BF16, nullptr), FP8BW_ERR_SHAPE);
  EXPECT_STATUS(fp8_scaled_grouped_gemm_blockwise(buf_a, 128, s, 256, buf_b, 128, 128 * 128, s,
                                                  1, 1, 1, 2, nullptr, 256, 128, 128, buf_out,
                                                  128, FP8BW_OUT_BF16, nullptr), FP8BW_ERR_NULL);
  // Group stride inside a group, and group strides whose products overflow.
  EXPECT_STATUS(fp8_scaled_grouped_gemm_blockwise(buf_a, 128, s, 256, buf_b, 128, 128 * 127, s,
                                                  1, 1, 1, 2, ends, 256, 128, 128, buf_out, 128,
                                                  FP8BW_OUT_BF16, nullptr), FP8BW_ERR_LAYOUT);
  EXPECT_STATUS(fp8_scaled_grouped_gemm_blockwise(buf_a, 128, s, 256, buf_b, 128,
                                                  kI64Max - 15, s, 1, 1, 1, 3, ends, 256, 128,
                                                  128, buf_out, 128, FP8BW_OUT_BF16, nullptr),
                FP8BW_ERR_LAYOUT);
  EXPECT_STATUS(fp8_scaled_grouped_gemm_blockwise(buf_a, 128, s, 256, buf_b, 128, 128 * 128, s,
                                                  1, 1, kI64Max, 3, ends, 256, 128, 128, buf_out,
                                                  128, FP8BW_OUT_BF16, nullptr), FP8BW_ERR_LAYOUT);
  EXPECT_STATUS(fp8_scaled_grouped_gemm_blockwise(buf_a, 128, s, kI64Max, buf_b, 128, 128 * 128,
                                                  s, 1, 2, 2, 2, ends, 256, 128, 256, buf_out, 128,
                                                  FP8BW_OUT_BF16, nullptr), FP8BW_ERR_LAYOUT);
  // Largest group strides that still fit below 2^48: accepted (fails at launch).
  EXPECT_STATUS(fp8_scaled_grouped_gemm_blockwise(buf_a, 128, s, 256, buf_b, 128,
                                                  (k2p48 - 128 * 128) / 16 * 16, s, 1, 1, 1, 2,
                                                  ends, 256, 128, 128, buf_out, 128,
                                                  FP8BW_OUT_BF16, nullptr), FP8BW_ERR_HIP);
  for (int64_t M : kDims)
    for (int64_t N : kDims)
      for (int64_t st : kStrides)
        for (int groups : {-1, 0, 1, 2, 1 << 20, (1 << 20) + 1}) {
          CHECK(known_status(fp8_scaled_grouped_gemm_blockwise(
              buf_a, 128, s, st, buf_b, 128, st, s, 1, st, st, groups, ends, M, N, 128, buf_out,
              N > 0 ? N : 1, FP8BW_OUT_BF16, nullptr)));
        }
}

void queries() {
  for (int64_t M : kDims)
    for (int64_t N : kDims)
      for (int64_t K : kDims) {
        const size_t ws = fp8bw_gemm_blockwise_ws_bytes(M, N, K);
        for (int sp : {-1, 0, 1, 2, 65535, 1 << 30}) {
          const size_t w = fp8bw_gemm_ws_bytes_for_split(M, N, sp);
          if (sp <= 1 || M <= 0 || N <= 0) CHECK(w == 0);
          else CHECK(w >= (size_t)sp * sizeof(float));   // saturates, never wraps
        }
        for (int which = -1; which <= 5; ++which) {
          const size_t lw = fp8bw_linear_ws_bytes(M, N, K, which);
          CHECK(lw % 256 == 0);
          if (which < 0 || which > 4) CHECK(lw == 0);
        }
        CHECK(fp8bw_linear_saved_bytes(M, N, K) % 256 == 0);
        for (int b_block : {FP8BW_BLOCK_1x128, FP8BW_BLOCK_128x128}) {
          int64_t info[6] = {-7, -7, -7, -7, -7, -7};
          const int st = fp8bw_gemm_blockwise_plan(M, N, K, b_block, info);
          const bool valid = M > 0 && N > 0 && K > 0 && M <= (1 << 30) && N <= (1 << 30) &&
                             K <= (1 << 30) && K % 128 == 0;
          CHECK((st == FP8BW_OK) == valid);
          if (st != FP8BW_OK) {
            CHECK(info[0] == -7);
            continue;
          }
          CHECK(info[0] >= 0 && info[0] < fp8bw_gemm_num_configs());
          CHECK(info[1] >= 1 && info[2] >= 1 && !(info[1] > 1 && info[2] > 1));
          CHECK(info[1] <= K / 128 && info[2] <= K / 128);
          CHECK(info[4] >= 0 && info[4] <= info[3] && info[3] >= 1);
          CHECK((info[4] < info[3]) == (info[2] > 1));
          CHECK((info[5] > 0) == (info[1] > 1 || info[2] > 1));
          CHECK((size_t)info[5] <= ws);
          if (info[1] > 1) CHECK((size_t)info[5] == fp8bw_gemm_ws_bytes_for_split(M, N, (int)info[1]));
        }
      }
  CHECK(fp8bw_gemm_blockwise_plan(128, 128, 128, FP8BW_BLOCK_1x128, nullptr) == FP8BW_ERR_NULL);
  CHECK(fp8bw_gemm_blockwise_plan(128, 128, 128, 3, nullptr) == FP8BW_ERR_NULL);
  int64_t info[6];
  CHECK(fp8bw_gemm_blockwise_plan(128, 128, 128, 3, info) == FP8BW_ERR_UNSUPPORTED);
  for (int s = -3; s < 12; ++s) CHECK(std::strlen(fp8bw_status_str(s)) > 0);
}

void linear_validation() {
  for (int64_t M : kDims)
    for (int64_t N : kDims)
      for (int64_t K : kDims) {
        // Too-small workspace: every nonzero problem is rejected before any launch.
        CHECK(known_status(fp8_linear_fwd(buf_a, buf_b, buf_out, M, N, K, buf_ws, 0, nullptr)));
        CHECK(known_status(fp8_linear_dgrad(buf_a, buf_b, buf_out, M, N, K, buf_ws, 0, nullptr)));
        CHECK(known_status(fp8_linear_wgrad(buf_a, buf_b, buf_out, M, N, K, buf_ws, 0, nullptr)));
        CHECK(known_status(fp8_linear_fwd_save(buf_a, buf_b, buf_out, M, N, K, buf_ws, 0, buf_ws,
                                               0, nullptr)));
        CHECK(known_status(fp8_linear_bwd(buf_a, buf_b, buf_ws, 0, buf_out, buf_out, M, N, K,
                                          buf_ws, 0, nullptr)));
      }
  EXPECT_STATUS(fp8_linear_fwd(buf_a, buf_b, buf_out, 128, 128, 128, buf_ws, 0, nullptr),
                FP8BW_ERR_WORKSPACE);
  EXPECT_STATUS(fp8_linear_fwd(buf_a, buf_b, buf_out, 128, 128, 100, buf_ws, 0, nullptr),
                FP8BW_ERR_SHAPE);
  EXPECT_STATUS(fp8_linear_fwd(buf_a, buf_b, buf_out, 0, 128, 128, nullptr, 0, nullptr), FP8BW_OK);
  EXPECT_STATUS(fp8_linear_bwd(buf_a, buf_b, buf_ws, 16, buf_out, buf_out, 128, 128, 128, buf_ws,
                               0, nullptr), FP8BW_ERR_WORKSPACE);
}

// fp8bw_last_error() is per thread: concurrent rejected calls each see their
// own message, and a message stays valid while other threads fail.
void threaded_errors() {
  std::vector<std::thread> ts;
  std::vector<int> bad(8, 0);
  for (int t = 0; t < 8; ++t) {
    ts.emplace_back([t, &bad] {
      for (int i = 0; i < 2000; ++i) {
        const int64_t cols = 16 * (t + 1) + 1;   // never a multiple of 16
        const int st = fp8_blockwise_quant(buf_a, 16, cols, 4096, FP8BW_BLOCK_1x128, 0, buf_out,
                                           4096, buf_s, 1, 16, nullptr);
        const std::string want = "cols=" + std::to_string(cols);
        if (st != FP8BW_ERR_SHAPE || std::strncmp(fp8bw_last_error(), want.c_str(), want.size()))
          ++bad[t];
        fp8bw_gemm_blockwise_ws_bytes(4096 + 128 * t, 4096, 8192);
      }
    });
  }
  for (auto& th : ts) th.join();
  for (int t = 0; t < 8; ++t) CHECK(bad[t] == 0);
}

}  // namespace

int main() {
  int devices = 0;
  if (hipGetDeviceCount(&devices) == hipSuccess && devices > 0) {
    std::printf("abi sanitize driver: %d GPU(s) visible; runs only on hosts without one\n",
                devices);
    return 77;
  }
  CHECK(fp8bw_abi_version() >= 1);
  quant_validation();
  tensorwise_validation();
  gemm_validation();
  gemm_kn_validation();
  grouped_validation();
  queries();
  linear_validation();
  threaded_errors();
  std::printf("abi sanitize driver: %d checks, %d failures\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
