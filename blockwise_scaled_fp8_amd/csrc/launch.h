// Internal host-side launchers shared by the C ABI (api.cpp) and the kernel
// translation units.  Arguments are validated by the caller (api.cpp); the
// launchers only size grids and enqueue on `stream`.  Each returns the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fp8bw {

// ---- quantization (quant.hip) ----
// 1x128 blocks along columns: q[r, c], recip[r*rs_row + kb*rs_kb].
hipError_t launch_quant_1x128_rows(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                   void* q, int64_t ld_q, float* recip, int64_t rs_row,
                                   int64_t rs_kb, hipStream_t stream);
// 128x128 tiles; transpose=1 writes q = x^T [cols, rows] and indexes recip by
// (output row block, output column block).
hipError_t launch_quant_128x128(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                int transpose, void* q, int64_t ld_q, float* recip,
                                int64_t rs_row, int64_t rs_kb, hipStream_t stream);
// 1x128 blocks running down the rows; output transposed q = x^T [cols, rows],
// recip[c*rs_row + mb*rs_kb].
hipError_t launch_quant_1x128_cols_t(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                     void* q, int64_t ld_q, float* recip, int64_t rs_row,
                                     int64_t rs_kb, hipStream_t stream);
// Both layouts from one read: block_128 = 0 writes the 1x128 row-block codes
// (q, recip[r*rs_row + kb*rs_kb]) and the transposed 1x128 column-block codes
// (qt = x^T, recip_t[c*rst_row + mb*rst_kb]); block_128 = 1 writes the
// 128x128 codes and the transposed codes with the tile scale in both orders.
// stream_t: the transposed codes go out with nontemporal stores.
hipError_t launch_quant_dual(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int block_128,
                             void* q, int64_t ld_q, float* recip, int64_t rs_row, int64_t rs_kb,
                             void* qt, int64_t ld_qt, float* recip_t, int64_t rst_row,
                             int64_t rst_kb, bool stream_t, hipStream_t stream);
// Per-tensor: partial amax into ws (n_partials floats, at most
// kMaxTensorwisePartials), then quantize.
constexpr int kMaxTensorwisePartials = 1024;
constexpr int kMaxDevices = 64;
int tensorwise_partials(int64_t rows, int64_t cols);
hipError_t launch_quant_tensorwise(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                   void* q, int64_t ld_q, float* recip, float* ws,
                                   hipStream_t stream);
// The same with the partials in the library's own per-device array (no
// workspace; calls that overlap on one GPU race on it).
hipError_t launch_quant_tensorwise_noalloc(const void* x, int64_t rows, int64_t cols,
                                           int64_t ld_x, void* q, int64_t ld_q, float* recip,
                                           hipStream_t stream);

// ---- GEMM (gemm.hip) ----
enum ScaleMode { kBlockB128 = 0, kBlockB1x128 = 1, kTensorwise = 2 };
enum OutKind { kOutBf16 = 0, kOutF32 = 1 };

struct GemmProblem {
  const void* a; int64_t lda;
  const void* b; int64_t ldb;
  const float* ra; int64_t ra_s_row, ra_s_kb;
  const float* rb; int64_t rb_s_row, rb_s_kb;
  void* out; int64_t ldo;
  int64_t M, N, K;
  int mode;       // ScaleMode
  int out_kind;   // OutKind
  const void* bias = nullptr;   // optional bf16 [N] added before the output cast
  int b_kn = 0;                 // B given as [K, N] (b[k * ldb + n]) instead of [N, K]
};

// Tile configurations; the table lives in gemm.hip.
int gemm_num_configs();
// Whether config `cfg` accepts this problem.
bool gemm_config_ok(const GemmProblem& p, int cfg);

// How one GEMM call is run: the tile configuration, a whole-problem split-K
// count (fp32 partials [splits, M, N], then an ordered reduce), or a tail
// split (tiles_full tiles unsplit, the remaining tiles split tail_splits
// ways into tile-local partials, then reduced), and the workspace it needs.
struct GemmPlan {
  int cfg;
  int splits;
  int tail_splits;
  int64_t tiles;
  int64_t tiles_full;
  size_t ws_bytes;
};
// config < 0: built-in choice; splits > 0 forces a whole-problem split
// (no tail split); splits == 0 lets the plan choose when allow_split.
GemmPlan gemm_plan(const GemmProblem& p, int config, int splits, bool allow_split);
hipError_t launch_gemm(const GemmProblem& p, const GemmPlan& plan, void* ws, hipStream_t stream);
// Fill a contiguous bf16 [rows, cols] matrix with +0.
// Grouped blockwise GEMM: row groups of A / out ending at device int32
// group_end[g] (cumulative), each with B + g*b_s_group and rb + g*rb_s_group.
bool grouped_gemm_ok(const GemmProblem& p, int groups);
hipError_t launch_grouped_gemm(const GemmProblem& p, int groups, const int* group_end,
                               int64_t b_s_group, int64_t rb_s_group, hipStream_t stream);
hipError_t launch_zero_bf16(void* out, int64_t rows, int64_t cols, hipStream_t stream);

}  // namespace fp8bw
