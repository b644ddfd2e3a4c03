// Dynamic E4M3 quantization kernels for gfx950.
//
// Per block: amax = max|x|, s = 448 / max(amax, 1e-12), codes =
// satRNE_e4m3(x * s), recip = 1 / s (the reciprocal is what the GEMM
// consumes; pytorch/ao PR "integrate torch._scaled_mm into
// Float8BlockwiseLinear and add bench script", Summary).  Block shapes:
// 1x128 for activations/gradients and 128x128 for weights (pytorch/ao PR
// "add more generic kernel for fp8 blockwise scaling", Performance table),
// plus one scale per tensor (ROCm/aiter issue "Does gemm_a8w8 support
// per-tensor quant?").
//
// All kernels are HBM-bound streaming kernels: every input byte is read once
// with 16-byte nontemporal loads, codes are written once with ordinary
// stores, the reductions are DPP / readlane / shuffles in registers plus a
// few words of LDS.  Lanes past a ragged edge load a clamped in-bounds
// address and have their values masked before use, so no load sits behind a
// branch and the compiler's waits stay exact.

#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace fp8bw {

__device__ __forceinline__ float bf16_elem(const uint4& v, int c) {
  const uint32_t w = c < 2 ? v.x : c < 4 ? v.y : c < 6 ? v.z : v.w;
  return (c & 1) ? bf16hi(w) : bf16lo(w);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const uint16_t* p) {
  const u32x4 t = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(t.x, t.y, t.z, t.w);
}

// ---------------------------------------------------------------------------
// 1x128 blocks along the columns (activation X, gradient dY).
//
// The input is cut into 512-column pieces of a row (4 column blocks; a
// row's last piece may be short) numbered row-major, and workgroup b takes
// pieces 16b .. 16b+15, so workgroups run over memory in dispatch order
// (one workgroup = one row when cols = 8192).  256 threads = 4 waves; load u
// of wave w reads piece 16b + 4u + w, and within a wave a 16-lane DPP row
// owns one 1x128 block (16 lanes x 8 bf16 = 256 B): every load instruction
// reads 1 KB of contiguous input and every store writes 512 B of contiguous
// codes.  Each block's reciprocal scale is written by its DPP row's first
// lane.
__global__ __launch_bounds__(256) void quant_1x128_rows_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ recip, int64_t rs_row,
    int64_t rs_kb, int64_t pieces_per_row) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 4, lig = lane & 15;
  const int64_t kblocks = (cols + 127) >> 7;
  const int64_t total = rows * pieces_per_row;
  uint4 v[4];
  int64_t rr[4], cc[4], kk[4];
  bool in[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t piece = (int64_t)blockIdx.x * 16 + 4 * u + wave;
    const int64_t r = piece / pieces_per_row;
    const int64_t kb = (piece - r * pieces_per_row) * 4 + grp;
    const int64_t col = kb * 128 + lig * 8;
    in[u] = piece < total && kb < kblocks && col < cols;
    rr[u] = r; cc[u] = col; kk[u] = kb;
    v[u] = load_stream16(x + (in[u] ? r * ld_x + col : 0));
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint4 w = in[u] ? v[u] : make_uint4(0, 0, 0, 0);
    const float s = scale_from_amax(row16_max(absmax8(w)));
    const uint2 code = quant8(w, s);
    if (in[u]) {
      *(uint2*)(q + rr[u] * ld_q + cc[u]) = code;
      if (lig == 0) recip[rr[u] * rs_row + kk[u] * rs_kb] = recip_of_scale(s);
    }
  }
}

hipError_t launch_quant_1x128_rows(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                   void* q, int64_t ld_q, float* recip, int64_t rs_row,
                                   int64_t rs_kb, hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const int64_t ppr = ((cols + 127) / 128 + 3) / 4;
  const int64_t wgs = (rows * ppr + 15) / 16;
  hipLaunchKernelGGL(quant_1x128_rows_kernel, dim3((unsigned)wgs), dim3(256), 0, stream,
                     (const uint16_t*)x, rows, cols, ld_x, (uint8_t*)q, ld_q, recip, rs_row,
                     rs_kb, ppr);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 128x128 input tiles: the weight quantizer (one scale per tile, codes as
// they are or transposed for the dgrad operand W^T) and the 1x128 blocks
// running down the rows, written transposed (the wgrad operands dY^T and
// X^T: one scale per input column per 128 rows).
//
// One workgroup per tile, 256 threads.  Thread t owns input columns
// 8g .. 8g+7 (g = t % 16) of input rows 4j .. 4j+3 and 64+4j .. 64+4j+3
// (j = t / 16): each load instruction of a wave reads four 256-byte row
// segments.  Amax: a tile scale reduces the thread maxima with DPP / readlane
// and LDS across the 4 waves; column scales reduce each column's 8 rows in
// registers, the 4 row quads of a wave with shuffles and the 4 waves in LDS.
//
// Transposed outputs: for each of its 8 columns a thread quantizes its rows
// into two dwords (4 consecutive output bytes each) and writes them to an
// LDS tile stored as [input column][input row] (128 rows = 32 dwords per
// column); dword d of column c sits at d ^ 4((c / 8) % 8), which spreads the
// 16 column groups of a store over the banks and keeps every 16-byte group
// of 4 dwords intact.  The tile is then read back as 16-byte segments of
// output rows, 8 lanes per 128-byte row.
// Dual outputs from one read of the tile: W and W^T codes with the one tile
// scale (written in both index orders), or the 1x128 row blocks (a row's 128
// columns of the tile are one block; its 16 threads are one DPP row) and the
// transposed 1x128 column blocks of X or dY together.
enum TileMode {
  kTileScale = 0,       // codes as they are, tile scale
  kTileScaleT = 1,      // transposed codes, tile scale
  kColScaleT = 2,       // transposed codes, one scale per column per 128 rows
  kTileScaleBoth = 3,   // both code layouts, tile scale
  kRowColBoth = 4       // codes with 1x128 row scales + transposed codes with column scales
};

struct TileOut {
  uint8_t* q;           // codes as they are [rows, cols] (ld_q)
  int64_t ld_q;
  float* recip;         // their scales (rs_row, rs_kb)
  int64_t rs_row, rs_kb;
  uint8_t* qt;          // transposed codes [cols, rows] (ld_qt)
  int64_t ld_qt;
  float* recip_t;       // their scales (rst_row, rst_kb)
  int64_t rst_row, rst_kb;
};

// STREAM_T: the transposed codes are written with nontemporal stores, for
// a caller that will not read them until much later (the X^T codes a
// training forward keeps for its backward): they then pass the 256 MB
// memory-side cache by instead of evicting the operands of the GEMM that
// runs next (the forward GEMM of the 16640 x 5120 x 8192 linear step ran
// 576-578 us after the plain stores, 558-562 us after these).
template <int MODE, bool STREAM_T = false>
__global__ __launch_bounds__(256) void quant_tile_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x, const TileOut o) {
  constexpr bool PLAIN = MODE == kTileScale || MODE == kTileScaleBoth || MODE == kRowColBoth;
  constexpr bool T = MODE != kTileScale;
  constexpr bool COLS = MODE == kColScaleT || MODE == kRowColBoth;
  constexpr bool ROWS = MODE == kRowColBoth;
  __shared__ float red[4][COLS ? 128 : 1];
  __shared__ float ssc[COLS ? 128 : 1];
  __shared__ __attribute__((aligned(16))) uint32_t tile[T ? 128 * 32 : 4];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = tid & 15, j = tid >> 4;
  const int64_t cb = blockIdx.x, rb = blockIdx.y;
  const int64_t col = cb * 128 + g * 8;
  const bool col_in = col < cols;

  uint4 v[8];                          // v[4p + i]: input row 64p + 4j + i of the tile
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int64_t r = rb * 128 + 64 * (k >> 2) + 4 * j + (k & 3);
    const bool in = col_in && r < rows;
    v[k] = load_stream16(x + (in ? r * ld_x + col : 0));
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int64_t r = rb * 128 + 64 * (k >> 2) + 4 * j + (k & 3);
    if (!(col_in && r < rows)) v[k] = make_uint4(0, 0, 0, 0);
  }

  float s = 0.f;
  if constexpr (!COLS) {
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, absmax8(v[k]));
    m = wave_max(m);
    if (lane == 0) red[wave][0] = m;
    __syncthreads();
    s = scale_from_amax(fmaxf(fmaxf(red[0][0], red[1][0]), fmaxf(red[2][0], red[3][0])));
    if (tid == 0) {
      if (PLAIN) o.recip[rb * o.rs_row + cb * o.rs_kb] = recip_of_scale(s);
      if (T) o.recip_t[cb * o.rst_row + rb * o.rst_kb] = recip_of_scale(s);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float m = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(bf16_elem(v[k], c)));
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      if (lane < 16) red[wave][8 * g + c] = m;
    }
    __syncthreads();
    if (tid < 128) {
      const float a = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
      const float sc = scale_from_amax(a);
      ssc[tid] = sc;
      if (cb * 128 + tid < cols)
        o.recip_t[(cb * 128 + tid) * o.rst_row + rb * o.rst_kb] = recip_of_scale(sc);
    }
    __syncthreads();
  }

  if constexpr (PLAIN) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t r = rb * 128 + 64 * (k >> 2) + 4 * j + (k & 3);
      float sr = s;
      if constexpr (ROWS) {
        // 1x128 row block: this row's 128 columns live in this DPP row
        sr = scale_from_amax(row16_max(absmax8(v[k])));
        if (g == 0 && r < rows) o.recip[r * o.rs_row + cb * o.rs_kb] = recip_of_scale(sr);
      }
      const uint2 code = quant8(v[k], sr);
      if (col_in && r < rows) *(uint2*)(o.q + r * o.ld_q + col) = code;
    }
  }
  if constexpr (T) {
    const int sw = 4 * (g & 7);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float sc = COLS ? ssc[8 * g + c] : s;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint32_t w = cvt4_e4m3(bf16_elem(v[4 * p + 0], c) * sc, bf16_elem(v[4 * p + 1], c) * sc,
                                     bf16_elem(v[4 * p + 2], c) * sc, bf16_elem(v[4 * p + 3], c) * sc);
        tile[(8 * g + c) * 32 + ((16 * p + j) ^ sw)] = w;
      }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int id = tid + 256 * m;
      const int oc = id >> 3, seg = id & 7;       // output row in the tile, 16-row segment
      const uint4 val = *(const uint4*)&tile[oc * 32 + ((4 * seg) ^ (4 * ((oc >> 3) & 7)))];
      const int64_t orow = cb * 128 + oc, ocol = rb * 128 + 16 * seg;
      if (orow < cols && ocol < rows) {
        if constexpr (STREAM_T) {
          const u32x4 t = {val.x, val.y, val.z, val.w};
          __builtin_nontemporal_store(t, (u32x4*)(o.qt + orow * o.ld_qt + ocol));
        } else {
          *(uint4*)(o.qt + orow * o.ld_qt + ocol) = val;
        }
      }
    }
  }
}

template <int MODE, bool STREAM_T = false>
static hipError_t launch_tile(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                              const TileOut& o, hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const dim3 grid((unsigned)((cols + 127) / 128), (unsigned)((rows + 127) / 128));
  hipLaunchKernelGGL((quant_tile_kernel<MODE, STREAM_T>), grid, dim3(256), 0, stream,
                     (const uint16_t*)x, rows, cols, ld_x, o);
  return hipGetLastError();
}

static TileOut plain_out(void* q, int64_t ld_q, float* recip, int64_t rs_row, int64_t rs_kb) {
  return TileOut{(uint8_t*)q, ld_q, recip, rs_row, rs_kb, nullptr, 0, nullptr, 0, 0};
}
static TileOut trans_out(void* q, int64_t ld_q, float* recip, int64_t rs_row, int64_t rs_kb) {
  return TileOut{nullptr, 0, nullptr, 0, 0, (uint8_t*)q, ld_q, recip, rs_row, rs_kb};
}

hipError_t launch_quant_128x128(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                int transpose, void* q, int64_t ld_q, float* recip,
                                int64_t rs_row, int64_t rs_kb, hipStream_t stream) {
  return transpose
             ? launch_tile<kTileScaleT>(x, rows, cols, ld_x, trans_out(q, ld_q, recip, rs_row, rs_kb), stream)
             : launch_tile<kTileScale>(x, rows, cols, ld_x, plain_out(q, ld_q, recip, rs_row, rs_kb), stream);
}

hipError_t launch_quant_1x128_cols_t(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                     void* q, int64_t ld_q, float* recip, int64_t rs_row,
                                     int64_t rs_kb, hipStream_t stream) {
  return launch_tile<kColScaleT>(x, rows, cols, ld_x, trans_out(q, ld_q, recip, rs_row, rs_kb), stream);
}

hipError_t launch_quant_dual(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int block_128,
                             void* q, int64_t ld_q, float* recip, int64_t rs_row, int64_t rs_kb,
                             void* qt, int64_t ld_qt, float* recip_t, int64_t rst_row,
                             int64_t rst_kb, bool stream_t, hipStream_t stream) {
  const TileOut o{(uint8_t*)q, ld_q, recip, rs_row, rs_kb, (uint8_t*)qt, ld_qt, recip_t, rst_row, rst_kb};
  if (block_128)
    return stream_t ? launch_tile<kTileScaleBoth, true>(x, rows, cols, ld_x, o, stream)
                    : launch_tile<kTileScaleBoth>(x, rows, cols, ld_x, o, stream);
  return stream_t ? launch_tile<kRowColBoth, true>(x, rows, cols, ld_x, o, stream)
                  : launch_tile<kRowColBoth>(x, rows, cols, ld_x, o, stream);
}

// ---------------------------------------------------------------------------
// Per-tensor: a grid of partial amaxes, then a quantize pass in which every
// workgroup reduces the partials itself (fixed order, no atomics, no
// memset) before quantizing its grid-stride share.  Both passes stream: a
// workgroup takes 16 KB blocks of 1024 consecutive 16-byte chunks in a grid
// stride, each thread holding four independent nontemporal loads in flight
// (one per 4 KB quarter of the block); the chunks past the last whole block
// go one per thread.  A contiguous input is indexed linearly, a strided one
// by row.
constexpr int kTwUnroll = 4;
constexpr int kTwBlock = 256 * kTwUnroll;   // chunks per workgroup block

// Address of 16-byte chunk c (8 bf16 values) of a rows x cols input.
__device__ __forceinline__ const uint16_t* tw_chunk(const uint16_t* x, int64_t c, int64_t cpr,
                                                    int64_t ld_x, bool contiguous) {
  if (contiguous) return x + c * 8;
  const int64_t r = c / cpr;
  return x + r * ld_x + (c - r * cpr) * 8;
}

__global__ __launch_bounds__(256) void amax_partial_kernel(const uint16_t* __restrict__ x,
                                                           int64_t rows, int64_t cols,
                                                           int64_t ld_x, float* __restrict__ ws) {
  __shared__ float red[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t cpr = cols >> 3;
  const int64_t total = rows * cpr;
  const bool contiguous = ld_x == cols;
  const int64_t whole = total / kTwBlock * kTwBlock;
  float m = 0.f;
  for (int64_t b = (int64_t)blockIdx.x * kTwBlock + tid; b < whole; b += (int64_t)gridDim.x * kTwBlock) {
    uint4 v[kTwUnroll];
#pragma unroll
    for (int u = 0; u < kTwUnroll; ++u) v[u] = load_stream16(tw_chunk(x, b + 256 * u, cpr, ld_x, contiguous));
#pragma unroll
    for (int u = 0; u < kTwUnroll; ++u) m = fmaxf(m, absmax8(v[u]));
  }
  for (int64_t c = whole + (int64_t)blockIdx.x * 256 + tid; c < total; c += (int64_t)gridDim.x * 256)
    m = fmaxf(m, absmax8(load_stream16(tw_chunk(x, c, cpr, ld_x, contiguous))));
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (tid == 0) ws[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ __launch_bounds__(256) void quant_tensorwise_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ recip,
    const float* __restrict__ ws, int nparts) {
  __shared__ float red[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  float m = 0.f;
  for (int i = tid; i < nparts; i += 256) m = fmaxf(m, ws[i]);
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = scale_from_amax(amax);
  if (blockIdx.x == 0 && tid == 0) *recip = recip_of_scale(s);
  const int64_t cpr = cols >> 3;
  const int64_t total = rows * cpr;
  const bool contiguous = ld_x == cols && ld_q == cols;
  const int64_t whole = total / kTwBlock * kTwBlock;
  auto qptr = [&](int64_t c) -> uint2* {
    if (contiguous) return (uint2*)(q + c * 8);
    const int64_t r = c / cpr;
    return (uint2*)(q + r * ld_q + (c - r * cpr) * 8);
  };
  for (int64_t b = (int64_t)blockIdx.x * kTwBlock + tid; b < whole; b += (int64_t)gridDim.x * kTwBlock) {
    uint4 v[kTwUnroll];
#pragma unroll
    for (int u = 0; u < kTwUnroll; ++u) v[u] = load_stream16(tw_chunk(x, b + 256 * u, cpr, ld_x, contiguous));
#pragma unroll
    for (int u = 0; u < kTwUnroll; ++u) *qptr(b + 256 * u) = quant8(v[u], s);
  }
  for (int64_t c = whole + (int64_t)blockIdx.x * 256 + tid; c < total; c += (int64_t)gridDim.x * 256)
    *qptr(c) = quant8(load_stream16(tw_chunk(x, c, cpr, ld_x, contiguous)), s);
}

int tensorwise_partials(int64_t rows, int64_t cols) {
  const int64_t chunks = rows * (cols / 8);
  int64_t p = (chunks + 256 * 8 - 1) / (256 * 8);
  if (p < 1) p = 1;
  if (p > kMaxTensorwisePartials) p = kMaxTensorwisePartials;
  return (int)p;
}

hipError_t launch_quant_tensorwise(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                   void* q, int64_t ld_q, float* recip, float* ws,
                                   hipStream_t stream) {
  const int p = tensorwise_partials(rows, cols);
  hipLaunchKernelGGL(amax_partial_kernel, dim3(p), dim3(256), 0, stream, (const uint16_t*)x,
                     rows, cols, ld_x, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quant_tensorwise_kernel, dim3(p), dim3(256), 0, stream, (const uint16_t*)x,
                     rows, cols, ld_x, (uint8_t*)q, ld_q, recip, (const float*)ws, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Allocation-free per-tensor quantization: the partial amaxes live in a
// library-owned device array instead of caller workspace.  Each GPU the
// library runs on holds its own copy of `scratch` (4 KiB) until the process
// ends.  In host code `scratch` names a host-side stand-in, not device
// memory: its device address on each GPU comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// passed to the kernels.  Every call on a GPU shares the array; the amax
// pass writes every partial the quantize pass reads, so nothing needs
// clearing between calls, but two calls that overlap on one GPU (different
// streams) race on it.
static __device__ __align__(256) float scratch[kMaxTensorwisePartials];

static std::mutex g_scratch_mu;
static float* g_scratch_dev[kMaxDevices];   // guarded by g_scratch_mu

static hipError_t scratch_of_current_device(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = (float*)ptr;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

hipError_t launch_quant_tensorwise_noalloc(const void* x, int64_t rows, int64_t cols,
                                           int64_t ld_x, void* q, int64_t ld_q, float* recip,
                                           hipStream_t stream) {
  if (tensorwise_partials(rows, cols) > kMaxTensorwisePartials) return hipErrorInvalidValue;
  float* ws = nullptr;
  const hipError_t e = scratch_of_current_device(&ws);
  if (e != hipSuccess) return e;
  return launch_quant_tensorwise(x, rows, cols, ld_x, q, ld_q, recip, ws, stream);
}

}  // namespace fp8bw
