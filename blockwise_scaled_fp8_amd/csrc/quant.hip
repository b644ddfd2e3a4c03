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
// with 16-byte loads, codes are written once, the reductions are DPP /
// readlane in registers plus a few words of LDS.

#include "device_common.h"
#include "launch.h"

namespace fp8bw {

// ---------------------------------------------------------------------------
// 1x128 blocks along the columns (activation X, gradient dY).
//
// 256 threads = 4 waves; a 16-lane DPP row owns one 1x128 block (16 lanes x
// 8 bf16 = 256 B).  The 4 DPP rows of a wave take 4 consecutive column
// blocks of the same input row, so every load instruction reads 1 KB of
// contiguous input and every store writes 512 B of contiguous codes.  A
// workgroup covers ROWS rows x 4 column blocks; each wave walks ROWS/4 rows
// with all its loads in flight before the first reduction.  The reciprocal
// scales are staged in LDS and written out so that consecutive threads
// write consecutive rows of one column block (column-major scales).
template <int ROWS>
__global__ __launch_bounds__(256) void quant_1x128_rows_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ recip, int64_t rs_row,
    int64_t rs_kb) {
  constexpr int U = ROWS / 4;
  __shared__ float sc[4][ROWS];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 4, lig = lane & 15;
  const int64_t kblocks = (cols + 127) >> 7;
  const int64_t kb = (int64_t)blockIdx.y * 4 + grp;
  const int64_t row0 = (int64_t)blockIdx.x * ROWS + wave * U;
  const int64_t col = kb * 128 + lig * 8;
  const bool col_ok = (kb < kblocks) && (col < cols);

  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t r = row0 + u;
    v[u] = make_uint4(0, 0, 0, 0);
    if (col_ok && r < rows) v[u] = *(const uint4*)(x + r * ld_x + col);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float amax = row16_max(absmax8(v[u]));
    const float s = scale_from_amax(amax);
    if (lig == 0) sc[grp][wave * U + u] = recip_of_scale(s);
    const uint2 c = quant8(v[u], s);
    const int64_t r = row0 + u;
    if (col_ok && r < rows) *(uint2*)(q + r * ld_q + col) = c;
  }
  __syncthreads();
  for (int t = tid; t < 4 * ROWS; t += 256) {
    const int g2 = t / ROWS, rr = t % ROWS;
    const int64_t kb2 = (int64_t)blockIdx.y * 4 + g2;
    const int64_t r = (int64_t)blockIdx.x * ROWS + rr;
    if (kb2 < kblocks && r < rows) recip[r * rs_row + kb2 * rs_kb] = sc[g2][rr];
  }
}

hipError_t launch_quant_1x128_rows(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                   void* q, int64_t ld_q, float* recip, int64_t rs_row,
                                   int64_t rs_kb, hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const int64_t kgroups = ((cols + 127) / 128 + 3) / 4;
  const int64_t tiles64 = (rows + 63) / 64;
  if (tiles64 * kgroups >= 2048) {
    dim3 grid((unsigned)tiles64, (unsigned)kgroups);
    hipLaunchKernelGGL(quant_1x128_rows_kernel<64>, grid, dim3(256), 0, stream,
                       (const uint16_t*)x, rows, cols, ld_x, (uint8_t*)q, ld_q, recip, rs_row,
                       rs_kb);
  } else {
    dim3 grid((unsigned)((rows + 15) / 16), (unsigned)kgroups);
    hipLaunchKernelGGL(quant_1x128_rows_kernel<16>, grid, dim3(256), 0, stream,
                       (const uint16_t*)x, rows, cols, ld_x, (uint8_t*)q, ld_q, recip, rs_row,
                       rs_kb);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 128x128 tiles (weights).  One workgroup per tile: thread t reads 16 B
// chunks (row t/16 + 16 i, chunk t%16) for i = 0..7, so each load
// instruction of a wave reads four 256-byte row segments.  amax: per-thread
// max, DPP row max + readlane across the wave, LDS across the 4 waves.
//
// TRANSPOSE writes q = x^T (the dgrad operand W^T).  The codes are staged in
// LDS as [row][col] bytes and gathered by output row; block amax is the same
// in either orientation, so the codes equal the transpose of the
// non-transposed codes.
template <bool TRANSPOSE>
__global__ __launch_bounds__(256) void quant_128x128_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ recip, int64_t rs_row,
    int64_t rs_kb) {
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[TRANSPOSE ? 128 * 128 : 16];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int c16 = tid & 15, rr = tid >> 4;
  const int64_t cb = blockIdx.x, rb = blockIdx.y;
  const int64_t col = cb * 128 + c16 * 8;
  const bool col_ok = col < cols;

  uint4 v[8];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = rb * 128 + rr + 16 * i;
    v[i] = make_uint4(0, 0, 0, 0);
    if (col_ok && r < rows) v[i] = *(const uint4*)(x + r * ld_x + col);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, absmax8(v[i]));
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = scale_from_amax(amax);
  if (tid == 0) {
    if (TRANSPOSE)
      recip[cb * rs_row + rb * rs_kb] = recip_of_scale(s);
    else
      recip[rb * rs_row + cb * rs_kb] = recip_of_scale(s);
  }
  if (!TRANSPOSE) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t r = rb * 128 + rr + 16 * i;
      const uint2 c = quant8(v[i], s);
      if (col_ok && r < rows) *(uint2*)(q + r * ld_q + col) = c;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *(uint2*)(tile + (rr + 16 * i) * 128 + c16 * 8) = quant8(v[i], s);
    __syncthreads();
    // Output row oc (= input column), input rows 64h .. 64h+63.
    const int oc = tid & 127, h = tid >> 7;
    const int64_t orow = cb * 128 + oc;
    if (orow < cols) {
#pragma unroll
      for (int seg = 0; seg < 4; ++seg) {
        const int r0 = 64 * h + 16 * seg;
        uint32_t w[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int rbase = r0 + 4 * d;
          w[d] = (uint32_t)tile[(rbase + 0) * 128 + oc] | ((uint32_t)tile[(rbase + 1) * 128 + oc] << 8) |
                 ((uint32_t)tile[(rbase + 2) * 128 + oc] << 16) |
                 ((uint32_t)tile[(rbase + 3) * 128 + oc] << 24);
        }
        const int64_t ocol = rb * 128 + r0;
        if (ocol < rows) *(uint4*)(q + orow * ld_q + ocol) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
}

hipError_t launch_quant_128x128(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                int transpose, void* q, int64_t ld_q, float* recip,
                                int64_t rs_row, int64_t rs_kb, hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  dim3 grid((unsigned)((cols + 127) / 128), (unsigned)((rows + 127) / 128));
  if (transpose)
    hipLaunchKernelGGL(quant_128x128_kernel<true>, grid, dim3(256), 0, stream,
                       (const uint16_t*)x, rows, cols, ld_x, (uint8_t*)q, ld_q, recip, rs_row,
                       rs_kb);
  else
    hipLaunchKernelGGL(quant_128x128_kernel<false>, grid, dim3(256), 0, stream,
                       (const uint16_t*)x, rows, cols, ld_x, (uint8_t*)q, ld_q, recip, rs_row,
                       rs_kb);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 1x128 blocks running down the rows, written transposed (wgrad operands
// dY^T and X^T: the 1x128 x 1x128 recipe).  One workgroup per 128 input rows
// x 64 input columns.  Thread t owns input columns 8(t%8)..+7 of input rows
// 4(t/8)..+3, so after quantization each of its 8 columns yields one dword
// holding 4 consecutive output bytes.  Column amax: register max over the 4
// rows, cross-lane max over the 8 lanes sharing the column group, LDS over
// the 4 waves.  The codes are transposed through an XOR-swizzled LDS tile
// and written as 16-byte segments of the output rows.
__device__ __forceinline__ float bf16_elem(const uint4& v, int c) {
  const uint32_t w = c < 2 ? v.x : c < 4 ? v.y : c < 6 ? v.z : v.w;
  return (c & 1) ? bf16hi(w) : bf16lo(w);
}

__global__ __launch_bounds__(256) void quant_1x128_cols_t_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ recip, int64_t rs_row,
    int64_t rs_kb) {
  __shared__ float red[4][64];
  __shared__ float ssc[64];
  __shared__ __attribute__((aligned(16))) uint32_t tile[64 * 32];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = tid & 7, j = tid >> 3;
  const int64_t mb = blockIdx.y, c0 = (int64_t)blockIdx.x * 64;
  const int64_t col = c0 + g * 8;
  const bool col_ok = col < cols;

  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = mb * 128 + 4 * j + i;
    v[i] = make_uint4(0, 0, 0, 0);
    if (col_ok && r < rows) v[i] = *(const uint4*)(x + r * ld_x + col);
  }
  float cm[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float mm = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) mm = fmaxf(mm, fabsf(bf16_elem(v[i], c)));
    mm = fmaxf(mm, __shfl_xor(mm, 8));
    mm = fmaxf(mm, __shfl_xor(mm, 16));
    mm = fmaxf(mm, __shfl_xor(mm, 32));
    cm[c] = mm;
  }
  if (lane < 8) {
#pragma unroll
    for (int c = 0; c < 8; ++c) red[wave][8 * lane + c] = cm[c];
  }
  __syncthreads();
  if (tid < 64) {
    const float a = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
    const float s = scale_from_amax(a);
    ssc[tid] = s;
    if (c0 + tid < cols) recip[(c0 + tid) * rs_row + mb * rs_kb] = recip_of_scale(s);
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float s = ssc[8 * g + c];
    const uint32_t w = cvt4_e4m3(bf16_elem(v[0], c) * s, bf16_elem(v[1], c) * s,
                                 bf16_elem(v[2], c) * s, bf16_elem(v[3], c) * s);
    const int orow = 8 * g + c;          // local output row; orow >> 3 == g
    const int seg = j >> 2;              // 16-byte segment of the 128-byte output row
    tile[orow * 32 + ((seg ^ g) << 2) + (j & 3)] = w;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int id = tid + 256 * k;
    const int orow = id >> 3, seg = id & 7;
    const uint4 val = *(const uint4*)&tile[orow * 32 + ((seg ^ (orow >> 3)) << 2)];
    const int64_t ocol = mb * 128 + seg * 16;
    if (c0 + orow < cols && ocol < rows) *(uint4*)(q + (c0 + orow) * ld_q + ocol) = val;
  }
}

hipError_t launch_quant_1x128_cols_t(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                     void* q, int64_t ld_q, float* recip, int64_t rs_row,
                                     int64_t rs_kb, hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 127) / 128));
  hipLaunchKernelGGL(quant_1x128_cols_t_kernel, grid, dim3(256), 0, stream, (const uint16_t*)x,
                     rows, cols, ld_x, (uint8_t*)q, ld_q, recip, rs_row, rs_kb);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-tensor: a grid of partial amaxes, then a quantize pass in which every
// workgroup reduces the partials itself (fixed order, no atomics, no
// memset) before quantizing its grid-stride share.
__global__ __launch_bounds__(256) void amax_partial_kernel(const uint16_t* __restrict__ x,
                                                           int64_t rows, int64_t cols,
                                                           int64_t ld_x, float* __restrict__ ws) {
  __shared__ float red[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t cpr = cols >> 3;
  const int64_t total = rows * cpr;
  float m = 0.f;
  for (int64_t c = (int64_t)blockIdx.x * 256 + tid; c < total; c += (int64_t)gridDim.x * 256) {
    const int64_t r = c / cpr, k = c - r * cpr;
    m = fmaxf(m, absmax8(*(const uint4*)(x + r * ld_x + k * 8)));
  }
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
  for (int64_t c = (int64_t)blockIdx.x * 256 + tid; c < total; c += (int64_t)gridDim.x * 256) {
    const int64_t r = c / cpr, k = c - r * cpr;
    *(uint2*)(q + r * ld_q + k * 8) = quant8(*(const uint4*)(x + r * ld_x + k * 8), s);
  }
}

int tensorwise_partials(int64_t rows, int64_t cols) {
  const int64_t chunks = rows * (cols / 8);
  int64_t p = (chunks + 256 * 8 - 1) / (256 * 8);
  if (p < 1) p = 1;
  if (p > 1024) p = 1024;
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

}  // namespace fp8bw
