// Blockwise- and tensorwise-scaled FP8 GEMM for gfx950 (CDNA4).
//
//   out[m, n] = sum_kb ra[m, kb] * rb[beta(n), kb] * sum_{k in kb} a[m, k] b[n, k]
//
// with A[M, K] and B[N, K] E4M3 codes (both K-contiguous, out = A B^T as in
// F.linear), ra the per-row (1x128) reciprocal scales of A and rb the
// reciprocal scales of B, either per 128x128 tile (beta(n) = n / 128; the
// forward and dgrad recipe) or per row (beta(n) = n; the 1x128 x 1x128
// weight-gradient recipe) -- pytorch/ao PR "add repro for blockwise
// _scaled_mm investigation", What Changed / Findings So Far.  The
// per-tensor variant multiplies the whole fp32 accumulator by ra * rb once
// (ROCm/aiter issue "Does gemm_a8w8 support per-tensor quant?").
//
// Design (see the design notes for the roofline):
//  * One K block (128 codes) is exactly one V_MFMA_F32_16X16X128_F8F6F4 per
//    16x16 output sub-tile.  Its fp32 result P goes to a fresh accumulator
//    and is folded into the running sum with one FMA per element:
//    acc += P * (ra * rb).  The tensorwise variant accumulates in the MFMA.
//  * A and B tiles for one K block are staged in LDS, double buffered, with
//    the 16-byte chunk index XOR-swizzled by (row & 7) so both the 16-byte
//    global->LDS writes and the 16-byte fragment reads are bank-conflict
//    free.  The scales of the K block travel with the tile through LDS.
//  * Each lane feeds the MFMA 32 contiguous K bytes of its row for both A
//    and B (the same byte->k assignment on both sides, so the dot product
//    is over matching k whatever order the instruction uses internally).
//  * Any number of K blocks: the loop runs [kb_begin, kb_end) with no
//    unrolling assumption, so 1001 or 1002 blocks need nothing special.
//  * Split-K writes fp32 partials [split, M, N]; a separate kernel sums them
//    in split order (deterministic, no atomics).

#include "device_common.h"
#include "launch.h"

namespace fp8bw {

struct GemmArgs {
  const uint8_t* a;
  const uint8_t* b;
  const float* ra;
  const float* rb;
  void* out;
  float* partial;
  int64_t lda, ldb, ldo;
  int64_t ra_s_kb;   // ra row stride is 1 (column-major scales)
  int64_t rb_s_row, rb_s_kb;
  int M, N, K;
  int kblocks;
  int tiles_m, tiles_n;
  int kb_per_split;
};

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  // Scale operands 0 select the unscaled V_MFMA_F32_16X16X128_F8F6F4;
  // format 0 = FP8 E4M3 for both A and B.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i load_frag(const uint8_t* tile, int row, int half) {
  // 32 K-bytes of `row`: 16-byte chunks 2*half and 2*half+1, swizzled.
  const int c0 = (2 * half) ^ (row & 7);
  const int c1 = (2 * half + 1) ^ (row & 7);
  const uint4 lo = *(const uint4*)(tile + row * 128 + (c0 << 4));
  const uint4 hi = *(const uint4*)(tile + row * 128 + (c1 << 4));
  v8i f;
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
  f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  return f;
}

template <int BM, int BN, int MODE, int OUT, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int ACH = BM / 32, BCH = BN / 32;   // 16-byte chunks per thread per K block
  constexpr int NBT = (BN + 127) / 128;         // 128-wide B scale blocks per tile
  constexpr int SB = (MODE == kBlockB1x128) ? BN : NBT;

  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * 128];
  __shared__ __attribute__((aligned(16))) float sRa[2][BM];
  __shared__ __attribute__((aligned(16))) float sRb[2][SB];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm0 = (wave >> 1) * WM, wn0 = (wave & 1) * WN;
  const int tile = blockIdx.x;
  const int tm = tile / p.tiles_n, tn = tile - tm * p.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb_begin = blockIdx.y * p.kb_per_split;
  const int kb_end = min(p.kblocks, kb_begin + p.kb_per_split);

  // Loader mapping: chunk (row = tid/8 + 32 i, 16-byte column tid%8).
  const int lrow = tid >> 3, lc = tid & 7;
  const uint8_t* pa[ACH];
  const uint8_t* pb[BCH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int r = min(m0 + lrow + 32 * i, p.M - 1);
    pa[i] = p.a + (int64_t)r * p.lda + lc * 16;
  }
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int r = min(n0 + lrow + 32 * i, p.N - 1);
    pb[i] = p.b + (int64_t)r * p.ldb + lc * 16;
  }

  uint4 rA[ACH], rB[BCH];
  float rsa = 0.f, rsb = 0.f;

  auto load_global = [&](int kb) {
    const int64_t koff = (int64_t)kb * 128;
    const bool kok = (MODE != kTensorwise) || (koff + lc * 16 < p.K);
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      rA[i] = make_uint4(0, 0, 0, 0);
      if (kok) rA[i] = *(const uint4*)(pa[i] + koff);
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      rB[i] = make_uint4(0, 0, 0, 0);
      if (kok) rB[i] = *(const uint4*)(pb[i] + koff);
    }
    if (MODE != kTensorwise) {
      if (tid < BM) rsa = p.ra[(int64_t)kb * p.ra_s_kb + min(m0 + tid, p.M - 1)];
      if (MODE == kBlockB128) {
        if (tid < SB) {
          const int nb = min(n0 / 128 + tid, (p.N - 1) / 128);
          rsb = p.rb[(int64_t)nb * p.rb_s_row + (int64_t)kb * p.rb_s_kb];
        }
      } else {
        if (tid < SB) rsb = p.rb[min(n0 + tid, p.N - 1) + (int64_t)kb * p.rb_s_kb];
      }
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int r = lrow + 32 * i;
      *(uint4*)(&sA[buf][r * 128 + ((lc ^ (r & 7)) << 4)]) = rA[i];
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int r = lrow + 32 * i;
      *(uint4*)(&sB[buf][r * 128 + ((lc ^ (r & 7)) << 4)]) = rB[i];
    }
    if (MODE != kTensorwise) {
      if (tid < BM) sRa[buf][tid] = rsa;
      if (tid < SB) sRb[buf][tid] = rsb;
    }
  };

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15, fhalf = lane >> 4;
  if (kb_begin < kb_end) {
    load_global(kb_begin);
    store_lds(0);
  }
  __syncthreads();
  for (int kb = kb_begin; kb < kb_end; ++kb) {
    const int buf = (kb - kb_begin) & 1;
    const bool more = kb + 1 < kb_end;
    if (more) load_global(kb + 1);

    v8i bf[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[j] = load_frag(sB[buf], wn0 + 16 * j + frow, fhalf);
    float sbn = 0.f;
    if (MODE == kBlockB128) sbn = sRb[buf][(n0 + wn0) / 128 - n0 / 128];
    float sbc[TN];
    if (MODE == kBlockB1x128) {
#pragma unroll
      for (int j = 0; j < TN; ++j) sbc[j] = sRb[buf][wn0 + 16 * j + frow];
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const v8i af = load_frag(sA[buf], wm0 + 16 * i + frow, fhalf);
      v4f sa = v4f{0.f, 0.f, 0.f, 0.f};
      if (MODE != kTensorwise) sa = *(const v4f*)&sRa[buf][wm0 + 16 * i + 4 * fhalf];
      if (MODE == kBlockB128) sa = sa * sbn;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if (MODE == kTensorwise) {
          acc[i][j] = mfma_fp8(af, bf[j], acc[i][j]);
        } else {
          const v4f pp = mfma_fp8(af, bf[j], v4f{0.f, 0.f, 0.f, 0.f});
          if (MODE == kBlockB128) {
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(pp[v], sa[v], acc[i][j][v]);
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[i][j][v] = __builtin_fmaf(pp[v] * sbc[j], sa[v], acc[i][j][v]);
          }
        }
      }
    }
    if (more) store_lds(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  Output layout of a 16x16 MFMA tile: lane l holds column l%16,
  // rows 4(l/16) .. 4(l/16)+3.
  float tscale = 1.f;
  if (MODE == kTensorwise) tscale = p.ra[0] * p.rb[0];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn0 + 16 * j + frow;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm0 + 16 * i + 4 * fhalf + v;
        if (m < p.M && n < p.N) {
          float val = acc[i][j][v];
          if (MODE == kTensorwise) val *= tscale;
          if (SPLIT) {
            p.partial[((int64_t)blockIdx.y * p.M + m) * p.N + n] = val;
          } else if (OUT == kOutBf16) {
            ((uint16_t*)p.out)[(int64_t)m * p.ldo + n] = (uint16_t)f32_to_bf16_rne(val);
          } else {
            ((float*)p.out)[(int64_t)m * p.ldo + n] = val;
          }
        }
      }
    }
  }
}

// Sum the split partials in split order and convert.
template <int OUT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, int M, int N,
                                                            void* __restrict__ out,
                                                            int64_t ldo) {
  const int64_t total = (int64_t)M * N;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    float s = 0.f;
    for (int k = 0; k < splits; ++k) s += part[(int64_t)k * total + idx];
    const int64_t m = idx / N, n = idx - m * N;
    if (OUT == kOutBf16)
      ((uint16_t*)out)[m * ldo + n] = (uint16_t)f32_to_bf16_rne(s);
    else
      ((float*)out)[m * ldo + n] = s;
  }
}

__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* __restrict__ out, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    out[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero_bf16(void* out, int64_t rows, int64_t cols, hipStream_t stream) {
  const int64_t n16 = rows * cols * 2 / 16;   // cols % 16 == 0
  if (n16 == 0) return hipSuccess;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint4*)out, n16);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Config table.
struct Cfg {
  int bm, bn;
};
static const Cfg kCfgs[] = {
    {128, 128},
    {64, 64},
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

int gemm_num_configs() { return kNumCfgs; }

bool gemm_config_ok(const GemmProblem&, int cfg) { return cfg >= 0 && cfg < kNumCfgs; }

size_t gemm_ws_bytes(int64_t M, int64_t N, int splits) {
  return splits > 1 ? (size_t)splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

void gemm_choose(const GemmProblem& p, int* config, int* splits) {
  const int64_t kblocks = (p.K + 127) / 128;
  const int64_t t128 = ((p.M + 127) / 128) * ((p.N + 127) / 128);
  int cfg = (t128 >= 128 || (p.M >= 128 && p.N >= 128 && t128 >= 64)) ? 0 : 1;
  const int bm = kCfgs[cfg].bm, bn = kCfgs[cfg].bn;
  const int64_t tiles = ((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn);
  int s = 1;
  if (tiles < 256 && kblocks >= 16) {
    int64_t want = (512 + tiles - 1) / tiles;
    int64_t maxs = kblocks / 8;
    s = (int)(want < maxs ? want : maxs);
    if (s < 1) s = 1;
    const int64_t per = (kblocks + s - 1) / s;
    s = (int)((kblocks + per - 1) / per);
  }
  *config = cfg;
  *splits = s;
}

template <int BM, int BN, int MODE>
static hipError_t launch_cfg(const GemmArgs& a, int splits, int out_kind, hipStream_t stream) {
  dim3 grid((unsigned)(a.tiles_m * a.tiles_n), (unsigned)splits);
  if (splits > 1)
    hipLaunchKernelGGL((gemm_kernel<BM, BN, MODE, kOutF32, true>), grid, dim3(256), 0, stream, a);
  else if (out_kind == kOutBf16)
    hipLaunchKernelGGL((gemm_kernel<BM, BN, MODE, kOutBf16, false>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_kernel<BM, BN, MODE, kOutF32, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int BM, int BN>
static hipError_t launch_mode(const GemmArgs& a, int mode, int splits, int out_kind,
                              hipStream_t stream) {
  switch (mode) {
    case kBlockB128: return launch_cfg<BM, BN, kBlockB128>(a, splits, out_kind, stream);
    case kBlockB1x128: return launch_cfg<BM, BN, kBlockB1x128>(a, splits, out_kind, stream);
    default: return launch_cfg<BM, BN, kTensorwise>(a, splits, out_kind, stream);
  }
}

hipError_t launch_gemm(const GemmProblem& p, int cfg, int splits, void* ws, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  const int bm = kCfgs[cfg].bm, bn = kCfgs[cfg].bn;
  GemmArgs a;
  a.a = (const uint8_t*)p.a;
  a.b = (const uint8_t*)p.b;
  a.ra = p.ra;
  a.rb = p.rb;
  a.out = p.out;
  a.partial = (float*)ws;
  a.lda = p.lda;
  a.ldb = p.ldb;
  a.ldo = p.ldo;
  a.ra_s_kb = p.ra_s_kb;
  a.rb_s_row = p.rb_s_row;
  a.rb_s_kb = p.rb_s_kb;
  a.M = (int)p.M;
  a.N = (int)p.N;
  a.K = (int)p.K;
  a.kblocks = (int)((p.K + 127) / 128);
  a.tiles_m = (int)((p.M + bm - 1) / bm);
  a.tiles_n = (int)((p.N + bn - 1) / bn);
  if (splits < 1) splits = 1;
  a.kb_per_split = (a.kblocks + splits - 1) / splits;
  if (a.kblocks == 0) a.kb_per_split = 0;
  hipError_t e;
  switch (cfg) {
    case 0: e = launch_mode<128, 128>(a, p.mode, splits, p.out_kind, stream); break;
    default: e = launch_mode<64, 64>(a, p.mode, splits, p.out_kind, stream); break;
  }
  if (e != hipSuccess || splits <= 1) return e;
  const int64_t total = p.M * p.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (p.out_kind == kOutBf16)
    hipLaunchKernelGGL(splitk_reduce_kernel<kOutBf16>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, (const float*)ws, splits, (int)p.M, (int)p.N, p.out, p.ldo);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<kOutF32>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, (const float*)ws, splits, (int)p.M, (int)p.N, p.out, p.ldo);
  return hipGetLastError();
}

}  // namespace fp8bw
