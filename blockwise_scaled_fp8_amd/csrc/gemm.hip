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
//  * A and B tiles for one K block are staged in LDS with the 16-byte chunk
//    index XOR-swizzled by row (see swz) so both the 16-byte direct-to-LDS
//    writes and the 16-byte fragment reads are bank-conflict free.  The
//    scales of the K block travel with the tile through LDS.
//  * Each lane feeds the MFMA 32 contiguous K bytes of its row for both A
//    and B (the same byte->k assignment on both sides, so the dot product
//    is over matching k whatever order the instruction uses internally).
//  * Any number of K blocks: the loop runs [kb_begin, kb_end) with no
//    unrolling assumption, so 1001 or 1002 blocks need nothing special.
//  * Split-K writes fp32 partials [split, M, N]; a separate kernel sums them
//    in split order (deterministic, no atomics).

#include <atomic>
#include <type_traits>

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
  int64_t ra_s_row, ra_s_kb;   // ra[m * ra_s_row + kb * ra_s_kb]
  int64_t rb_s_row, rb_s_kb;   // rb[beta(n) * rb_s_row + kb * rb_s_kb]
  int M, N, K;
  int kblocks;
  int tiles_m, tiles_n;
  int kb_per_split;
  // Large-tile kernel only: this launch covers grouped tile ids
  // [tile_base, tile_base + gridDim.x); with part_tiled the split partials
  // are stored tile-locally, [split][tile - tile_base][BM][BN], instead of
  // [split][M][N].
  int tile_base;
  int part_tiled;
  // Optional bf16 bias [N], added to each output row after scaling and before
  // the output cast; nullptr for none.  Split-K adds it in the reduce.
  const uint16_t* bias;
  // Grouped GEMM (large-tile kernel, no split): groups > 0 row groups of A
  // and out, group g covering rows [group_end[g-1], group_end[g]) (device
  // int32, cumulative, clamped to M), each with its own B (b + g*b_s_group)
  // and B scales (rb + g*rb_s_group).
  int groups;
  const int* group_end;
  int64_t b_s_group, rb_s_group;
  // Which rows of each group a grouped launch covers (group_part_rows), and
  // what grouped_split_pays weighs: the CUs one round of large tiles
  // occupies and the large tiles' column width.
  int group_part;
  int group_cus, group_big_bn;
  // B given in [K, N] layout (b[k * ldb + n], N contiguous) instead of
  // [N, K]; large 256x256 tiles only.
  int b_kn;
  // Persistent launch (gemm_v2_kernel with PERSIST): each workgroup runs
  // `rounds` tiles in turn, those a grid of rounds x gridDim.x workgroups
  // would have run; other launches leave it at 1.  Then workgroups
  // 0 .. tail_pieces - 1 each run one K piece of the leftover tiles
  // [tail_base, tail_base + tail_tiles) (tail_kbps K blocks a piece, fp32
  // tile-local partials [piece split][tile - tail_base][BM][BN], the same
  // pieces and workgroup order as the separate split launch); 0: none.
  int rounds;
  int tail_pieces, tail_kbps, tail_base, tail_tiles;
};

// A grouped GEMM on the large tiles runs as two launches: the large-tile
// kernel takes every group's whole 256-row tiles, and its last partial tile
// too when that holds more than 128 rows (part 1); the 64x64 small-tile
// kernel takes the remaining last partial tiles of at most 128 rows (part 2).
// A group's last tile of a few rows then costs a few 64-row tiles instead of
// a whole 256-row tile.  Part 0 is every row of every group in one launch.
constexpr int kGroupBigRows = 256;
constexpr int kGroupSmallRows = 128;

// Rows [first, first + rows) of a group of mg rows that part `part` covers.
__host__ __device__ __forceinline__ void group_part_rows(int part, int mg, int* first, int* rows) {
  if (part == 0) {
    *first = 0;
    *rows = mg;
    return;
  }
  const int full = mg / kGroupBigRows * kGroupBigRows, rem = mg - full;
  const bool big = rem > kGroupSmallRows;
  if (part == 1) {
    *first = 0;
    *rows = big ? mg : full;
  } else {
    *first = full;
    *rows = big ? 0 : rem;
  }
}

// Whether the two-launch split of a grouped GEMM pays for this group table:
// it does when the groups' last partial tiles of at most 128 rows, left on
// the large tiles, would take one more round of the chip's CUs than the
// large tiles take without them.  Otherwise they fit in the last round's
// idle CUs, and the second launch, which reads each such group's B once
// more, would only add time; both launches then run part 0 and nothing.
// Every workgroup of both launches reaches the same answer from the same
// table.
__device__ __forceinline__ bool grouped_split_pays(const GemmArgs& p) {
  int all = 0, big = 0, row0 = 0;
  for (int g = 0; g < p.groups; ++g) {
    const int end = max(row0, min(p.group_end[g], p.M));
    int first, rows;
    group_part_rows(1, end - row0, &first, &rows);
    all += (end - row0 + kGroupBigRows - 1) / kGroupBigRows;
    big += (rows + kGroupBigRows - 1) / kGroupBigRows;
    row0 = end;
  }
  const int64_t tn = (p.N + p.group_big_bn - 1) / p.group_big_bn;
  const int64_t rounds_all = ((int64_t)all * tn + p.group_cus - 1) / p.group_cus;
  const int64_t rounds_big = ((int64_t)big * tn + p.group_cus - 1) / p.group_cus;
  return rounds_big < rounds_all;
}

__device__ __forceinline__ float bias_at(const uint16_t* bias, int n) {
  return bias ? bf16lo(bias[n]) : 0.f;
}

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  // Scale operands 0 select the unscaled V_MFMA_F32_16X16X128_F8F6F4;
  // format 0 = FP8 E4M3 for both A and B.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// LDS tile layout: rows of 128 K-bytes; the logical 16-byte chunk c of row r
// is stored at physical chunk c ^ swz(r).  gfx950's LDS returns 256 bytes a
// clock (64 four-byte banks), so a 16-byte-per-lane read takes four passes
// of 16 lanes.  The lanes of a pass are not 16 consecutive ones: the bank
// conflict counter, over a set of probe patterns, matches passes of lanes
// {0-3, 8-11, 20-23, 28-31}, {4-7, 12-15, 16-19, 24-27} and the same sets
// + 32.  A fragment read has lane l on row l % 16 at logical chunk
// 2 (l / 16) + j, so one pass reads rows {0-3, 8-11} at chunk c and rows
// {4-7, 12-15} at chunk c ^ 2.  Rows 128 bytes apart alternate between the
// two 32-bank halves, so among the 8 even (and the 8 odd) rows of a pass
// the physical chunks must differ: swz(r) = (r >> 1) & 5 (bits 1 and 3 of
// r) does, for every c.  ((r >> 1) & 7 leaves a 2-way conflict.)
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 5; }

__device__ __forceinline__ v8i load_frag(const uint8_t* tile, int row, int half) {
  // 32 K-bytes of `row`: logical 16-byte chunks 2*half and 2*half+1.
  const int c0 = (2 * half) ^ swz(row);
  const int c1 = (2 * half + 1) ^ swz(row);
  const uint4 lo = *(const uint4*)(tile + row * 128 + (c0 << 4));
  const uint4 hi = *(const uint4*)(tile + row * 128 + (c1 << 4));
  v8i f;
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
  f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  return f;
}

// How many 16-row A sub-tiles ahead the large-tile kernel reads fragments.
constexpr int kRowPrefetch = 1;
// MFMA steps between a partial's MFMA and its rescale (ring of delay + 1).
constexpr int kRingDelay = 2;

// Fragment of a B tile stored in [K, N] layout (see gemm_v2_kernel): four
// transposing 8-byte LDS reads (ds_read_b64_tr_b8) 8 rows apart.  Within
// each 16-lane group, result byte b of lane i is byte i % 8 of the 8 bytes
// that lane 2 b + i / 8 addresses, so lanes 2 b and 2 b + 1 point at row
// r0 + b, columns c and c + 8, and lane i receives column c + i of rows
// r0 .. r0 + 7: 8 consecutive K values of its output column.
__device__ __forceinline__ v8i load_frag_kn(const uint8_t* tile, uint32_t off) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) v2i lds_v2i;
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  lds_u8* t = (lds_u8*)(uint8_t*)tile + off;
  const v2i r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(t));
  const v2i r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(t + 2048));
  const v2i r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(t + 4096));
  const v2i r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(t + 6144));
  v8i f;
  f[0] = r0.x; f[1] = r0.y; f[2] = r1.x; f[3] = r1.y;
  f[4] = r2.x; f[5] = r2.y; f[6] = r3.x; f[7] = r3.y;
  return f;
}

// Fragment read at precomputed byte offsets of its two 16-byte chunks.
__device__ __forceinline__ v8i load_frag_at(const uint8_t* tile, uint32_t lo, uint32_t hi) {
  const uint4 a = *(const uint4*)(tile + lo);
  const uint4 b = *(const uint4*)(tile + hi);
  v8i f;
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  return f;
}

template <int BM, int OUT>
__device__ __forceinline__ bool locate_group_tile(GemmArgs& p, int t, int* tm, int* tn, int* row0);

template <int BM, int BN, int MODE, int OUT, bool SPLIT>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs p_in) {
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
  GemmArgs p = p_in;
  int tm, tn;
  if (p.groups > 0) {
    // Grouped GEMM: p now addresses this tile's group (rows clamp to it).
    if (p.group_part == 2 && !grouped_split_pays(p)) return;
    int row0;
    if (!locate_group_tile<BM, OUT>(p, blockIdx.x, &tm, &tn, &row0)) return;
  } else {
    tm = blockIdx.x / p.tiles_n;
    tn = blockIdx.x - tm * p.tiles_n;
  }
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
      if (tid < BM) rsa = p.ra[(int64_t)kb * p.ra_s_kb + (int64_t)min(m0 + tid, p.M - 1) * p.ra_s_row];
      if (MODE == kBlockB128) {
        if (tid < SB) {
          const int nb = min(n0 / 128 + tid, (p.N - 1) / 128);
          rsb = p.rb[(int64_t)nb * p.rb_s_row + (int64_t)kb * p.rb_s_kb];
        }
      } else {
        if (tid < SB) rsb = p.rb[(int64_t)min(n0 + tid, p.N - 1) * p.rb_s_row + (int64_t)kb * p.rb_s_kb];
      }
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int r = lrow + 32 * i;
      *(uint4*)(&sA[buf][r * 128 + ((lc ^ swz(r)) << 4)]) = rA[i];
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int r = lrow + 32 * i;
      *(uint4*)(&sB[buf][r * 128 + ((lc ^ swz(r)) << 4)]) = rB[i];
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
          if (!SPLIT) val += bias_at(p.bias, n);
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

// ---------------------------------------------------------------------------
// Large-tile kernel: BM x BN workgroup tile, WGM x WGN waves, STAGES-deep
// LDS ring filled by direct buffer->LDS loads (buffer_load_dwordx4 ... lds:
// each lane's 16 bytes land at LDS base + 16 * lane, so a wave instruction
// fills one 1 KB "row octet" = 8 rows x 128 bytes; the XOR swizzle is
// applied by choosing which global chunk each lane fetches).  Scales ride
// the same ring via 4-byte direct loads.  The buffer (MUBUF) form is used
// rather than the global (FLAT) one because the compiler's wait insertion
// treats an outstanding FLAT load into LDS as possibly pending on the LDS
// counter too and then waits for every LDS read to return (lgkmcnt(0))
// before using any; with MUBUF loads the fragment reads get exact counts.
// The compiler does not order these LDS writes against later LDS reads, so
// the kernel waits with explicit vmcnt counts: every wave issues exactly
// LPS loads per stage, and before consuming stage kb+1 it waits until at
// most the loads of later stages are outstanding.

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt with vmcnt = N and no wait on expcnt / lgkmcnt (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// End of a K block: this wave's loads of the next stage have landed (vmcnt
// <= N) and its LDS reads of the current stage have returned (lgkmcnt 0),
// then the barrier makes both hold for every wave before any wave issues
// loads into the stage just read.
template <int N>
__device__ __forceinline__ void stage_sync() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
  __builtin_amdgcn_s_barrier();
}

// End of a K block for a wave that issues no direct loads: its LDS reads have
// returned, then the barrier.  It does not wait on vmcnt, so output stores it
// left in flight (persistent launch) keep draining under the K loop.
__device__ __forceinline__ void stage_sync_noload() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
  __builtin_amdgcn_s_barrier();
}

// Which copy of the K loop a wave runs: 0 the common one (every wave, loads
// issued by waves < LW), 1 a loader wave's, 2 a non-loader wave's.
template <int R> struct kloop_role { static constexpr int value = R; };

// Tile order: XCD-aware (the dispatcher deals workgroups round-robin to the
// 8 XCDs in linear workgroup order; xcd_remap gives each XCD a contiguous
// range of ids) then
// grouped (tile_to_mn: GROUP_M row-blocks per column sweep) so that
// concurrently running tiles on one XCD share A and B slices in that XCD's
// L2.
__device__ __forceinline__ void tile_to_mn(int tile, int tiles_m, int tiles_n, int* tm, int* tn) {
  constexpr int kGroupM = 8;
  const int per_group = kGroupM * tiles_n;
  const int group = tile / per_group;
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in_group = tile - group * per_group;
  *tm = first_m + in_group % gm;
  *tn = in_group / gm;
}

__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  constexpr int kXcds = 8;
  const int x = bid % kXcds, q = bid / kXcds;
  const int full = nwg / kXcds, rem = nwg % kXcds;
  return x * full + min(x, rem) + q;
}

// Raw buffer descriptor over `bytes` bytes from `base` (stride 0; gfx9
// dword3: 32-bit data format, no swizzle).  The large-tile kernels never
// rely on its range check: every direct load they issue addresses a row
// that exists (ragged edge tiles move their operand window back inside the
// matrix, see gemm_v2_kernel), because the check covers only the per-lane
// vector offset and not the scalar offset the row octets and K blocks use.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// One stage of direct buffer->LDS loads for K block kb (see gemm_v2_kernel).
// ars / brs cover the tile's BM rows of A / BN rows of B; a_voff / b_voff
// are this lane's byte offsets in its wave's first row octet, and octet i is
// 8 NW rows further (soffset), K block kb 128 bytes further.  ra_voff /
// rb_voff are this lane's byte offsets of its scale slots (row times the
// scale row stride), precomputed by the caller; ra_base / rb_base point at
// the scales of the tile's first row (row block) in K block 0.
template <int AI, int BI, int RAI, int RBI, int RAB, int RBB, int NW, int MODE, bool BKN>
__device__ __forceinline__ void issue_stage(const GemmArgs& p, int kb, uint8_t* sa, uint8_t* sb,
                                            float* sra, float* srb, __amdgpu_buffer_rsrc_t ars,
                                            __amdgpu_buffer_rsrc_t brs, uint32_t a_voff,
                                            uint32_t b_voff, uint32_t b_voff_hi,
                                            const uint8_t* bkn_base, int bkn_cols,
                                            const uint32_t (&ra_voff)[RAI > 0 ? RAI : 1],
                                            const uint32_t (&rb_voff)[RBI > 0 ? RBI : 1],
                                            const float* ra_base, int64_t ra_bytes,
                                            const float* rb_base, int64_t rb_bytes, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the kernel stub
  const int ko = kb * 128;
#pragma unroll
  for (int i = 0; i < AI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (lds_void_t*)(sa + (wave + NW * i) * 1024), 16,
                                             a_voff, ko + 8 * NW * i * (int)p.lda, 0, 0);
  if constexpr (BKN) {
    // B in [K, N] layout: the stage holds the K block's 128 rows of B, each
    // of the tile's 256 columns (row-major, 256 bytes a row); load i fills
    // rows 4 o .. 4 o + 3, o = wave + NW i.  The descriptor starts at the K
    // block's first row, so every offset stays below 128 rows.
    const __amdgpu_buffer_rsrc_t bk =
        buffer_rsrc(bkn_base + (int64_t)ko * p.ldb, (int64_t)127 * p.ldb + bkn_cols);
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int o = wave + NW * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(bk, (lds_void_t*)(sb + o * 1024), 16,
                                               ((o >> 3) & 1) ? b_voff_hi : b_voff,
                                               4 * o * (int)p.ldb, 0, 0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < BI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (lds_void_t*)(sb + (wave + NW * i) * 1024), 16,
                                               b_voff, ko + 8 * NW * i * (int)p.ldb, 0, 0);
  }
  if constexpr (MODE != kTensorwise) {
    const __amdgpu_buffer_rsrc_t rars = buffer_rsrc(ra_base + (int64_t)kb * p.ra_s_kb, ra_bytes);
#pragma unroll
    for (int i = 0; i < RAI; ++i) {
      const int blk = (wave + NW * i) % RAB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rars, (lds_void_t*)(sra + 64 * blk), 4, ra_voff[i],
                                               0, 0, 0);
    }
    const __amdgpu_buffer_rsrc_t rbrs = buffer_rsrc(rb_base + (int64_t)kb * p.rb_s_kb, rb_bytes);
#pragma unroll
    for (int i = 0; i < RBI; ++i) {
      const int blk = MODE == kBlockB128 ? 0 : (wave + NW * i) % RBB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rbrs, (lds_void_t*)(srb + 64 * blk), 4, rb_voff[i],
                                               0, 0, 0);
    }
  }
#endif
}

// Epilogue of the large-tile kernels: lane (frow, fhalf) holds, for each
// sub-tile (i, j), row mb + 16 i + frow and the four columns
// nb + 16 j + 4 fhalf + v.  The four are stored with one 8-byte (bf16) or
// 16-byte (fp32) store when the output rows allow it, else one by one.
// GUARD: only rows in [m_lo, M) and columns in [n_lo, N) are stored (an
// edge tile computes rows and columns of its neighbour, see gemm_v2_kernel);
// a quad is stored with one vector store only if it lies wholly inside and
// starts on a 4-column boundary.
template <bool GUARD, int TM, int TN, int MODE, int OUT, bool SPLIT>
__device__ __forceinline__ void store_acc(const GemmArgs& p, const v4f (&acc)[TM][TN], float tscale,
                                          int mb, int nb, int m_lo, int n_lo, int frow, int fhalf,
                                          float* pbase, int64_t pld, int pm0, int pn0) {
  const bool vec = SPLIT ? ((pld & 3) == 0 && ((size_t)pbase & 15) == 0)
                         : ((p.ldo & 3) == 0 && ((size_t)p.out & 15) == 0);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = mb + 16 * i + frow;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int nq = nb + 16 * j + 4 * fhalf;
      float val[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        val[v] = acc[i][j][v];
        if constexpr (MODE == kTensorwise) val[v] *= tscale;
        if constexpr (!SPLIT) {
          if (!GUARD || nq + v < p.N) val[v] += bias_at(p.bias, nq + v);
        }
      }
      if (vec && (!GUARD || (m >= m_lo && m < p.M && nq >= n_lo && nq + 3 < p.N &&
                             (nq & 3) == 0))) {
        if constexpr (SPLIT) {
          *(float4*)(pbase + (int64_t)(m - pm0) * pld + (nq - pn0)) =
              make_float4(val[0], val[1], val[2], val[3]);
        } else if constexpr (OUT == kOutBf16) {
          uint2 w;
          w.x = pack_bf16x2_rne(val[0], val[1]);
          w.y = pack_bf16x2_rne(val[2], val[3]);
          *(uint2*)((uint16_t*)p.out + (int64_t)m * p.ldo + nq) = w;
        } else {
          *(float4*)((float*)p.out + (int64_t)m * p.ldo + nq) =
              make_float4(val[0], val[1], val[2], val[3]);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int n = nq + v;
          if (!GUARD || (m >= m_lo && m < p.M && n >= n_lo && n < p.N)) {
            if constexpr (SPLIT) {
              pbase[(int64_t)(m - pm0) * pld + (n - pn0)] = val[v];
            } else if constexpr (OUT == kOutBf16) {
              ((uint16_t*)p.out)[(int64_t)m * p.ldo + n] = (uint16_t)f32_to_bf16_rne(val[v]);
            } else {
              ((float*)p.out)[(int64_t)m * p.ldo + n] = val[v];
            }
          }
        }
      }
    }
  }
}

// Epilogue of an interior 256x256 tile with bf16 output, through LDS.  The
// tile's 256 rows x 512 bytes go into the four 32 KB stage arrays, 64 rows
// each (array q holds rows 64 q .. 64 q + 63); within a row the 16-byte
// chunk c lies at c ^ (row & 15), so the 8-byte writes of 16 rows x one
// chunk and the 16-byte reads of 32 chunks of one row both meet every bank
// once per 256 bytes.  Wave (wm, wn) writes its 128 x 64 outputs (rows
// 128 wm .., columns 64 wn ..); after the barrier wave w reads rows
// 64 (w / 2) + 32 (w % 2) .. + 31, two rows per instruction, and stores
// them with 16-byte nontemporal stores, 32 lanes per 512-byte row.  Each
// wave must have waited for its own direct loads (vmcnt 0) before the call;
// the first barrier orders every wave's last fragment reads before the
// first write.
// With STORERS0 > 0 (persistent launch) only waves STORERS0 .. 7 (the ones
// that issue no direct loads) store, two rows per instruction over the 256
// rows, and nothing waits for the stores: the call ends with their LDS reads
// returned and a barrier, so the next tile's loads may fill the stages while
// the stores drain.  (A wave's s_endpgm waits for all its outstanding stores;
// with one tile per workgroup every round of tiles ended with the whole
// chip's output, 32 MB, draining while no CU computed.)
template <int TM, int TN, int MODE, int STORERS0 = 0>
__device__ __forceinline__ void store_tile_bf16_lds(const GemmArgs& p, const v4f (&acc)[TM][TN],
                                                    float tscale, uint8_t* s0, uint8_t* s1,
                                                    uint8_t* s2, uint8_t* s3, int m0, int n0,
                                                    int wave, int lane) {
  static_assert(TM == 8 && TN == 4, "256x256 tile of 8 waves of 128x64");
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  auto arr = [&](int q) -> uint8_t* { return q == 0 ? s0 : q == 1 ? s1 : q == 2 ? s2 : s3; };
  const int wmi = wave / 4, wni = wave % 4;
  const int frow = lane & 15, fhalf = lane >> 4;
  // (On gfx950 a workgroup-scope fence waits for LDS accesses only, so the
  // barriers below leave the storing waves' global stores in flight.)
  __syncthreads();   // every wave is done reading the stages
  // The lane's 16 columns are the same in every sub-tile row: their bias
  // values are read once, and without a bias nothing is added.
  auto write_tile = [&](auto with_bias) {
    constexpr bool kBias = decltype(with_bias)::value;
    float bv[TN][4];
    if constexpr (kBias) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) bv[j][v] = bf16lo(p.bias[n0 + 64 * wni + 16 * j + 4 * fhalf + v]);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      uint8_t* const qb = arr(2 * wmi + i / 4);
      const int rq = 16 * (i % 4) + frow;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        float val[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          val[v] = acc[i][j][v];
          if constexpr (MODE == kTensorwise) val[v] *= tscale;
          if constexpr (kBias) val[v] += bv[j][v];
        }
        u32x2 w;
        w.x = pack_bf16x2_rne(val[0], val[1]);
        w.y = pack_bf16x2_rne(val[2], val[3]);
        const int chunk = 8 * wni + 2 * j + (fhalf >> 1);
        *(u32x2*)(qb + rq * 512 + 16 * (chunk ^ frow) + 8 * (fhalf & 1)) = w;
      }
    }
  };
  if (p.bias)
    write_tile(std::true_type{});
  else
    write_tile(std::false_type{});
  const int c = lane & 31;
  __syncthreads();
  if constexpr (STORERS0 > 0) {
    if (wave >= STORERS0) {
      uint16_t* const ob = (uint16_t*)p.out + (int64_t)m0 * p.ldo + n0;
      for (int pr = wave - STORERS0; pr < 128; pr += 8 - STORERS0) {
        const int row = 2 * pr + (lane >> 5);   // tile row, in array row / 64
        const int rr = row & 63;
        const u32x4 d = *(const u32x4*)(arr(row >> 6) + rr * 512 + 16 * (c ^ (rr & 15)));
        __builtin_nontemporal_store(d, (u32x4*)(ob + (int64_t)row * p.ldo + 8 * c));
      }
    }
    __syncthreads();   // the stages are free again
  } else {
    const int q = wave >> 1, rbase = 32 * (wave & 1);
    const uint8_t* const qr = arr(q);
    uint16_t* const ob = (uint16_t*)p.out + (int64_t)(m0 + 64 * q) * p.ldo + n0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int row = rbase + 2 * k + (lane >> 5);
      const u32x4 d = *(const u32x4*)(qr + row * 512 + 16 * (c ^ (row & 15)));
      __builtin_nontemporal_store(d, (u32x4*)(ob + (int64_t)row * p.ldo + 8 * c));
    }
  }
}

// Epilogue of an interior 256x256 tile with fp32 values (an fp32 output with
// its bias, or a K piece's partial), through LDS like the bf16 epilogue but
// in two passes, the 256 KB tile being twice the 128 KB of stage arrays:
// pass h takes the sub-tile rows 4h .. 4h + 3 of every wave, i.e. tile rows
// 64 h .. 64 h + 63 and 128 + 64 h .. 128 + 64 h + 63, as 128 LDS rows of
// 1 KB (LDS row r = 64 wm + 16 i' + frow in array r / 32; 16-byte chunk c at
// c ^ (r & 15)).  Then wave w reads LDS rows 16 w .. 16 w + 15, one 1 KB row
// per instruction, and stores each as eight whole lines (16-byte
// nontemporal stores: the reduce that reads the partials runs on other
// XCDs' L2s anyway).  base addresses the tile's element (0, 0), ld its row
// stride in floats.
template <int TM, int TN, int MODE, bool BIAS>
__device__ __forceinline__ void store_tile_f32_lds(const GemmArgs& p, const v4f (&acc)[TM][TN],
                                                   float tscale, uint8_t* s0, uint8_t* s1,
                                                   uint8_t* s2, uint8_t* s3, float* base,
                                                   int64_t ld, int n0, int wave, int lane) {
  static_assert(TM == 8 && TN == 4, "256x256 tile of 8 waves of 128x64");
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  auto arr = [&](int q) -> uint8_t* { return q == 0 ? s0 : q == 1 ? s1 : q == 2 ? s2 : s3; };
  const int wmi = wave / 4, wni = wave % 4;
  const int frow = lane & 15, fhalf = lane >> 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    __syncthreads();   // the stages (pass 0) or the previous pass are read
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = 4 * h + ii;
      const int lr = 64 * wmi + 16 * ii + frow;
      uint8_t* const rowp = arr(lr >> 5) + (lr & 31) * 1024;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = 64 * wni + 16 * j + 4 * fhalf;
        float val[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          val[v] = acc[i][j][v];
          if constexpr (MODE == kTensorwise) val[v] *= tscale;
          if constexpr (BIAS) val[v] += bias_at(p.bias, n0 + col + v);
        }
        *(float4*)(rowp + 16 * ((col >> 2) ^ frow)) = make_float4(val[0], val[1], val[2], val[3]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int lr = 16 * wave + k;
      const int trow = 128 * (lr >> 6) + 64 * h + (lr & 63);
      const u32x4 d = *(const u32x4*)(arr(lr >> 5) + (lr & 31) * 1024 + 16 * (lane ^ (lr & 15)));
      __builtin_nontemporal_store(d, (u32x4*)(base + (int64_t)trow * ld + 4 * lane));
    }
  }
}

// Number of tiles of a grouped GEMM's group table (each group's row tiles
// times the column tiles), with the same clamping as locate_group_tile.
template <int BM>
__device__ __forceinline__ int grouped_tile_count(const GemmArgs& p) {
  int tiles = 0, row0 = 0;
  for (int g = 0; g < p.groups; ++g) {
    const int end = max(row0, min(p.group_end[g], p.M));
    int first, rows;
    group_part_rows(p.group_part, end - row0, &first, &rows);
    tiles += (rows + BM - 1) / BM;
    row0 = end;
  }
  return tiles * p.tiles_n;
}

// Grouped GEMM: find the group and tile of (remapped) tile id t, and point
// p at the rows of that group this launch covers (group_part_rows) in A, ra
// and out, and at its B and B scales.  Tiles are numbered group by group
// (tiles_m(g) x tiles_n each, grouped order inside a group).  Returns false
// for ids past the last tile (the grid is sized for the worst case of every
// group's last row tile being partial).
template <int BM, int OUT>
__device__ __forceinline__ bool locate_group_tile(GemmArgs& p, int t, int* tm, int* tn, int* row0_out) {
  int start = 0, row0 = 0;
  for (int g = 0; g < p.groups; ++g) {
    const int end = max(row0, min(p.group_end[g], p.M));
    int first, mg;
    group_part_rows(p.group_part, end - row0, &first, &mg);
    const int mt = (mg + BM - 1) / BM;
    const int nt = mt * p.tiles_n;
    if (t < start + nt) {
      const int r0 = row0 + first;
      tile_to_mn(t - start, mt, p.tiles_n, tm, tn);
      *row0_out = r0;
      p.a += (int64_t)r0 * p.lda;
      p.ra += (int64_t)r0 * p.ra_s_row;
      p.out = (uint8_t*)p.out + (int64_t)r0 * p.ldo * (OUT == kOutBf16 ? 2 : 4);
      p.b += (int64_t)g * p.b_s_group;
      p.rb += (int64_t)g * p.rb_s_group;
      p.M = mg;
      p.tiles_m = mt;
      return true;
    }
    start += nt;
    row0 = end;
  }
  return false;
}

template <int BM, int BN, int WGM, int WGN, int STAGES, int MODE, int OUT, bool SPLIT,
          bool BKN = false, bool PERSIST = false>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_v2_kernel(const GemmArgs p_in) {
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int AOCT = BM / 8, BOCT = BN / 8;
  // Waves that issue the direct loads.  Issuing a 1 KB direct load occupies
  // the CU's vector memory address path for about 16 cycles, and a wave that
  // issues a stage's loads stalls until they are taken in; with 8 waves only
  // waves 0 and 1 issue them, so the other wave on their SIMD and both waves
  // on the other SIMDs go straight to their MFMAs.
  constexpr int LW = NW == 8 ? 2 : NW;
  static_assert(AOCT % LW == 0 && BOCT % LW == 0, "row octets must split evenly over waves");
  constexpr int AI = AOCT / LW, BI = BOCT / LW;
  constexpr bool SCALED = MODE != kTensorwise;
  constexpr int RAB = BM / 64;                       // 64-row blocks of ra
  constexpr int RAI = SCALED ? (RAB + LW - 1) / LW : 0;
  constexpr int RBB = MODE == kBlockB1x128 ? BN / 64 : 1;
  constexpr int RBI = SCALED ? (RBB + LW - 1) / LW : 0;
  constexpr int LPS = AI + BI + RAI + RBI;           // loads per loading wave per stage
  constexpr int SBS = MODE == kBlockB1x128 ? BN : 64;
  static_assert(STAGES == 2 || STAGES == 3, "2 or 3 stages");
  static_assert(TN >= 2, "the rescale ring assumes at least two column sub-tiles");
  static_assert(LPS < 64, "vmcnt range");

  // Every stage is an LDS variable of its own and the stage loop below is
  // unrolled, so each access names its stage statically.  The compiler can
  // then tell that a stage's fragment reads do not alias the direct loads
  // in flight into another stage and does not wait for those loads before
  // the reads; the explicit vmcnt wait + barrier at the end of each K block
  // orders the loads before the reads of their own stage.
  constexpr int S3 = STAGES == 3;
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[BM * 128], sA1[BM * 128], sA2[S3 ? BM * 128 : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[BN * 128], sB1[BN * 128], sB2[S3 ? BN * 128 : 16];
  __shared__ __attribute__((aligned(16))) float sRa0[SCALED ? BM : 4], sRa1[SCALED ? BM : 4],
      sRa2[SCALED && S3 ? BM : 4];
  __shared__ __attribute__((aligned(16))) float sRb0[SCALED ? SBS : 4], sRb1[SCALED ? SBS : 4],
      sRb2[SCALED && S3 ? SBS : 4];
  uint8_t* const sA[3] = {sA0, sA1, sA2};
  uint8_t* const sB[3] = {sB0, sB1, sB2};
  float* const sRa[3] = {sRa0, sRa1, sRa2};
  float* const sRb[3] = {sRb0, sRb1, sRb2};

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm0 = (wave / WGN) * WM, wn0 = (wave % WGN) * WN;
  // Persistent launch (full rounds of interior 256x256 tiles, bf16 out, no
  // split): one workgroup per CU runs p_in.rounds tiles, the ones that
  // workgroups blockIdx.x + r * gridDim.x of a one-tile-per-workgroup grid
  // would run, so the tile order is unchanged.
  static_assert(!PERSIST || (BM == 256 && BN == 256 && NW == 8 && OUT == kOutBf16 && !SPLIT &&
                             !BKN),
                "persistent launch: 256x256 bf16 tiles only");
  const int rounds = PERSIST ? p_in.rounds : 1;
  auto run_tile = [&](int rnd, bool piece) {
  int tm, tn;
  GemmArgs p = p_in;
  if (piece) {   // persistent launch: a leftover tile's K piece
    p.tile_base = p_in.tail_base;
    p.kb_per_split = p_in.tail_kbps;
  }
  // Workgroup -> (K split, tile): the whole grid, split-major, dealt out
  // XCD-contiguously, so the workgroups an XCD runs together mostly share
  // one K range and read the same A and B slices through its L2 (with the
  // tiles of a split spread over XCDs, a long-K split-K GEMM streamed
  // nearly every operand byte from the fabric).
  // A grouped GEMM's grid covers the worst case of its group table; its
  // tiles are dealt out over the tiles that exist, so that the workgroups
  // past them are the last of every XCD rather than a run on the last XCDs
  // (which left the other XCDs a partly filled extra round).
  const int gx = gridDim.x * rounds;
  const int nwg = gx * gridDim.y;
  int wg;
  if (p.groups > 0) {
    if (p.group_part == 1 && !grouped_split_pays(p)) p.group_part = 0;
    const int T = grouped_tile_count<BM>(p);
    constexpr int kXcds = 8;
    const int x = blockIdx.x % kXcds, q = blockIdx.x / kXcds;
    const int full = T / kXcds, rem = T % kXcds;
    if (q >= full + (x < rem ? 1 : 0)) return;
    wg = x * full + min(x, rem) + q;
  } else {
    wg = xcd_remap(blockIdx.y * gx + blockIdx.x + rnd * gridDim.x, nwg);
  }
  int split = wg / gx;
  int tile_local = wg - split * gx;
  if (piece) {
    const int w2 = xcd_remap(blockIdx.x, p_in.tail_pieces);
    split = w2 / p_in.tail_tiles;
    tile_local = w2 - split * p_in.tail_tiles;
  }
  // Output tile [m0, m0 + BM) x [n0, n0 + BN).  The operand window the tile
  // loads, [ml, ml + BM) x [nl, nl + BN), is the same except at a ragged
  // edge, where it moves back to end exactly at the last row of A (of B):
  // every direct load then reads an existing row, and the edge tile stores
  // only its own rows and columns.  The host guarantees M >= BM and
  // N >= BN (the whole A of a grouped GEMM has at least BM rows) and, for
  // 128x128 B scales, N % 64 == 0, so nl stays a multiple of 64 and a
  // wave's 64 columns keep a single B scale block.
  int ml;
  if (p.groups > 0) {
    int row0;
    if (!locate_group_tile<BM, OUT>(p, tile_local, &tm, &tn, &row0)) return;
    ml = min(row0 + tm * BM, p_in.M - BM) - row0;   // may reach into earlier groups
  } else {
    tile_to_mn(p.tile_base + tile_local, p.tiles_m, p.tiles_n, &tm, &tn);
    ml = min(tm * BM, p.M - BM);
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int nl = min(n0, p.N - BN);
  const int kb_begin = split * p.kb_per_split;
  const int kb_end = min(p.kblocks, kb_begin + p.kb_per_split);

  // Per-lane byte offsets of this wave's first row octets of A and B.  Lane
  // 8q + c of a direct-load instruction fills physical chunk c of row 8o + q
  // (o = octet index), which holds logical chunk c ^ swz(8o + q); swz(8o + q)
  // = (4 (o & 1) + (q >> 1)) & 5 and o & 1 == wave & 1 because the octets of
  // a loading wave step by LW (even).
  static_assert(LW % 2 == 0, "octet parity must be the wave parity");
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ ((4 * (wave & 1) + (lrow >> 1)) & 5);
  const uint32_t a_voff = (uint32_t)((8 * wave + lrow) * p.lda + lchunk * 16);
  const uint32_t b_voff = (uint32_t)((8 * wave + lrow) * p.ldb + lchunk * 16);
  const __amdgpu_buffer_rsrc_t ars =
      buffer_rsrc(p.a + (int64_t)ml * p.lda, (int64_t)BM * p.lda);
  const __amdgpu_buffer_rsrc_t brs =
      buffer_rsrc(p.b + (int64_t)nl * p.ldb, (int64_t)BN * p.ldb);
  // B in [K, N] layout: row r of a K block's B tile (256 bytes, the tile's
  // columns) is stored with 16-byte chunk c at c ^ swz_kn(r), swz_kn(r) =
  // (r & 7) | (((r >> 5) & 1) << 3), so that each pass of a transposing
  // fragment read (32 lanes: 16 rows, one chunk each) meets every bank once.
  // Lane 16 q + c of a direct load fills physical chunk c of row 4 o + q;
  // (4 o + q) & 7 = 4 (o & 1) + q with o & 1 == wave & 1, and bit 3 of the
  // swizzle is bit 3 of o (two offsets).
  static_assert(!BKN || (BN == 256 && LW % 2 == 0), "[K, N] B tiles are 256 columns wide");
  uint32_t b_voff_hi = 0;
  uint32_t bkn_voff = 0;
  if constexpr (BKN) {
    const int q = lane >> 4, c = lane & 15, f0 = 4 * (wave & 1) + q;
    bkn_voff = (uint32_t)(q * p.ldb + 16 * (c ^ f0));
    b_voff_hi = (uint32_t)(q * p.ldb + 16 * (c ^ (f0 | 8)));
  }
  // Scale slots of this lane.  ra lands transposed per wave row band of 16 TM
  // rows, in groups of four sub-tiles: LDS slot k = 16 TM h + 64 q + 4 r + v
  // holds row 16 TM h + 16 (4 q + v) + r, so a lane (fragment row r) finds
  // the scales of sub-tiles 4q .. 4q + 3 in one 16-byte chunk, and the 16
  // rows' chunks of one group are 256 consecutive bytes (one conflict-free
  // pass).  128x128 B scales: lane l loads column block nl / 128 + l
  // (clamped to the last block); per-row B scales: slot 64 blk + l holds row
  // 64 blk + l of the window.
  static_assert(TM % 4 == 0, "scales grouped by four sub-tiles");
  uint32_t ra_voff[RAI > 0 ? RAI : 1];
  uint32_t rb_voff[RBI > 0 ? RBI : 1];
#pragma unroll
  for (int i = 0; i < RAI; ++i) {
    const int k = 64 * ((wave + LW * i) % RAB) + lane;
    const int kb16 = k % (16 * TM);
    const int row = (k / (16 * TM)) * (16 * TM) + 16 * (4 * (kb16 / 64) + kb16 % 4) + (kb16 % 64) / 4;
    ra_voff[i] = (uint32_t)(row * p.ra_s_row * 4);
  }
#pragma unroll
  for (int i = 0; i < RBI; ++i) {
    const int r = MODE == kBlockB128 ? min(nl / 128 + lane, (p.N - 1) / 128)
                                     : 64 * ((wave + LW * i) % RBB) + lane;
    rb_voff[i] = (uint32_t)(r * p.rb_s_row * 4);
  }
  const float* ra_base = p.ra + (int64_t)ml * p.ra_s_row;
  const int64_t ra_bytes = ((int64_t)(BM - 1) * p.ra_s_row + 1) * 4;
  const float* rb_base = MODE == kBlockB128 ? p.rb : p.rb + (int64_t)nl * p.rb_s_row;
  const int64_t rb_bytes = MODE == kBlockB128 ? ((int64_t)((p.N - 1) / 128) * p.rb_s_row + 1) * 4
                                              : ((int64_t)(BN - 1) * p.rb_s_row + 1) * 4;

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15, fhalf = lane >> 4;
  const int nkb = kb_end - kb_begin;
  // Every iteration issues one stage of loads, STAGES-1 K blocks ahead; past
  // the end it re-loads the last K block into a stage nobody reads again, so
  // the loop body has no branches (one scheduling region) and every wave
  // always has exactly LPS loads per stage in flight.
  const int kb_last = kb_end - 1;

  // The K loop.  A persistent launch runs it in two copies, one per wave
  // role, so that neither has a branch on the role inside the loop (one
  // there made the compiler spill): the loader waves issue the direct loads
  // and wait for them, the other waves never wait on vmcnt, which lets the
  // output stores they issued for the previous tile drain meanwhile.
#define FP8BW_ISSUE_ROLE(kb, st)                                                              \
  if (kRole == 1 || (kRole == 0 && wave < LW))                                                \
  issue_stage<AI, BI, RAI, RBI, RAB, RBB, LW, MODE, BKN>(                                     \
      p, (kb), sA[st], sB[st], sRa[st], sRb[st], ars, brs, a_voff, BKN ? bkn_voff : b_voff,    \
      b_voff_hi, p.b + nl, BN, ra_voff, rb_voff, ra_base, ra_bytes, rb_base, rb_bytes, wave)
  auto kloop = [&](auto role) {
  constexpr int kRole = decltype(role)::value;
  if (nkb > 0) {
    FP8BW_ISSUE_ROLE(kb_begin, 0);
    if constexpr (STAGES == 3) {
      FP8BW_ISSUE_ROLE(min(kb_begin + 1, kb_last), 1);
      if constexpr (kRole != 2) wait_vmcnt<LPS>();
    } else {
      if constexpr (kRole != 2) wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
  }
  for (int it0 = 0; it0 < nkb; it0 += STAGES) {
#pragma unroll
  for (int st = 0; st < STAGES; ++st) {
    const int it = it0 + st;
    if (it >= nkb) break;
    FP8BW_ISSUE_ROLE(min(kb_begin + it + STAGES - 1, kb_last), (st + STAGES - 1) % STAGES);

    // LDS byte offsets of this lane's fragment chunks and scales.  Sub-tile
    // i of a wave is 16 rows (2 KB) further down and keeps the same swizzle,
    // so every read is a base offset plus a constant.  The offsets are made
    // opaque each K block: otherwise the compiler hoists one address per
    // fragment and stage out of the loop and runs out of registers.
    uint32_t a_lo = (wm0 + frow) * 128 + (((2 * fhalf) ^ swz(wm0 + frow)) << 4);
    uint32_t a_hi = (wm0 + frow) * 128 + (((2 * fhalf + 1) ^ swz(wm0 + frow)) << 4);
    uint32_t b_lo = (wn0 + frow) * 128 + (((2 * fhalf) ^ swz(wn0 + frow)) << 4);
    uint32_t b_hi = (wn0 + frow) * 128 + (((2 * fhalf + 1) ^ swz(wn0 + frow)) << 4);
    uint32_t ra_off = (wm0 + 4 * frow) * 4;
    uint32_t rb_off = (wn0 + 4 * fhalf) * 4;
    asm volatile("" : "+v"(a_lo), "+v"(a_hi), "+v"(b_lo), "+v"(b_hi), "+v"(ra_off), "+v"(rb_off));
    // [K, N] B tiles: sub-tile j's transposing reads (see load_frag_kn) --
    // lanes 2 b and 2 b + 1 of group g = fhalf address row 32 g + b (+ 8 per
    // read), the two halves of the chunk holding columns wn0 + 16 j ..
    uint32_t bkn[BKN ? TN : 1];
    if constexpr (BKN) {
      const int r = 32 * fhalf + (frow >> 1);
      const int sw = (frow >> 1) | ((fhalf & 1) << 3);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        bkn[j] = (uint32_t)(r * 256 + 16 * (((wn0 >> 4) + j) ^ sw) + 8 * (frow & 1));
        asm volatile("" : "+v"(bkn[j]));
      }
    }
    auto load_b = [&](const uint8_t* tB_, int j) -> v8i {
      if constexpr (BKN) return load_frag_kn(tB_, bkn[j]);
      else return load_frag_at(tB_, b_lo + 2048 * j, b_hi + 2048 * j);
    };
    const uint8_t* tA = sA[st];
    const uint8_t* tB = sB[st];
    const uint8_t* tRa = (const uint8_t*)sRa[st];
    const uint8_t* tRb = (const uint8_t*)sRb[st];

    constexpr int PF = kRowPrefetch < TM ? kRowPrefetch : TM - 1;
    constexpr int NS = PF + 1;
    v8i bf[TN];
    v8i af[NS];
    if constexpr (MODE == kTensorwise) {
      // Fragment reads in the order the first MFMAs use them (B column 0,
      // A row 0, the other B columns, the prefetched A rows): LDS reads
      // complete in order, so the first MFMA waits for two fragments, not
      // for all of the K block's head (tensorwise +2%; with block scales,
      // whose products the head also computes, it measured slower).
      bf[0] = load_b(tB, 0);
      af[0] = load_frag_at(tA, a_lo, a_hi);
#pragma unroll
      for (int j = 1; j < TN; ++j) bf[j] = load_b(tB, j);
#pragma unroll
      for (int i = 1; i < PF; ++i) af[i] = load_frag_at(tA, a_lo + 2048 * i, a_hi + 2048 * i);
      __builtin_amdgcn_sched_barrier(0);   // keep that order
    } else {
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[j] = load_b(tB, j);
    }
    // Row scales of this lane's TM sub-tile rows (one row per sub-tile:
    // the partials are computed transposed, see below), times the 128x128
    // B scale of the wave's columns; per-row B scales of the lane's four
    // columns of each column sub-tile.
    float sa[TM];
    v4f sbc[TN];
    if constexpr (SCALED) {
#pragma unroll
      for (int q = 0; q < TM / 4; ++q) {
        const v4f s4 = *(const v4f*)(tRa + ra_off + 256 * q);
#pragma unroll
        for (int v = 0; v < 4; ++v) sa[4 * q + v] = s4[v];
      }
      if constexpr (MODE == kBlockB128) {
        const float sbn = sRb[st][(nl + wn0) / 128 - nl / 128];
#pragma unroll
        for (int i = 0; i < TM; ++i) sa[i] *= sbn;
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) sbc[j] = *(const v4f*)(tRb + rb_off + 64 * j);
      }
    }
    // MFMA-granularity pipeline over the TM x TN sub-tiles (row-major): the
    // partial of sub-tile t lands in ring slot t % 3 and is folded into its
    // accumulator two MFMAs later, when it is complete, so each MFMA issues
    // with the previous partials' rescale FMAs in its shadow.  The MFMA
    // takes the B fragment as its first operand, so it computes the sub-tile
    // transposed: lane l holds row 16 i + l % 16 and columns
    // 16 j + 4 (l / 16) + v, one A row (one row scale) per lane.
    constexpr int T = TM * TN;
    // A rows are read PF rows ahead into a ring of PF + 1 fragment slots:
    // row i + PF goes into the slot of row i - 1 as soon as row i starts
    // (row i - 1's MFMAs are issued).
    if constexpr (MODE != kTensorwise) {
#pragma unroll
      for (int i = 0; i < PF; ++i) af[i] = load_frag_at(tA, a_lo + 2048 * i, a_hi + 2048 * i);
    }
    v4f ring[kRingDelay + 1];
#pragma unroll
    for (int t = 0; t < T + kRingDelay; ++t) {
      const int i = t / TN, j = t % TN;
      if (t < T && j == 0 && i + PF < TM) {
        af[(i + PF) % NS] = load_frag_at(tA, a_lo + 2048 * (i + PF), a_hi + 2048 * (i + PF));
        // Keep the read here, ahead of the row's MFMAs: left alone, the
        // scheduler sinks it below them and reuses the current row's
        // fragment registers, and every row then waits for its own read.
        // (With per-row B scales the compiler's own order measured faster.)
        if constexpr (MODE != kBlockB1x128) __builtin_amdgcn_sched_barrier(0);
      }
      if (t < T) {
        if (MODE == kTensorwise)
          acc[i][j] = mfma_fp8(bf[j], af[i % NS], acc[i][j]);
        else
          ring[t % (kRingDelay + 1)] = mfma_fp8(bf[j], af[i % NS], v4f{0.f, 0.f, 0.f, 0.f});
      }
      if constexpr (SCALED) {
        if (t >= kRingDelay) {
          const int u = t - kRingDelay, iu = u / TN, ju = u % TN;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            if constexpr (MODE == kBlockB128)
              acc[iu][ju][v] = __builtin_fmaf(ring[u % (kRingDelay + 1)][v], sa[iu], acc[iu][ju][v]);
            else
              acc[iu][ju][v] = __builtin_fmaf(ring[u % (kRingDelay + 1)][v] * sbc[ju][v], sa[iu],
                                              acc[iu][ju][v]);
          }
        }
      }
      // 128x128 B blocks: one MFMA, then the 4 rescale FMAs of an earlier
      // partial.  (For per-row B scales the compiler's own interleave of the
      // 8 VALU ops per MFMA measured faster.)
      if constexpr (MODE == kBlockB128) {
        if (t < T) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
    }
    if constexpr (kRole == 2)
      stage_sync_noload();
    else if constexpr (STAGES == 3)
      stage_sync<LPS>();
    else
      stage_sync<0>();
  }
  }
  if constexpr (kRole != 2) wait_vmcnt<0>();
  };
  if constexpr (PERSIST) {
    if (wave < LW) kloop(kloop_role<1>{});
    else kloop(kloop_role<2>{});
  } else {
    kloop(kloop_role<0>{});
  }
#undef FP8BW_ISSUE_ROLE

  float tscale = 1.f;
  if constexpr (MODE == kTensorwise) tscale = p.ra[0] * p.rb[0];
  // Interior tiles store without per-element checks; edge tiles check rows
  // and columns.
  float* pbase = nullptr;
  int64_t pld = 0;
  int pm0 = 0, pn0 = 0;
  if constexpr (SPLIT) {
    if (p.part_tiled) {
      pbase = p.partial + ((int64_t)split * gridDim.x + tile_local) * (BM * BN);
      pld = BN;
      pm0 = m0;
      pn0 = n0;
    } else {
      pbase = p.partial + (int64_t)split * p.M * p.N;
      pld = p.N;
    }
  }
  const bool interior = ml == m0 && nl == n0 && m0 + BM <= p.M && n0 + BN <= p.N;
  if constexpr (PERSIST) {
    // Every tile of a persistent launch is interior (the host checks M, N,
    // the output stride and alignment).  (A second bf16 epilogue for the
    // last tile, stored by all eight waves, made the kernel spill.)
    if (piece) {
      float* const pb = p.partial + ((int64_t)split * p_in.tail_tiles + tile_local) * (BM * BN);
      store_tile_f32_lds<TM, TN, MODE, false>(p, acc, tscale, sA0, sA1, sB0, sB1, pb, BN, n0,
                                              wave, lane);
      return;
    }
    store_tile_bf16_lds<TM, TN, MODE, LW>(p, acc, tscale, sA0, sA1, sB0, sB1, m0, n0, wave, lane);
    return;
  }
  // An interior 256x256 tile is staged through LDS (free once the K loop is
  // done) so that every global store writes whole 128-byte lines, 16 bytes
  // a lane, instead of the quads of four columns the MFMA layout leaves in
  // each lane (a row of a wave's output then arriving in 32-byte (bf16) or
  // 64-byte (fp32) pieces).  The stores are nontemporal: nothing in this
  // launch reads the output again, and keeping it out of the L2 leaves the
  // L2 to the operands.  Same bits; on the linear step's shapes the bf16
  // tiles made the fwd and dgrad calls 2.6-2.8% faster, the fp32 partials
  // of the leftover tiles another 0.7-1.6%.
  if constexpr (BM == 256 && BN == 256 && WGM == 2 && WGN == 4) {
    if constexpr (SPLIT) {
      if (interior && (pld & 3) == 0 && ((size_t)pbase & 15) == 0) {
        store_tile_f32_lds<TM, TN, MODE, false>(p, acc, tscale, sA0, sA1, sB0, sB1,
                                                pbase + (int64_t)(m0 - pm0) * pld + (n0 - pn0),
                                                pld, n0, wave, lane);
        return;
      }
    } else if constexpr (OUT == kOutBf16) {
      if (interior && (p.ldo & 7) == 0 && ((size_t)p.out & 15) == 0) {
        store_tile_bf16_lds<TM, TN, MODE>(p, acc, tscale, sA0, sA1, sB0, sB1, m0, n0, wave, lane);
        return;
      }
    } else {
      if (interior && (p.ldo & 3) == 0 && ((size_t)p.out & 15) == 0) {
        store_tile_f32_lds<TM, TN, MODE, true>(p, acc, tscale, sA0, sA1, sB0, sB1,
                                               (float*)p.out + (int64_t)m0 * p.ldo + n0, p.ldo,
                                               n0, wave, lane);
        return;
      }
    }
  }
  if (interior)
    store_acc<false, TM, TN, MODE, OUT, SPLIT>(p, acc, tscale, m0 + wm0, n0 + wn0, m0, n0, frow,
                                               fhalf, pbase, pld, pm0, pn0);
  else
    store_acc<true, TM, TN, MODE, OUT, SPLIT>(p, acc, tscale, ml + wm0, nl + wn0, m0, n0, frow,
                                              fhalf, pbase, pld, pm0, pn0);
  };
  if constexpr (PERSIST) {
#pragma nounroll
    for (int rnd = 0; rnd < rounds; ++rnd) run_tile(rnd, false);
    if ((int)blockIdx.x < p_in.tail_pieces) run_tile(0, true);
  } else {
    run_tile(0, false);
  }
}

// Sum the split partials [split][M][N] in split order and convert.  With
// N % 4 == 0 a thread takes four consecutive columns (16-byte partial loads,
// one 8- or 16-byte store where the output row allows it); otherwise one
// element.  The sums are the same either way.
template <int OUT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, int M, int N,
                                                            void* __restrict__ out,
                                                            int64_t ldo,
                                                            const uint16_t* __restrict__ bias) {
  const int64_t total = (int64_t)M * N;
  if ((N & 3) == 0 && ((size_t)part & 15) == 0) {
    const bool vec = (ldo & 3) == 0 && ((size_t)out & 15) == 0;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total / 4;
         q += (int64_t)gridDim.x * 256) {
      float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int k = 0; k < splits; ++k) {
        const float4 v = *(const float4*)(part + (int64_t)k * total + 4 * q);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
      }
      const int64_t m = 4 * q / N, n = 4 * q - m * N;
      float val[4] = {s.x + bias_at(bias, (int)n), s.y + bias_at(bias, (int)n + 1),
                      s.z + bias_at(bias, (int)n + 2), s.w + bias_at(bias, (int)n + 3)};
      if (vec) {
        if (OUT == kOutBf16) {
          uint2 w;
          w.x = pack_bf16x2_rne(val[0], val[1]);
          w.y = pack_bf16x2_rne(val[2], val[3]);
          *(uint2*)((uint16_t*)out + m * ldo + n) = w;
        } else {
          *(float4*)((float*)out + m * ldo + n) = make_float4(val[0], val[1], val[2], val[3]);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (OUT == kOutBf16)
            ((uint16_t*)out)[m * ldo + n + v] = (uint16_t)f32_to_bf16_rne(val[v]);
          else
            ((float*)out)[m * ldo + n + v] = val[v];
        }
      }
    }
    return;
  }
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    float s = 0.f;
    for (int k = 0; k < splits; ++k) s += part[(int64_t)k * total + idx];
    const int64_t m = idx / N, n = idx - m * N;
    s += bias_at(bias, (int)n);
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

// Sum tile-local split partials ([split][tile][BM][BN], grouped tile ids
// tile_base ..) in split order and write the output tiles.  One thread per
// four consecutive columns of a tile row: 16-byte partial loads, one 8-byte
// (bf16) or 16-byte (fp32) store where the output row allows it.  Indices
// are 32-bit (the host keeps ntiles * BM * BN below 2^31).
template <int BM, int BN, int OUT>
__global__ __launch_bounds__(256) void splitk_reduce_tiled_kernel(
    const float* __restrict__ part, int splits, int ntiles, int tile_base, int tiles_m,
    int tiles_n, int M, int N, void* __restrict__ out, int64_t ldo,
    const uint16_t* __restrict__ bias) {
  static_assert(BN % 4 == 0, "quads of columns");
  constexpr int QPT = BM * BN / 4;   // quads per tile
  const int total = BM * BN * ntiles;
  const int nq = QPT * ntiles;
  const bool vec = (ldo & 3) == 0 && ((size_t)out & 15) == 0;
  for (int q = blockIdx.x * 256 + threadIdx.x; q < nq; q += gridDim.x * 256) {
    const int tl = q / QPT;
    const int e = (q - tl * QPT) * 4;
    const int r = e / BN, c = e - r * BN;
    int tm, tn;
    tile_to_mn(tile_base + tl, tiles_m, tiles_n, &tm, &tn);
    const int m = tm * BM + r, n = tn * BN + c;
    if (m >= M || n >= N) continue;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < splits; ++k) {
      const float4 v = *(const float4*)(part + (int64_t)k * total + 4 * q);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    float val[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (n + v < N) val[v] += bias_at(bias, n + v);
    if (vec && n + 3 < N) {
      if (OUT == kOutBf16) {
        uint2 w;
        w.x = pack_bf16x2_rne(val[0], val[1]);
        w.y = pack_bf16x2_rne(val[2], val[3]);
        *(uint2*)((uint16_t*)out + (int64_t)m * ldo + n) = w;
      } else {
        *(float4*)((float*)out + (int64_t)m * ldo + n) = make_float4(val[0], val[1], val[2], val[3]);
      }
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (n + v >= N) break;
        if (OUT == kOutBf16)
          ((uint16_t*)out)[(int64_t)m * ldo + n + v] = (uint16_t)f32_to_bf16_rne(val[v]);
        else
          ((float*)out)[(int64_t)m * ldo + n + v] = val[v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Config table.
struct Cfg {
  int bm, bn;
  int kind;   // 0: small-tile kernel, 1: large-tile kernel
};
static const Cfg kCfgs[] = {
    {128, 128, 0},   // 0: 4 waves of 64x64, register-staged double buffer
    {64, 64, 0},     // 1: small problems and tails
    {256, 128, 1},   // 2: 4 waves of 128x64, 3-stage direct-to-LDS ring
    {256, 256, 1},   // 3: 8 waves (2 per SIMD) of 128x64, 2-stage ring
};
constexpr int kNumCfgs = sizeof(kCfgs) / sizeof(kCfgs[0]);

int gemm_num_configs() { return kNumCfgs; }

bool gemm_config_ok(const GemmProblem& p, int cfg) {
  if (cfg < 0 || cfg >= kNumCfgs) return false;
  if (p.b_kn) {
    // B in [K, N] layout: 256x256 tiles only; 16-byte column chunks of B
    // rows (N % 16), and the offsets of a K block's 128 rows in 31 bits.
    if (cfg != 3 || p.K % 128 || p.M < 256 || p.N < 256 || p.N % 16) return false;
    if (p.ldb < 0 || p.ldb > (((int64_t)1 << 31) - 1 - 256) / 128) return false;
  }
  if (kCfgs[cfg].kind == 1) {
    // The large-tile kernels load whole 128-byte K blocks (no K tail), need
    // at least one whole tile in each dimension (an edge tile's operand
    // window moves back inside the matrix), and address a row tile of A or
    // B (at most 256 rows) and the scales of a tile with signed 32-bit
    // buffer offsets.
    if (p.K % 128) return false;
    if (p.M < kCfgs[cfg].bm || p.N < kCfgs[cfg].bn) return false;
    // 128x128 B scales: a wave's 64 columns must stay inside one scale
    // block when the last column tile moves back to end at row N - 1.
    if (p.mode == kBlockB128 && p.N % 64) return false;
    // n * stride + extra < 2^31, without forming the product
    auto fits31 = [](int64_t n, int64_t stride, int64_t extra) {
      const int64_t room = ((int64_t)1 << 31) - 1 - extra;
      return stride >= 0 && room >= 0 && stride <= room / n;
    };
    if (!fits31(256, p.lda, p.K) || !fits31(256, p.ldb, p.K)) return false;
    if (p.mode != kTensorwise) {
      if (!fits31(256 * 4, p.ra_s_row, 0)) return false;
      const int64_t rb_rows = p.mode == kBlockB128 ? (p.N + 127) / 128 : 256;
      if (!fits31(rb_rows * 4, p.rb_s_row, 0)) return false;
    }
  }
  return true;
}

// Compute units of the current device (the number of workgroups that run
// concurrently with one large-tile workgroup per CU); 256 when unknown.
// Cached per device; calls from several host threads may race to fill an
// entry, all with the same value, hence the relaxed atomics.
static int num_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Built-in tile configuration: the largest tiles that still give the chip
// at least half a round of workgroups, counting K splits where the call may
// split (each piece at least 8 K blocks).  Measured: M = N = 1024 with 1000
// K blocks runs 167 us on 256x256 tiles x 16 splits against 267 us on
// 256x128 x 16; the 256 x 4096 x 1024 per-tensor GEMM 10.4 us on 64x64
// tiles against 14.4 us on 256x128.
static int heuristic_config(const GemmProblem& p, bool allow_split, int cus) {
  if (p.b_kn) return 3;
  auto tiles = [&](int bm, int bn) { return ((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn); };
  const int64_t kblocks = (p.K + 127) / 128;
  const int64_t half = cus / 2;
  auto fills = [&](int bm, int bn) {
    const int64_t t = tiles(bm, bn);
    return t >= half || (allow_split && t * (kblocks / 8) >= cus);
  };
  if (gemm_config_ok(p, 3) && fills(256, 256)) return 3;
  if (gemm_config_ok(p, 2) && fills(256, 128)) return 2;
  if (p.M >= 128 && p.N >= 128 && fills(128, 128)) return 0;
  return 1;
}

// The main launch may run persistent (gemm_v2_kernel with PERSIST): 256x256
// tiles, [N, K] B, bf16 output, no K split, at least two whole rounds of
// tiles (one per CU), every tile interior (M and N multiples of 256) and
// output rows the staged epilogue can store whole (16-byte aligned rows).
static bool persistent_ok(const GemmProblem& p, int cfg, int splits, int nmain, int cus) {
  return cfg == 3 && !p.b_kn && splits == 1 && p.out_kind == kOutBf16 && cus > 0 &&
         nmain >= 2 * cus && nmain % cus == 0 && p.K >= 128 && p.M % 256 == 0 &&
         p.N % 256 == 0 && p.ldo % 8 == 0 && ((size_t)p.out & 15) == 0;
}

GemmPlan gemm_plan(const GemmProblem& p, int config, int splits, bool allow_split) {
  GemmPlan pl;
  const int cus = num_cus();
  pl.cfg = config >= 0 ? config : heuristic_config(p, allow_split && splits == 0, cus);
  const int bm = kCfgs[pl.cfg].bm, bn = kCfgs[pl.cfg].bn;
  const int64_t kblocks = (p.K + 127) / 128;
  pl.tiles = ((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn);
  pl.splits = 1;
  pl.tail_splits = 1;
  pl.tiles_full = pl.tiles;
  if (splits > 0) {
    pl.splits = splits;
  } else if (allow_split) {
    if (pl.tiles < cus && kblocks >= 16) {
      // Too few tiles to fill the chip: split K over the whole problem, one
      // round of pieces (a large-tile workgroup fills its CU's LDS; the
      // small-tile kernel runs two workgroups per CU).
      const int64_t slots = kCfgs[pl.cfg].kind == 1 ? cus : 2 * cus;
      int64_t want = (slots + pl.tiles - 1) / pl.tiles;
      int64_t maxs = kblocks / 8;
      int64_t sp = want < maxs ? want : maxs;
      if (sp < 1) sp = 1;
      const int64_t per = (kblocks + sp - 1) / sp;
      pl.splits = (int)((kblocks + per - 1) / per);
    } else if (kCfgs[pl.cfg].kind == 1 && pl.tiles > cus) {
      // Full rounds of one tile per CU run unsplit; the leftover tiles of
      // the last, partial round are split over K across the idle CUs.  Where
      // four or more pieces per tile would fit, half as many (twice as long)
      // measured faster: each piece writes a whole fp32 tile of partials,
      // so fewer pieces write and reduce fewer bytes (fwd call +0.8%, dgrad
      // +2.2% at the 16640 x 5120 x 8192 linear shapes).
      const int64_t full = pl.tiles / cus * cus, rem = pl.tiles - full;
      if (rem > 0) {
        int64_t sp = cus / rem;
        if (sp >= 4) sp /= 2;
        const int64_t maxs = kblocks / 4;
        if (sp > maxs) sp = maxs;
        if (sp >= 2) {
          const int64_t per = (kblocks + sp - 1) / sp;
          pl.tail_splits = (int)((kblocks + per - 1) / per);
          if (pl.tail_splits >= 2) pl.tiles_full = full;
          else pl.tail_splits = 1;
        }
      }
    }
  }
  size_t mn, part;
  if (pl.splits > 1)   // SIZE_MAX when it does not fit (no workspace is that large)
    pl.ws_bytes = __builtin_mul_overflow((size_t)p.M, (size_t)p.N, &mn) ||
                          __builtin_mul_overflow(mn, (size_t)pl.splits * sizeof(float), &part)
                      ? SIZE_MAX
                      : part;
  else if (pl.tail_splits > 1)
    pl.ws_bytes = (size_t)pl.tail_splits * (size_t)(pl.tiles - pl.tiles_full) * bm * bn * sizeof(float);
  else
    pl.ws_bytes = 0;
  return pl;
}

template <int BM, int BN, int WGM, int WGN, int STAGES, int MODE, bool BKN = false>
static hipError_t launch_v2(const GemmArgs& a, int ntiles, int splits, int out_kind,
                            hipStream_t stream) {
  dim3 grid((unsigned)ntiles, (unsigned)splits);
  dim3 block(64 * WGM * WGN);
  if constexpr (BM == 256 && BN == 256 && WGM == 2 && WGN == 4 && !BKN) {
    if (a.rounds > 1) {   // persistent: ntiles workgroups of a.rounds tiles each
      hipLaunchKernelGGL((gemm_v2_kernel<BM, BN, WGM, WGN, STAGES, MODE, kOutBf16, false, false, true>),
                         grid, block, 0, stream, a);
      return hipGetLastError();
    }
  }
  if (splits > 1)
    hipLaunchKernelGGL((gemm_v2_kernel<BM, BN, WGM, WGN, STAGES, MODE, kOutF32, true, BKN>), grid, block, 0, stream, a);
  else if (out_kind == kOutBf16)
    hipLaunchKernelGGL((gemm_v2_kernel<BM, BN, WGM, WGN, STAGES, MODE, kOutBf16, false, BKN>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_v2_kernel<BM, BN, WGM, WGN, STAGES, MODE, kOutF32, false, BKN>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int STAGES, bool BKN = false>
static hipError_t launch_v2_mode(const GemmArgs& a, int mode, int ntiles, int splits,
                                 int out_kind, hipStream_t stream) {
  switch (mode) {
    case kBlockB128: return launch_v2<BM, BN, WGM, WGN, STAGES, kBlockB128, BKN>(a, ntiles, splits, out_kind, stream);
    case kBlockB1x128: return launch_v2<BM, BN, WGM, WGN, STAGES, kBlockB1x128, BKN>(a, ntiles, splits, out_kind, stream);
    default: return launch_v2<BM, BN, WGM, WGN, STAGES, kTensorwise, BKN>(a, ntiles, splits, out_kind, stream);
  }
}

template <int BM, int BN>
static hipError_t launch_tiled_reduce(const GemmArgs& a, int splits, int ntiles, int out_kind,
                                      hipStream_t stream) {
  const int64_t total = (int64_t)BM * BN * ntiles;
  if (total >= ((int64_t)1 << 31)) return hipErrorInvalidValue;   // 32-bit indices
  int64_t blocks = (total / 4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (out_kind == kOutBf16)
    hipLaunchKernelGGL((splitk_reduce_tiled_kernel<BM, BN, kOutBf16>), dim3((unsigned)blocks),
                       dim3(256), 0, stream, (const float*)a.partial, splits, ntiles, a.tile_base,
                       a.tiles_m, a.tiles_n, a.M, a.N, a.out, a.ldo, a.bias);
  else
    hipLaunchKernelGGL((splitk_reduce_tiled_kernel<BM, BN, kOutF32>), dim3((unsigned)blocks),
                       dim3(256), 0, stream, (const float*)a.partial, splits, ntiles, a.tile_base,
                       a.tiles_m, a.tiles_n, a.M, a.N, a.out, a.ldo, a.bias);
  return hipGetLastError();
}

// One launch of large-tile config `cfg` over grouped tiles [base, base + ntiles).
static hipError_t launch_v2_cfg(int cfg, const GemmArgs& a, int mode, int ntiles, int splits,
                                int out_kind, hipStream_t stream) {
  if (a.b_kn) return launch_v2_mode<256, 256, 2, 4, 2, true>(a, mode, ntiles, splits, out_kind, stream);
  if (cfg == 2) return launch_v2_mode<256, 128, 2, 2, 3>(a, mode, ntiles, splits, out_kind, stream);
  return launch_v2_mode<256, 256, 2, 4, 2>(a, mode, ntiles, splits, out_kind, stream);
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

hipError_t launch_gemm(const GemmProblem& p, const GemmPlan& pl, void* ws, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  const int cfg = pl.cfg;
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
  a.ra_s_row = p.ra_s_row;
  a.ra_s_kb = p.ra_s_kb;
  a.rb_s_row = p.rb_s_row;
  a.rb_s_kb = p.rb_s_kb;
  a.M = (int)p.M;
  a.N = (int)p.N;
  a.K = (int)p.K;
  a.kblocks = (int)((p.K + 127) / 128);
  a.tiles_m = (int)((p.M + bm - 1) / bm);
  a.tiles_n = (int)((p.N + bn - 1) / bn);
  a.tile_base = 0;
  a.part_tiled = 0;
  a.bias = (const uint16_t*)p.bias;
  a.b_kn = p.b_kn;
  a.rounds = 1;
  a.tail_pieces = 0;
  a.groups = 0;
  a.group_part = 0;
  a.group_cus = 1;
  a.group_big_bn = bn;
  a.group_end = nullptr;
  a.b_s_group = a.rb_s_group = 0;
  const int splits = pl.splits < 1 ? 1 : pl.splits;
  a.kb_per_split = a.kblocks == 0 ? 0 : (a.kblocks + splits - 1) / splits;
  hipError_t e;
  if (kCfgs[cfg].kind == 0) {
    e = cfg == 0 ? launch_mode<128, 128>(a, p.mode, splits, p.out_kind, stream)
                 : launch_mode<64, 64>(a, p.mode, splits, p.out_kind, stream);
  } else {
    // Full rounds (or the whole problem) unsplit or whole-problem split-K.
    const int nmain = (int)(pl.tail_splits > 1 ? pl.tiles_full : pl.tiles);
    const int cus = num_cus();
    // Leftover tiles split over K into tile-local partials, then reduced.
    GemmArgs t = a;
    const int ntail = (int)(pl.tiles - pl.tiles_full);
    t.tile_base = (int)pl.tiles_full;
    t.part_tiled = 1;
    t.kb_per_split = (a.kblocks + pl.tail_splits - 1) / pl.tail_splits;
    // (Every piece needs a workgroup of the persistent grid: ntail * tail
    // splits <= cus, which the plan's choice of splits gives.)
    const bool persist = persistent_ok(p, cfg, splits, nmain, cus) &&
                         (pl.tail_splits <= 1 || (int64_t)ntail * pl.tail_splits <= cus);
    if (persist) {
      // Two or more full rounds of interior tiles: one workgroup per CU runs
      // its tiles of every round, then the leftover tiles' K pieces (each
      // piece's workgroup is free from its last tile on, with that tile's
      // stores still draining): bit-identical output, 1-2% faster.
      GemmArgs m = a;
      m.rounds = nmain / cus;
      if (pl.tail_splits > 1) {
        m.tail_pieces = ntail * pl.tail_splits;
        m.tail_kbps = t.kb_per_split;
        m.tail_base = t.tile_base;
        m.tail_tiles = ntail;
      }
      e = launch_v2_cfg(cfg, m, p.mode, cus, 1, p.out_kind, stream);
    } else {
      e = nmain > 0 ? launch_v2_cfg(cfg, a, p.mode, nmain, splits, p.out_kind, stream) : hipSuccess;
    }
    if (e == hipSuccess && pl.tail_splits > 1) {
      if (!persist) e = launch_v2_cfg(cfg, t, p.mode, ntail, pl.tail_splits, p.out_kind, stream);
      if (e == hipSuccess)
        e = cfg == 2 ? launch_tiled_reduce<256, 128>(t, pl.tail_splits, ntail, p.out_kind, stream)
                     : launch_tiled_reduce<256, 256>(t, pl.tail_splits, ntail, p.out_kind, stream);
    }
  }
  if (e != hipSuccess || splits <= 1) return e;
  const int64_t total = p.M * p.N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (p.out_kind == kOutBf16)
    hipLaunchKernelGGL(splitk_reduce_kernel<kOutBf16>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, (const float*)ws, splits, (int)p.M, (int)p.N, p.out, p.ldo,
                       (const uint16_t*)p.bias);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<kOutF32>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, (const float*)ws, splits, (int)p.M, (int)p.N, p.out, p.ldo,
                       (const uint16_t*)p.bias);
  return hipGetLastError();
}

// Grouped GEMM launch (see GemmArgs::groups).  The grid covers the worst
// case, sum over groups of ceil(M_g / BM) <= ceil(M / BM) + groups row tiles,
// times the column tiles; workgroups past the last tile return at once.
// Problems with fewer rows or columns than a large tile run on the
// small-tile kernel, which clamps its loads to each group's rows.
static int grouped_config(const GemmProblem& p) {
  if (p.N >= 256 && gemm_config_ok(p, 3)) return 3;
  if (p.N >= 128 && gemm_config_ok(p, 2)) return 2;
  return (p.M >= 128 && p.N >= 128) ? 0 : 1;
}

// Groups up to this count run as the two launches of group_part_rows; more
// run as one (each workgroup scans the group table, and the small-tile
// launch's grid grows with the count).
constexpr int kMaxSplitGroups = 64;

static bool grouped_split(const GemmProblem& p, int groups) {
  return kCfgs[grouped_config(p)].kind == 1 && groups <= kMaxSplitGroups;
}

bool grouped_gemm_ok(const GemmProblem& p, int groups) {
  if (groups <= 0 || p.K % 128) return false;
  // Grids: (row tiles + groups) x column tiles workgroups, in 31 bits.
  const int cfg = grouped_config(p);
  const int64_t grid = ((p.M + kCfgs[cfg].bm - 1) / kCfgs[cfg].bm + groups) *
                       ((p.N + kCfgs[cfg].bn - 1) / kCfgs[cfg].bn);
  const int64_t grid2 = grouped_split(p, groups) ? 2 * (int64_t)groups * ((p.N + 63) / 64) : 0;
  const int64_t lim = ((int64_t)1 << 31) - 1;
  return grid <= lim && grid2 <= lim;
}

hipError_t launch_grouped_gemm(const GemmProblem& p, int groups, const int* group_end,
                               int64_t b_s_group, int64_t rb_s_group, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return hipSuccess;
  const int cfg = grouped_config(p);
  const int bm = kCfgs[cfg].bm, bn = kCfgs[cfg].bn;
  GemmArgs a = {};
  a.a = (const uint8_t*)p.a;
  a.b = (const uint8_t*)p.b;
  a.ra = p.ra;
  a.rb = p.rb;
  a.out = p.out;
  a.lda = p.lda;
  a.ldb = p.ldb;
  a.ldo = p.ldo;
  a.ra_s_row = p.ra_s_row;
  a.ra_s_kb = p.ra_s_kb;
  a.rb_s_row = p.rb_s_row;
  a.rb_s_kb = p.rb_s_kb;
  a.M = (int)p.M;
  a.N = (int)p.N;
  a.K = (int)p.K;
  a.kblocks = (int)(p.K / 128);
  a.kb_per_split = a.kblocks;
  a.tiles_n = (int)((p.N + bn - 1) / bn);
  a.groups = groups;
  a.group_end = group_end;
  a.b_s_group = b_s_group;
  a.rb_s_group = rb_s_group;
  const int64_t tiles_m = (p.M + bm - 1) / bm + groups;
  if (kCfgs[cfg].kind == 0) {
    a.group_part = 0;
    a.group_cus = 1;
    a.group_big_bn = bn;
    a.tiles_m = (int)tiles_m;   // grid only; each tile's group sets its own
    return cfg == 0 ? launch_mode<128, 128>(a, p.mode, 1, p.out_kind, stream)
                    : launch_mode<64, 64>(a, p.mode, 1, p.out_kind, stream);
  }
  static_assert(kGroupBigRows == 256 && kGroupSmallRows <= kGroupBigRows,
                "part 1 runs on the 256-row large tiles");
  const bool split = grouped_split(p, groups);
  a.group_part = split ? 1 : 0;
  a.group_cus = num_cus();
  a.group_big_bn = bn;
  a.tiles_m = 0;
  hipError_t e = launch_v2_cfg(cfg, a, p.mode, (int)(tiles_m * a.tiles_n), 1, p.out_kind, stream);
  if (e != hipSuccess || !split) return e;
  // Part 2: the groups' last partial tiles of at most 128 rows, at most two
  // 64-row tiles per group.
  GemmArgs s2 = a;
  s2.group_part = 2;
  s2.tiles_n = (int)((p.N + 63) / 64);
  s2.tiles_m = 2 * groups;   // grid only
  return launch_mode<64, 64>(s2, p.mode, 1, p.out_kind, stream);
}

}  // namespace fp8bw
