// Device helpers for the gfx950 (CDNA4) kernels: bf16 unpacking, the
// saturating E4M3 cast, wavefront reductions.  HIP for gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bw {

// Largest finite OCP E4M3 magnitude and the amax floor that keeps
// 448/amax finite for an all-zero block.
constexpr float kFp8Max = 448.0f;
constexpr float kAmaxEps = 1e-12f;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even, in hardware: gfx950's
// v_cvt_pk_bf16_f32 converts a pair in one instruction (the same bits as
// rounding the fp32 pattern by hand for every finite input, at a fifth of
// the VALU work, which the GEMM epilogues pay for every output element).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
// One value: bf16 bits in the low half.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  return pack_bf16x2_rne(f, 0.f) & 0xFFFFu;
}

// Scale from a block amax: s = 448 / max(amax, eps), IEEE fp32 division
// (correctly rounded: the library is built without fast-math), and the
// reciprocal handed to the GEMM, recip = 1 / s.
__device__ __forceinline__ float scale_from_amax(float amax) {
  return kFp8Max / fmaxf(amax, kAmaxEps);
}
__device__ __forceinline__ float recip_of_scale(float s) { return 1.0f / s; }

// Saturating round-to-nearest-even cast of two fp32 values to E4M3,
// packed into byte lane `hi ? 2,3 : 0,1` of `old`.  The clamp to +-448
// comes first (v_med3), so the convert never sees an out-of-range value;
// v_cvt_pk_fp8_f32 then rounds to nearest even with the OCP encoding on
// gfx950.
template <bool HI>
__device__ __forceinline__ int cvt2_e4m3(float a, float b, int old) {
  a = __builtin_amdgcn_fmed3f(a, -kFp8Max, kFp8Max);
  b = __builtin_amdgcn_fmed3f(b, -kFp8Max, kFp8Max);
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// Four fp32 values -> one dword of E4M3 codes (byte i = value i).
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
  int r = cvt2_e4m3<false>(a, b, 0);
  r = cvt2_e4m3<true>(c, d, r);
  return (uint32_t)r;
}

// Max over the 16 lanes of a DPP row (lanes 16r..16r+15); every lane of the
// row receives the result.  Values are non-negative floats.
__device__ __forceinline__ float row16_max(float v) {
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}

// Max over the whole wavefront (64 lanes); uniform result.
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Max of |x| over the 8 bf16 values packed in a 16-byte vector.
__device__ __forceinline__ float absmax8(uint4 w) {
  float m0 = fmaxf(fabsf(bf16lo(w.x)), fabsf(bf16hi(w.x)));
  float m1 = fmaxf(fabsf(bf16lo(w.y)), fabsf(bf16hi(w.y)));
  float m2 = fmaxf(fabsf(bf16lo(w.z)), fabsf(bf16hi(w.z)));
  float m3 = fmaxf(fabsf(bf16lo(w.w)), fabsf(bf16hi(w.w)));
  return fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
}

// Quantize 8 bf16 values with scale s: 8 E4M3 codes in a uint2.
__device__ __forceinline__ uint2 quant8(uint4 w, float s) {
  uint2 r;
  r.x = cvt4_e4m3(bf16lo(w.x) * s, bf16hi(w.x) * s, bf16lo(w.y) * s, bf16hi(w.y) * s);
  r.y = cvt4_e4m3(bf16lo(w.z) * s, bf16hi(w.z) * s, bf16lo(w.w) * s, bf16hi(w.w) * s);
  return r;
}

}  // namespace fp8bw
