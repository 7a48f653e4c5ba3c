// Device-side helpers shared by the gfx950 kernels of libpagedkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// c + a.lo * b.lo + a.hi * b.hi over packed bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Max / sum over the 16 lanes of each row (lanes 16 r .. 16 r + 15), the
// result in all of them: quad swaps, then the mirror inside each half row,
// then the mirror of the row (DPP moves, no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm(1, 0, 3, 2)
  v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm(2, 3, 0, 1)
  v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
  return fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  return v + dpp_f32<0x140>(v);
}

// Value of v in lane `src` (any lane of the wave), per lane.
__device__ __forceinline__ float lane_get(float v, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src * 4, __float_as_int(v)));
}

// Symmetric integer code of x for a row scale s = absmax / MAXC (IEEE fp32
// division, round half to even, clamp to +-MAXC); s == 0 means an all-zero
// (or underflowed) row and gives 0.  MAXC is 127 for int8 and 7 for INT4.
// Used by every writer of those caches so their codes agree bit for bit.
template <int MAXC>
__device__ __forceinline__ int quantize_sym(float x, float s) {
  if (!(s > 0.f)) return 0;
  return static_cast<int>(fminf(fmaxf(rintf(x / s), -static_cast<float>(MAXC)), static_cast<float>(MAXC)));
}
__device__ __forceinline__ int quantize_code(float x, float s) { return quantize_sym<127>(x, s); }

// Byte of two INT4 codes: lo in bits 0..3, hi in bits 4..7, two's complement.
__device__ __forceinline__ uint32_t pack_int4_pair(int lo, int hi) {
  return (static_cast<uint32_t>(lo) & 0xfu) | ((static_cast<uint32_t>(hi) & 0xfu) << 4);
}

// FP8 code of x for scale s: x / s (IEEE fp32 division) rounded to the
// nearest OCP E4M3 value (bias 7, largest finite 448, ties to the even code)
// by the hardware conversion.  x / s is clamped to +-448 first: it can pass
// 448 only through the rounding of s, where 448 is the nearest code anyway,
// and the conversion does not saturate.  s == 0 (all-zero or underflowed
// row) gives code 0.  Used by every FP8 writer so their codes agree.
__device__ __forceinline__ uint32_t fp8_code(float x, float s) {
  if (!(s > 0.f)) return 0u;
  const float r = fminf(fmaxf(x / s, -448.f), 448.f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(r, 0.f, 0, false)) & 0xffu;
}

// E5M2 code of x for scale s = absmax / 57344: x / s rounded to the nearest
// E5M2 value (bias 15, largest finite 57344, ties to the even code) by the
// hardware conversion, after clamping to +-57344 so that it never yields an
// infinity; s == 0 gives code 0.
__device__ __forceinline__ uint32_t e5m2_code(float x, float s) {
  if (!(s > 0.f)) return 0u;
  const float r = fminf(fmaxf(x / s, -57344.f), 57344.f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_bf8_f32(r, 0.f, 0, false)) & 0xffu;
}

// Combine a value across the four 16-lane groups of a wave (lanes l, l^16,
// l^32, l^48) with two VALU lane swaps, no LDS traffic: v_permlane16_swap
// of a register with itself hands every lane its value and that of the lane
// 16 away (rows 0 <-> 1, 2 <-> 3), v_permlane32_swap that of the lane 32
// away.  Every lane ends with the same bits ((v0 op v1) op (v2 op v3)).
__device__ __forceinline__ float groups_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

__device__ __forceinline__ float groups_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

}  // namespace pkv
