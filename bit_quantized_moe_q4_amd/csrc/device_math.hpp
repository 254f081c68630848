// device_math.hpp -- small device helpers of the HIP path (gfx950 only).
//
// The fp32 programs here are evaluated bit-for-bit the same way as the
// library's published definitions (moe_q4.h): build with -ffp-contract=off,
// no fast-math, correctly rounded fp32 '/' and sqrtf (the HIP defaults), and
// denormals kept.  Every fused multiply-add is spelled __builtin_fmaf.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq4 {

constexpr int BLK = 32;       // elements per quantisation block
constexpr int Q4B = 18;       // bytes per Q4_0 block

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  _Float16 h;
  uint16_t b = (uint16_t)bits16;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;                       // exact
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;              // round to nearest even, subnormals kept
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);  // exact
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;                  // round to nearest even
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

// Two floats rounded to bf16 (nearest, ties to even) by one packed
// conversion: a in the low half, b in the high half.
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const f32x2v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

#if defined(__HIP_DEVICE_COMPILE__)   // buffer descriptors exist only in the device pass
// Buffer resource of a wave-uniform byte range; readfirstlane makes its
// uniformity explicit so the descriptor lives in scalar registers.  Raw
// accesses at offsets past `bytes` read zeros and drop stores.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* u = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, 0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
#endif

// Fixed fp32 exponential.  Cody & Waite range reduction (Software Manual for
// the Elementary Functions, 1980): n = rint(x*log2 e), r = x - n*ln2 with ln2
// split into a 15-bit-significand head (n*head exact for |n| < 2^9) and a
// tail; exp(r) by the degree-7 Taylor polynomial (fp32-rounded 1/i!) in
// Horner form with fused multiply-adds; result = ldexp(p, n).  x is first
// clamped to [-104, 89] (ldexp then yields 0 and +inf at the ends).
__device__ __forceinline__ float exp_p(float x) {
  const float kLog2e = 1.44269502162933349609375f;
  const float kLn2Hi = 0.693145751953125f;
  const float kLn2Lo = 1.428606765330187045e-06f;
  x = fminf(fmaxf(x, -104.0f), 89.0f);
  float n = rintf(x * kLog2e);
  float r = __builtin_fmaf(-n, kLn2Hi, x);
  r = __builtin_fmaf(-n, kLn2Lo, r);
  float p = (float)(1.0 / 5040.0);
  p = __builtin_fmaf(p, r, (float)(1.0 / 720.0));
  p = __builtin_fmaf(p, r, (float)(1.0 / 120.0));
  p = __builtin_fmaf(p, r, (float)(1.0 / 24.0));
  p = __builtin_fmaf(p, r, (float)(1.0 / 6.0));
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return ldexpf(p, (int)n);
}

// silu(g) = g / (1 + exp_p(-g)), IEEE division.
__device__ __forceinline__ float silu_p(float g) { return g / (1.0f + exp_p(-g)); }

__device__ __forceinline__ uint32_t next_pow2_u32(uint32_t n) {
  uint32_t m = 1;
  while (m < n) m <<= 1;
  return m;
}

// Pairwise tree over the lanes of one 64-wide wavefront: lane i holds leaf i
// of an aligned group of `width` lanes (a power of two <= 64).  After the
// butterfly every lane of the group holds the level-by-level pairwise sum of
// the group's leaves (IEEE addition is commutative, so v[i] + v[i^m] and
// v[i^m] + v[i] are the same value).
__device__ __forceinline__ float wave_tree_sum(float v, int width) {
  for (int m = 1; m < width; m <<= 1) v = v + __shfl_xor(v, m, 64);
  return v;
}

template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  const int l2 = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWMASK, 0xf, false);
  const int h2 = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWMASK, 0xf, false);
  return ((uint64_t)(uint32_t)h2 << 32) | (uint32_t)l2;
}

// Maximum of v over the 64 lanes (all active), by DPP lane moves: xor 1 and
// 2 inside quads, mirrors inside 8 and 16 lanes, then row broadcasts that
// leave the maximum in lane 63; returned in every lane.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  auto mx = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  v = mx(v, dpp_u64<0xb1, 0xf>(v));      // quad_perm [1,0,3,2]
  v = mx(v, dpp_u64<0x4e, 0xf>(v));      // quad_perm [2,3,0,1]
  v = mx(v, dpp_u64<0x141, 0xf>(v));     // row_half_mirror
  v = mx(v, dpp_u64<0x140, 0xf>(v));     // row_mirror
  v = mx(v, dpp_u64<0x142, 0xa>(v));     // row_bcast:15 into rows 1, 3
  v = mx(v, dpp_u64<0x143, 0xc>(v));     // row_bcast:31 into rows 2, 3
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

}  // namespace moeq4
