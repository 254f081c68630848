// decode_common.hpp -- pieces shared by the single-token and the batched
// decode kernels: the LDS layout of activation codes, the pinned router tree
// over chunk leaves, and the order key of the top-k.
#pragma once
#include "device_math.hpp"

namespace moeq4 {

// Activation codes in LDS: block b of a row of activation blocks starts at
// dword act_off(b) = 8b + 4*floor(b/8).  A lane owns 8 consecutive blocks,
// so the lanes of one row start 68 dwords apart (4 banks apart) and their
// 16-byte reads do not collide; without the pad they all hit one bank.
__device__ __forceinline__ int act_off(int b) { return 8 * b + 4 * (b >> 3); }
__host__ __device__ inline int act_row_dwords(int nb) { return 8 * nb + 4 * ((nb + 7) / 8); }

// Pairwise tree over v[0 .. n-1] (n a power of two <= 64); returns the root.
__device__ __forceinline__ float tree64(float (&v)[64], int n) {
#pragma unroll
  for (int w = 64; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; i++)
      if (w <= n) v[i] = v[2 * i] + v[2 * i + 1];
  return v[0];
}

// Order key: larger key = earlier in (logit desc, index asc); -0 and +0 tie
// as they do under a float comparison.
__device__ __forceinline__ uint64_t rank_key(float l, int e) {
  uint32_t u = __float_as_uint(l == 0.0f ? 0.0f : l);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
}

// Pairwise tree over the leaves c0 .. c0+L-1 of one expert (src = partials
// + e, leaf stride E); leaves >= nc are +0.
template <int L>
__device__ __forceinline__ float leaf_run(const float* __restrict__ src, int E, int c0, int nc) {
  float v[L];
#pragma unroll
  for (int j = 0; j < L; j++) {
    const int cc = c0 + j;
    const float t = src[(size_t)min(cc, nc - 1) * E];
    v[j] = cc < nc ? t : 0.0f;
  }
#pragma unroll
  for (int w = L; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; i++) v[i] = v[2 * i] + v[2 * i + 1];
  return v[0];
}

__device__ __forceinline__ float leaf_tree(const float* src, int E, int c0, int L, int nc) {
  switch (L) {
    case 1: return leaf_run<1>(src, E, c0, nc);
    case 2: return leaf_run<2>(src, E, c0, nc);
    case 4: return leaf_run<4>(src, E, c0, nc);
    case 8: return leaf_run<8>(src, E, c0, nc);
    case 16: return leaf_run<16>(src, E, c0, nc);
    default: return leaf_run<32>(src, E, c0, nc);
  }
}

// The router's pinned tree for one expert: the pairwise, level-by-level sum of
// its nc leaves (src = leaf 0, leaf stride E) padded with +0 to m =
// next_pow2(nc), taken as runs of up to 32 leaves and then pairwise over the
// runs (the same tree).  nc <= 512.
__device__ __forceinline__ float root_tree(const float* __restrict__ src, int E, int nc) {
  const int m = (int)next_pow2_u32((uint32_t)nc);
  if (m <= 32) return leaf_tree(src, E, 0, m, nc);
  const int nr = m / 32;                  // <= 16 runs (nc <= 512)
  float r[16];
#pragma unroll
  for (int i = 0; i < 16; i++) r[i] = i < nr ? leaf_run<32>(src, E, 32 * i, nc) : 0.0f;
#pragma unroll
  for (int w = 16; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; i++)
      if (w <= nr) r[i] = r[2 * i] + r[2 * i + 1];
  return r[0];
}

// The RMSNorm scale r = sqrtf(ss / H + eps) of one row y [H] (H/32 <= 512):
// ss is the per-32-chunk fused chain y*y from +0, the chunk partials summed
// pairwise level by level (padded with +0 to a power of two), the program of
// the library's RMSNorm.  Every thread of the block returns r; part and tmp
// are 512-float LDS buffers.  Contains barriers: call from the whole block.
__device__ __forceinline__ float rms_scale(const float* __restrict__ row, int H, float eps,
                                           float* part, float* tmp) {
  const int nc = H / BLK;
  const int m = (int)next_pow2_u32((uint32_t)nc);
  for (int c = threadIdx.x; c < m; c += blockDim.x) {
    float acc = 0.0f;
    if (c < nc)
      for (int i = 0; i < BLK; i++) {
        const float v = row[c * BLK + i];
        acc = __builtin_fmaf(v, v, acc);
      }
    part[c] = acc;
  }
  __syncthreads();
  float* src = part;
  float* dst = tmp;
  for (int w = m; w > 1; w >>= 1) {      // one level: dst[i] = src[2i] + src[2i+1]
    for (int i = threadIdx.x; i < w / 2; i += blockDim.x) dst[i] = src[2 * i] + src[2 * i + 1];
    __syncthreads();
    float* t = src;
    src = dst;
    dst = t;
  }
  return sqrtf(src[0] / (float)H + eps);
}

// Inverse of rank_key's logit part (-0 comes back as +0).
__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t u = (uint32_t)(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

}  // namespace moeq4
