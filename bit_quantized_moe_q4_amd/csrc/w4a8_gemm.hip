// w4a8_gemm.hip -- the W4A8 row program for many tokens on int8 MFMA.
//
// "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU",
// technical summary, Methodology 1-2: the decode kernel is W4A8 (4-bit
// weights, 8-bit activations, integer dots) and prefill a GEMM.  Here the
// W4A8 program runs as a GEMM: an int8 MFMA with K = 32 spans exactly one
// Q4_0 block, so one instruction yields the int32 dots of one block for a
// tile of (token, weight row) pairs.  Every dot is then rescaled on its own:
// value = (d_w * d_a) * (float)dot, and the values of a row are summed in the
// pinned pairwise tree over its blocks (+0 leaves past K/32) -- the decode
// row program, so out[m][n] is bit-identical to the one-token GEMV of token m
// against weight row n.  The per-block rescale is the cost: every
// accumulator value needs a correction, a conversion, two multiplies and a
// tree step in VALU after each MFMA.
//
// Operands: weights in the tile order of q4_tile (piece s of a 32-row group
// holds blocks 2s and 2s+1: lane l's 16 nibble bytes at 16 l, its scale at
// 1024 + 2 l); activations q [M][K] int8 with per-block scales d [M][K/32].
// The weight codes enter the MFMA unsigned (0..15) and the dot is corrected
// by -8 * (sum of the block's activation codes), exact in int32.
//
// Block: 4 waves, 32 tokens x 32 weight rows (one 32-row group of the tile
// order); wave w owns tokens m0 + 16 (w & 1) .. +15 and weight rows
// n0 + 16 (w >> 1) .. +15 and issues v_mfma_i32_16x16x32_i8 per block, which
// keeps four outputs per lane, so the tree's pending subtrees fit in 32
// registers.  MFMA lane l supplies token row l%16 (A) and weight row l%16 (B)
// with the block's K quarter g = l/16; its four results are the (token, row)
// pairs (4 g + r, l%16), r = 0..3.  K is taken in the same order on both
// sides: quarter g is the low (g < 2) or high (g >= 2) nibbles of weight bytes
// 8 (g%2) .. +7, i.e. block elements 8 g .. 8 g + 7.
//
// Activations are read four blocks at a time: lane quarter g loads all 32
// bytes of block b0 + g of its token row (whole cache lines), and a 4 x 4
// transpose across the lane quarters (two rounds of permlane swaps) leaves
// quarter g holding elements 8 g .. +7 of each of the four blocks.  The code
// sums for the -8 correction come from a second MFMA against weights that
// are all 8, so it yields 8 x the sum, already in the output layout.  The next four blocks' operands are
// in flight while the current four are reduced.
#include "launch.hpp"
#include "device_math.hpp"

namespace moeq4 {

typedef int w8_v4i __attribute__((ext_vector_type(4)));

constexpr int kW8Levels = 8;                 // tree levels: up to 128 blocks (K <= 4096)
constexpr long kW8Eights = 0x0808080808080808L;     // B operand of the code-sum MFMA: 8 x the sum

struct W8Quad {
  uint4 a0, a1;                              // 32 activation bytes: block b0 + g of the lane's token row
  long w[4];                                 // 8 weight nibble bytes of blocks b0 .. b0+3
  uint32_t sc[4];                            // the weight row's fp16 scale bits of blocks b0 .. b0+3
};

// CLAMP: blocks past the row read its last block (their leaves are +0)
template <bool CLAMP>
__device__ __forceinline__ W8Quad w8_load_quad(const int8_t* arow, const uint8_t* wrow, const uint8_t* srow,
                                               int b0, int nb, int g) {
  W8Quad o;
  const int ba = CLAMP ? min(b0 + g, nb - 1) : b0 + g;
  const uint4* ap = reinterpret_cast<const uint4*>(arow + 32 * ba);
  o.a0 = ap[0];
  o.a1 = ap[1];
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const int bw = CLAMP ? min(b0 + t, nb - 1) : b0 + t;
    const int piece = (bw >> 1) * 1152;
    o.w[t] = *reinterpret_cast<const long*>(wrow + piece + 512 * (bw & 1));
    o.sc[t] = *reinterpret_cast<const uint16_t*>(srow + piece + 64 * (bw & 1));
  }
  return o;
}

// slot t of quarter q holds bytes 8t..8t+7 of block b0+q; afterwards slot t
// of quarter g holds bytes 8g..8g+7 of block b0+t
__device__ __forceinline__ void w8_transpose(const W8Quad& q, long (&R)[4]) {
  uint32_t r[4][2] = {{q.a0.x, q.a0.y}, {q.a0.z, q.a0.w}, {q.a1.x, q.a1.y}, {q.a1.z, q.a1.w}};
#pragma unroll
  for (int t = 0; t < 2; t++)
#pragma unroll
    for (int d = 0; d < 2; d++) {            // quarters 2,3 of slot t <-> quarters 0,1 of slot t+2
      const auto p = __builtin_amdgcn_permlane32_swap(r[t][d], r[t + 2][d], false, false);
      r[t][d] = p[0];
      r[t + 2][d] = p[1];
    }
#pragma unroll
  for (int t = 0; t < 4; t += 2)
#pragma unroll
    for (int d = 0; d < 2; d++) {            // quarters 1,3 of slot t <-> quarters 0,2 of slot t+1
      const auto p = __builtin_amdgcn_permlane16_swap(r[t][d], r[t + 1][d], false, false);
      r[t][d] = p[0];
      r[t + 1][d] = p[1];
    }
#pragma unroll
  for (int t = 0; t < 4; t++) R[t] = (long)(((unsigned long)r[t][1] << 32) | r[t][0]);
}

// Leaves are taken in groups of G = 2^LG (G <= the padded leaf count, a
// power of two, so groups never straddle the tree's top).  Inside a group
// the merges are fixed at compile time; the group's total then joins the
// pending subtrees above level LG, whose depth depends on the group index.
template <int LG>
__device__ __forceinline__ void w8_leaf(float (&st)[4][kW8Levels], const float (&v)[4], int i, int grp) {
  // i: the leaf's index inside its group (a compile-time constant after unrolling)
  int t = 0;
  while (t < LG && ((i >> t) & 1)) t++;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    float x = v[r];
#pragma unroll
    for (int q = 0; q < LG; q++)
      if (q < t) x = st[r][q] + x;
    if (t < LG) {
      st[r][t] = x;
    } else {                                 // the group's last leaf: x is its total at level LG
      int lvl = LG;
#pragma unroll
      for (int q = 0; q < kW8Levels - 1 - LG; q++) {
        if (((grp >> q) & 1) == 0) break;
        lvl = LG + q + 1;
      }
#pragma unroll
      for (int q = LG; q < kW8Levels - 1; q++)
        if (q < lvl) x = st[r][q] + x;
#pragma unroll
      for (int q = LG; q < kW8Levels; q++)
        if (q == lvl) st[r][q] = x;
    }
  }
}

// One block of the row: the MFMAs, the correction and rescale of the four
// dots, and the leaf's merge.  LIVE = false: b may lie past the row (then the
// leaf is +0 and no dot is written).
template <int LG, bool LIVE, bool DOTS>
__device__ __forceinline__ void w8_block(float (&st)[4][kW8Levels], long a, long w, uint32_t sc, int b, int nb,
                                         int i, int grp, const float* da_l, int t0, int sh, int m0, int M, int N,
                                         int n, int32_t* dots) {
  const w8_v4i zero = {};
  const uint32_t lo = (uint32_t)w, hi = (uint32_t)((unsigned long)w >> 32);
  const long bw = (long)(((unsigned long)((hi >> sh) & 0x0f0f0f0fu) << 32) | ((lo >> sh) & 0x0f0f0f0fu));
  const w8_v4i acc = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, bw, zero, 0, 0, 0);
  const w8_v4i sum8 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, kW8Eights, zero, 0, 0, 0);
  const float dw = f16_bits_to_f32(sc);
  const int bc = LIVE ? b : min(b, nb - 1);
  const float4 d4 = *reinterpret_cast<const float4*>(da_l + bc * 32 + t0);
  const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
  const bool live = LIVE || b < nb;                          // (uniform)
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int32_t dot = acc[r] - sum8[r];
    if (DOTS && live) {
      const int m = m0 + t0 + r;
      if (m < M) dots[((size_t)m * N + n) * nb + b] = dot;
    }
    v[r] = (dw * dv[r]) * (float)dot;
    if (!LIVE) v[r] = live ? v[r] : 0.0f;                    // +0 leaves past the row
  }
  w8_leaf<LG>(st, v, i, grp);
}

template <int LG, bool DOTS>
__global__ void __launch_bounds__(256, 2) w4a8_gemm_kernel(const uint8_t* __restrict__ Wt, int N, int K,
                                                       const int8_t* __restrict__ qa,
                                                       const float* __restrict__ da, int M,
                                                       int32_t* __restrict__ dots, float* __restrict__ out) {
  constexpr int G = 1 << LG;
  constexpr int NQ = G >= 4 ? G / 4 : 1;                     // quads per group
  constexpr int TQ = G >= 4 ? 4 : G;                         // leaves per quad
  extern __shared__ __align__(16) uint8_t dyn[];
  const int nb = K / 32, nsteps = K / 64;
  float* da_l = reinterpret_cast<float*>(dyn);               // [nb][32] activation block scales per token
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int m0 = blockIdx.x * 32;
  for (int i0 = tid; i0 < nb * 32; i0 += 4 * 256) {
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int i = min(i0 + 256 * u, nb * 32 - 1);
      x[u] = da[(size_t)min(m0 + i % 32, M - 1) * nb + i / 32];
    }
#pragma unroll
    for (int u = 0; u < 4; u++)
      if (i0 + 256 * u < nb * 32) da_l[i0 + 256 * u] = x[u];   // index b * 32 + r
  }
  __syncthreads();

  const int j = lane % 16, g = lane / 16;
  const int tw = 16 * (wave & 1), rw = 16 * (wave >> 1);    // the wave's token and weight-row offsets
  const int n = blockIdx.y * 32 + rw + j;                    // this lane's weight row (N % 32 == 0: in range)
  const uint8_t* grp = Wt + (size_t)blockIdx.y * (size_t)nsteps * 1152;
  const uint8_t* wrow = grp + 16 * (rw + j) + 8 * (g & 1);
  const uint8_t* srow = grp + 1024 + 2 * (rw + j);
  const int8_t* arow = qa + (size_t)min(m0 + tw + j, M - 1) * K;
  const int sh = 4 * (g >> 1);
  const int t0 = tw + 4 * g;                                 // the lane's first output token in the tile
  int m2 = 1;
  while (m2 < nb) m2 <<= 1;

  float st[4][kW8Levels];
#pragma unroll
  for (int r = 0; r < 4; r++)
#pragma unroll
    for (int q = 0; q < kW8Levels; q++) st[r][q] = 0.0f;
  W8Quad nx = w8_load_quad<true>(arow, wrow, srow, 0, nb, g);
  for (int c = 0; c < m2; c += G) {
    if (c + G + 3 < nb) {                                    // (uniform) every leaf and every load in the row
#pragma unroll
      for (int qd = 0; qd < NQ; qd++) {
        const W8Quad cur = nx;
        nx = w8_load_quad<false>(arow, wrow, srow, c + 4 * qd + 4, nb, g);
        long R[4];
        w8_transpose(cur, R);
#pragma unroll
        for (int t = 0; t < TQ; t++)
          w8_block<LG, true, DOTS>(st, R[t], cur.w[t], cur.sc[t], c + 4 * qd + t, nb, 4 * qd + t, c >> LG, da_l, t0,
                             sh, m0, M, N, n, dots);
      }
    } else {                                                 // the row's end: clamped loads, +0 leaves
#pragma unroll
      for (int qd = 0; qd < NQ; qd++) {
        const W8Quad cur = nx;
        nx = w8_load_quad<true>(arow, wrow, srow, c + 4 * qd + 4, nb, g);
        long R[4];
        w8_transpose(cur, R);
#pragma unroll
        for (int t = 0; t < TQ; t++)
          w8_block<LG, false, DOTS>(st, R[t], cur.w[t], cur.sc[t], c + 4 * qd + t, nb, 4 * qd + t, c >> LG, da_l, t0,
                              sh, m0, M, N, n, dots);
      }
    }
  }
  int L = 0;
  while ((1 << L) < m2) L++;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int m = m0 + t0 + r;
    float res = 0.0f;
#pragma unroll
    for (int q = 0; q < kW8Levels; q++)
      if (q == L) res = st[r][q];
    if (m < M) out[(size_t)m * N + n] = res;
  }
}

size_t w4a8_gemm_lds_bytes(int K) { return (size_t)(K / 32) * 32 * 4; }

hipError_t launch_w4a8_gemm(const uint8_t* Wt, int N, int K, const int8_t* qa, const float* da, int M,
                            int32_t* dots, float* out, hipStream_t stream) {
  // token tiles along x: consecutive blocks go to different XCDs, so each
  // XCD's L2 holds its own token tiles' activations (N / 32 <= 65535)
  dim3 grid((M + 31) / 32, N / 32);
  int m2 = 1;
  while (m2 < K / 32) m2 <<= 1;                              // K >= 64: m2 >= 2
  const size_t lds = w4a8_gemm_lds_bytes(K);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), lds, stream, Wt, N, K, qa, da, M, dots, out);
  };
  if (dots) {
    if (m2 >= 8) go(w4a8_gemm_kernel<3, true>);
    else if (m2 == 4) go(w4a8_gemm_kernel<2, true>);
    else go(w4a8_gemm_kernel<1, true>);
  } else {
    if (m2 >= 8) go(w4a8_gemm_kernel<3, false>);
    else if (m2 == 4) go(w4a8_gemm_kernel<2, false>);
    else go(w4a8_gemm_kernel<1, false>);
  }
  return hipGetLastError();
}

}  // namespace moeq4
