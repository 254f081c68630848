// w4a8_gemm.hip -- the W4A8 row program for many tokens on int8 MFMA.
//
// "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU",
// technical summary, Methodology 1-2: the decode kernel is W4A8 (4-bit
// weights, 8-bit activations, integer dots) and prefill a GEMM.  Here the
// W4A8 program runs as a GEMM: v_mfma_i32_32x32x32_i8 takes K = 32, exactly
// one Q4_0 block, so one instruction yields the int32 dots of one block for
// a 32 x 32 tile of (token, weight row) pairs.  Every dot is then rescaled on
// its own: value = (d_w * d_a) * (float)dot, and the values of a row are
// summed in the pinned pairwise tree over its blocks (+0 leaves past K/32)
// -- the decode row program, so out[m][n] is bit-identical to the one-token
// GEMV of token m against weight row n.  The per-block rescale is the cost:
// 16 accumulator values per lane and block need a correction, a conversion,
// two multiplies and a tree step in VALU against one 32-cycle MFMA.
//
// Operands: weights in the tile order of q4_tile (piece s of a 32-row group
// holds blocks 2s and 2s+1: lane l's 16 nibble bytes at 16 l, its scale at
// 1024 + 2 l); activations q [M][K] int8 with per-block scales d [M][K/32].
// The weight codes enter the MFMA unsigned (0..15) and the dot is corrected
// by -8 * (sum of the block's activation codes), exact in int32.
//
// Block: 4 waves, 32 tokens x 128 weight rows; wave w owns weight rows
// n0 + 32 w .. +31.  MFMA lane l supplies token row l%32 (A) and weight row
// l%32 (B), K half l/32 of the block; its 16 results are the (token, row)
// pairs (8 (r/4) + 4 (l/32) + r%4, l%32), r = 0..15.
#include "launch.hpp"
#include "device_math.hpp"

namespace moeq4 {

typedef int w8_v4i __attribute__((ext_vector_type(4)));
typedef int w8_v16i __attribute__((ext_vector_type(16)));

constexpr int kW8Levels = 8;                 // tree levels: up to 128 blocks (K <= 4096)

__global__ void __launch_bounds__(256) w4a8_gemm_kernel(const uint8_t* __restrict__ Wt, int N, int K,
                                                       const int8_t* __restrict__ qa,
                                                       const float* __restrict__ da, int M,
                                                       int32_t* __restrict__ dots, float* __restrict__ out) {
  extern __shared__ __align__(16) uint8_t dyn[];
  const int nb = K / 32, nsteps = K / 64;
  int32_t* sa_l = reinterpret_cast<int32_t*>(dyn);          // [nb][32] sum of a block's codes per token
  float* da_l = reinterpret_cast<float*>(sa_l + nb * 32);     // [nb][32]
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int m0 = blockIdx.y * 32;
  const int n0 = blockIdx.x * 128 + wave * 32;
  // per token row of the tile and block: the codes' sum and the scale
  for (int i = tid; i < nb * 32; i += blockDim.x) {
    const int r = i % 32, b = i / 32;
    const int m = min(m0 + r, M - 1);
    const uint4* q = reinterpret_cast<const uint4*>(qa + (size_t)m * K + 32 * b);
    const uint4 u0 = q[0], u1 = q[1];
    int s = 0;
    s = __builtin_amdgcn_sdot4((int)u0.x, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4((int)u0.y, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4((int)u0.z, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4((int)u0.w, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4((int)u1.x, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4((int)u1.y, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4((int)u1.z, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4((int)u1.w, 0x01010101, s, false);
    sa_l[b * 32 + r] = s;
    da_l[b * 32 + r] = da[(size_t)m * nb + b];
  }
  __syncthreads();

  const int j = lane % 32, h = lane / 32;
  const bool live_n = n0 < N;                                // (N % 32 == 0: a wave's rows are all in or out)
  const int nw = live_n ? n0 : N - 32;                       // dead waves read valid rows
  const uint8_t* wg = Wt + (size_t)(nw / 32) * (size_t)nsteps * 1152;   // the wave's 32-row group
  const int8_t* arow = qa + (size_t)min(m0 + j, M - 1) * K + 16 * h;
  int m2 = 1;
  while (m2 < nb) m2 <<= 1;

  float st[16][kW8Levels];
#pragma unroll
  for (int r = 0; r < 16; r++)
#pragma unroll
    for (int q = 0; q < kW8Levels; q++) st[r][q] = 0.0f;
  const w8_v16i zero = {};
  for (int b = 0; b < m2; b++) {
    float v[16];
    if (b < nb) {                                            // (uniform)
      const uint8_t* piece = wg + (size_t)(b / 2) * 1152;
      const uint4 nib = *reinterpret_cast<const uint4*>(piece + 16 * (j + 32 * (b & 1)));
      const uint32_t sc = *reinterpret_cast<const uint16_t*>(piece + 1024 + 2 * (j + 32 * (b & 1)));
      // K half h of the block: element k of the half is the low (h = 0) or
      // high (h = 1) nibble of byte k
      const int sh = 4 * h;
      const w8_v4i bw = {(int)((nib.x >> sh) & 0x0f0f0f0fu), (int)((nib.y >> sh) & 0x0f0f0f0fu),
                         (int)((nib.z >> sh) & 0x0f0f0f0fu), (int)((nib.w >> sh) & 0x0f0f0f0fu)};
      const w8_v4i aw = *reinterpret_cast<const w8_v4i*>(arow + 32 * b);
      const w8_v16i acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(aw, bw, zero, 0, 0, 0);
      const float dw = f16_bits_to_f32(sc);
#pragma unroll
      for (int g = 0; g < 4; g++) {
        const int r0 = 8 * g + 4 * h;                        // token rows r0 .. r0+3 of this lane
        const int4 s4 = *reinterpret_cast<const int4*>(sa_l + b * 32 + r0);
        const float4 d4 = *reinterpret_cast<const float4*>(da_l + b * 32 + r0);
        const int sv[4] = {s4.x, s4.y, s4.z, s4.w};
        const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const int r = 4 * g + e;
          const int32_t dot = acc[r] - 8 * sv[e];
          if (dots) {
            const int m = m0 + r0 + e, n = nw + j;
            if (live_n && m < M) dots[((size_t)m * N + n) * nb + b] = dot;
          }
          v[r] = (dw * dv[e]) * (float)dot;
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; r++) v[r] = 0.0f;              // +0 leaves past the row
    }
    // binary-counter merge: leaf b joins the pending subtrees of equal size
    int lvl = 0;
#pragma unroll
    for (int q = 0; q < kW8Levels - 1; q++) {
      if (((b >> q) & 1) == 0) break;
      lvl = q + 1;
    }
#pragma unroll
    for (int r = 0; r < 16; r++) {
      float x = v[r];
#pragma unroll
      for (int q = 0; q < kW8Levels - 1; q++)
        if (q < lvl) x = st[r][q] + x;
#pragma unroll
      for (int q = 0; q < kW8Levels; q++)
        if (q == lvl) st[r][q] = x;
    }
  }
  int L = 0;
  while ((1 << L) < m2) L++;
  if (!live_n) return;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int m = m0 + 8 * (r / 4) + 4 * h + r % 4;
    float res = 0.0f;
#pragma unroll
    for (int q = 0; q < kW8Levels; q++)
      if (q == L) res = st[r][q];
    if (m < M) out[(size_t)m * N + nw + j] = res;
  }
}

size_t w4a8_gemm_lds_bytes(int K) { return (size_t)(K / 32) * 32 * 8; }

hipError_t launch_w4a8_gemm(const uint8_t* Wt, int N, int K, const int8_t* qa, const float* da, int M,
                            int32_t* dots, float* out, hipStream_t stream) {
  dim3 grid((N + 127) / 128, (M + 31) / 32);
  hipLaunchKernelGGL(w4a8_gemm_kernel, grid, dim3(256), w4a8_gemm_lds_bytes(K), stream, Wt, N, K, qa, da, M,
                     dots, out);
  return hipGetLastError();
}

}  // namespace moeq4
