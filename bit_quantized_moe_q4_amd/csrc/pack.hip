// pack.hip -- Q4_0 weight packing and 8-bit activation quantisation.
//
// Formats ("A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011
// GPU", technical summary, Methodology 2: group-wise symmetric 4-bit Q4_0
// weights, 8-bit activations on the decode path); the exact block layout and
// rounding rules are the ones stated in moe_q4.h.
//
// Both kernels are one thread per 32-element block: packing runs once per
// weight load and activation quantisation of a decode step is 64 blocks, so
// neither is on a bandwidth-critical path.
#include "launch.hpp"
#include "device_math.hpp"

namespace moeq4 {

__global__ void __launch_bounds__(256) q4_pack_kernel(const float* __restrict__ w, int64_t nblocks,
                                                      uint16_t* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nblocks) return;
  const float4* src = reinterpret_cast<const float4*>(w + i * BLK);
  float v[BLK];
#pragma unroll
  for (int c = 0; c < BLK / 4; c++) {
    float4 t = src[c];
    v[4 * c] = t.x; v[4 * c + 1] = t.y; v[4 * c + 2] = t.z; v[4 * c + 3] = t.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < BLK; j++) amax = fmaxf(amax, fabsf(v[j]));
  uint16_t dh = f32_to_f16_bits(amax / 7.0f);
  float df = f16_bits_to_f32(dh);
  uint32_t q[BLK];
#pragma unroll
  for (int j = 0; j < BLK; j++) {
    float t = roundf(v[j] / df);
    t = fminf(fmaxf(t, -8.0f), 7.0f);
    q[j] = (df == 0.0f) ? 8u : (uint32_t)((int)t + 8);
  }
  // 18 bytes = 9 little-endian halfwords: d, then bytes (q_j | q_{j+16} << 4)
  uint16_t* dst = out + i * (Q4B / 2);
  dst[0] = dh;
#pragma unroll
  for (int p = 0; p < 8; p++) {
    uint32_t lo = q[2 * p] | (q[2 * p + 16] << 4);
    uint32_t hi = q[2 * p + 1] | (q[2 * p + 17] << 4);
    dst[1 + p] = (uint16_t)(lo | (hi << 8));
  }
}

// Q8_0 weights ("A Modern Multimodal Assistant on a 6 GB 2011 GPU", abstract:
// 8-bit weights): d = fp16(amax/127), q = clamp(roundf(w/d), -127, 127);
// 34 bytes = d then the 32 int8 codes in element order.
__global__ void __launch_bounds__(256) q8w_pack_kernel(const float* __restrict__ w, int64_t nblocks,
                                                       uint16_t* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nblocks) return;
  const float4* src = reinterpret_cast<const float4*>(w + i * BLK);
  float v[BLK];
#pragma unroll
  for (int c = 0; c < BLK / 4; c++) {
    float4 t = src[c];
    v[4 * c] = t.x; v[4 * c + 1] = t.y; v[4 * c + 2] = t.z; v[4 * c + 3] = t.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < BLK; j++) amax = fmaxf(amax, fabsf(v[j]));
  uint16_t dh = f32_to_f16_bits(amax / 127.0f);
  float df = f16_bits_to_f32(dh);
  uint32_t q[BLK];
#pragma unroll
  for (int j = 0; j < BLK; j++) {
    float t = (df == 0.0f) ? 0.0f : roundf(v[j] / df);
    t = fminf(fmaxf(t, -127.0f), 127.0f);
    q[j] = (uint32_t)(int)t & 0xffu;
  }
  // 34 bytes = 17 little-endian halfwords: d, then code pairs (q_2p | q_2p+1 << 8)
  uint16_t* dst = out + i * 17;
  dst[0] = dh;
#pragma unroll
  for (int p = 0; p < 16; p++) dst[1 + p] = (uint16_t)(q[2 * p] | (q[2 * p + 1] << 8));
}

hipError_t launch_q8w_pack(const float* w, int64_t rows, int64_t K, void* packed, hipStream_t stream) {
  int64_t nblocks = rows * (K / BLK);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(q8w_pack_kernel, dim3((uint32_t)((nblocks + 255) / 256)), dim3(256), 0, stream, w,
                     nblocks, static_cast<uint16_t*>(packed));
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) q8_quantize_kernel(const float* __restrict__ x,
                                                          int64_t nblocks, int8_t* __restrict__ q,
                                                          float* __restrict__ d) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nblocks) return;
  const float4* src = reinterpret_cast<const float4*>(x + i * BLK);
  float v[BLK];
#pragma unroll
  for (int c = 0; c < BLK / 4; c++) {
    float4 t = src[c];
    v[4 * c] = t.x; v[4 * c + 1] = t.y; v[4 * c + 2] = t.z; v[4 * c + 3] = t.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < BLK; j++) amax = fmaxf(amax, fabsf(v[j]));
  float dd = amax / 127.0f;
  d[i] = dd;
  uint32_t packed[BLK / 4];
#pragma unroll
  for (int c = 0; c < BLK / 4; c++) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; b++) {
      int qi = (dd == 0.0f) ? 0 : (int)roundf(v[4 * c + b] / dd);
      word |= ((uint32_t)qi & 0xffu) << (8 * b);
    }
    packed[c] = word;
  }
  uint4* dst = reinterpret_cast<uint4*>(q + i * BLK);
  dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
}

hipError_t launch_q4_pack(const float* w, int64_t rows, int64_t K, void* packed,
                          hipStream_t stream) {
  int64_t nblocks = rows * (K / BLK);
  if (nblocks == 0) return hipSuccess;
  int64_t grid = (nblocks + 255) / 256;
  hipLaunchKernelGGL(q4_pack_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, w, nblocks,
                     static_cast<uint16_t*>(packed));
  return hipGetLastError();
}

// Grouped-GEMM tile order (layout stated in moe_q4.h at q4_tile): one thread
// per block; thread i = (G * nsteps + s) * 64 + l moves block 2s + l/32 of
// row 32G + l%32.  Source blocks are 2-byte aligned, so the 16 nibble bytes
// are read as halfwords and written as one 16-byte store.
__global__ void __launch_bounds__(256) q4_tile_kernel(const uint16_t* __restrict__ q4, int64_t nblocks,
                                                      int nsteps, uint8_t* __restrict__ tiled) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nblocks) return;
  const int l = (int)(i & 63);
  const int64_t gs = i >> 6;                       // G * nsteps + s
  const int64_t G = gs / nsteps;
  const int st = (int)(gs - G * nsteps);
  const int64_t rbh = (int64_t)nsteps * 18;        // row bytes / 2 (halfwords per row)
  const int64_t row = 32 * G + (l & 31);
  const int blk = 2 * st + (l >> 5);
  const uint16_t* src = q4 + row * rbh + (int64_t)blk * 9;
  uint32_t w[4];
#pragma unroll
  for (int c = 0; c < 4; c++) w[c] = (uint32_t)src[1 + 2 * c] | ((uint32_t)src[2 + 2 * c] << 16);
  uint8_t* piece = tiled + gs * 1152;
  *reinterpret_cast<uint4*>(piece + 16 * l) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint16_t*>(piece + 1024 + 2 * l) = src[0];
}

hipError_t launch_q4_tile(const void* q4, int64_t rows, int64_t K, void* tiled, hipStream_t stream) {
  const int64_t nblocks = rows * (K / BLK);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(q4_tile_kernel, dim3((uint32_t)((nblocks + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q4), nblocks, (int)(K / 64), static_cast<uint8_t*>(tiled));
  return hipGetLastError();
}

// The same tile order for Q8_0 blocks (layout stated in moe_q4.h at
// q8w_tile): a step of 32 rows is one 2176-byte piece, lane l's 32 code
// bytes at 32 * l, its fp16 scale at 2048 + 2 * l.  Source blocks are 2-byte
// aligned: the codes are read as halfwords and written as two 16-byte stores.
__global__ void __launch_bounds__(256) q8w_tile_kernel(const uint16_t* __restrict__ q8, int64_t nblocks,
                                                       int nsteps, uint8_t* __restrict__ tiled) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nblocks) return;
  const int l = (int)(i & 63);
  const int64_t gs = i >> 6;                       // G * nsteps + s
  const int64_t G = gs / nsteps;
  const int st = (int)(gs - G * nsteps);
  const int64_t rbh = (int64_t)nsteps * 34;        // row bytes / 2 (halfwords per row)
  const int64_t row = 32 * G + (l & 31);
  const int blk = 2 * st + (l >> 5);
  const uint16_t* src = q8 + row * rbh + (int64_t)blk * 17;
  uint32_t w[8];
#pragma unroll
  for (int c = 0; c < 8; c++) w[c] = (uint32_t)src[1 + 2 * c] | ((uint32_t)src[2 + 2 * c] << 16);
  uint8_t* piece = tiled + gs * 2176;
  *reinterpret_cast<uint4*>(piece + 32 * l) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint4*>(piece + 32 * l + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  *reinterpret_cast<uint16_t*>(piece + 2048 + 2 * l) = src[0];
}

hipError_t launch_q8w_tile(const void* q8, int64_t rows, int64_t K, void* tiled, hipStream_t stream) {
  const int64_t nblocks = rows * (K / BLK);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(q8w_tile_kernel, dim3((uint32_t)((nblocks + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q8), nblocks, (int)(K / 64), static_cast<uint8_t*>(tiled));
  return hipGetLastError();
}

hipError_t launch_q8_quantize(const float* x, int64_t rows, int64_t K, int8_t* q, float* d,
                              hipStream_t stream) {
  int64_t nblocks = rows * (K / BLK);
  if (nblocks == 0) return hipSuccess;
  int64_t grid = (nblocks + 255) / 256;
  hipLaunchKernelGGL(q8_quantize_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, x, nblocks,
                     q, d);
  return hipGetLastError();
}

}  // namespace moeq4
