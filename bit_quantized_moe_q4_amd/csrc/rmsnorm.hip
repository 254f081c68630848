// rmsnorm.hip -- unit-gain RMSNorm between stacked MoE layers:
//   out = y / sqrt(mean(y^2) + eps)
// evaluated as the library's fp32 program (moe_q4.h): per 32-chunk a
// sequential fused chain y*y from +0, chunk partials summed pairwise level by
// level (padded with +0 to a power of two), r = sqrtf(ss / H + eps) and
// out = y / r, both correctly rounded.  One block per row.
#include "launch.hpp"
#include "device_math.hpp"

namespace moeq4 {

__global__ void __launch_bounds__(256) rmsnorm_kernel(const float* __restrict__ y, int H, float eps,
                                                      float* __restrict__ out_f32,
                                                      uint16_t* __restrict__ out_bf16) {
  __shared__ float part[512];
  const int nc = H / BLK;
  const int m = (int)next_pow2_u32((uint32_t)nc);
  const float* row = y + (size_t)blockIdx.x * H;
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
  // m <= 512, so one level never has more than blockDim (256) sums
  for (int w = m; w > 1; w >>= 1) {
    const bool act = (int)threadIdx.x < w / 2;
    float s = 0.0f;
    if (act) s = part[2 * threadIdx.x] + part[2 * threadIdx.x + 1];
    __syncthreads();
    if (act) part[threadIdx.x] = s;
    __syncthreads();
  }
  const float r = sqrtf(part[0] / (float)H + eps);
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    const float o = row[h] / r;
    if (out_f32) out_f32[(size_t)blockIdx.x * H + h] = o;
    if (out_bf16) out_bf16[(size_t)blockIdx.x * H + h] = f32_to_bf16_bits(o);
  }
}

hipError_t launch_rmsnorm(const float* y, int T, int H, float eps, float* out_f32,
                          uint16_t* out_bf16, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, stream, y, H, eps, out_f32, out_bf16);
  return hipGetLastError();
}

}  // namespace moeq4
