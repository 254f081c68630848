// rmsnorm.hip -- unit-gain RMSNorm between stacked MoE layers:
//   out = y / sqrt(mean(y^2) + eps)
// evaluated as the library's fp32 program (moe_q4.h): per 32-chunk a
// sequential fused chain y*y from +0, chunk partials summed pairwise level by
// level (padded with +0 to a power of two), r = sqrtf(ss / H + eps) and
// out = y / r, both correctly rounded.  One block per row.
#include "launch.hpp"
#include "device_math.hpp"
#include "decode_common.hpp"

namespace moeq4 {

__global__ void __launch_bounds__(256) rmsnorm_kernel(const float* __restrict__ y, int H, float eps,
                                                      float* __restrict__ out_f32,
                                                      uint16_t* __restrict__ out_bf16) {
  __shared__ float part[512], tmp[512];
  const float* row = y + (size_t)blockIdx.x * H;
  const float r = rms_scale(row, H, eps, part, tmp);
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
