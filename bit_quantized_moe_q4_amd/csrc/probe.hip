// probe.hip -- matrix-core rate probes: what the MI355X sustains for the three
// MFMA shapes the kernels of this library issue, so a kernel's rate can be
// read against a measured ceiling next to the published one.
//
// The companion report ("A Modern Multimodal Assistant on a 6 GB 2011 GPU",
// abstract) argues for performance work built on measured foundations: it
// found its best hand-written GEMM had been wrongly taken for the ceiling.
//
// Each wave runs kChains independent accumulator chains of `iters` MFMAs of
// one shape on lane-dependent operands (no memory traffic inside the loop),
// then stores one checksum per lane so the work cannot be dropped.  A block
// is 4 waves; the caller picks the grid (2 blocks per CU = 2 waves per SIMD,
// the occupancy of the grouped GEMM).  Shapes:
//   kind 0  v_mfma_f32_32x32x16_bf16   the bf16 grouped GEMM's
//   kind 1  v_mfma_i32_32x32x32_i8     the W4A8 prefill's
//   kind 2  v_mfma_f32_32x32x1_2b_f32  the router leaves' (K = 1 chains)
#include "launch.hpp"

namespace moeq4 {

constexpr int kProbeChains = 8;

typedef __bf16 pr_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pr_f32x16 __attribute__((ext_vector_type(16)));
typedef float pr_f32x32 __attribute__((ext_vector_type(32)));
typedef int pr_i32x4 __attribute__((ext_vector_type(4)));
typedef int pr_i32x16 __attribute__((ext_vector_type(16)));

template <int KIND>
__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x % 64;
  float s = 0.0f;
  if constexpr (KIND == 0) {
    pr_bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      a[i] = (__bf16)(0.001f * (float)(lane + i));
      b[i] = (__bf16)(0.002f * (float)(lane - i));
    }
    pr_f32x16 acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; c++) acc[c] = pr_f32x16{};
    for (int it = 0; it < iters; it++)
#pragma unroll
      for (int c = 0; c < kProbeChains; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < kProbeChains; c++)
#pragma unroll
      for (int r = 0; r < 16; r++) s += acc[c][r];
  } else if constexpr (KIND == 1) {
    const pr_i32x4 a = {lane, lane + 1, lane + 2, lane + 3}, b = {3 - lane, 5, -lane, 7};
    pr_i32x16 acc[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; c++) acc[c] = pr_i32x16{};
    for (int it = 0; it < iters; it++)
#pragma unroll
      for (int c = 0; c < kProbeChains; c++) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < kProbeChains; c++)
#pragma unroll
      for (int r = 0; r < 16; r++) s += (float)acc[c][r];
  } else {
    const float a = 1.0f + 1e-7f * (float)lane, b = 0.5f - 1e-7f * (float)lane;
    // (32 outputs per lane: half the chains keep the register count that of the others)
    pr_f32x32 acc[kProbeChains / 2];
#pragma unroll
    for (int c = 0; c < kProbeChains / 2; c++) acc[c] = pr_f32x32{};
    for (int it = 0; it < iters; it++)
#pragma unroll
      for (int c = 0; c < kProbeChains / 2; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x1f32(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < kProbeChains / 2; c++)
#pragma unroll
      for (int r = 0; r < 32; r++) s += acc[c][r];
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

int64_t probe_mfma_count(int kind, int blocks, int iters) {
  const int chains = kind == 2 ? kProbeChains / 2 : kProbeChains;
  return (int64_t)blocks * 4 * chains * iters;
}

hipError_t launch_probe_mfma(int kind, int blocks, int iters, float* out, hipStream_t stream) {
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(blocks), dim3(256), 0, stream, iters, out); break;
    case 1: hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(blocks), dim3(256), 0, stream, iters, out); break;
    default: hipLaunchKernelGGL(mfma_probe_kernel<2>, dim3(blocks), dim3(256), 0, stream, iters, out); break;
  }
  return hipGetLastError();
}

}  // namespace moeq4
