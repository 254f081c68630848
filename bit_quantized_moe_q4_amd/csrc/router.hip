// router.hip -- prefill routing: router logits, top-k + softmax weights,
// expert histogram, segment offsets and the token permutation.
//
// The pages route each prompt token to experts before the grouped 4-bit GEMM
// ("A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU",
// technical summary, Methodology 1) and give no routing arithmetic; the
// library's fp32 programs (moe_q4.h) are reproduced here bit for bit:
//   logit = pairwise tree over 32-wide chunks of a sequential FMA chain,
//   then + bias; top-k by (logit desc, index asc); weights by the fixed exp.
// The companion report ("A Modern Multimodal Assistant on a 6 GB 2011 GPU",
// abstract) is the reason every tie and summation order is pinned.
//
// Kernels (one stream, no host round trip):
//   router_partials  the per-chunk FMA chains as chained K=1 fp32 MFMAs (32
//                    tokens x 64 experts per wave), one aligned subtree of
//                    cw chunks per grid z
//   topk_hist        finishes the chunk tree, top-k (k rounds of a DPP
//                    wave maximum over 64-bit order keys), weights, and a
//                    wavefront-ballot histogram of the block's tokens with
//                    each assignment's stable rank inside the block
//   route_colscan    per expert (one block each): prefix of its counts over
//                    the token tiles, and its total
//   route_scatter    offsets from the totals (in every block), perm / inv_perm
#include "launch.hpp"
#include "device_math.hpp"

namespace moeq4 {

RouterSplit prefill_router_split(int H) {
  RouterSplit s;
  s.nc = H / BLK;
  s.m = 1;
  while (s.m < s.nc) s.m <<= 1;
  s.cw = s.m < 8 ? s.m : 8;
  s.nsplit = s.m / s.cw;
  return s;
}

// ---------------------------------------------------------------- partials
template <int CW>
struct Log2 { static constexpr int v = 1 + Log2<CW / 2>::v; };
template <>
struct Log2<1> { static constexpr int v = 0; };

// Leaves on v_mfma_f32_32x32x1f32: one instruction is an outer
// product of 32 values by 32 values for each of two blocks, and each output
// gets exactly one fmaf per instruction (checked bit for bit against fmaf
// chains on gfx950), so 32 instructions over k = 0..31 are the chunk's
// sequential FMA chain, at twice the fp32 VALU rate.  A wave covers 32 tokens
// x 64 experts: lane l supplies token t0 + l%32 (both lane halves) and
// expert e0 + l; block b's output (row i, column j) sits in register
// 16b + 4*(i/8) + i%4 of lane 32*((i/4)%2) + j.
//
// Block = 4 waves = 2 token tiles x 2 halves of the grid z's aligned subtree
// of CW chunks: half h computes the subtree of chunks h*CW/2 .. (h+1)*CW/2-1
// and the two halves meet in LDS as (left + right), the subtree's own top
// node.  The two waves of a half read the same router rows: the block stages
// each chunk's 32 rows x 64 experts per half in LDS with direct
// global->LDS loads (one 256-byte row per wave instruction), double
// buffered, so a lane reads its weight per k with one conflict-free LDS
// read.  A lane's token values come from global memory one chunk ahead.
// Splitting the subtree over two waves keeps a wave's pending subtrees to
// log2(CW/2) + 1 accumulators, so three waves fit on a SIMD.
constexpr int RPW = 4;                    // waves per block
constexpr int RPT = 2;                    // token tiles of 32 per block

__device__ __forceinline__ void wait_vm_router() {
  // s_waitcnt vmcnt(0), expcnt/lgkmcnt untouched (gfx9 encoding)
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

template <int CW>
struct RouterSmem {
  static constexpr int NH = CW >= 2 ? 2 : 1;   // halves
  float w[2][NH][BLK * 64];                     // [buffer][half][k][expert]
};

template <bool BF16, int CW>
__global__ void __launch_bounds__(64 * RPW) router_partials_mfma_kernel(const void* __restrict__ xv, int T,
                                                                         int H, const float* __restrict__ Wr,
                                                                         int E, int nc, int nsplit,
                                                                         float* __restrict__ partials) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef float f32x32_t __attribute__((ext_vector_type(32)));
  constexpr int NH = RouterSmem<CW>::NH;
  constexpr int HC = CW / NH;                   // chunks per half
  constexpr int L = Log2<HC>::v;
  __shared__ RouterSmem<CW> sm;
  // Block b -> (expert tile ex, group g = token group * nsplit + split): the
  // expert tiles of one group are 8 blocks apart, so they land on the same
  // XCD (blocks are dealt to the 8 XCDs round robin) close in time, and the
  // group's token rows are fetched into that XCD's L2 once.
  const int nx = (E + 63) / 64;
  const int q = blockIdx.x / 8;
  const int ex = q % nx, g = 8 * (q / nx) + blockIdx.x % 8;
  const int ty = g / nsplit, split = g % nsplit;
  if (ty * RPT * 32 >= T) return;               // padding of the last 8 groups (uniform per block)
  const int lane = threadIdx.x % 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int tt = wave % RPT, h = wave / RPT;
  const int t0 = (ty * RPT + tt) * 32, e0 = ex * 64;
  const int t = t0 + lane % 32, e = e0 + lane;
  const int tc = t < T ? t : T - 1, ec = e < E ? e : E - 1;   // clamped: loads stay in bounds
  const int cbase = split * CW + h * HC;        // this wave's first chunk (uniform)
  const bool active = h < NH;                   // NH == 1: waves of half 1 only stage rows

  // router rows: wave w stages rows k = tt + RPT*j of its half's chunk
  // (readfirstlane returns int: each half goes through uint32_t, so the low
  // word is not sign-extended into the high one)
  const uint64_t wp = reinterpret_cast<uint64_t>(Wr);
  const uint32_t wlo = __builtin_amdgcn_readfirstlane((uint32_t)wp);
  const uint32_t whi = __builtin_amdgcn_readfirstlane((uint32_t)(wp >> 32));
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uint64_t)whi << 32) | wlo), 0,
      (int)__builtin_amdgcn_readfirstlane((uint32_t)((size_t)H * E * 4)), 0x00020000);
  const uint32_t vw = 4u * (uint32_t)ec;
  const int hs = h < NH ? h : 0;                // half whose rows this wave stages
  constexpr int SW = NH == 2 ? RPT : RPW;       // waves staging one half's rows
  const int sbase = split * CW + hs * HC;
  auto stage_w = [&](int i, int buf) {
    const int c = sbase + i;
    if (c >= nc) return;                        // uniform
#pragma unroll
    for (int j = 0; j < BLK / SW; j++) {
      const int k = (NH == 2 ? tt : wave) + SW * j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (__attribute__((address_space(3))) void*)(&sm.w[buf][hs][k * 64]), 4, vw,
          (uint32_t)((c * BLK + k) * E) * 4u, 0, 0);
    }
  };
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  constexpr int XR = BF16 ? BLK / 2 : BLK;      // registers of one chunk of the lane's token
  uint32_t xr[2][XR];
  auto load_x = [&](int i, int slot) {
    const int c = cbase + i;
    if (!active || c >= nc) return;
    if (BF16) {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(xv) + (size_t)tc * H + c * BLK);
#pragma unroll
      for (int q = 0; q < XR / 4; q++) {
        const u32x4_t v = src[q];
        xr[slot][4 * q] = v.x; xr[slot][4 * q + 1] = v.y; xr[slot][4 * q + 2] = v.z; xr[slot][4 * q + 3] = v.w;
      }
    } else {
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(static_cast<const float*>(xv) + (size_t)tc * H + c * BLK);
#pragma unroll
      for (int q = 0; q < XR / 4; q++) {
        const u32x4_t v = src[q];
        xr[slot][4 * q] = v.x; xr[slot][4 * q + 1] = v.y; xr[slot][4 * q + 2] = v.z; xr[slot][4 * q + 3] = v.w;
      }
    }
  };
  auto xval = [&](int slot, int k) -> float {
    if (BF16) {
      const uint32_t p = xr[slot][k / 2];
      return __uint_as_float((k & 1) ? (p & 0xffff0000u) : (p << 16));
    }
    return __uint_as_float(xr[slot][k]);
  };

  f32x32_t st[L + 1];
  stage_w(0, 0);
  load_x(0, 0);
#pragma unroll
  for (int i = 0; i < HC; i++) {
    wait_vm_router();                           // own rows and token values of chunk i landed
    __syncthreads();                            // every wave's rows of chunk i landed; chunk i-1 done
    if (i + 1 < HC) {
      stage_w(i + 1, (i + 1) & 1);
      load_x(i + 1, (i + 1) & 1);
    }
    f32x32_t acc = {};
    const int c = cbase + i;
    if (active && c < nc) {                     // padded leaves stay +0.0
      const float* wl = &sm.w[i & 1][h][lane];
#pragma unroll
      for (int k = 0; k < BLK; k++) acc = __builtin_amdgcn_mfma_f32_32x32x1f32(xval(i & 1, k), wl[k * 64], acc, 0, 0, 0);
    }
    // binary-counter merge: leaf i joins the pending subtrees of equal size
    int lvl = 0;
#pragma unroll
    for (int b = 0; b < L; b++) {
      if (((i >> b) & 1) == 0) break;
      lvl = b + 1;
    }
#pragma unroll
    for (int b = 0; b < L; b++)
      if (b < lvl) acc = st[b] + acc;
#pragma unroll
    for (int b = 0; b <= L; b++)
      if (b == lvl) st[b] = acc;
  }
  f32x32_t res = st[L];
  if (NH == 2) {
    // the right half's subtree meets the left one's: (left + right)
    float* ex = &sm.w[0][0][0];                 // RPT waves x 32 registers x 64 lanes
    __syncthreads();                            // every wave is done with the staged rows
    if (h == 1) {
#pragma unroll
      for (int r = 0; r < 32; r++) ex[(tt * 32 + r) * 64 + lane] = res[r];
    }
    __syncthreads();
    if (h == 1) return;
#pragma unroll
    for (int r = 0; r < 32; r++) res[r] = res[r] + ex[(tt * 32 + r) * 64 + lane];
  } else if (h != 0) {
    return;
  }
  float* out = partials + (size_t)split * T * E;
#pragma unroll
  for (int r = 0; r < 32; r++) {
    const int blk = r / 16, i = 8 * ((r % 16) / 4) + 4 * (lane / 32) + (r % 4), j = lane % 32;
    const int to = t0 + i, eo = e0 + 32 * blk + j;
    if (to < T && eo < E) out[(size_t)to * E + eo] = res[r];
  }
#endif
}

hipError_t launch_router_partials(const void* x, int x_bf16, int T, int H, const float* w_router,
                                  int E, const RouterSplit& sp, float* partials,
                                  hipStream_t stream) {
  const int groups = (T + 32 * RPT - 1) / (32 * RPT) * sp.nsplit;
  dim3 grid((uint32_t)(8 * ((groups + 7) / 8) * ((E + 63) / 64)));
#define MOEQ4_RP(BF, CWV)                                                                         \
  hipLaunchKernelGGL((router_partials_mfma_kernel<BF, CWV>), grid, dim3(64 * RPW), 0, stream, x, T, H, \
                     w_router, E, sp.nc, sp.nsplit, partials)
#define MOEQ4_RP_CW(BF)                      \
  switch (sp.cw) {                           \
    case 1: MOEQ4_RP(BF, 1); break;          \
    case 2: MOEQ4_RP(BF, 2); break;          \
    case 4: MOEQ4_RP(BF, 4); break;          \
    default: MOEQ4_RP(BF, 8); break;         \
  }
  if (x_bf16) {
    MOEQ4_RP_CW(true)
  } else {
    MOEQ4_RP_CW(false)
  }
#undef MOEQ4_RP_CW
#undef MOEQ4_RP
  return hipGetLastError();
}

// ---------------------------------------------------------------- top-k
constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;

// Logit of (row idx, expert e): pairwise tree over the NS (a power of two)
// aligned subtree partials at idx + s*stride, loads all issued together.
template <int NS>
__device__ __forceinline__ float finish_logit(const float* __restrict__ partials, size_t stride,
                                              size_t idx, const float* bias, int e) {
  float v[NS];
#pragma unroll
  for (int s = 0; s < NS; s++) v[s] = partials[(size_t)s * stride + idx];
#pragma unroll
  for (int w = NS; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; i++) v[i] = v[2 * i] + v[2 * i + 1];
  float l = v[0];
  if (bias) l = l + bias[e];
  return l;
}

// Order key: larger key = earlier in (logit desc, index asc); -0 and +0 tie
// as under a float comparison.  Unique per expert.
__device__ __forceinline__ uint64_t topk_key(float l, int e) {
  uint32_t u = __float_as_uint(l == 0.0f ? 0.0f : l);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
}

// Top-k of one token's logits held as lane + 64*j (all 64 lanes active).
// Round s takes the largest remaining key: the same pick as "first maximum
// among the rest".  Returns, in lane s < k, the s-th pick (my_v, my_e) and
// its weight my_w.
template <int NJ>
__device__ __forceinline__ void wave_topk(const float (&lv)[NJ], int E, int k, float& my_v,
                                          int& my_e, float& my_w) {
  const int lane = threadIdx.x % 64;
  uint64_t key[NJ];
#pragma unroll
  for (int j = 0; j < NJ; j++) {
    const int e = lane + 64 * j;
    key[j] = (e < E) ? topk_key(lv[j], e) : 0ull;
  }
  my_v = 0.0f;
  my_e = -1;
  float l0 = 0.0f;
  for (int s = 0; s < k; s++) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < NJ; j++) best = key[j] > best ? key[j] : best;
    const uint64_t win = wave_max_u64(best);
    const int we = (int)(0xffffffffu - (uint32_t)win);
    const int wj = we >> 6, wl = we & 63;
    float sel = lv[0];
#pragma unroll
    for (int j = 1; j < NJ; j++) sel = (j == wj) ? lv[j] : sel;   // wj is uniform
    const float wv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel), wl));
#pragma unroll
    for (int j = 0; j < NJ; j++)
      if (j == wj && lane == wl) key[j] = 0ull;
    if (s == 0) l0 = wv;
    if (lane == s) { my_v = wv; my_e = we; }
  }
  // weights: e_s = exp(l_s - l_0), S = e_0 + e_1 + ... left to right
  const float ex = (lane < k) ? exp_p(my_v - l0) : 0.0f;
  float S = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), 0));
  for (int s = 1; s < k; s++) S = S + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), s));
  my_w = ex / S;
}

// Block = kTopkTokensPerBlock waves, one token per wave; then the block's
// expert histogram by ballots over its tokens (lane = token) and each
// assignment's stable rank inside the block.
template <int NJ, int NS>
__global__ void __launch_bounds__(1024) topk_hist_kernel(
    const float* __restrict__ partials, const float* __restrict__ bias, int T, int E, int k,
    float* __restrict__ logits_out, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ counts_w, int32_t* __restrict__ rank) {
  constexpr int TPB = kTopkTokensPerBlock;
  __shared__ int32_t ids_l[TPB][kMaxK];
  __shared__ uint32_t mask_l[TPB][kMaxE / 32 + 1];
  __shared__ unsigned long long bal_l[kMaxE];
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int t0 = blockIdx.x * TPB;
  const size_t stride = (size_t)T * E;
  {
    const int t = t0 + wave;
    if (t < T) {                          // uniform per wave
      float lv[NJ];
#pragma unroll
      for (int j = 0; j < NJ; j++) {
        const int e = lane + 64 * j;
        lv[j] = 0.0f;
        if (e < E) lv[j] = finish_logit<NS>(partials, stride, (size_t)t * E + e, bias, e);
      }
      if (logits_out) {
#pragma unroll
        for (int j = 0; j < NJ; j++) {
          const int e = lane + 64 * j;
          if (e < E) logits_out[(size_t)t * E + e] = lv[j];
        }
      }
      float my_v, my_w;
      int my_e;
      wave_topk<NJ>(lv, E, k, my_v, my_e, my_w);
      if (lane < k) {
        ids[(size_t)t * k + lane] = my_e;
        w[(size_t)t * k + lane] = my_w;
        ids_l[wave][lane] = my_e;
      }
    }
  }
  const int nwords = (E + 31) / 32;
  for (int i = threadIdx.x; i < TPB * (kMaxE / 32 + 1); i += blockDim.x)
    (&mask_l[0][0])[i] = 0u;
  __syncthreads();
  if (threadIdx.x < TPB && t0 + (int)threadIdx.x < T) {
    for (int s = 0; s < k; s++) {
      const int e = ids_l[threadIdx.x][s];
      mask_l[threadIdx.x][e >> 5] |= 1u << (e & 31);
    }
  }
  __syncthreads();
  // one ballot per expert over the block's tokens (lane = token, lanes >= TPB read 0)
  for (int wd = wave; wd < nwords; wd += blockDim.x / 64) {
    const uint32_t word = (lane < TPB) ? mask_l[lane][wd] : 0u;
    for (int b = 0; b < 32; b++) {
      const int e = wd * 32 + b;
      if (e >= E) break;
      const unsigned long long bal = __ballot((word >> b) & 1u);
      if (lane == 0) {
        bal_l[e] = bal;
        counts_w[(size_t)blockIdx.x * E + e] = (int32_t)__popcll(bal);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < TPB && t0 + (int)threadIdx.x < T) {
    const int tl = threadIdx.x;
    const unsigned long long below = (tl == 0) ? 0ull : (~0ull >> (64 - tl));
    for (int s = 0; s < k; s++) {
      const int e = ids_l[tl][s];
      rank[(size_t)(t0 + tl) * k + s] = (int32_t)__popcll(bal_l[e] & below);
    }
  }
}

hipError_t launch_topk_hist(const float* partials, const RouterSplit& sp, const float* bias,
                            int T, int E, int k, float* logits_out, int32_t* ids, float* w,
                            int32_t* counts_w, int32_t* rank, hipStream_t stream) {
  dim3 grid((T + kTopkTokensPerBlock - 1) / kTopkTokensPerBlock);
  dim3 block(64 * kTopkTokensPerBlock);
  const int nj = (E + 63) / 64;
#define MOEQ4_TK(NJV, NSV)                                                                    \
  hipLaunchKernelGGL((topk_hist_kernel<NJV, NSV>), grid, block, 0, stream, partials, bias, T, E, \
                     k, logits_out, ids, w, counts_w, rank)
#define MOEQ4_TK_NS(NJV)                          \
  switch (sp.nsplit) {                            \
    case 1: MOEQ4_TK(NJV, 1); break;              \
    case 2: MOEQ4_TK(NJV, 2); break;              \
    case 4: MOEQ4_TK(NJV, 4); break;              \
    case 8: MOEQ4_TK(NJV, 8); break;              \
    case 16: MOEQ4_TK(NJV, 16); break;            \
    case 32: MOEQ4_TK(NJV, 32); break;            \
    default: MOEQ4_TK(NJV, 64); break;            \
  }
  if (nj <= 1) { MOEQ4_TK_NS(1) }
  else if (nj <= 2) { MOEQ4_TK_NS(2) }
  else if (nj <= 4) { MOEQ4_TK_NS(4) }
  else if (nj <= 8) { MOEQ4_TK_NS(8) }
  else { MOEQ4_TK_NS(16) }
#undef MOEQ4_TK_NS
#undef MOEQ4_TK
  return hipGetLastError();
}

// ---------------------------------------------------------------- scan
// Block e: the exclusive prefix of expert e's counts over the nt token tiles,
// counts_w [nt][E] in place (tile b's first assignment to e is then
// offsets[e] + counts_w[b][e] in perm), and the expert's total in tot[e].
// One block per expert: the count matrix (512 KB at 8192 tokens and 256
// experts) is read and rewritten by E blocks, not by one.  Thread i takes
// tiles i*per .. (i+1)*per - 1, loads issued CH at a time.
__global__ void __launch_bounds__(1024) route_colscan_kernel(int32_t* __restrict__ counts_w, int nt, int E,
                                                             int32_t* __restrict__ tot) {
  constexpr int CH = 16;
  __shared__ int32_t wsum[16];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int per = (nt + blockDim.x - 1) / blockDim.x;
  const int b0 = tid * per, b1 = min(nt, b0 + per);
  int run = 0;
  for (int b = b0; b < b1; b += CH) {
    int c[CH];
#pragma unroll
    for (int i = 0; i < CH; i++) c[i] = (b + i < b1) ? counts_w[(size_t)(b + i) * E + e] : 0;
#pragma unroll
    for (int i = 0; i < CH; i++) run += c[i];
  }
  // exclusive prefix of the thread sums: inside each wave, then over waves
  int incl = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = incl - run;
  const int nw = blockDim.x / 64;
  int total = 0;
  for (int w = 0; w < nw; w++) {
    const int v = wsum[w];
    if (w < wave) before += v;
    total += v;
  }
  if (tid == 0) tot[e] = total;
  int acc = before;
  for (int b = b0; b < b1; b += CH) {
    int c[CH];
#pragma unroll
    for (int i = 0; i < CH; i++) c[i] = (b + i < b1) ? counts_w[(size_t)(b + i) * E + e] : 0;
#pragma unroll
    for (int i = 0; i < CH; i++)
      if (b + i < b1) {
        counts_w[(size_t)(b + i) * E + e] = acc;
        acc += c[i];
      }
  }
}

hipError_t launch_route_colscan(int32_t* counts_w, int n_tiles, int E, int32_t* tot, hipStream_t stream) {
  hipLaunchKernelGGL(route_colscan_kernel, dim3(E), dim3(1024), 0, stream, counts_w, n_tiles, E, tot);
  return hipGetLastError();
}

// ---------------------------------------------------------------- scatter
// Every block first turns the E expert totals into segment offsets in LDS
// (exclusive scan; block 0 also writes offsets [E+1]), then places its
// assignments: perm[pos] = f, inv_perm[f] = pos with pos = offsets[e] +
// (tile prefix of e) + (rank of f among the tile's assignments to e).
// tot == nullptr: no assignments (T == 0), every offset 0.
__global__ void __launch_bounds__(256) route_scatter_kernel(const int32_t* __restrict__ ids,
                                                            const int32_t* __restrict__ rank,
                                                            const int32_t* __restrict__ base_w,
                                                            const int32_t* __restrict__ tot, int T, int k, int E,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ inv_perm) {
  __shared__ int32_t off_l[kMaxE];
  __shared__ int32_t wsum[4];
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  // exclusive scan of tot: thread t takes experts 4t .. 4t+3
  int v[4], run = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int e = 4 * tid + i;
    v[i] = (tot && e < E) ? tot[e] : 0;
    run += v[i];
  }
  int incl = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int acc = incl - run;
  for (int w = 0; w < wave; w++) acc += wsum[w];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int e = 4 * tid + i;
    if (e < E) {
      off_l[e] = acc;
      if (blockIdx.x == 0) offsets[e] = acc;
    }
    acc += v[i];
  }
  if (blockIdx.x == 0 && tid == 0) offsets[E] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  const int64_t f = (int64_t)blockIdx.x * blockDim.x + tid;
  if (f >= (int64_t)T * k) return;
  const int t = (int)(f / k);
  const int e = ids[f];
  if (e < 0 || e >= E) return;            // unreachable for the ids the top-k writes
  const int pos = off_l[e] + base_w[(size_t)(t / kTopkTokensPerBlock) * E + e] + rank[f];
  if (pos < 0 || (int64_t)pos >= (int64_t)T * k) return;   // unreachable for valid ranks
  perm[pos] = (int32_t)f;
  inv_perm[f] = pos;
}

hipError_t launch_route_scatter(const int32_t* ids, const int32_t* rank, const int32_t* base_w,
                                const int32_t* tot, int T, int k, int E, int32_t* offsets, int32_t* perm,
                                int32_t* inv_perm, hipStream_t stream) {
  const int64_t n = (int64_t)T * k;
  const uint32_t blocks = n > 0 ? (uint32_t)((n + 255) / 256) : 1u;
  hipLaunchKernelGGL(route_scatter_kernel, dim3(blocks), dim3(256), 0, stream, ids, rank, base_w, tot, T, k, E,
                     offsets, perm, inv_perm);
  return hipGetLastError();
}

}  // namespace moeq4
