// decode.hip -- single-token decode step of the Q4_0 MoE layer (W4A8).
//
// "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU",
// technical summary, Methodology 1 (decode of single tokens by a W4A8 integer
// kernel over 4-bit weights read straight from memory) and Key Contribution 2.
// On the pages the weights are read from host RAM by the CPU; here every
// expert stays resident in HBM and the step is bound by streaming the k+S
// selected experts' 18-byte blocks.
//
// Three launches on the caller's stream:
//   decode_router   router GEMV split over aligned chunk subtrees; block 0
//                   also quantises x; the last block to finish (atomic
//                   ticket) completes the chunk tree, picks the top-k and
//                   computes the weights, then re-arms the ticket
//   decode_gateup   one block per (slot, 32 rows of I): gate and up rows by
//                   the W4A8 row program, h = silu(g) * u, q8(h) of the block
//   decode_down     one block per few output rows, all slots: down rows by
//                   the row program, then the fixed-order weighted combine
#include "launch.hpp"
#include "w4a8.hpp"

namespace moeq4 {

RouterSplit decode_router_split(int H, int E) {
  RouterSplit s;
  s.nc = H / BLK;
  s.m = 1;
  while (s.m < s.nc) s.m <<= 1;
  int cw = 256 / E;
  if (cw < 1) cw = 1;
  int c = 1;
  while (c * 2 <= cw) c *= 2;            // power of two <= 256/E
  if (c > s.m) c = s.m;
  while (s.m / c > 64) c *= 2;           // at most 64 subtrees
  s.cw = c;
  s.nsplit = s.m / c;
  return s;
}

// Wave-wide (value desc, index asc) argmax.
__device__ __forceinline__ void dec_wave_argmax(float& v, int& e) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const float ov = __shfl_xor(v, m, 64);
    const int oe = __shfl_xor(e, m, 64);
    if (ov > v || (ov == v && oe < e)) { v = ov; e = oe; }
  }
}

// ---------------------------------------------------------------- router
template <int NS>
__global__ void __launch_bounds__(256) decode_router_kernel(DecodeArgs a, int nc, int cw) {
  constexpr int nsplit = NS;
  __shared__ float xs[256 * BLK];         // cw * 32 inputs (cw <= 256)
  __shared__ float part[1024];            // [cl][e] chain results (cw * E <= 1024)
  __shared__ float logit_l[1024];
  __shared__ int s_last;
  const int tid = threadIdx.x, split = blockIdx.x;
  const int E = a.E, H = a.H;
  const int c0 = split * cw;

  for (int i = tid; i < cw * BLK; i += blockDim.x) {
    const int h = c0 * BLK + i;
    xs[i] = (h < H) ? a.x[h] : 0.0f;
  }
  __syncthreads();
  // chunk chains: pair p = (cl, e)
  for (int p = tid; p < cw * E; p += blockDim.x) {
    const int cl = p / E, e = p % E;
    const int c = c0 + cl;
    float acc = 0.0f;
    if (c < nc) {
      const float* w = a.w_router + (size_t)c * BLK * E + e;
#pragma unroll 8
      for (int i = 0; i < BLK; i++) acc = __builtin_fmaf(xs[cl * BLK + i], w[(size_t)i * E], acc);
    }
    part[cl * E + e] = acc;
  }
  __syncthreads();
  // subtree of cw leaves per expert, level by level
  for (int e = tid; e < E; e += blockDim.x) {
    for (int w = cw; w > 1; w >>= 1)
      for (int i = 0; i < w / 2; i++) part[i * E + e] = part[2 * i * E + e] + part[(2 * i + 1) * E + e];
    a.partials[(size_t)split * E + e] = part[e];
  }
  // block 0 also quantises x: one thread per 32-block
  if (split == 0) {
    for (int b = tid; b < H / BLK; b += blockDim.x) {
      const float* src = a.x + b * BLK;
      float v[BLK];
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < BLK; j++) { v[j] = src[j]; amax = fmaxf(amax, fabsf(v[j])); }
      const float d = amax / 127.0f;
      int32_t sum = 0;
      uint32_t words[8];
#pragma unroll
      for (int c = 0; c < 8; c++) {
        uint32_t wd = 0;
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int qi = (d == 0.0f) ? 0 : (int)roundf(v[4 * c + q] / d);
          sum += qi;
          wd |= ((uint32_t)qi & 0xffu) << (8 * q);
        }
        words[c] = wd;
      }
      uint4* dst = reinterpret_cast<uint4*>(a.qx + b * BLK);
      dst[0] = make_uint4(words[0], words[1], words[2], words[3]);
      dst[1] = make_uint4(words[4], words[5], words[6], words[7]);
      a.dx[b] = d;
      a.sx[b] = sum;
      if (a.t_qx) {
        uint4* tq = reinterpret_cast<uint4*>(a.t_qx + b * BLK);
        tq[0] = dst[0];
        tq[1] = dst[1];
      }
      if (a.t_dx) a.t_dx[b] = d;
    }
  }
  // last block to finish completes the tree and routes
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (uint32_t)(nsplit - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  // each thread finishes experts e = tid, tid+256, ...: NS loads in flight
  for (int e = tid; e < E; e += blockDim.x) {
    float v[NS];
#pragma unroll
    for (int s = 0; s < NS; s++) v[s] = __builtin_nontemporal_load(a.partials + (size_t)s * E + e);
#pragma unroll
    for (int w = NS; w > 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w / 2; i++) v[i] = v[2 * i] + v[2 * i + 1];
    float l = v[0];
    if (a.bias) l = l + a.bias[e];
    logit_l[e] = l;
    if (a.t_logits) a.t_logits[e] = l;
  }
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    constexpr int NJ = 16;                // E <= 1024
    float lv[NJ];
    const int nj = (E + 63) / 64;
#pragma unroll
    for (int j = 0; j < NJ; j++) {
      const int e = lane + 64 * j;
      lv[j] = (j < nj && e < E) ? logit_l[e] : -__builtin_inff();
    }
    uint32_t taken = 0;
    float my_v = 0.0f;
    int my_e = -1;
    for (int s = 0; s < a.k; s++) {
      float bv = -__builtin_inff();
      int be = 0x7fffffff;
      for (int j = 0; j < nj; j++) {
        const int e = lane + 64 * j;
        if (e < E && !((taken >> j) & 1u) && (be == 0x7fffffff || lv[j] > bv)) { bv = lv[j]; be = e; }
      }
      dec_wave_argmax(bv, be);
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      if (lane == s) { my_v = bv; my_e = be; }
    }
    const float l0 = __shfl(my_v, 0, 64);
    const float ex = (lane < a.k) ? exp_p(my_v - l0) : 0.0f;
    float S = __shfl(ex, 0, 64);
    for (int s = 1; s < a.k; s++) S = S + __shfl(ex, s, 64);
    const float wv = ex / S;
    if (lane < a.k) {
      a.ids[lane] = my_e;
      a.w[lane] = wv;
      if (a.t_ids) a.t_ids[lane] = my_e;
      if (a.t_w) a.t_w[lane] = wv;
    }
    if (lane == 0)
      __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------- gate/up
// Block: 64 rows (32 gate rows + the 32 matching up rows) x LPR lanes each.
template <int BPL, bool FAST>
__global__ void __launch_bounds__(1024) decode_gateup_kernel(DecodeArgs a, int lpr) {
  extern __shared__ uint8_t dyn[];
  const int H = a.H, I = a.I, nbh = H / BLK;
  uint32_t* qx_l = reinterpret_cast<uint32_t*>(dyn);            // H bytes
  float* dx_l = reinterpret_cast<float*>(dyn + H);              // nbh
  int32_t* sx_l = reinterpret_cast<int32_t*>(dyn + H + 4 * nbh);
  __shared__ float val[64];
  const int tid = threadIdx.x;
  const int slot = blockIdx.y, i0 = blockIdx.x * BLK;

  for (int i = tid; i < H / 4; i += blockDim.x) qx_l[i] = reinterpret_cast<const uint32_t*>(a.qx)[i];
  for (int i = tid; i < nbh; i += blockDim.x) { dx_l[i] = a.dx[i]; sx_l[i] = a.sx[i]; }
  __syncthreads();

  const int row = tid / lpr, lr = tid % lpr;
  const bool is_up = row >= 32;
  const int i = i0 + (row & 31);
  const size_t rb = (size_t)nbh * Q4B;
  const uint8_t* base;
  if (slot < a.k) {
    const int e = min(max(a.ids[slot], 0), a.E - 1);
    base = (is_up ? a.w_up : a.w_gate) + ((size_t)e * I + i) * rb;
  } else {
    base = (is_up ? a.s_up : a.s_gate) + (size_t)i * rb;
  }
  auto act = [&](int b) {
    ActBlock A;
#pragma unroll
    for (int q = 0; q < 8; q++) A.a[q] = qx_l[b * 8 + q];
    A.d = dx_l[b];
    A.s = sx_l[b];
    return A;
  };
  float v = w4a8_lane<BPL, FAST>(base, nbh, lr * BPL, act, nullptr);
  v = wave_tree_sum(v, lpr);
  if (lr == 0) val[row] = v;
  __syncthreads();
  if (tid < 32) {
    const float g = val[tid], u = val[32 + tid];
    const float h = silu_p(g) * u;
    float amax = fabsf(h);
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 32));
    const float d = amax / 127.0f;
    const int q = (d == 0.0f) ? 0 : (int)roundf(h / d);
    int sum = q;
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) sum += __shfl_xor(sum, m, 32);
    a.qh[(size_t)slot * I + i0 + tid] = (int8_t)q;
    if (a.t_qh) a.t_qh[(size_t)slot * I + i0 + tid] = (int8_t)q;
    if (tid == 0) {
      a.dh[(size_t)slot * (I / BLK) + blockIdx.x] = d;
      a.sh[(size_t)slot * (I / BLK) + blockIdx.x] = sum;
      if (a.t_dh) a.t_dh[(size_t)slot * (I / BLK) + blockIdx.x] = d;
    }
  }
}

// ---------------------------------------------------------------- down + combine
// Block: `rows` output rows x ns slots, LPR lanes per (row, slot).
template <int BPL, bool FAST>
__global__ void __launch_bounds__(1024) decode_down_kernel(DecodeArgs a, int lpr, int rows) {
  extern __shared__ uint8_t dyn[];
  const int H = a.H, I = a.I, nbi = I / BLK;
  const int ns = a.k + (a.has_shared ? 1 : 0);
  uint32_t* qh_l = reinterpret_cast<uint32_t*>(dyn);                     // ns * I bytes
  float* dh_l = reinterpret_cast<float*>(dyn + (size_t)ns * I);           // ns * nbi
  int32_t* sh_l = reinterpret_cast<int32_t*>(dyn + (size_t)ns * I + 4 * (size_t)ns * nbi);
  float* o_l = reinterpret_cast<float*>(dyn + (size_t)ns * I + 8 * (size_t)ns * nbi);  // rows*ns
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * rows;

  for (int i = tid; i < ns * I / 4; i += blockDim.x) qh_l[i] = reinterpret_cast<const uint32_t*>(a.qh)[i];
  for (int i = tid; i < ns * nbi; i += blockDim.x) { dh_l[i] = a.dh[i]; sh_l[i] = a.sh[i]; }
  __syncthreads();

  const int item = tid / lpr, lr = tid % lpr;
  const int rl = item / ns, slot = item % ns;
  const int r = r0 + rl;
  const bool live = rl < rows && r < H;
  float v = 0.0f;
  if (live) {
    const size_t rb = (size_t)nbi * Q4B;
    const uint8_t* base = (slot < a.k)
        ? a.w_down + ((size_t)min(max(a.ids[slot], 0), a.E - 1) * H + r) * rb
        : a.s_down + (size_t)r * rb;
    auto act = [&](int b) {
      ActBlock A;
#pragma unroll
      for (int q = 0; q < 8; q++) A.a[q] = qh_l[(slot * I) / 4 + b * 8 + q];
      A.d = dh_l[slot * nbi + b];
      A.s = sh_l[slot * nbi + b];
      return A;
    };
    v = w4a8_lane<BPL, FAST>(base, nbi, lr * BPL, act, nullptr);
  }
  v = wave_tree_sum(v, lpr);
  if (live && lr == 0) o_l[rl * ns + slot] = v;
  __syncthreads();
  if (tid < rows && r0 + tid < H) {
    const float* o = o_l + tid * ns;
    float acc = a.w[0] * o[0];
    for (int s = 1; s < a.k; s++) acc = acc + a.w[s] * o[s];
    if (a.has_shared) acc = acc + o[a.k];
    a.y[r0 + tid] = acc;
  }
}

// ---------------------------------------------------------------- launch
hipError_t launch_decode(const DecodeArgs& a, const RouterSplit& sp, hipStream_t stream) {
#define MOEQ4_DR(NSV) \
  hipLaunchKernelGGL((decode_router_kernel<NSV>), dim3(NSV), dim3(256), 0, stream, a, sp.nc, sp.cw)
  switch (sp.nsplit) {
    case 1: MOEQ4_DR(1); break;
    case 2: MOEQ4_DR(2); break;
    case 4: MOEQ4_DR(4); break;
    case 8: MOEQ4_DR(8); break;
    case 16: MOEQ4_DR(16); break;
    case 32: MOEQ4_DR(32); break;
    default: MOEQ4_DR(64); break;
  }
#undef MOEQ4_DR
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  const int ns = a.k + (a.has_shared ? 1 : 0);
  // gate/up
  {
    const RowSplit rs = row_split(a.H, 16);
    const bool fast = (rs.bpl % 8 == 0) && (rs.nb % rs.bpl == 0);
    const size_t lds = (size_t)a.H + 8 * (size_t)(a.H / BLK);
    dim3 grid(a.I / BLK, ns);
    dim3 block(64 * rs.lpr);
#define MOEQ4_GU(B, F) \
  hipLaunchKernelGGL((decode_gateup_kernel<B, F>), grid, block, lds, stream, a, rs.lpr)
    if (fast) {
      if (rs.bpl == 8) MOEQ4_GU(8, true);
      else if (rs.bpl == 16) MOEQ4_GU(16, true);
      else MOEQ4_GU(32, true);
    } else {
      if (rs.bpl == 1) MOEQ4_GU(1, false);
      else if (rs.bpl == 2) MOEQ4_GU(2, false);
      else if (rs.bpl == 4) MOEQ4_GU(4, false);
      else if (rs.bpl == 8) MOEQ4_GU(8, false);
      else if (rs.bpl == 16) MOEQ4_GU(16, false);
      else MOEQ4_GU(32, false);
    }
#undef MOEQ4_GU
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // down + combine
  {
    const RowSplit rs = row_split(a.I, 16);
    const bool fast = (rs.bpl % 8 == 0) && (rs.nb % rs.bpl == 0);
    int threads = 128;
    while (threads / rs.lpr < ns) threads *= 2;
    const int rows = (threads / rs.lpr) / ns;
    const int nbi = a.I / BLK;
    const size_t lds = (size_t)ns * a.I + 8 * (size_t)ns * nbi + 4 * (size_t)rows * ns;
    dim3 grid((a.H + rows - 1) / rows);
    dim3 block(threads);
#define MOEQ4_DN(B, F) \
  hipLaunchKernelGGL((decode_down_kernel<B, F>), grid, block, lds, stream, a, rs.lpr, rows)
    if (fast) {
      if (rs.bpl == 8) MOEQ4_DN(8, true);
      else if (rs.bpl == 16) MOEQ4_DN(16, true);
      else MOEQ4_DN(32, true);
    } else {
      if (rs.bpl == 1) MOEQ4_DN(1, false);
      else if (rs.bpl == 2) MOEQ4_DN(2, false);
      else if (rs.bpl == 4) MOEQ4_DN(4, false);
      else if (rs.bpl == 8) MOEQ4_DN(8, false);
      else if (rs.bpl == 16) MOEQ4_DN(16, false);
      else MOEQ4_DN(32, false);
    }
#undef MOEQ4_DN
    err = hipGetLastError();
  }
  return err;
}

// ---------------------------------------------------------------- test GEMV
template <int BPL, bool FAST>
__global__ void __launch_bounds__(256) w4a8_gemv_kernel(const uint8_t* __restrict__ W, int N, int K,
                                                        const int8_t* __restrict__ qa,
                                                        const float* __restrict__ da,
                                                        int32_t* __restrict__ dots,
                                                        float* __restrict__ out, int lpr) {
  extern __shared__ uint8_t dyn[];
  const int nb = K / BLK;
  uint32_t* qa_l = reinterpret_cast<uint32_t*>(dyn);
  float* da_l = reinterpret_cast<float*>(dyn + K);
  int32_t* sa_l = reinterpret_cast<int32_t*>(dyn + K + 4 * nb);
  const int tid = threadIdx.x;
  for (int i = tid; i < K / 4; i += blockDim.x) qa_l[i] = reinterpret_cast<const uint32_t*>(qa)[i];
  for (int b = tid; b < nb; b += blockDim.x) {
    da_l[b] = da[b];
    int32_t s = 0;
    for (int j = 0; j < BLK; j++) s += qa[b * BLK + j];
    sa_l[b] = s;
  }
  __syncthreads();
  const int rows_per_block = blockDim.x / lpr;
  const int r = blockIdx.x * rows_per_block + tid / lpr, lr = tid % lpr;
  float v = 0.0f;
  if (r < N) {
    auto act = [&](int b) {
      ActBlock A;
#pragma unroll
      for (int q = 0; q < 8; q++) A.a[q] = qa_l[b * 8 + q];
      A.d = da_l[b];
      A.s = sa_l[b];
      return A;
    };
    v = w4a8_lane<BPL, FAST>(W + (size_t)r * nb * Q4B, nb, lr * BPL, act,
                             dots ? dots + (size_t)r * nb : nullptr);
  }
  v = wave_tree_sum(v, lpr);
  if (r < N && lr == 0) out[r] = v;
}

hipError_t launch_w4a8_gemv(const uint8_t* W, int N, int K, const int8_t* qa, const float* da,
                            int32_t* dots, float* out, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const RowSplit rs = row_split(K, 64);
  const bool fast = (rs.bpl % 8 == 0) && (rs.nb % rs.bpl == 0) &&
                    (((uintptr_t)W & 15u) == 0) && (((size_t)rs.nb * Q4B) % 16 == 0);
  const int threads = 256 < rs.lpr ? rs.lpr : 256;
  const int rpb = threads / rs.lpr;
  dim3 grid((N + rpb - 1) / rpb);
  const size_t lds = (size_t)K + 8 * (size_t)rs.nb;
#define MOEQ4_GV(B, F)                                                                        \
  hipLaunchKernelGGL((w4a8_gemv_kernel<B, F>), grid, dim3(threads), lds, stream, W, N, K, qa, da, \
                     dots, out, rs.lpr)
  if (fast) {
    if (rs.bpl == 8) MOEQ4_GV(8, true);
    else if (rs.bpl == 16) MOEQ4_GV(16, true);
    else MOEQ4_GV(32, true);
  } else {
    if (rs.bpl == 1) MOEQ4_GV(1, false);
    else if (rs.bpl == 2) MOEQ4_GV(2, false);
    else if (rs.bpl == 4) MOEQ4_GV(4, false);
    else if (rs.bpl == 8) MOEQ4_GV(8, false);
    else if (rs.bpl == 16) MOEQ4_GV(16, false);
    else MOEQ4_GV(32, false);
  }
#undef MOEQ4_GV
  return hipGetLastError();
}

}  // namespace moeq4
