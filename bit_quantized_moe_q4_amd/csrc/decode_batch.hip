// decode_batch.hip -- decode of a small batch of tokens (1..32) in one call.
//
// "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU",
// technical summary, Methodology 1 (single tokens through the W4A8 integer
// kernel) and Results (the thin-M regime between a GEMV and a grouped GEMM).
// Every token goes through exactly the single-token program of decode.hip:
// the same router leaves and tree, top-k order and softmax, the same W4A8
// row program for gate/up and down and the same fixed-order combine, so each
// token's y is bit-identical to a moe_q4_decode of that token alone.  What
// changes is the memory traffic: an expert selected by several tokens is
// read once per call, not once per token.
//
// Four launches on the caller's stream:
//   dbatch_router   one block per 32-element chunk c: W_r's chunk rows are
//                   read once and every token's FMA chain (a leaf of the
//                   pinned tree) is taken; q8 of chunk c of every token.
//   dbatch_route    one block: per token (one wave) the tree over the leaves,
//                   bias, the top-k in (logit desc, index asc) order and the
//                   softmax weights; then per expert the ascending list of
//                   its (token, slot) pairs and the ascending list of the
//                   experts that have pairs.
//   dbatch_gateup   one block per (listed expert, 32 values of i): the 32 gate
//                   and 32 up rows stay in registers while the block runs the
//                   row program for each of the expert's tokens (codes in
//                   LDS), then h = silu(g) * u and its q8 per pair.
//   dbatch_down     one block per few output rows: (row, listed expert) items
//                   whose weights stay in registers over the expert's pairs,
//                   then each token's combine in slot order.
#include "launch.hpp"
#include "w4a8.hpp"
#include "decode_common.hpp"

namespace moeq4 {

// ---------------------------------------------------------------- router
__global__ void __launch_bounds__(1024) dbatch_router_kernel(DecodeBatchArgs a) {
  __shared__ float xs[kDecodeBatchMax][BLK + 1];
  const int tid = threadIdx.x, c = blockIdx.x;
  const int M = a.M, E = a.E, H = a.H, nc = H / BLK;
  for (int i = tid; i < M * BLK; i += blockDim.x) xs[i / BLK][i % BLK] = a.x[(size_t)(i / BLK) * H + c * BLK + i % BLK];
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    const float* w = a.w_router + (size_t)c * BLK * E + e;
    float wv[BLK];
#pragma unroll
    for (int i = 0; i < BLK; i++) wv[i] = w[(size_t)i * E];
    for (int t = 0; t < M; t++) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < BLK; i++) acc = __builtin_fmaf(xs[t][i], wv[i], acc);
      a.partials[((size_t)t * nc + c) * E + e] = acc;
    }
  }
  // q8 of chunk c of every token: a 32-lane group per token (blockDim % 32 == 0,
  // so the lanes of a group take the same pass of the loop)
  for (int i = tid; i < M * BLK; i += blockDim.x) {
    const int t = i / BLK, j = i % BLK;
    const float v = xs[t][j];
    float amax = fabsf(v);
#pragma unroll
    for (int m = 1; m < BLK; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, BLK));
    const float d = amax / 127.0f;
    const int q = (d == 0.0f) ? 0 : (int)roundf(v / d);
    int sum = q;
#pragma unroll
    for (int m = 1; m < BLK; m <<= 1) sum += __shfl_xor(sum, m, BLK);
    a.qx[(size_t)t * H + c * BLK + j] = (int8_t)q;
    if (j == 0) {
      a.dx[t * nc + c] = d;
      a.sx[t * nc + c] = sum;
    }
  }
}

// ---------------------------------------------------------------- routing
// 64-bit wave maximum (keys are unique: the low word encodes the expert).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, 64), hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    const uint64_t u = ((uint64_t)hi << 32) | lo;
    v = u > v ? u : v;
  }
  return v;
}

constexpr int kRouteKeysPerLane = 16;     // E <= 1024

__global__ void __launch_bounds__(1024) dbatch_route_kernel(DecodeBatchArgs a) {
  __shared__ int ids_l[kDecodeBatchMax * 32];
  __shared__ float vals_l[kDecodeBatchMax * 32];
  __shared__ int scan_l[1024];
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64, nw = blockDim.x / 64;
  const int M = a.M, E = a.E, k = a.k, nc = a.H / BLK;
  const int nj = (E + 63) / 64;
  for (int t = wave; t < M; t += nw) {
    const float* P = a.partials + (size_t)t * nc * E;
    uint64_t kv[kRouteKeysPerLane];
#pragma unroll
    for (int j = 0; j < kRouteKeysPerLane; j++) {
      kv[j] = 0;
      const int e = lane + 64 * j;
      if (j < nj && e < E) {
        float l = root_tree(P + e, E, nc);
        if (a.bias) l = l + a.bias[e];
        kv[j] = rank_key(l, e);
      }
    }
    for (int r = 0; r < k; r++) {         // k rounds of the first maximum among the rest
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < kRouteKeysPerLane; j++) best = kv[j] > best ? kv[j] : best;
      best = wave_max_u64(best);
      const int e = (int)(0xffffffffu - (uint32_t)best);
#pragma unroll
      for (int j = 0; j < kRouteKeysPerLane; j++)
        if (kv[j] == best) kv[j] = 0;
      if (lane == 0) {
        ids_l[t * k + r] = min(max(e, 0), E - 1);
        vals_l[t * k + r] = key_logit(best);
      }
    }
  }
  __syncthreads();
  // softmax weights: w_s = e_s / ((e_0 + e_1) + ...), e_s = exp(l_s - l_0)
  for (int i = tid; i < M * k; i += blockDim.x) {
    const int t = i / k;
    const float l0 = vals_l[t * k];
    float S = exp_p(vals_l[t * k] - l0);
    for (int s = 1; s < k; s++) S = S + exp_p(vals_l[t * k + s] - l0);
    const float wv = exp_p(vals_l[i] - l0) / S;
    a.ids[i] = ids_l[i];
    a.w[i] = wv;
    if (a.t_ids) a.t_ids[i] = ids_l[i];
    if (a.t_w) a.t_w[i] = wv;
  }
  // per-expert pair lists: expert e counts its pairs in pair order, an
  // exclusive scan over (listed << 16 | count) places lists and hits
  const int np = M * k;
  int cnt = 0;
  const int e = tid;
  if (e < E)
    for (int p = 0; p < np; p++) cnt += ids_l[p] == e ? 1 : 0;
  int v = (e < E) ? (((cnt > 0) ? 1 : 0) << 16) | cnt : 0;
  scan_l[tid] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {    // inclusive Hillis-Steele scan over 1024 entries
    const int add = (tid >= o && tid < (int)blockDim.x) ? scan_l[tid - o] : 0;
    __syncthreads();
    scan_l[tid] += add;
    __syncthreads();
  }
  const int excl = scan_l[tid] - v;
  if (e < E) {
    const int off = excl & 0xffff, h = excl >> 16;
    a.elist_off[e] = off;
    if (cnt > 0) {
      a.hit[h] = e;
      int n = 0;
      for (int p = 0; p < np && n < cnt; p++)
        if (ids_l[p] == e) a.elist[off + n++] = p;
    }
  }
  if (tid == 0) {
    a.elist_off[E] = np;
    a.nhit[0] = scan_l[E - 1] >> 16;
  }
}

// ---------------------------------------------------------------- gate/up
// The n pairs of block row j: a listed expert's pairs, or (j == hb) every
// token for the shared expert.  Pair u: index into qh, and its token.
struct PairSet {
  int n, p0, shared, e;
};

__device__ __forceinline__ PairSet pair_set(const DecodeBatchArgs& a, int j) {
  PairSet ps;
  ps.shared = a.has_shared && j == a.hb;
  ps.n = 0;
  ps.p0 = 0;
  ps.e = 0;
  if (ps.shared) {
    ps.n = a.M;
  } else if (j < a.nhit[0]) {
    ps.e = a.hit[j];
    ps.p0 = a.elist_off[ps.e];
    ps.n = a.elist_off[ps.e + 1] - ps.p0;
  }
  return ps;
}

__device__ __forceinline__ int pair_index(const DecodeBatchArgs& a, const PairSet& ps, int u) {
  return ps.shared ? a.M * a.k + u : a.elist[ps.p0 + u];
}

__device__ __forceinline__ int pair_token(const DecodeBatchArgs& a, const PairSet& ps, int u) {
  return ps.shared ? u : a.elist[ps.p0 + u] / a.k;
}

constexpr int DBG_ROWS = 32;

// ALDS: every token's x codes staged in LDS; otherwise read from the workspace.
template <int BPL, bool FAST, bool ALDS>
__global__ void __launch_bounds__(1024) dbatch_gateup_kernel(DecodeBatchArgs a, int lpr) {
  extern __shared__ __align__(16) uint8_t dyn[];
  const int H = a.H, I = a.I, nbh = H / BLK, M = a.M;
  const int SS = act_row_dwords(nbh);
  uint32_t* qa_l = reinterpret_cast<uint32_t*>(dyn);                       // [M][SS] (ALDS)
  float* da_l = reinterpret_cast<float*>(qa_l + (ALDS ? (size_t)M * SS : 0));  // [M][nbh]
  int32_t* sa_l = reinterpret_cast<int32_t*>(da_l + (ALDS ? (size_t)M * nbh : 0));
  float* val = reinterpret_cast<float*>(sa_l + (ALDS ? (size_t)M * nbh : 0));  // [64][M]
  const int tid = threadIdx.x;
  const int ngrp = I / DBG_ROWS, j = blockIdx.x / ngrp, gx = blockIdx.x % ngrp, i0 = gx * DBG_ROWS;
  const PairSet ps = pair_set(a, j);
  if (ps.n == 0) return;                  // uniform over the block
  const int n = ps.n;
  for (int g = tid; ALDS && g < n * nbh; g += blockDim.x) {
    const int u = g / nbh, b = g % nbh, t = pair_token(a, ps, u);
    const uint4* src = reinterpret_cast<const uint4*>(a.qx + (size_t)t * H) + 2 * b;
    uint4* dst = reinterpret_cast<uint4*>(qa_l + (size_t)u * SS + act_off(b));
    dst[0] = src[0];
    dst[1] = src[1];
    da_l[u * nbh + b] = a.dx[t * nbh + b];
    sa_l[u * nbh + b] = a.sx[t * nbh + b];
  }
  const int row = tid / lpr, lr = tid % lpr;
  const bool is_up = row >= DBG_ROWS;
  const int i = i0 + (row % DBG_ROWS);
  const size_t rb = (size_t)nbh * Q4B;
  const uint8_t* base = ps.shared ? (is_up ? a.s_up : a.s_gate) + (size_t)i * rb
                                  : (is_up ? a.w_up : a.w_gate) + ((size_t)ps.e * I + i) * rb;
  constexpr int NV = FAST ? 18 * BPL / 16 : 1;
  uint32_t D[4 * NV + 1] = {};
  if (FAST && lr * BPL < nbh) {
    const uint4* src = reinterpret_cast<const uint4*>(base + (size_t)lr * BPL * Q4B);
#pragma unroll
    for (int v = 0; v < NV; v++) {
      const uint4 q = src[v];
      D[4 * v] = q.x; D[4 * v + 1] = q.y; D[4 * v + 2] = q.z; D[4 * v + 3] = q.w;
    }
  }
  __syncthreads();
  for (int u = 0; u < n; u++) {
    const int t = pair_token(a, ps, u);
    auto act = [&](int b) {
      ActBlock A;
      const uint4* q = ALDS ? reinterpret_cast<const uint4*>(qa_l + (size_t)u * SS + act_off(b))
                            : reinterpret_cast<const uint4*>(a.qx + (size_t)t * H) + 2 * b;
      const uint4 u0 = q[0], u1 = q[1];
      A.a[0] = u0.x; A.a[1] = u0.y; A.a[2] = u0.z; A.a[3] = u0.w;
      A.a[4] = u1.x; A.a[5] = u1.y; A.a[6] = u1.z; A.a[7] = u1.w;
      A.d = ALDS ? da_l[u * nbh + b] : a.dx[t * nbh + b];
      A.s = ALDS ? sa_l[u * nbh + b] : a.sx[t * nbh + b];
      return A;
    };
    float v;
    if constexpr (FAST) v = w4a8_regs<BPL>(D, nbh, lr * BPL, act);
    else v = w4a8_lane<BPL, false>(base, nbh, lr * BPL, act, nullptr);
    v = wave_tree_sum(v, lpr);
    if (lr == 0) val[row * M + u] = v;
  }
  __syncthreads();
  // h of one 32-group per pair, then its q8 (a 32-lane group per pair)
  for (int idx = tid; idx < n * DBG_ROWS; idx += blockDim.x) {
    const int u = idx / DBG_ROWS, r = idx % DBG_ROWS;
    const float h = silu_p(val[r * M + u]) * val[(DBG_ROWS + r) * M + u];
    float amax = fabsf(h);
#pragma unroll
    for (int m = 1; m < BLK; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, BLK));
    const float d = amax / 127.0f;
    const int q = (d == 0.0f) ? 0 : (int)roundf(h / d);
    int sum = q;
#pragma unroll
    for (int m = 1; m < BLK; m <<= 1) sum += __shfl_xor(sum, m, BLK);
    const int p = pair_index(a, ps, u);
    a.qh[(size_t)p * I + i0 + r] = (int8_t)q;
    if (r == 0) {
      a.dh[(size_t)p * (I / BLK) + gx] = d;
      a.sh[(size_t)p * (I / BLK) + gx] = sum;
    }
  }
}

// ---------------------------------------------------------------- down + combine
// Block: `rows` output rows x (hb + S) listed experts, LPR lanes per (row,
// expert) item; an item's weight span stays in registers over its pairs.
template <int BPL, bool FAST>
__global__ void __launch_bounds__(1024) dbatch_down_kernel(DecodeBatchArgs a, int lpr, int rows) {
  extern __shared__ __align__(16) float o_l[];          // [rows][np + M*S]
  const int H = a.H, I = a.I, nbi = I / BLK, M = a.M, k = a.k;
  const int nlist = a.hb + (a.has_shared ? 1 : 0);
  const int npair = M * k + (a.has_shared ? M : 0);
  const int tid = threadIdx.x, r0 = blockIdx.x * rows;
  const int lr = tid % lpr, stride = blockDim.x / lpr;
  const size_t rb = (size_t)nbi * Q4B;
  // items (row, listed expert), lpr lanes each; the lanes of an item run the
  // same number of pairs, so the shuffles stay inside the item's lanes
  for (int item = tid / lpr; item < rows * nlist; item += stride) {
    const int rl = item / nlist, j = item % nlist, r = r0 + rl;
    if (r >= H) continue;
    const PairSet ps = pair_set(a, j);
    if (ps.n == 0) continue;
    const uint8_t* base = ps.shared ? a.s_down + (size_t)r * rb : a.w_down + ((size_t)ps.e * H + r) * rb;
    constexpr int NV = FAST ? 18 * BPL / 16 : 1;
    uint32_t D[4 * NV + 1] = {};
    if (FAST && lr * BPL < nbi) {
      const uint4* src = reinterpret_cast<const uint4*>(base + (size_t)lr * BPL * Q4B);
#pragma unroll
      for (int v = 0; v < NV; v++) {
        const uint4 q = src[v];
        D[4 * v] = q.x; D[4 * v + 1] = q.y; D[4 * v + 2] = q.z; D[4 * v + 3] = q.w;
      }
    }
    for (int u = 0; u < ps.n; u++) {
      const int p = pair_index(a, ps, u);
      auto act = [&](int b) {
        ActBlock A;
        const uint4* q = reinterpret_cast<const uint4*>(a.qh + (size_t)p * I) + 2 * b;
        const uint4 u0 = q[0], u1 = q[1];
        A.a[0] = u0.x; A.a[1] = u0.y; A.a[2] = u0.z; A.a[3] = u0.w;
        A.a[4] = u1.x; A.a[5] = u1.y; A.a[6] = u1.z; A.a[7] = u1.w;
        A.d = a.dh[(size_t)p * nbi + b];
        A.s = a.sh[(size_t)p * nbi + b];
        return A;
      };
      float v;
      if constexpr (FAST) v = w4a8_regs<BPL>(D, nbi, lr * BPL, act);
      else v = w4a8_lane<BPL, false>(base, nbi, lr * BPL, act, nullptr);
      v = wave_tree_sum(v, lpr);
      if (lr == 0) o_l[(size_t)rl * npair + p] = v;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < rows * M; idx += blockDim.x) {
    const int rr = idx / M, t = idx % M, ro = r0 + rr;
    if (ro >= H) continue;
    const float* o = o_l + (size_t)rr * npair;
    const float* w = a.w + (size_t)t * k;
    float acc = w[0] * o[t * k];
    for (int s = 1; s < k; s++) acc = acc + w[s] * o[t * k + s];
    if (a.has_shared) acc = acc + o[M * k + t];
    a.y[(size_t)t * H + ro] = acc;
  }
}

// ---------------------------------------------------------------- launch
DecodeBatchGeometry decode_batch_geometry(int M, int H, int I, int E, int k, int has_shared) {
  DecodeBatchGeometry g;
  const int hb = E < M * k ? E : M * k;
  const int nlist = hb + (has_shared ? 1 : 0);
  int rt = (E + 63) / 64 * 64;
  if (rt < 32 * M) rt = 32 * M;
  g.router_threads = rt;
  const RowSplit gu = row_split(H, 16);
  g.gu_lpr = gu.lpr;
  g.gu_bpl = gu.bpl;
  g.gu_fast = (gu.bpl % 8 == 0) && (gu.nb % gu.bpl == 0);
  g.gu_threads = 2 * DBG_ROWS * gu.lpr;
  const int nbh = H / BLK;
  const size_t act = 4 * ((size_t)M * act_row_dwords(nbh) + 2 * (size_t)M * nbh);
  const size_t val = 4 * (size_t)2 * DBG_ROWS * M;
  g.gu_alds = act + val <= kDecodeLdsMax;
  g.gu_lds = (g.gu_alds ? act : 0) + val;
  const RowSplit dn = row_split(I, 16);
  g.dn_lpr = dn.lpr;
  g.dn_bpl = dn.bpl;
  g.dn_fast = (dn.bpl % 8 == 0) && (dn.nb % dn.bpl == 0);
  const int per_row = nlist * dn.lpr;
  int rows = 1024 / per_row;
  if (rows < 1) rows = 1;
  if (rows > 64) rows = 64;
  g.dn_rows = rows;
  g.dn_threads = (rows * per_row + 63) / 64 * 64;
  if (g.dn_threads > 1024) g.dn_threads = 1024;   // the kernel loops over its items
  const int npair = M * k + (has_shared ? M : 0);
  g.dn_lds = 4 * (size_t)rows * npair;
  return g;
}

hipError_t launch_decode_batch(const DecodeBatchArgs& a, hipStream_t stream) {
  const DecodeBatchGeometry g = decode_batch_geometry(a.M, a.H, a.I, a.E, a.k, a.has_shared);
  const int nc = a.H / BLK;
  hipLaunchKernelGGL(dbatch_router_kernel, dim3(nc), dim3(g.router_threads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dbatch_route_kernel, dim3(1), dim3(1024), 0, stream, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nlist = a.hb + (a.has_shared ? 1 : 0);
  {
    dim3 grid(nlist * (a.I / DBG_ROWS));
    dim3 block(g.gu_threads);
#define MOEQ4_GU(B, F, L) \
  hipLaunchKernelGGL((dbatch_gateup_kernel<B, F, L>), grid, block, g.gu_lds, stream, a, g.gu_lpr)
#define MOEQ4_GU_L(B, F) \
  if (g.gu_alds) MOEQ4_GU(B, F, true); else MOEQ4_GU(B, F, false)
    if (g.gu_fast) {
      if (g.gu_bpl == 8) { MOEQ4_GU_L(8, true); }
      else if (g.gu_bpl == 16) { MOEQ4_GU_L(16, true); }
      else { MOEQ4_GU_L(32, true); }
    } else {
      if (g.gu_bpl == 1) { MOEQ4_GU_L(1, false); }
      else if (g.gu_bpl == 2) { MOEQ4_GU_L(2, false); }
      else if (g.gu_bpl == 4) { MOEQ4_GU_L(4, false); }
      else if (g.gu_bpl == 8) { MOEQ4_GU_L(8, false); }
      else if (g.gu_bpl == 16) { MOEQ4_GU_L(16, false); }
      else { MOEQ4_GU_L(32, false); }
    }
#undef MOEQ4_GU_L
#undef MOEQ4_GU
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  {
    dim3 grid((a.H + g.dn_rows - 1) / g.dn_rows);
    dim3 block(g.dn_threads);
#define MOEQ4_DN(B, F) \
  hipLaunchKernelGGL((dbatch_down_kernel<B, F>), grid, block, g.dn_lds, stream, a, g.dn_lpr, g.dn_rows)
    if (g.dn_fast) {
      if (g.dn_bpl == 8) MOEQ4_DN(8, true);
      else if (g.dn_bpl == 16) MOEQ4_DN(16, true);
      else MOEQ4_DN(32, true);
    } else {
      if (g.dn_bpl == 1) MOEQ4_DN(1, false);
      else if (g.dn_bpl == 2) MOEQ4_DN(2, false);
      else if (g.dn_bpl == 4) MOEQ4_DN(4, false);
      else if (g.dn_bpl == 8) MOEQ4_DN(8, false);
      else if (g.dn_bpl == 16) MOEQ4_DN(16, false);
      else MOEQ4_DN(32, false);
    }
#undef MOEQ4_DN
    err = hipGetLastError();
  }
  return err;
}

}  // namespace moeq4
