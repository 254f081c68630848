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
// Five launches on the caller's stream:
//   dbatch_router   one block per 32-element chunk c: W_r's chunk rows are
//                   read once and every token's FMA chain (a leaf of the
//                   pinned tree) is taken; q8 of chunk c of every token.
//   dbatch_route    one block per token: the tree over its leaves (P lanes
//                   per expert, as in the one-token kernel), bias, the top-k
//                   by rank in (logit desc, index asc) order and the softmax.
//   dbatch_gateup   one block per (expert, 32 values of i): the block finds
//                   the expert's tokens in ascending order (one ballot),
//                   stages their x codes in LDS, keeps its 32 gate and 32 up
//                   rows in registers over those tokens, then h = silu(g) * u
//                   and its q8 per (token, slot) pair.  Experts no token
//                   chose exit at once.
//   dbatch_down     one block per (expert, 128 output rows): the pairs' q8(h)
//                   in LDS, the rows in registers, fp32 outputs per pair.
//   dbatch_combine  y[t] = ((w_0 o_0 + w_1 o_1) + ...) + o_shared per token,
//                   in slot order.
#include "launch.hpp"
#include "w4a8.hpp"
#include "decode_common.hpp"
#include "decode_tile.hpp"

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
__global__ void __launch_bounds__(1024) dbatch_route_kernel(DecodeBatchArgs a, int P) {
  extern __shared__ __align__(16) uint8_t dyn[];
  uint64_t* key = reinterpret_cast<uint64_t*>(dyn);                 // [E]
  float* logit = reinterpret_cast<float*>(key + a.E);                // [E]
  __shared__ int ids_l[32];
  __shared__ float vals_l[32], ex_l[32];
  const int tid = threadIdx.x, nt = blockDim.x, t = blockIdx.x;
  const int E = a.E, k = a.k, nc = a.H / BLK;
  const int m = (int)next_pow2_u32((uint32_t)nc), L = m / P;
  const float* src = a.partials + (size_t)t * nc * E;
  const int items = E * P;                // item = e * P + p; the loop is uniform over the block
  for (int b0 = 0; b0 < items; b0 += nt) {
    const int it = b0 + tid;
    const bool ok = it < items;
    const int e = ok ? it / P : 0, p = it % P;
    float lv = ok ? leaf_tree(src + e, E, p * L, L, nc) : 0.0f;
    for (int o = 1; o < P; o <<= 1) lv = lv + __shfl_xor(lv, o, 64);
    if (ok && p == 0) {
      const float lg = a.bias ? lv + a.bias[e] : lv;
      logit[e] = lg;
      key[e] = rank_key(lg, e);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += nt) {     // rank = experts before e in (logit desc, index asc)
    const uint64_t ke = key[e];
    int rank = 0;
    for (int j = 0; j < E; j++) rank += key[j] > ke ? 1 : 0;
    if (rank < k) {
      ids_l[rank] = e;
      vals_l[rank] = logit[e];
    }
  }
  __syncthreads();
  if (tid < k) ex_l[tid] = exp_p(vals_l[tid] - vals_l[0]);
  __syncthreads();
  if (tid < k) {                          // w_s = e_s / ((e_0 + e_1) + ...)
    float S = ex_l[0];
    for (int s = 1; s < k; s++) S = S + ex_l[s];
    const float wv = ex_l[tid] / S;
    a.ids[t * k + tid] = ids_l[tid];
    a.w[t * k + tid] = wv;
    if (a.t_ids) a.t_ids[t * k + tid] = ids_l[tid];
    if (a.t_w) a.t_w[t * k + tid] = wv;
  }
}

// ---------------------------------------------------------------- pairs of one expert
// The (token, slot) pairs of expert e in token order (a token chooses an
// expert at most once), found by wave 0 with one ballot over the tokens;
// e == E is the shared expert (every token, pair M*k + t).  Returns n; the
// pair indices land in pairs_l.  Ends with a barrier.
__device__ __forceinline__ int expert_pairs(const DecodeBatchArgs& a, int e, int* pairs_l, int* n_l) {
  const int tid = threadIdx.x, M = a.M, k = a.k;
  if (tid < 64) {
    int p = -1;
    if (tid < M) {
      if (e == a.E) {
        p = M * k + tid;
      } else {
        for (int s = 0; s < k; s++)
          if (a.ids[tid * k + s] == e) p = tid * k + s;
      }
    }
    const unsigned long long mask = __ballot(p >= 0);
    if (p >= 0) pairs_l[__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u))] = p;
    if (tid == 0) *n_l = __builtin_popcountll(mask);
  }
  __syncthreads();
  return *n_l;
}

// ---------------------------------------------------------------- gate/up
// ---------------------------------------------------------------- tile order
// A lane's blocks b0 .. b0+BPL-1 of row n (0..31) of a 32-row group in tile
// order (`grp` = the group's first piece): block b is half b%2 of piece b/2,
// the lane's codes at code * (n + 32 (b%2)), its scale at scale + 2 (n + 32
// (b%2)).  Blocks >= nb are +0 leaves; the leaves and their pairwise tree are
// those of wxa8_regs, so a row's value is the same bit for bit.
template <int BPL, int FMT>
struct TileSpan {
  TileCodes<FMT> c[BPL];
  uint32_t sc[BPL];
};

template <int BPL, int FMT, bool SCALES = true>
__device__ __forceinline__ void tile_span_load(TileSpan<BPL, FMT>& t, const uint8_t* grp, int n, int nb, int b0) {
  using TF = TileFmt<FMT>;
#pragma unroll
  for (int j = 0; j < BPL; j++) {
    const int b = min(b0 + j, nb - 1);    // (loads past the row re-read its last block)
    const uint8_t* pc = grp + (size_t)(b >> 1) * TF::piece;
    const int l = n + 32 * (b & 1);
    t.c[j] = tile_codes<FMT>(pc + TF::code * l);
    if (SCALES) t.sc[j] = *reinterpret_cast<const uint16_t*>(pc + TF::scale + 2 * l);
  }
}

// WHOLE: nb % BPL == 0, so a lane's span lies wholly inside or wholly past
// the row and no block needs its own test.
template <int BPL, int FMT, bool WHOLE, typename ActFn>
__device__ __forceinline__ float tile_span_value(const TileSpan<BPL, FMT>& t, int nb, int b0, ActFn act) {
  if (b0 >= nb) return 0.0f;              // a lane of padding leaves only
  float p[BPL];
#pragma unroll
  for (int j = 0; j < BPL; j++) {
    const int b = b0 + j;
    p[j] = 0.0f;
    if (WHOLE || b < nb) {
      const ActBlock A = act(b);
      const int32_t dot = tile_dot<FMT>(t.c[j], A.a, A.s);
      const float sd = f16_bits_to_f32(t.sc[j]) * A.d;
      p[j] = sd * (float)dot;
    }
  }
  return reg_tree<BPL>(p);
}

constexpr int DBG_ROWS = 32;

// tb: tokens whose codes fit the block's LDS at once; the expert's tokens are
// taken tb at a time.
// TILED: the weights are read from the tile-order copies (FAST then says
// that nb % BPL == 0; the lane's span is held in registers when BPL <= 8,
// else read per token from the caches).
// sc_off (tile order, BPL <= 8): byte offset in LDS of a copy of the scale
// sections of the block's two 32-row groups, staged by 16-byte loads (a
// lane's scale loads would each touch a cache line for 2 bytes); 0: none.
template <int BPL, bool FAST, int FMT, bool TILED>
__global__ void __launch_bounds__(1024) dbatch_gateup_kernel(DecodeBatchArgs a, int lpr, int tb, int sc_off) {
  extern __shared__ __align__(16) uint8_t dyn[];
  __shared__ int pairs_l[kDecodeBatchMax];
  __shared__ int n_l;
  const int H = a.H, I = a.I, nbh = H / BLK, M = a.M, k = a.k;
  const int SS = act_row_dwords(nbh);
  float* val = reinterpret_cast<float*>(dyn);                              // [64][M]
  uint32_t* qa_l = reinterpret_cast<uint32_t*>(val + 2 * DBG_ROWS * M);   // [tb][SS]
  float* da_l = reinterpret_cast<float*>(qa_l + (size_t)tb * SS);          // [tb][nbh]
  int32_t* sa_l = reinterpret_cast<int32_t*>(da_l + (size_t)tb * nbh);     // [tb][nbh]
  const int tid = threadIdx.x;
  const int ngrp = I / DBG_ROWS, e = blockIdx.x / ngrp, gx = blockIdx.x % ngrp, i0 = gx * DBG_ROWS;
  const bool shared = e == a.E;
  const int n = expert_pairs(a, e, pairs_l, &n_l);
  if (n == 0) return;                     // uniform over the block
  const int row = tid / lpr, lr = tid % lpr;
  const bool is_up = row >= DBG_ROWS;
  const int i = i0 + (row % DBG_ROWS);
  constexpr int QB = WFmt<FMT>::bytes;
  const size_t rb = (size_t)nbh * QB;
  const uint8_t* base = shared ? (is_up ? a.s_up : a.s_gate) + (size_t)i * rb
                               : (is_up ? a.w_up : a.w_gate) + ((size_t)e * I + i) * rb;
  constexpr bool REGS = FAST && !TILED;
  constexpr int NV = REGS ? QB * BPL / 16 : 1;
  uint32_t D[4 * NV + 1] = {};
  if (REGS && lr * BPL < nbh) {
    const uint4* src = reinterpret_cast<const uint4*>(base + (size_t)lr * BPL * QB);
#pragma unroll
    for (int v = 0; v < NV; v++) {
      const uint4 q = src[v];
      D[4 * v] = q.x; D[4 * v + 1] = q.y; D[4 * v + 2] = q.z; D[4 * v + 3] = q.w;
    }
  }
  // tile order: the row's 32-row group (matrix [E][I][H], groups of 32 rows)
  constexpr bool TREGS = TILED && BPL <= 8;
  const size_t gbytes = (size_t)(nbh / 2) * TileFmt<FMT>::piece;
  const uint8_t* grp = nullptr;
  if (TILED)
    grp = shared ? (is_up ? a.ts_up : a.ts_gate) + (size_t)(i / 32) * gbytes
                 : (is_up ? a.t_up : a.t_gate) + ((size_t)e * (I / 32) + i / 32) * gbytes;
  TileSpan<(TILED ? BPL : 1), FMT> ts;
  if constexpr (TREGS) {
    using TF = TileFmt<FMT>;
    if (sc_off) {                         // (uniform: a kernel argument)
      uint8_t* sct = dyn + sc_off;         // [2][nbh / 2 pieces][64 scales]
      const int nsec = nbh / 2;
      const size_t g0 = shared ? (size_t)(i0 / 32) * gbytes : ((size_t)e * (I / 32) + i0 / 32) * gbytes;
      const uint8_t* gg = (shared ? a.ts_gate : a.t_gate) + g0;
      const uint8_t* gu = (shared ? a.ts_up : a.t_up) + g0;
      for (int idx = tid; idx < 2 * nsec * 8; idx += blockDim.x) {
        const int m = idx / (nsec * 8), rem = idx % (nsec * 8), sp = rem / 8, c = rem % 8;
        const uint8_t* src = (m ? gu : gg) + (size_t)sp * TF::piece + TF::scale + 16 * c;
        *reinterpret_cast<uint4*>(sct + ((size_t)m * nsec + sp) * 128 + 16 * c) =
            *reinterpret_cast<const uint4*>(src);
      }
      tile_span_load<BPL, FMT, false>(ts, grp, i % 32, nbh, lr * BPL);
      __syncthreads();
      const uint16_t* sc16 = reinterpret_cast<const uint16_t*>(sct) + (size_t)(is_up ? nsec : 0) * 64;
#pragma unroll
      for (int j = 0; j < BPL; j++) {
        const int b = min(lr * BPL + j, nbh - 1);
        ts.sc[j] = sc16[(b >> 1) * 64 + (i % 32) + 32 * (b & 1)];
      }
    } else {
      tile_span_load<BPL, FMT>(ts, grp, i % 32, nbh, lr * BPL);
    }
  }
  for (int u0 = 0; u0 < n; u0 += tb) {
    const int nu = min(tb, n - u0);
    for (int g = tid; g < nu * nbh; g += blockDim.x) {
      const int u = g / nbh, b = g % nbh;
      const int p = pairs_l[u0 + u], t = shared ? p - M * k : p / k;
      const uint4* src = reinterpret_cast<const uint4*>(a.qx + (size_t)t * H) + 2 * b;
      uint4* dst = reinterpret_cast<uint4*>(qa_l + (size_t)u * SS + act_off(b));
      dst[0] = src[0];
      dst[1] = src[1];
      da_l[u * nbh + b] = a.dx[t * nbh + b];
      sa_l[u * nbh + b] = a.sx[t * nbh + b];
    }
    __syncthreads();
    for (int u = 0; u < nu; u++) {
      auto act = [&](int b) {
        ActBlock A;
        const uint4* q = reinterpret_cast<const uint4*>(qa_l + (size_t)u * SS + act_off(b));
        const uint4 q0 = q[0], q1 = q[1];
        A.a[0] = q0.x; A.a[1] = q0.y; A.a[2] = q0.z; A.a[3] = q0.w;
        A.a[4] = q1.x; A.a[5] = q1.y; A.a[6] = q1.z; A.a[7] = q1.w;
        A.d = da_l[u * nbh + b];
        A.s = sa_l[u * nbh + b];
        return A;
      };
      float v;
      if constexpr (TILED) {
        if constexpr (TREGS) {
          v = tile_span_value<BPL, FMT, FAST>(ts, nbh, lr * BPL, act);
        } else {
          TileSpan<BPL, FMT> tu;
          tile_span_load<BPL, FMT>(tu, grp, i % 32, nbh, lr * BPL);
          v = tile_span_value<BPL, FMT, FAST>(tu, nbh, lr * BPL, act);
        }
      } else if constexpr (FAST) {
        v = wxa8_regs<BPL, FMT>(D, nbh, lr * BPL, act);
      } else {
        v = wxa8_lane<BPL, false, FMT>(base, nbh, lr * BPL, act, nullptr);
      }
      v = wave_tree_sum(v, lpr);
      if (lr == 0) val[row * M + u0 + u] = v;
    }
    __syncthreads();                      // the chunk's codes are read; val is complete
  }
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
    const int p = pairs_l[u];
    a.qh[(size_t)p * I + i0 + r] = (int8_t)q;
    if (r == 0) {
      a.dh[(size_t)p * (I / BLK) + gx] = d;
      a.sh[(size_t)p * (I / BLK) + gx] = sum;
    }
  }
}

// ---------------------------------------------------------------- down
// Block: `rows` (<= 128) output rows of one expert, lpr lanes per row, the
// rows' weights in registers over the expert's pairs; o[pair][r] fp32.
template <int BPL, bool FAST, int FMT, bool TILED>
__global__ void __launch_bounds__(1024) dbatch_down_kernel(DecodeBatchArgs a, int lpr, int tb, int rows) {
  extern __shared__ __align__(16) uint8_t dyn[];
  __shared__ int pairs_l[kDecodeBatchMax];
  __shared__ int n_l;
  const int H = a.H, I = a.I, nbi = I / BLK, M = a.M;
  const int SS = act_row_dwords(nbi);
  uint32_t* qh_l = reinterpret_cast<uint32_t*>(dyn);                       // [tb][SS]
  float* dh_l = reinterpret_cast<float*>(qh_l + (size_t)tb * SS);          // [tb][nbi]
  int32_t* sh_l = reinterpret_cast<int32_t*>(dh_l + (size_t)tb * nbi);     // [tb][nbi]
  const int tid = threadIdx.x;
  const int ngrp = (H + rows - 1) / rows, e = blockIdx.x / ngrp, r0 = (blockIdx.x % ngrp) * rows;
  const bool shared = e == a.E;
  const int n = expert_pairs(a, e, pairs_l, &n_l);
  if (n == 0) return;                     // uniform over the block
  const int rl = tid / lpr, lr = tid % lpr, r = r0 + rl;
  const bool live = rl < rows && r < H;
  constexpr int QB = WFmt<FMT>::bytes;
  const size_t rb = (size_t)nbi * QB;
  const uint8_t* base = shared ? a.s_down + (size_t)min(r, H - 1) * rb
                               : a.w_down + ((size_t)e * H + min(r, H - 1)) * rb;
  constexpr bool REGS = FAST && !TILED;
  constexpr int NV = REGS ? QB * BPL / 16 : 1;
  uint32_t D[4 * NV + 1] = {};
  if (REGS && live && lr * BPL < nbi) {
    const uint4* src = reinterpret_cast<const uint4*>(base + (size_t)lr * BPL * QB);
#pragma unroll
    for (int v = 0; v < NV; v++) {
      const uint4 q = src[v];
      D[4 * v] = q.x; D[4 * v + 1] = q.y; D[4 * v + 2] = q.z; D[4 * v + 3] = q.w;
    }
  }
  // tile order: matrix [E][H][I], groups of 32 output rows
  constexpr bool TREGS = TILED && BPL <= 8;
  const int rr = min(r, H - 1);
  const size_t gbytes = (size_t)(nbi / 2) * TileFmt<FMT>::piece;
  const uint8_t* grp = nullptr;
  if (TILED)
    grp = shared ? a.ts_down + (size_t)(rr / 32) * gbytes : a.t_down + ((size_t)e * (H / 32) + rr / 32) * gbytes;
  TileSpan<(TILED ? BPL : 1), FMT> ts;
  if (TREGS) tile_span_load<(TILED ? BPL : 1), FMT>(ts, grp, rr % 32, nbi, lr * BPL);
  for (int u0 = 0; u0 < n; u0 += tb) {
    const int nu = min(tb, n - u0);
    if (u0 > 0) __syncthreads();          // the previous chunk's activations are read
    for (int g = tid; g < nu * nbi; g += blockDim.x) {
      const int u = g / nbi, b = g % nbi, p = pairs_l[u0 + u];
      const uint4* src = reinterpret_cast<const uint4*>(a.qh + (size_t)p * I) + 2 * b;
      uint4* dst = reinterpret_cast<uint4*>(qh_l + (size_t)u * SS + act_off(b));
      dst[0] = src[0];
      dst[1] = src[1];
      dh_l[u * nbi + b] = a.dh[(size_t)p * nbi + b];
      sh_l[u * nbi + b] = a.sh[(size_t)p * nbi + b];
    }
    __syncthreads();
    for (int u = 0; u < nu; u++) {
      auto act = [&](int b) {
        ActBlock A;
        const uint4* q = reinterpret_cast<const uint4*>(qh_l + (size_t)u * SS + act_off(b));
        const uint4 q0 = q[0], q1 = q[1];
        A.a[0] = q0.x; A.a[1] = q0.y; A.a[2] = q0.z; A.a[3] = q0.w;
        A.a[4] = q1.x; A.a[5] = q1.y; A.a[6] = q1.z; A.a[7] = q1.w;
        A.d = dh_l[u * nbi + b];
        A.s = sh_l[u * nbi + b];
        return A;
      };
      float v;
      if constexpr (TILED) {
        if constexpr (TREGS) {
          v = tile_span_value<BPL, FMT, FAST>(ts, nbi, lr * BPL, act);
        } else {
          TileSpan<BPL, FMT> tu;
          tile_span_load<BPL, FMT>(tu, grp, rr % 32, nbi, lr * BPL);
          v = tile_span_value<BPL, FMT, FAST>(tu, nbi, lr * BPL, act);
        }
      } else if constexpr (FAST) {
        v = wxa8_regs<BPL, FMT>(D, nbi, lr * BPL, act);
      } else {
        v = wxa8_lane<BPL, false, FMT>(base, nbi, lr * BPL, act, nullptr);
      }
      v = wave_tree_sum(v, lpr);
      if (live && lr == 0) a.o[(size_t)pairs_l[u0 + u] * H + r] = v;
    }
  }
}

// ---------------------------------------------------------------- combine
__global__ void __launch_bounds__(256) dbatch_combine_kernel(DecodeBatchArgs a) {
  const int H = a.H, M = a.M, k = a.k;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * H) return;
  const int t = (int)(i / H), r = (int)(i % H);
  const float* w = a.w + (size_t)t * k;
  const float* o = a.o + (size_t)t * k * H + r;
  float acc = w[0] * o[0];
  for (int s = 1; s < k; s++) acc = acc + w[s] * o[(size_t)s * H];
  if (a.has_shared) acc = acc + a.o[((size_t)M * k + t) * H + r];
  a.y[(size_t)t * H + r] = acc;
}

// ---------------------------------------------------------------- launch
DecodeBatchGeometry decode_batch_geometry(int M, int H, int I, int E, int k, int has_shared) {
  DecodeBatchGeometry g;
  int rt = (E + 63) / 64 * 64;
  if (rt < 32 * M) rt = 32 * M;
  g.router_threads = rt;
  const int nc = H / BLK;
  int m = 1;
  while (m < nc) m <<= 1;
  int P = 1;                              // lanes per expert: runs of <= 32 leaves
  while (P < 64 && P < m && E * P * 2 <= 1024) P <<= 1;
  while (m / P > 32) P <<= 1;
  g.route_parts = P;
  int rth = (E * P + 63) / 64 * 64;
  g.route_threads = rth > 1024 ? 1024 : rth;
  g.route_lds = 12 * (size_t)E;
  const RowSplit gu = row_split(H, 16);
  g.gu_lpr = gu.lpr;
  g.gu_bpl = gu.bpl;
  g.gu_fast = (gu.bpl % 8 == 0) && (gu.nb % gu.bpl == 0);
  g.gu_threads = 2 * DBG_ROWS * gu.lpr;
  const size_t gu_tok = 4 * ((size_t)act_row_dwords(nc) + 2 * (size_t)nc);   // LDS bytes per staged token
  const size_t gu_val = 4 * (size_t)2 * DBG_ROWS * M;
  size_t tb = (kDecodeBatchLds - gu_val) / gu_tok;
  g.gu_tb = (int)(tb < 1 ? 1 : (tb > (size_t)M ? (size_t)M : tb));
  g.gu_lds = gu_val + gu_tok * g.gu_tb;
  const RowSplit dn = row_split(I, 16);
  g.dn_lpr = dn.lpr;
  g.dn_bpl = dn.bpl;
  g.dn_fast = (dn.bpl % 8 == 0) && (dn.nb % dn.bpl == 0);
  g.dn_rows = 1024 / dn.lpr < 128 ? 1024 / dn.lpr : 128;
  g.dn_threads = g.dn_rows * dn.lpr;
  const int nbi = I / BLK;
  const size_t dn_tok = 4 * ((size_t)act_row_dwords(nbi) + 2 * (size_t)nbi);
  tb = kDecodeBatchLds / dn_tok;
  g.dn_tb = (int)(tb < 1 ? 1 : (tb > (size_t)M ? (size_t)M : tb));
  g.dn_lds = dn_tok * g.dn_tb;
  (void)has_shared;
  return g;
}

// gate/up and down launches for one weight format
template <int FMT>
hipError_t launch_dbatch_experts(const DecodeBatchArgs& a, const DecodeBatchGeometry& g, int nexp,
                                 hipStream_t stream) {
  hipError_t err = hipSuccess;
  // the tile-order copies when the layer carries them (H and I are then
  // multiples of 64, so a lane's span covers whole pieces: bpl >= 2)
  const bool tiled = a.t_gate && a.t_up && a.t_down && (!a.has_shared || (a.ts_gate && a.ts_up && a.ts_down)) &&
                     g.gu_bpl >= 2 && g.dn_bpl >= 2;
  {
    dim3 grid(nexp * (a.I / DBG_ROWS));
    dim3 block(g.gu_threads);
    // the tile-order kernel's LDS copy of the scale sections (2 groups x H/64
    // pieces x 128 bytes) after the rest, when the lane spans are in registers
    const int nbh = a.H / BLK;
    const int sc_off = (tiled && g.gu_bpl <= 8 && nbh * 128 <= 16 * 1024) ? (int)((g.gu_lds + 15) / 16 * 16) : 0;
    const size_t lds_t = sc_off ? (size_t)sc_off + (size_t)nbh * 128 : g.gu_lds;
#define MOEQ4_GU(B, F) \
  hipLaunchKernelGGL((dbatch_gateup_kernel<B, F, FMT, false>), grid, block, g.gu_lds, stream, a, g.gu_lpr, g.gu_tb, 0)
#define MOEQ4_GUT(B, W) \
  hipLaunchKernelGGL((dbatch_gateup_kernel<B, W, FMT, true>), grid, block, lds_t, stream, a, g.gu_lpr, g.gu_tb, sc_off)
#define MOEQ4_GUTW(B) \
  if ((a.H / BLK) % B == 0) MOEQ4_GUT(B, true); else MOEQ4_GUT(B, false);
    if (tiled) {
      if (g.gu_bpl == 2) { MOEQ4_GUTW(2) }
      else if (g.gu_bpl == 4) { MOEQ4_GUTW(4) }
      else if (g.gu_bpl == 8) { MOEQ4_GUTW(8) }
      else if (g.gu_bpl == 16) { MOEQ4_GUTW(16) }
      else { MOEQ4_GUTW(32) }
    } else if (g.gu_fast) {
      if (g.gu_bpl == 8) MOEQ4_GU(8, true);
      else if (g.gu_bpl == 16) MOEQ4_GU(16, true);
      else MOEQ4_GU(32, true);
    } else {
      if (g.gu_bpl == 1) MOEQ4_GU(1, false);
      else if (g.gu_bpl == 2) MOEQ4_GU(2, false);
      else if (g.gu_bpl == 4) MOEQ4_GU(4, false);
      else if (g.gu_bpl == 8) MOEQ4_GU(8, false);
      else if (g.gu_bpl == 16) MOEQ4_GU(16, false);
      else MOEQ4_GU(32, false);
    }
#undef MOEQ4_GUTW
#undef MOEQ4_GUT
#undef MOEQ4_GU
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  {
    dim3 grid(nexp * ((a.H + g.dn_rows - 1) / g.dn_rows));
    dim3 block(g.dn_threads);
#define MOEQ4_DN(B, F) \
  hipLaunchKernelGGL((dbatch_down_kernel<B, F, FMT, false>), grid, block, g.dn_lds, stream, a, g.dn_lpr, g.dn_tb, g.dn_rows)
#define MOEQ4_DNT(B, W) \
  hipLaunchKernelGGL((dbatch_down_kernel<B, W, FMT, true>), grid, block, g.dn_lds, stream, a, g.dn_lpr, g.dn_tb, g.dn_rows)
#define MOEQ4_DNTW(B) \
  if ((a.I / BLK) % B == 0) MOEQ4_DNT(B, true); else MOEQ4_DNT(B, false);
    if (tiled) {
      if (g.dn_bpl == 2) { MOEQ4_DNTW(2) }
      else if (g.dn_bpl == 4) { MOEQ4_DNTW(4) }
      else if (g.dn_bpl == 8) { MOEQ4_DNTW(8) }
      else if (g.dn_bpl == 16) { MOEQ4_DNTW(16) }
      else { MOEQ4_DNTW(32) }
    } else if (g.dn_fast) {
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
#undef MOEQ4_DNTW
#undef MOEQ4_DNT
#undef MOEQ4_DN
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return err;
}

hipError_t launch_decode_batch(const DecodeBatchArgs& a, hipStream_t stream) {
  const DecodeBatchGeometry g = decode_batch_geometry(a.M, a.H, a.I, a.E, a.k, a.has_shared);
  const int nc = a.H / BLK, nexp = a.E + (a.has_shared ? 1 : 0);
  hipLaunchKernelGGL(dbatch_router_kernel, dim3(nc), dim3(g.router_threads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dbatch_route_kernel, dim3(a.M), dim3(g.route_threads), g.route_lds, stream, a, g.route_parts);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = a.wfmt == kQ8 ? launch_dbatch_experts<kQ8>(a, g, nexp, stream)
                      : launch_dbatch_experts<kQ4>(a, g, nexp, stream);
  if (err != hipSuccess) return err;
  const int64_t n = (int64_t)a.M * a.H;
  hipLaunchKernelGGL(dbatch_combine_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moeq4
