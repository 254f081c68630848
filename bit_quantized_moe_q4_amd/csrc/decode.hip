// decode.hip -- single-token decode step of the Q4_0 MoE layer (W4A8).
//
// "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU",
// technical summary, Methodology 1 (decode of single tokens by a W4A8 integer
// kernel over 4-bit weights read straight from memory) and Key Contribution 2.
// On the pages the weights are read from host RAM by the CPU; here every
// expert stays resident in HBM and the step is bound by streaming the k+S
// selected experts' 18-byte blocks, behind a short chain of dependent steps
// (router -> expert choice -> gate/up -> down).  Each launch boundary is the
// only cross-CU synchronisation: no atomics, flags or cache maintenance.
//
// Three launches on the caller's stream:
//   decode_router   one block per 32-element chunk c of x, one thread per
//                   expert: the chunk's sequential FMA chain for every
//                   expert (a leaf of the pinned pairwise tree), and the q8
//                   codes of chunk c (a chunk is one q8 block).
//   decode_gateup   one block per (slot, 32 values of i).  A routed slot's
//                   block first finishes the router itself from the leaves
//                   (tree, bias, top-k, weights: a few microseconds of
//                   redundant work per block instead of a serial tail in
//                   one block plus another launch); block (0, 0) publishes
//                   ids and weights.  Then the 32 gate and 32 up rows by
//                   the W4A8 row program with x's codes staged in LDS, and
//                   h = silu(g) * u quantised to q8 -- the block holds
//                   exactly one 32-group of h.
//   decode_down     one block per few output rows: the down-row weights
//                   into registers, every slot's q8(h) into LDS, then the
//                   row program and the fixed-order weighted combine.
//
// Activation codes in LDS use the padded layout of decode_common.hpp.
#include "launch.hpp"
#include "w4a8.hpp"
#include "decode_common.hpp"
#include "decode_tile.hpp"

namespace moeq4 {

// ---------------------------------------------------------------- router
// With a.norm_in the input is the previous layer's y and the block first
// takes x = y / r, r the RMSNorm scale of y (every block computes r itself:
// the stack's glue without a launch of its own).
__global__ void __launch_bounds__(1024) decode_router_kernel(DecodeArgs a) {
  __shared__ float xs[BLK];
  __shared__ float part[512], tmp[512];
  const int tid = threadIdx.x, c = blockIdx.x;
  const int E = a.E;
  if (a.norm_in) {
    const float r = rms_scale(a.x, a.H, a.norm_eps, part, tmp);
    if (tid < BLK) xs[tid] = a.x[c * BLK + tid] / r;
  } else if (tid < BLK) {
    xs[tid] = a.x[c * BLK + tid];
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    const float* w = a.w_router + (size_t)c * BLK * E + e;
    float wv[BLK];
#pragma unroll
    for (int i = 0; i < BLK; i++) wv[i] = w[(size_t)i * E];
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < BLK; i++) acc = __builtin_fmaf(xs[i], wv[i], acc);
    a.partials[(size_t)c * E + e] = acc;
  }
  if (tid < BLK) {                        // q8 of chunk c: d = amax / 127, q = round(x / d)
    const float v = xs[tid];
    float amax = fabsf(v);
#pragma unroll
    for (int m = 1; m < BLK; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, BLK));
    const float d = amax / 127.0f;
    const int q = (d == 0.0f) ? 0 : (int)roundf(v / d);
    int sum = q;
#pragma unroll
    for (int m = 1; m < BLK; m <<= 1) sum += __shfl_xor(sum, m, BLK);
    a.qx[c * BLK + tid] = (int8_t)q;
    if (a.t_qx) a.t_qx[c * BLK + tid] = (int8_t)q;
    if (tid == 0) {
      a.dx[c] = d;
      a.sx[c] = sum;
      if (a.t_dx) a.t_dx[c] = d;
    }
  }
}

// ---------------------------------------------------------------- gate/up
// Block: 32 values of i; rows 0..31 gate, 32..63 up, LPR lanes per row.

// Router completion inside a gate/up block.  The nc leaves of expert e
// (padded with +0 to m = next_pow2(nc)) are split into P aligned runs of
// L = m / P <= 32 leaves, one run per lane of a group of P adjacent lanes;
// each lane takes its run's pairwise tree, and log2(P) xor-shuffle levels
// finish the same tree (the two operands of a level are the two subtree
// sums, added in either order).  The top-k is taken by rank: expert e's
// rank is the number of experts before it in (logit desc, index asc) order,
// which for non-NaN logits picks the same experts in the same order as k
// rounds of "first maximum among the rest".  The P lanes of a group split
// the E comparisons.
struct GuLds {
  uint32_t* qa;    // act_row_dwords(nbh)   x's codes
  float* da;       // nbh
  int32_t* sa;     // nbh
  float* logit;    // E
  uint64_t* key;   // E
};

// (the key array is padded to an even count so that qa is 16-byte aligned)
__host__ __device__ inline size_t gu_lds_bytes(int nbh, int E) {
  return 8 * (size_t)((E + 1) & ~1) + 4 * ((size_t)act_row_dwords(nbh) + 2 * (size_t)nbh + (size_t)E);
}

__device__ __forceinline__ GuLds gu_lds(uint8_t* dyn, int nbh, int E) {
  GuLds l;
  l.key = reinterpret_cast<uint64_t*>(dyn);
  l.qa = reinterpret_cast<uint32_t*>(l.key + ((E + 1) & ~1));
  l.da = reinterpret_cast<float*>(l.qa + act_row_dwords(nbh));
  l.sa = reinterpret_cast<int32_t*>(l.da + nbh);
  l.logit = reinterpret_cast<float*>(l.sa + nbh);
  return l;
}

// Stages x's q8 blocks into LDS and, for a routed slot, finishes the router:
// ids_l / vals_l receive the chosen experts and their logits.  Ends with a
// barrier.
__device__ void decode_gu_prologue(const DecodeArgs& a, const GuLds& l, int P, bool route,
                                   int* ids_l, float* vals_l, bool publish) {
  const int tid = threadIdx.x, nt = blockDim.x, E = a.E;
  const int nbh = a.H / BLK, nc = nbh;
  const int m = (int)next_pow2_u32((uint32_t)nc);
  const int L = m / P;
  // one memory round trip: x's codes, and each thread's first leaf run and bias
  const bool stg = tid < nbh;             // nbh <= blockDim.x by the launch shape
  uint4 q0 = {0, 0, 0, 0}, q1 = {0, 0, 0, 0};
  float dv = 0.0f;
  int32_t sv = 0;
  if (stg) {
    const uint4* src = reinterpret_cast<const uint4*>(a.qx) + 2 * tid;
    q0 = src[0];
    q1 = src[1];
    dv = a.dx[tid];
    sv = a.sx[tid];
  }
  const int items = E * P;                // item = e * P + p
  float lv = 0.0f, bv = 0.0f;
  if (route && tid < items) {
    const int e = tid / P, p = tid % P;
    lv = leaf_tree(a.partials + e, E, p * L, L, nc);
    if (a.bias) bv = a.bias[e];
  }
  if (stg) {
    uint4* dst = reinterpret_cast<uint4*>(l.qa + act_off(tid));
    dst[0] = q0;
    dst[1] = q1;
    l.da[tid] = dv;
    l.sa[tid] = sv;
  }
  if (!route) {
    __syncthreads();
    return;
  }
  // logits and order keys; the loop is uniform over the block (shuffles)
  for (int b0 = 0; b0 < items; b0 += nt) {
    const int it = b0 + tid;
    const bool ok = it < items;
    const int e = it / P, p = it % P;
    if (b0 > 0 && ok) {
      lv = leaf_tree(a.partials + e, E, p * L, L, nc);
      if (a.bias) bv = a.bias[e];
    }
    for (int o = 1; o < P; o <<= 1) lv = lv + __shfl_xor(lv, o, 64);
    if (ok && p == 0) {
      const float lg = a.bias ? lv + bv : lv;
      l.logit[e] = lg;
      l.key[e] = rank_key(lg, e);
      if (publish && a.t_logits) a.t_logits[e] = lg;
    }
  }
  __syncthreads();
  rank_topk(l.key, l.logit, E, a.k, ids_l, vals_l);
}

// h = silu(g) * u of the block's 32-group from val[0..31] (gate) and
// val[32..63] (up), then its q8; block 0 also publishes ids and weights.
// Called by every thread after the barrier that completes val.
__device__ __forceinline__ void gu_epilogue(const DecodeArgs& a, const float* val, int slot, int i0,
                                            bool publish, const int* ids_l, const float* vals_l,
                                            float* ex_l) {
  const int tid = threadIdx.x, I = a.I;
  if (tid < DGU_ROWS) {                   // h of one 32-group, then its q8
    const float h = silu_p(val[tid]) * val[DGU_ROWS + tid];
    float amax = fabsf(h);
#pragma unroll
    for (int m = 1; m < BLK; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, BLK));
    const float d = amax / 127.0f;
    const int q = (d == 0.0f) ? 0 : (int)roundf(h / d);
    int sum = q;
#pragma unroll
    for (int m = 1; m < BLK; m <<= 1) sum += __shfl_xor(sum, m, BLK);
    const size_t hi = (size_t)slot * I + i0 + tid;
    a.qh[hi] = (int8_t)q;
    if (a.t_qh) a.t_qh[hi] = (int8_t)q;
    if (tid == 0) {
      const size_t g = hi / BLK;
      a.dh[g] = d;
      a.sh[g] = sum;
      if (a.t_dh) a.t_dh[g] = d;
    }
  }
  if (publish) {                          // w_s = e_s / ((e_0 + e_1) + ...), e_s = exp(l_s - l_0)
    if (tid < a.k) ex_l[tid] = exp_p(vals_l[tid] - vals_l[0]);
    __syncthreads();
    if (tid < a.k) {
      float S = ex_l[0];
      for (int s = 1; s < a.k; s++) S = S + ex_l[s];
      const float wv = ex_l[tid] / S;
      a.ids[tid] = ids_l[tid];
      a.w[tid] = wv;
      if (a.t_ids) a.t_ids[tid] = ids_l[tid];
      if (a.t_w) a.t_w[tid] = wv;
    }
  }
}

template <int BPL, bool FAST, int FMT>
__global__ void __launch_bounds__(1024) decode_gateup_kernel(DecodeArgs a, int lpr, int P) {
  extern __shared__ __align__(16) uint8_t dyn[];
  const int H = a.H, I = a.I, nbh = H / BLK;
  const GuLds l = gu_lds(dyn, nbh, a.E);
  __shared__ float val[2 * DGU_ROWS];
  __shared__ int ids_l[32];
  __shared__ float vals_l[32], ex_l[32];
  const int tid = threadIdx.x;
  const int ngrp = I / DGU_ROWS, j = blockIdx.x;
  const int slot = j / ngrp, gx = j % ngrp, i0 = gx * DGU_ROWS;
  const bool publish = j == 0;
  decode_gu_prologue(a, l, P, slot < a.k, ids_l, vals_l, publish);

  const int row = tid / lpr, lr = tid % lpr;
  const bool is_up = row >= DGU_ROWS;
  const int i = i0 + (row % DGU_ROWS);
  const size_t rb = (size_t)nbh * WFmt<FMT>::bytes;
  const uint8_t* base;
  if (slot < a.k) {                      // (clamped: a NaN logit leaves ranks unfilled)
    const int e = min(max(ids_l[slot], 0), a.E - 1);
    base = (is_up ? a.w_up : a.w_gate) + ((size_t)e * I + i) * rb;
  } else {
    base = (is_up ? a.s_up : a.s_gate) + (size_t)i * rb;
  }
  auto act = [&](int b) {
    ActBlock A;
    const uint4* q = reinterpret_cast<const uint4*>(l.qa + act_off(b));
    const uint4 u0 = q[0], u1 = q[1];
    A.a[0] = u0.x; A.a[1] = u0.y; A.a[2] = u0.z; A.a[3] = u0.w;
    A.a[4] = u1.x; A.a[5] = u1.y; A.a[6] = u1.z; A.a[7] = u1.w;
    A.d = l.da[b];
    A.s = l.sa[b];
    return A;
  };
  float v = wxa8_lane<BPL, FAST, FMT>(base, nbh, lr * BPL, act, nullptr);
  v = wave_tree_sum(v, lpr);
  if (lr == 0) val[row] = v;
  __syncthreads();
  gu_epilogue(a, val, slot, i0, publish, ids_l, vals_l, ex_l);
}

// Gate/up over the tile-order copies (Q4_0 or Q8_0, H % 64 == 0; layouts at
// q4_tile and q8w_tile in moe_q4.h).  Same blocks, prologue and epilogue as
// decode_gateup_kernel.  The block's W waves split the row's m =
// next_pow2(H/32) blocks (+0 leaves past H/32) into W aligned runs of 2*SP
// blocks, SP tile pieces per wave: in piece s, lane l holds block 2s + l/32
// of row l%32 of the gate group and of the up group -- one 16-byte (Q8_0:
// two) and one 2-byte load per lane and matrix, consecutive lanes on
// consecutive addresses (a row-major span load touches 64 cache lines per
// instruction).  The sums follow the row's pairwise tree:
// blocks 2s and 2s+1 (lanes l and l^32) first, then the lane's pieces
// pairwise (CH pieces loaded together, then the chunk sums), then the W wave
// sums pairwise.
constexpr int kGtWaves = 16, kGtRouteThreads = 512;

template <int SP, int FMT>
__global__ void __launch_bounds__(1024) decode_gateup_tiled_kernel(DecodeArgs a, int P) {
  using TF = TileFmt<FMT>;
  extern __shared__ __align__(16) uint8_t dyn[];
  constexpr int CHM = FMT == kQ4 ? 4 : 2;  // pieces whose loads are issued together
  constexpr int CH = SP < CHM ? SP : CHM;
  constexpr int NCH = SP / CH;
  const int H = a.H, I = a.I, nbh = H / BLK, nsteps = H / 64;
  const GuLds l = gu_lds(dyn, nbh, a.E);
  __shared__ float val[2 * DGU_ROWS];
  __shared__ float wsum[16][2 * DGU_ROWS];
  __shared__ int ids_l[32];
  __shared__ float vals_l[32], ex_l[32];
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), W = blockDim.x / 64;
  const int ngrp = I / DGU_ROWS, j = blockIdx.x;
  const int slot = j / ngrp, gx = j % ngrp, i0 = gx * DGU_ROWS;
  const bool publish = j == 0;
  decode_gu_prologue(a, l, P, slot < a.k, ids_l, vals_l, publish);

  const size_t gbytes = (size_t)DGU_ROWS * nbh * WFmt<FMT>::bytes;   // one 32-row group
  const uint8_t* gb;
  const uint8_t* ub;
  if (slot < a.k) {                      // (clamped: a NaN logit leaves ranks unfilled)
    const size_t G = (size_t)min(max(ids_l[slot], 0), a.E - 1) * ngrp + gx;
    gb = a.t_gate + G * gbytes;
    ub = a.t_up + G * gbytes;
  } else {
    gb = a.ts_gate + (size_t)gx * gbytes;
    ub = a.ts_up + (size_t)gx * gbytes;
  }
  const int half = lane >> 5;
  float cg[NCH], cu[NCH];
#pragma unroll
  for (int c = 0; c < NCH; c++) {
    TileCodes<FMT> gn[CH], un[CH];
    uint32_t gs[CH], us[CH];
    // every load unconditional (pieces past the row re-read its last piece
    // and are zeroed below): branches around loads make each piece wait
    // for the one before
#pragma unroll
    for (int q = 0; q < CH; q++) {
      const size_t o = (size_t)min(wave * SP + c * CH + q, nsteps - 1) * TF::piece;
      gn[q] = tile_codes<FMT>(gb + o + TF::code * lane);
      un[q] = tile_codes<FMT>(ub + o + TF::code * lane);
    }
#pragma unroll
    for (int q = 0; q < CH; q++) {
      const size_t o = (size_t)min(wave * SP + c * CH + q, nsteps - 1) * TF::piece;
      gs[q] = *reinterpret_cast<const uint16_t*>(gb + o + TF::scale + 2 * lane);
      us[q] = *reinterpret_cast<const uint16_t*>(ub + o + TF::scale + 2 * lane);
    }
    float gv[CH], uv[CH];
#pragma unroll
    for (int q = 0; q < CH; q++) {
      const int st = wave * SP + c * CH + q;
      const int b = 2 * min(st, nsteps - 1) + half;
      const uint4* qa = reinterpret_cast<const uint4*>(l.qa + act_off(b));
      const uint4 a0 = qa[0], a1 = qa[1];
      const uint32_t av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float da = l.da[b];
      const int32_t sa = l.sa[b];
      const int32_t dg = tile_dot<FMT>(gn[q], av, sa);
      const int32_t du = tile_dot<FMT>(un[q], av, sa);
      const bool ok = st < nsteps;
      gv[q] = ok ? (f16_bits_to_f32(gs[q]) * da) * (float)dg : 0.0f;
      uv[q] = ok ? (f16_bits_to_f32(us[q]) * da) * (float)du : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < CH; q++) {        // blocks 2s and 2s+1
      gv[q] = gv[q] + __shfl_xor(gv[q], 32, 64);
      uv[q] = uv[q] + __shfl_xor(uv[q], 32, 64);
    }
    cg[c] = reg_tree<CH>(gv);
    cu[c] = reg_tree<CH>(uv);
  }
  const float tg = reg_tree<NCH>(cg), tu = reg_tree<NCH>(cu);
  if (lane < DGU_ROWS) {
    wsum[wave][lane] = tg;
    wsum[wave][DGU_ROWS + lane] = tu;
  }
  __syncthreads();
  if (tid < 2 * DGU_ROWS) {               // the W wave sums, pairwise
    float t[16];
#pragma unroll
    for (int w = 0; w < 16; w++) t[w] = w < W ? wsum[w][tid] : 0.0f;
#pragma unroll
    for (int n = 16; n > 1; n >>= 1)
      if (n <= W) {
#pragma unroll
        for (int i = 0; i < n / 2; i++) t[i] = t[2 * i] + t[2 * i + 1];
      }
    val[tid] = t[0];
  }
  __syncthreads();
  gu_epilogue(a, val, slot, i0, publish, ids_l, vals_l, ex_l);
}

// ---------------------------------------------------------------- down + combine
// Block: `rows` output rows x ns slots, LPR lanes per (row, slot).  ALDS:
// every slot's q8(h) staged in LDS; otherwise read from the workspace.
template <int BPL, bool FAST, bool ALDS, int FMT>
__global__ void __launch_bounds__(1024) decode_down_kernel(DecodeArgs a, int lpr, int rows) {
  extern __shared__ __align__(16) uint8_t dyn[];
  const int H = a.H, I = a.I, nbi = I / BLK;
  const int ns = a.k + (a.has_shared ? 1 : 0);
  const int SS = act_row_dwords(nbi);
  const size_t nact = ALDS ? (size_t)ns * SS + 2 * (size_t)ns * nbi : 0;
  uint32_t* qh_l = reinterpret_cast<uint32_t*>(dyn);                     // ns * SS dwords
  float* dh_l = reinterpret_cast<float*>(qh_l + (size_t)ns * SS);         // ns * nbi
  int32_t* sh_l = reinterpret_cast<int32_t*>(dh_l + (size_t)ns * nbi);    // ns * nbi
  float* o_l = reinterpret_cast<float*>(dyn) + nact;                      // rows * ns
  __shared__ float w_l[32];
  const int tid = threadIdx.x;
  const int r0 = blockIdx.x * rows;
  const int item = tid / lpr, lr = tid % lpr;
  const int rl = item / ns, slot = item % ns;
  const int r = r0 + rl;
  const bool live = rl < rows && r < H;
  constexpr int QB = WFmt<FMT>::bytes;
  const size_t rb = (size_t)nbi * QB;
  // Straight-line loads, none behind a branch or in a loop (either makes
  // the compiler wait for loads issued earlier): the expert id first (lanes
  // past the block's rows mirror a valid row; their results are unused),
  // the routing weights and this thread's first q8(h) group, then the
  // weight span, then the LDS stores.
  const int rc = min(r, H - 1);
  const int eid = a.ids[min(slot, a.k - 1)];
  const float wr = a.w[min(tid, a.k - 1)];
  const int nq = ALDS ? ns * nbi : 0;
  const int g0 = min(tid, max(nq - 1, 0));
  uint4 h0 = make_uint4(0, 0, 0, 0), h1 = make_uint4(0, 0, 0, 0);
  float hd = 0.0f;
  int32_t hs = 0;
  if constexpr (ALDS) {
    h0 = reinterpret_cast<const uint4*>(a.qh)[2 * (size_t)g0];
    h1 = reinterpret_cast<const uint4*>(a.qh)[2 * (size_t)g0 + 1];
    hd = a.dh[g0];
    hs = a.sh[g0];
  }
  const uint8_t* base = (slot < a.k) ? a.w_down + ((size_t)min(max(eid, 0), a.E - 1) * H + rc) * rb
                                     : a.s_down + (size_t)rc * rb;
  // this lane's weight span into registers (fast shapes; a lane of padding
  // leaves, lr * BPL >= nbi, re-reads the row's last span and is zeroed in
  // the row program)
  constexpr int NV = FAST ? QB * BPL / 16 : 1;
  uint32_t D[4 * NV + 1] = {};
  if constexpr (FAST) {
    const int lrc = min(lr, nbi / BPL - 1);
    const uint4* src = reinterpret_cast<const uint4*>(base + (size_t)lrc * BPL * QB);
#pragma unroll
    for (int v = 0; v < NV; v++) {
      const uint4 t = src[v];
      D[4 * v] = t.x; D[4 * v + 1] = t.y; D[4 * v + 2] = t.z; D[4 * v + 3] = t.w;
    }
  }
  D[4 * NV] = 0u;
  // every slot's q8(h) into LDS
  if (ALDS && tid < nq) {
    uint4* dst = reinterpret_cast<uint4*>(qh_l + (size_t)(tid / nbi) * SS + act_off(tid % nbi));
    dst[0] = h0;
    dst[1] = h1;
    dh_l[tid] = hd;
    sh_l[tid] = hs;
  }
  for (int g = tid + (int)blockDim.x; ALDS && g < nq; g += blockDim.x) {    // wide rows only
    const int s = g / nbi, b = g % nbi;
    const uint4* src = reinterpret_cast<const uint4*>(a.qh) + 2 * (size_t)g;
    uint4* dst = reinterpret_cast<uint4*>(qh_l + (size_t)s * SS + act_off(b));
    dst[0] = src[0];
    dst[1] = src[1];
    dh_l[g] = a.dh[g];
    sh_l[g] = a.sh[g];
  }
  if (tid < a.k) w_l[tid] = wr;
  __syncthreads();
  float v = 0.0f;
  if (live) {
    const uint32_t* qs = qh_l + (size_t)slot * SS;
    const uint4* qg = reinterpret_cast<const uint4*>(a.qh) + 2 * (size_t)slot * nbi;
    auto act = [&](int b) {
      ActBlock A;
      const uint4* q = ALDS ? reinterpret_cast<const uint4*>(qs + act_off(b)) : qg + 2 * b;
      const uint4 u0 = q[0], u1 = q[1];
      A.a[0] = u0.x; A.a[1] = u0.y; A.a[2] = u0.z; A.a[3] = u0.w;
      A.a[4] = u1.x; A.a[5] = u1.y; A.a[6] = u1.z; A.a[7] = u1.w;
      A.d = ALDS ? dh_l[slot * nbi + b] : a.dh[slot * nbi + b];
      A.s = ALDS ? sh_l[slot * nbi + b] : a.sh[slot * nbi + b];
      return A;
    };
    if constexpr (FAST) v = wxa8_regs<BPL, FMT>(D, nbi, lr * BPL, act);
    else v = wxa8_lane<BPL, false, FMT>(base, nbi, lr * BPL, act, nullptr);
  }
  v = wave_tree_sum(v, lpr);
  if (live && lr == 0) o_l[rl * ns + slot] = v;
  __syncthreads();
  if (tid < rows && r0 + tid < H) {
    const float* o = o_l + tid * ns;
    float acc = w_l[0] * o[0];
    for (int s = 1; s < a.k; s++) acc = acc + w_l[s] * o[s];
    if (a.has_shared) acc = acc + o[a.k];
    a.y[r0 + tid] = acc;
  }
}

// Down + combine over the tile-order copies (Q4_0 or Q8_0, I % 64 == 0;
// layouts at q4_tile and q8w_tile in moe_q4.h).  Block: 8 output rows r0..r0+7 (inside one 32-row
// group) x every slot; wave w serves slots 4w..4w+3.  In piece s of a
// slot's row group, lane L = 32*half + 8*g + rr loads the piece lane
// 32*half + (r0 % 32) + rr of slot 4w+g: block 2s + half of row r0 + rr,
// so one load instruction reads 8 runs of 128 contiguous bytes.  Every lane
// covers the whole row (the padded m = next_pow2(I/32) blocks: SP = m/2
// pieces, +0 leaves past I/32); the sums follow the row's pairwise tree:
// blocks 2s and 2s+1 (lanes L and L^32) first, then the pieces pairwise
// (CH loaded together, then the chunk sums).  Then the fixed-order combine.
template <int SP, int FMT>
__global__ void __launch_bounds__(1024) decode_down_tiled_kernel(DecodeArgs a) {
  using TF = TileFmt<FMT>;
  extern __shared__ __align__(16) uint8_t dyn[];
  constexpr int CHM = FMT == kQ4 ? 8 : 4;  // pieces whose loads are issued together
  constexpr int CH = SP < CHM ? SP : CHM;
  constexpr int NCH = SP / CH;
  const int H = a.H, I = a.I, nbi = I / BLK, nsteps = I / 64;
  const int ns = a.k + (a.has_shared ? 1 : 0);
  const int SS = act_row_dwords(nbi);
  uint32_t* qh_l = reinterpret_cast<uint32_t*>(dyn);                     // ns * SS dwords
  float* dh_l = reinterpret_cast<float*>(qh_l + (size_t)ns * SS);         // ns * nbi
  int32_t* sh_l = reinterpret_cast<int32_t*>(dh_l + (size_t)ns * nbi);    // ns * nbi
  __shared__ float o_l[kDtRows * 33];
  __shared__ float w_l[32];
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  // The four blocks of a 32-row group share each piece's scale line: keep
  // them on one XCD (blocks are dealt to the 8 XCDs round robin) so that
  // line comes from HBM once.  b = 32*(G/8) + 8*quarter + G%8 when H/32 is
  // a multiple of 8; otherwise blocks in order.
  const int bx = blockIdx.x;
  const int r0 = (H % 256 == 0) ? 32 * (8 * (bx / 32) + bx % 8) + kDtRows * ((bx / 8) % 4) : bx * kDtRows;
  const int half = lane >> 5, g = (lane >> 3) & 3, rr = lane & 7;
  const int slot = 4 * wave + g;
  const bool live = slot < ns;
  const int sl = live ? slot : ns - 1;    // lanes past the last slot mirror it (results unused)
  // Straight-line loads, none behind a branch or in a loop (either makes
  // the compiler wait for loads issued earlier): the expert id first, then
  // the routing weights and this thread's first q8(h) group; once the id
  // is in, the first chunk of weights; then the LDS stores.
  const int eid = a.ids[min(sl, a.k - 1)];
  const float wr = a.w[min(tid, a.k - 1)];
  const int nact = ns * nbi;
  const int i0 = min(tid, nact - 1);
  const uint4 h0 = reinterpret_cast<const uint4*>(a.qh)[2 * (size_t)i0];
  const uint4 h1 = reinterpret_cast<const uint4*>(a.qh)[2 * (size_t)i0 + 1];
  const float hd = a.dh[i0];
  const int32_t hs = a.sh[i0];
  const size_t gbytes = (size_t)nsteps * TF::piece;                      // one 32-row group
  const int pl = 32 * half + (r0 % 32) + rr;                             // lane inside a piece
  const size_t G = (size_t)(r0 / 32);
  const uint8_t* base = (sl < a.k) ? a.t_down + ((size_t)min(max(eid, 0), a.E - 1) * (H / 32) + G) * gbytes
                                   : a.ts_down + G * gbytes;
  // pieces past the row re-read its last piece and are zeroed below
  TileCodes<FMT> wn[CH];
  uint32_t ws[CH];
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int q = 0; q < CH; q++)
      wn[q] = tile_codes<FMT>(base + (size_t)min(c * CH + q, nsteps - 1) * TF::piece + TF::code * pl);
#pragma unroll
    for (int q = 0; q < CH; q++)
      ws[q] = *reinterpret_cast<const uint16_t*>(base + (size_t)min(c * CH + q, nsteps - 1) * TF::piece + TF::scale + 2 * pl);
  };
  load_chunk(0);
  if (tid < nact) {                       // every slot's q8(h) into LDS
    uint4* dst = reinterpret_cast<uint4*>(qh_l + (size_t)(tid / nbi) * SS + act_off(tid % nbi));
    dst[0] = h0;
    dst[1] = h1;
    dh_l[tid] = hd;
    sh_l[tid] = hs;
  }
  for (int i = tid + (int)blockDim.x; i < nact; i += blockDim.x) {      // wide rows only
    const uint4* src = reinterpret_cast<const uint4*>(a.qh) + 2 * (size_t)i;
    uint4* dst = reinterpret_cast<uint4*>(qh_l + (size_t)(i / nbi) * SS + act_off(i % nbi));
    dst[0] = src[0];
    dst[1] = src[1];
    dh_l[i] = a.dh[i];
    sh_l[i] = a.sh[i];
  }
  if (tid < a.k) w_l[tid] = wr;
  __syncthreads();
  const uint32_t* qs = qh_l + (size_t)sl * SS;
  float cs[NCH];
#pragma unroll
  for (int c = 0; c < NCH; c++) {
    if (c > 0) load_chunk(c);
    float v[CH];
#pragma unroll
    for (int q = 0; q < CH; q++) {
      const int st = c * CH + q;
      const int b = 2 * min(st, nsteps - 1) + half;
      const uint4* qa = reinterpret_cast<const uint4*>(qs + act_off(b));
      const uint4 a0 = qa[0], a1 = qa[1];
      const uint32_t av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const int32_t dot = tile_dot<FMT>(wn[q], av, sh_l[sl * nbi + b]);
      v[q] = st < nsteps ? (f16_bits_to_f32(ws[q]) * dh_l[sl * nbi + b]) * (float)dot : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < CH; q++) v[q] = v[q] + __shfl_xor(v[q], 32, 64);   // blocks 2s and 2s+1
    cs[c] = reg_tree<CH>(v);
  }
  const float o = reg_tree<NCH>(cs);
  if (live && half == 0) o_l[rr * 33 + slot] = o;
  __syncthreads();
  if (tid < kDtRows && r0 + tid < H) {
    const float* ov = o_l + tid * 33;
    float acc = w_l[0] * ov[0];
    for (int s = 1; s < a.k; s++) acc = acc + w_l[s] * ov[s];
    if (a.has_shared) acc = acc + ov[a.k];
    a.y[r0 + tid] = acc;
  }
}

// ---------------------------------------------------------------- launch
DecodeGeometry decode_geometry(int H, int I, int E, int k, int has_shared) {
  DecodeGeometry g;
  const int ns = k + (has_shared ? 1 : 0);
  g.router_threads = (E + 63) / 64 * 64;
  const RowSplit gu = row_split(H, 16);
  g.gu_lpr = gu.lpr;
  g.gu_bpl = gu.bpl;
  g.gu_fast = (gu.bpl % 8 == 0) && (gu.nb % gu.bpl == 0);
  g.gu_threads = 2 * DGU_ROWS * gu.lpr;
  const int nc = H / BLK;
  int m = 1;
  while (m < nc) m <<= 1;
  // lanes per expert: as many as the block allows (<= 64, <= m), at least
  // enough for runs of <= 32 leaves
  int P = 1;
  while (P < 64 && P < m && E * P * 2 <= g.gu_threads) P <<= 1;
  while (m / P > 32) P <<= 1;
  g.gu_parts = P;
  g.gu_lds = gu_lds_bytes(nc, E);
  // tile-order gate/up: W = min(kGtWaves, m/2) waves of SP = m / (2W)
  // pieces.  The router finish keeps the lane split of a kGtRouteThreads
  // block: more lanes per expert make its leaf loads less coalesced.
  g.gt_sp = 0;
  g.gt_threads = 0;
  g.gt_parts = 0;
  if (H % 64 == 0) {
    const int W = m / 2 < kGtWaves ? m / 2 : kGtWaves;
    g.gt_threads = 64 * W;
    const int rt = g.gt_threads < kGtRouteThreads ? g.gt_threads : kGtRouteThreads;
    int Pt = 1;
    while (Pt < 64 && Pt < m && E * Pt * 2 <= rt) Pt <<= 1;
    while (m / Pt > 32) Pt <<= 1;
    g.gt_parts = Pt;
    g.gt_sp = m / (2 * W) <= 16 ? m / (2 * W) : 0;
  }
  const RowSplit dn = row_split(I, 16);
  g.dn_lpr = dn.lpr;
  g.dn_bpl = dn.bpl;
  g.dn_fast = (dn.bpl % 8 == 0) && (dn.nb % dn.bpl == 0);
  const int per_row = ns * dn.lpr;
  g.dn_rows = 256 / per_row < 1 ? 1 : 256 / per_row;
  g.dn_threads = (g.dn_rows * per_row + 63) / 64 * 64;
  const int nbi = I / BLK;
  const size_t act = 4 * ((size_t)ns * act_row_dwords(nbi) + 2 * (size_t)ns * nbi);
  const size_t out = 4 * (size_t)g.dn_rows * ns;
  g.dn_act_lds = act + out <= kDecodeLdsMax;
  g.dn_lds = (g.dn_act_lds ? act : 0) + out;
  // tile-order down: SP = m/2 pieces per lane, every slot's q8(h) in LDS
  g.dt_sp = 0;
  g.dt_threads = 64 * ((ns + 3) / 4);
  g.dt_lds = act;
  {
    int md = 1;
    while (md < nbi) md <<= 1;
    if (I % 64 == 0 && H % 64 == 0 && md / 2 <= 32 && act <= kDecodeLdsMax) g.dt_sp = md / 2;
  }
  return g;
}

// gate/up and down launches for one weight format
template <int FMT>
hipError_t launch_decode_experts(const DecodeArgs& a, const DecodeGeometry& g, hipStream_t stream) {
  hipError_t err = hipSuccess;
  const int ns = a.k + (a.has_shared ? 1 : 0);
  if (g.gt_sp > 0 && a.t_gate && a.t_up && (!a.has_shared || (a.ts_gate && a.ts_up))) {
    dim3 grid(a.I / DGU_ROWS * ns);
    dim3 block(g.gt_threads);
#define MOEQ4_GT(SPV) \
  hipLaunchKernelGGL((decode_gateup_tiled_kernel<SPV, FMT>), grid, block, g.gu_lds, stream, a, g.gt_parts)
    switch (g.gt_sp) {
      case 1: MOEQ4_GT(1); break;
      case 2: MOEQ4_GT(2); break;
      case 4: MOEQ4_GT(4); break;
      case 8: MOEQ4_GT(8); break;
      default: MOEQ4_GT(16); break;
    }
#undef MOEQ4_GT
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  } else {
    dim3 grid(a.I / DGU_ROWS * ns);
    dim3 block(g.gu_threads);
#define MOEQ4_GU(B, F) \
  hipLaunchKernelGGL((decode_gateup_kernel<B, F, FMT>), grid, block, g.gu_lds, stream, a, g.gu_lpr, g.gu_parts)
    if (g.gu_fast) {
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
#undef MOEQ4_GU
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (g.dt_sp > 0 && a.t_down && (!a.has_shared || a.ts_down)) {
    dim3 grid(a.H / kDtRows);
    dim3 block(g.dt_threads);
#define MOEQ4_DT(SPV) \
  hipLaunchKernelGGL((decode_down_tiled_kernel<SPV, FMT>), grid, block, g.dt_lds, stream, a)
    switch (g.dt_sp) {
      case 1: MOEQ4_DT(1); break;
      case 2: MOEQ4_DT(2); break;
      case 4: MOEQ4_DT(4); break;
      case 8: MOEQ4_DT(8); break;
      case 16: MOEQ4_DT(16); break;
      default: MOEQ4_DT(32); break;
    }
#undef MOEQ4_DT
    err = hipGetLastError();
  } else {
    dim3 grid((a.H + g.dn_rows - 1) / g.dn_rows);
    dim3 block(g.dn_threads);
#define MOEQ4_DN(B, F)                                                                     \
  do {                                                                                     \
    if (g.dn_act_lds)                                                                      \
      hipLaunchKernelGGL((decode_down_kernel<B, F, true, FMT>), grid, block, g.dn_lds, stream, a, \
                         g.dn_lpr, g.dn_rows);                                            \
    else                                                                                   \
      hipLaunchKernelGGL((decode_down_kernel<B, F, false, FMT>), grid, block, g.dn_lds, stream, a, \
                         g.dn_lpr, g.dn_rows);                                            \
  } while (0)
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

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const DecodeGeometry g = decode_geometry(a.H, a.I, a.E, a.k, a.has_shared);
  const int nc = a.H / BLK;
  hipLaunchKernelGGL(decode_router_kernel, dim3(nc), dim3(g.router_threads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return a.wfmt == kQ8 ? launch_decode_experts<kQ8>(a, g, stream) : launch_decode_experts<kQ4>(a, g, stream);
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
