// decode_fused.hip -- the single-token decode step of the Q4_0 MoE layer in
// ONE launch.
//
// "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU",
// technical summary, Methodology 1 and Key Contribution 2: single tokens go
// through a W4A8 integer kernel over 4-bit weights.  The arithmetic is the
// pinned program of decode.hip (the same router tree, top-k by rank, W4A8 row
// program, silu, q8(h) and combine), so y is bit-identical to the
// three-launch path; what changes is how the step's dependent pieces meet.
// A batch-1 step moves 17 MB, a few microseconds at HBM speed, behind a chain
// of dependent steps (router -> expert choice -> gate/up -> down); between
// launches each link costs a launch gap plus the next kernel's first memory
// round trip.  Here every link is one tagged-word handoff inside one launch.
//
// Block roles (every block kFuThreads threads; index ranges in launch order,
// so producers are dispatched before their consumers):
//   [0, nR)            router: the chunk chains of cpb consecutive 32-chunks
//                      of x for every expert (leaves of the pinned tree),
//                      summed pairwise into one subtree value per expert and
//                      published.
//   [base_gu, +n_gu)   gate/up unit (slot, 32 values of i): q8(x) from x
//                      itself; a routed slot's unit waits for the router's
//                      words and finishes the tree, the logits, the top-k and
//                      (unit 0, which publishes them) the weights; then the
//                      32 gate and 32 up rows, h = silu(g) * u and its q8,
//                      published.  The shared expert's units wait for nothing.
//   [base_dn, +n_dn)   down unit (8 output rows): waits for ids and weights,
//                      loads its weight pieces, waits for every slot's q8(h),
//                      then the row program and the fixed-order combine.
//
// Handoff words: 64 bits, (mark << 32) | payload with mark = tag ^ hash(payload),
// stored and loaded with relaxed device-scope atomics (global_store/load_dwordx2
// sc1).  One access carries mark and payload together, so a reader that sees
// this call's mark sees the payload stored with it: no fences and no cache
// writeback.  The tag
// is the call's epoch + 1.  The epoch lives in kFuSlots per-block slots of
// the workspace header, all equal between calls: block b reads slot b at its
// start and, at its end, stores epoch + 1 into slots b, b + n, b + 2n, ...
// (n = the grid), so every slot advances once per call whatever the grid, and
// no two blocks touch one address (a shared counter would serialise every
// block's start on one atomic).  The slots must be zero before the first call
// on a workspace.  Every wait is bounded; a wait that gives up counts itself
// in the header's failure word (read back by moe_q4_decode_status) and
// continues with zeros.
#include <string.h>

#include <mutex>

#include "launch.hpp"
#include "w4a8.hpp"
#include "decode_common.hpp"
#include "decode_tile.hpp"

namespace moeq4 {

constexpr int kFuThreads = 512;
constexpr int kFuWaves = kFuThreads / 64;
constexpr int kFuSpinMax = 1 << 20;   // polls of one wait (about half a second) before it gives up
constexpr int kFuQhWords = 10;        // words per published 32-group of q8(h): 8 code dwords, d, code sum
constexpr int kFuMaxSlots = 12;       // slots (k + shared) the one-launch step covers
// test only: waits look for tag + kFuTestTag, which no word of this or a
// neighbouring call or layer carries
constexpr uint32_t kFuTestTag = 0x40000000u;

// A word's high half is the tag mixed with a multiplicative hash of its
// payload, so bytes a workspace held before (other layers' or other paths'
// data) pass as this call's word with probability ~2^-32; a zero word never
// does (tags are >= 1).
__device__ __forceinline__ uint32_t ll_mark(uint32_t tag, uint32_t v) { return tag ^ (v * 0x9E3779B1u); }
__device__ __forceinline__ bool ll_ready(uint64_t w, uint32_t tag) {
  return (uint32_t)(w >> 32) == ll_mark(tag, (uint32_t)w);
}

__device__ __forceinline__ uint64_t ll_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void ll_store(uint64_t* p, uint32_t tag, uint32_t v) {
  __hip_atomic_store(p, ((uint64_t)ll_mark(tag, v) << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Header: [0] failure count (low 32 bits), [1 .. kFuSlots] the epoch slots.
__device__ __forceinline__ void fu_fail(const DecodeArgs& a) {
  __hip_atomic_fetch_add(reinterpret_cast<uint32_t*>(a.hdr), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits for the words base[i * stride], i < n (N >= n; words i >= n count as
// payload 0), every load issued before the first check.  Returns false if the
// bound ran out (the words not seen then read 0).  CACHED: the first read is
// a plain load, which may be served by this XCD's L2 (a word that many
// blocks read after its producer's indicator is fetched from memory once per
// XCD); it is only trusted if its mark checks, and the polls after it are
// device-scope loads (a plain load could keep hitting a stale L2 line).
template <int N, bool CACHED = false>
__device__ __forceinline__ bool ll_wait(const uint64_t* base, size_t stride, int n, uint32_t tag,
                                        uint32_t (&val)[N], int spin_max = kFuSpinMax) {
  uint64_t w[N];
  const uint64_t ready = (uint64_t)ll_mark(tag, 0u) << 32;
#pragma unroll
  for (int i = 0; i < N; i++) w[i] = i < n ? (CACHED ? base[i * stride] : ll_load(base + i * stride)) : ready;
  bool all = false;
  for (int it = 0; it <= spin_max; it++) {
    all = true;
#pragma unroll
    for (int i = 0; i < N; i++) all = all && ll_ready(w[i], tag);
    if (all) break;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int i = 0; i < N; i++)
      if (!ll_ready(w[i], tag)) w[i] = ll_load(base + i * stride);
  }
#pragma unroll
  for (int i = 0; i < N; i++) val[i] = ll_ready(w[i], tag) ? (uint32_t)w[i] : 0u;
  return all;
}

// x of a stacked layer after the first: the previous layer's y, handed over
// as one tagged word per value, into LDS xl [H].  Whole block (H % 64 == 0).
// Polls are device-scope loads that cross to memory, and every block of the
// next layer needs all of y: so wave 0 alone polls one word per 8-row group
// (a down unit stores its 8 words with one instruction) until all are there,
// then every thread reads its words once (each checked again).  Every thread
// polling all of its words took ~3 MB of loads per poll round over the grid
// and slowed the producers.
__device__ __forceinline__ void fu_stage_x(const uint64_t* llx, int H, uint32_t tag, float* xl, int spin_max,
                                           bool& ok) {
  if (threadIdx.x < 64) {
    const int ng = H / kDtRows, lane = threadIdx.x;
    for (int g0 = 0; g0 < ng; g0 += 64 * 4) {
      uint32_t v[4];
      const int n = max(0, min(4, (ng - g0 - lane + 63) / 64));
      ok = ll_wait<4>(llx + (size_t)(g0 + lane) * kDtRows, (size_t)64 * kDtRows, n, tag, v, spin_max) && ok;
    }
  }
  __syncthreads();
  for (int i0 = 4 * threadIdx.x; i0 < H; i0 += 4 * blockDim.x) {
    uint32_t v[4];
    ok = ll_wait<4>(llx + i0, 1, 4, tag, v, spin_max) && ok;
#pragma unroll
    for (int j = 0; j < 4; j++) xl[i0 + j] = __uint_as_float(v[j]);
  }
  __syncthreads();
}

// ---------------------------------------------------------------- router role
// Router block r = (expert group eg, chunk group cg): experts e0 = eg * EB ..
// e0 + EB - 1 over chunks c0 = cg * cpb .. c0 + cpb - 1 (chunks >= H/32 are
// +0 leaves).  Pair (chunk cl, expert el) -> the chunk's sequential fused
// chain; then per expert the pairwise tree over the cpb leaves (an aligned
// subtree of the router's tree), published at ll_leaf[cg * E + e].  A wave's
// lanes cover 16 experts of 4 chunks, so a load instruction reads runs of 64
// contiguous bytes of W_r.
// Pairwise tree of the N leaves lf[j * EB + el], j < N.
template <int N>
__device__ __forceinline__ float lds_subtree(const float* lf, int EB, int el) {
  float v[N];
#pragma unroll
  for (int j = 0; j < N; j++) v[j] = lf[j * EB + el];
  return reg_tree<N>(v);
}

// (llx: x comes from the previous stacked layer's words with tag xtag, staged
// in xl, after this block's first router weights are in flight)
__device__ void fu_router(const DecodeArgs& a, const StackLayer& LW, int norm_in, const FusedGeometry& g, int r,
                          const uint32_t* tag_s, uint8_t* dyn, float* part, float* tmp, const uint64_t* llx,
                          uint32_t xtag, float* xl, bool& ok) {
  const int tid = threadIdx.x, E = a.E, nc = a.H / BLK, cpb = g.cpb, EB = g.eb;
  const int eg = r % g.n_eg, cg = r / g.n_eg;
  const int e0 = eg * EB, ne = min(EB, E - e0);
  float* xs = reinterpret_cast<float*>(dyn);          // [cpb * 32]
  float* lf = xs + cpb * BLK;                          // [cpb][EB]
  const int c0 = cg * cpb, np = cpb * EB;
  // the first pair's weights are in flight while x is staged
  float wv[BLK];
  {
    const int p = min(tid, np - 1), cl = p / EB, el = min(p % EB, ne - 1);
    const int c = min(c0 + cl, nc - 1);
    const float* w = LW.w_router + (size_t)c * BLK * E + e0 + el;
#pragma unroll
    for (int i = 0; i < BLK; i++) wv[i] = w[(size_t)i * E];
  }
  const float* X = a.x;
  if (llx) {
    fu_stage_x(llx, a.H, xtag, xl, a.spin_max, ok);
    X = xl;
  }
  if (norm_in) {
    const float rr = rms_scale(X, a.H, a.norm_eps, part, tmp);
    for (int i = tid; i < cpb * BLK; i += blockDim.x)
      xs[i] = (c0 + i / BLK < nc) ? X[c0 * BLK + i] / rr : 0.0f;
  } else {
    for (int i = tid; i < cpb * BLK; i += blockDim.x)
      xs[i] = (c0 + i / BLK < nc) ? X[c0 * BLK + i] : 0.0f;
  }
  __syncthreads();
  const uint32_t tag = *tag_s;
  for (int p = tid; p < np; p += blockDim.x) {
    const int cl = p / EB, el = min(p % EB, ne - 1);
    if (p != tid) {
      const int c = min(c0 + cl, nc - 1);
      const float* w = LW.w_router + (size_t)c * BLK * E + e0 + el;
#pragma unroll
      for (int i = 0; i < BLK; i++) wv[i] = w[(size_t)i * E];
    }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < BLK; i++) acc = __builtin_fmaf(xs[cl * BLK + i], wv[i], acc);
    lf[p] = (c0 + cl < nc) ? acc : 0.0f;
  }
  __syncthreads();
  for (int el = tid; el < ne; el += blockDim.x) {
    float s;
    switch (cpb) {
      case 1: s = lf[el]; break;
      case 2: s = lds_subtree<2>(lf, EB, el); break;
      case 4: s = lds_subtree<4>(lf, EB, el); break;
      case 8: s = lds_subtree<8>(lf, EB, el); break;
      case 16: s = lds_subtree<16>(lf, EB, el); break;
      case 32: s = lds_subtree<32>(lf, EB, el); break;
      default: s = lds_subtree<64>(lf, EB, el); break;
    }
    ll_store(a.ll_leaf + (size_t)cg * E + e0 + el, tag, __float_as_uint(s));
  }
}

// ---------------------------------------------------------------- gate/up role
// Pairwise tree of expert e's L published subtree values r0 .. r0+L-1 (chunk
// groups r >= n_cg are +0), polled together.
template <int L>
__device__ __forceinline__ float ll_leaf_run(const DecodeArgs& a, int ncg, int e, int r0, uint32_t tag, bool& ok) {
  uint32_t u[L];
  const int n = max(0, min(L, ncg - r0));
  ok = ll_wait<L>(a.ll_leaf + (size_t)r0 * a.E + e, (size_t)a.E, n, tag, u, a.spin_max) && ok;
  float v[L];
#pragma unroll
  for (int j = 0; j < L; j++) v[j] = __uint_as_float(u[j]);
#pragma unroll
  for (int w = L; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; i++) v[i] = v[2 * i] + v[2 * i + 1];
  return v[0];
}

__device__ __forceinline__ float ll_leaf_tree(const DecodeArgs& a, int ncg, int L, int e, int r0, uint32_t tag,
                                              bool& ok) {
  switch (L) {
    case 1: return ll_leaf_run<1>(a, ncg, e, r0, tag, ok);
    case 2: return ll_leaf_run<2>(a, ncg, e, r0, tag, ok);
    case 4: return ll_leaf_run<4>(a, ncg, e, r0, tag, ok);
    case 8: return ll_leaf_run<8>(a, ncg, e, r0, tag, ok);
    default: return ll_leaf_run<16>(a, ncg, e, r0, tag, ok);
  }
}

// Top-k by rank (the same selection as rank_topk): the count of keys above
// expert e's own, split over Q key ranges.  Item it: expert e = it % E, range
// q = it / E, so the lanes of a wave share q and read the same key at once
// (an LDS broadcast; lanes on different ranges would hit the same banks);
// eight key pairs in flight at a time.  The Q partial counts meet in LDS.
// Top-k by k rounds of a wave maximum over the order keys, by wave 0 (E / 64
// keys per lane): keys are unique, so round s picks the s-th largest — the
// same experts in the same order as the rank pass — in k DPP reductions
// instead of E comparisons per expert (the faster of the two past 128
// experts).  ids_l / vals_l [k] in LDS; every thread of the block reaches
// the closing barrier.
template <int NJ>
__device__ __forceinline__ void fu_wave_topk_nj(const uint64_t* key, const float* logit, int E, int k,
                                                int* ids_l, float* vals_l) {
  if (threadIdx.x < 64) {                 // (wave 0, whole)
    const int lane = threadIdx.x;
    uint64_t kv[NJ];
#pragma unroll
    for (int j = 0; j < NJ; j++) {
      const int e = lane + 64 * j;
      kv[j] = (e < E) ? key[e] : 0ull;    // (real keys are never 0)
    }
    for (int s = 0; s < k; s++) {
      uint64_t best = kv[0];
#pragma unroll
      for (int j = 1; j < NJ; j++) best = kv[j] > best ? kv[j] : best;
      const uint64_t win = wave_max_u64(best);
      const int we = (int)(0xffffffffu - (uint32_t)win);
#pragma unroll
      for (int j = 0; j < NJ; j++)
        if (kv[j] == win) kv[j] = 0ull;
      if (lane == 0) {
        ids_l[s] = we;
        vals_l[s] = logit[we];
      }
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void fu_wave_topk(const uint64_t* key, const float* logit, int E, int k, int* ids_l,
                                             float* vals_l) {
  const int nj = (E + 63) / 64;
  if (nj <= 1) fu_wave_topk_nj<1>(key, logit, E, k, ids_l, vals_l);
  else if (nj <= 2) fu_wave_topk_nj<2>(key, logit, E, k, ids_l, vals_l);
  else if (nj <= 4) fu_wave_topk_nj<4>(key, logit, E, k, ids_l, vals_l);
  else if (nj <= 8) fu_wave_topk_nj<8>(key, logit, E, k, ids_l, vals_l);
  else fu_wave_topk_nj<16>(key, logit, E, k, ids_l, vals_l);
}

__device__ __forceinline__ void fu_rank_topk(const uint64_t* key, const float* logit, int E, int k,
                                             int* ids_l, float* vals_l, int32_t* rpart) {
  const int tid = threadIdx.x, nt = blockDim.x;
  int Q = 1;                              // Q * E <= nt (one item per thread), Q | E / 2, Q <= 8
  while (Q < 8 && E * Q * 2 <= nt && (E % (Q * 4)) == 0) Q <<= 1;
  const int span = E / Q;
  const ulonglong2* K2 = reinterpret_cast<const ulonglong2*>(key);
  for (int it = tid; it < E * Q; it += nt) {
    const int e = it % E, q = it / E;
    const uint64_t ke = key[e];
    int rank = 0;
    const int j0 = q * span, j1 = j0 + span;
    int j = j0;
    if ((j0 & 1) == 0) {
      for (; j + 16 <= j1; j += 16) {
        ulonglong2 kk[8];
#pragma unroll
        for (int i = 0; i < 8; i++) kk[i] = K2[(j >> 1) + i];
#pragma unroll
        for (int i = 0; i < 8; i++) rank += (kk[i].x > ke ? 1 : 0) + (kk[i].y > ke ? 1 : 0);
      }
    }
    for (; j < j1; j++) rank += key[j] > ke ? 1 : 0;
    rpart[it] = rank;
  }
  __syncthreads();
  for (int e = tid; e < E; e += nt) {
    int rp[8];                            // Q <= 8: every read in flight, then the sum
#pragma unroll
    for (int q = 0; q < 8; q++) rp[q] = rpart[min(q, Q - 1) * E + e];
    int rank = 0;
#pragma unroll
    for (int q = 0; q < 8; q++) rank += q < Q ? rp[q] : 0;
    if (rank < k) {
      ids_l[rank] = e;
      vals_l[rank] = logit[e];
    }
  }
  __syncthreads();
}

// LDS of a gate/up unit: the order keys, x's q8 codes (padded layout), their
// scales and code sums, the logits.
__host__ __device__ inline size_t fu_gu_lds_bytes(int nbh, int E) {
  return 8 * (size_t)((E + 1) & ~1) + 4 * ((size_t)act_row_dwords(nbh) + 2 * (size_t)nbh + (size_t)E);
}

template <int SP, int FMT>
__device__ void fu_gateup(const DecodeArgs& a, const StackLayer& LW, int norm_in, const FusedGeometry& g, int jj,
                          const uint32_t* tag_s, uint8_t* dyn, float* part, float* tmp, const uint64_t* llx,
                          uint32_t xtag, float* xl, bool& ok) {
  using TF = TileFmt<FMT>;
  constexpr int CHM = FMT == kQ4 ? 4 : 2;  // pieces whose loads are issued together
  constexpr int CH = SP < CHM ? SP : CHM;
  constexpr int NCH = SP / CH;
  __shared__ float val[2 * DGU_ROWS];
  __shared__ float wsum[kFuWaves][2 * DGU_ROWS];
  __shared__ int ids_l[32];
  __shared__ float vals_l[32], ex_l[32];
  __shared__ int32_t rpart[1024];
  const int tid = threadIdx.x, lane = tid % 64, nt = blockDim.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int H = a.H, I = a.I, E = a.E, nbh = H / BLK, nsteps = H / 64;
  // units in launch order: the shared expert's first (they wait for
  // nothing), then the routed slots'
  const int ngrp = I / DGU_ROWS, S = a.has_shared ? 1 : 0;
  const int j = jj < S * ngrp ? a.k * ngrp + jj : jj - S * ngrp;
  const int slot = j / ngrp, gx = j % ngrp, i0 = gx * DGU_ROWS;
  const bool routed = slot < a.k, publish = j == 0;
  uint64_t* key = reinterpret_cast<uint64_t*>(dyn);
  uint32_t* qa = reinterpret_cast<uint32_t*>(key + ((E + 1) & ~1));
  float* da = reinterpret_cast<float*>(qa + act_row_dwords(nbh));
  int32_t* sa = reinterpret_cast<int32_t*>(da + nbh);
  float* logit = reinterpret_cast<float*>(sa + nbh);

  // a routed unit with one subtree value per lane (the usual split) issues
  // its first poll of it now, so that round trip overlaps x's
  const bool pre1 = routed && g.L == 1 && E * g.P <= nt;
  uint64_t pre = 0;
  if (pre1 && tid < E * g.P) pre = ll_load(a.ll_leaf + (size_t)(tid % g.P) * E + tid / g.P);
  // q8 of x (x = y / r with the RMSNorm glue): 8 threads per 32-block, 4
  // elements each; amax and the code sum over the 8 threads by shuffles
  {
    const float* X = a.x;
    if (llx) {                            // (a stacked layer after the first)
      fu_stage_x(llx, H, xtag, xl, a.spin_max, ok);
      X = xl;
    }
    float rr = 1.0f;
    if (norm_in) rr = rms_scale(X, H, a.norm_eps, part, tmp);
    for (int t = tid; t < nbh * 8; t += nt) {
      const int c = t / 8, s = t % 8;
      const float4 v4 = *reinterpret_cast<const float4*>(X + c * BLK + 4 * s);
      float v[4] = {v4.x, v4.y, v4.z, v4.w};
      if (norm_in) {
#pragma unroll
        for (int i = 0; i < 4; i++) v[i] = v[i] / rr;
      }
      float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
      for (int m = 1; m < 8; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 8));
      const float d = amax / 127.0f;
      uint32_t packed = 0;
      int sum = 0;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int q = (d == 0.0f) ? 0 : (int)roundf(v[i] / d);
        packed |= ((uint32_t)q & 0xffu) << (8 * i);
        sum += q;
        if (publish && a.t_qx) a.t_qx[c * BLK + 4 * s + i] = (int8_t)q;
      }
#pragma unroll
      for (int m = 1; m < 8; m <<= 1) sum += __shfl_xor(sum, m, 8);
      qa[act_off(c) + s] = packed;
      if (s == 0) {
        da[c] = d;
        sa[c] = sum;
        if (publish && a.t_dx) a.t_dx[c] = d;
      }
    }
  }
  __syncthreads();                        // x's codes and the tag
  const uint32_t tag = *tag_s;            // this call's words carry it
  const uint32_t wtag = tag + (a.test_wait_fail ? kFuTestTag : 0u);   // waited for (test: a tag no word carries)
  if (routed) {
    // the published subtree values, polled directly: P lanes per expert, L
    // values per lane, then log2(P) shuffle levels of the tree
    const int P = g.P, L = g.L, items = E * P;
    for (int b0 = 0; b0 < items; b0 += nt) {     // uniform over the block (shuffles)
      const int it = b0 + tid;
      const bool in = it < items;
      const int e = in ? it / P : 0, p = it % P;
      float lv = 0.0f;
      if (pre1) {                         // (b0 == 0, L == 1: the word polled above)
        if (in) {
          if (p >= g.n_cg) {
            lv = 0.0f;
          } else if (ll_ready(pre, wtag)) {
            lv = __uint_as_float((uint32_t)pre);
          } else {
            uint32_t u[1];
            ok = ll_wait<1>(a.ll_leaf + (size_t)p * E + e, 1, 1, wtag, u, a.spin_max) && ok;
            lv = __uint_as_float(u[0]);
          }
        }
      } else {
        lv = in ? ll_leaf_tree(a, g.n_cg, L, e, p * L, wtag, ok) : 0.0f;
      }
      for (int o = 1; o < P; o <<= 1) lv = lv + __shfl_xor(lv, o, 64);
      if (in && p == 0) {
        const float lg = LW.bias ? lv + LW.bias[e] : lv;
        logit[e] = lg;
        key[e] = rank_key(lg, e);
        if (publish && a.t_logits) a.t_logits[e] = lg;
      }
    }
    __syncthreads();
    // (measured per step: at 128 experts the rank pass 1.2 us against 1.8 us
    // of wave rounds; at 256 the rank pass 2.4 us, the wave rounds faster)
    if (E > 128) fu_wave_topk(key, logit, E, a.k, ids_l, vals_l);
    else fu_rank_topk(key, logit, E, a.k, ids_l, vals_l, rpart);
    if (publish) {                        // w_s = e_s / ((e_0 + e_1) + ...), e_s = exp(l_s - l_0)
      if (tid < a.k) ex_l[tid] = exp_p(vals_l[tid] - vals_l[0]);
      __syncthreads();
      if (tid < a.k) {
        float S = ex_l[0];
        for (int s = 1; s < a.k; s++) S = S + ex_l[s];
        const float wv = ex_l[tid] / S;
        ll_store(a.ll_route + tid, tag, (uint32_t)ids_l[tid]);
        ll_store(a.ll_route + a.k + tid, tag, __float_as_uint(wv));
        if (a.t_ids) a.t_ids[tid] = ids_l[tid];
        if (a.t_w) a.t_w[tid] = wv;
      }
    }
  }

  // the 32 gate and 32 up rows: wave w takes pieces w*SP .. w*SP+SP-1 of the
  // row group (pieces past the row: re-read the last, zeroed), lanes l and
  // l^32 hold blocks 2s and 2s+1
  const size_t gbytes = (size_t)DGU_ROWS * nbh * WFmt<FMT>::bytes;   // one 32-row group
  const uint8_t* gb;
  const uint8_t* ub;
  if (routed) {                           // (clamped: a NaN logit leaves ranks unfilled)
    const size_t G = (size_t)min(max(ids_l[slot], 0), E - 1) * ngrp + gx;
    gb = LW.t_gate + G * gbytes;
    ub = LW.t_up + G * gbytes;
  } else {
    gb = LW.ts_gate + (size_t)gx * gbytes;
    ub = LW.ts_up + (size_t)gx * gbytes;
  }
  const int half = lane >> 5;
  float cg[NCH], cu[NCH];
#pragma unroll
  for (int c = 0; c < NCH; c++) {
    TileCodes<FMT> gn[CH], un[CH];
    uint32_t gs[CH], us[CH];
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
      const uint4* qp = reinterpret_cast<const uint4*>(qa + act_off(b));
      const uint4 a0 = qp[0], a1 = qp[1];
      const uint32_t av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float dav = da[b];
      const int32_t sav = sa[b];
      const int32_t dg = tile_dot<FMT>(gn[q], av, sav);
      const int32_t du = tile_dot<FMT>(un[q], av, sav);
      const bool in = st < nsteps;
      gv[q] = in ? (f16_bits_to_f32(gs[q]) * dav) * (float)dg : 0.0f;
      uv[q] = in ? (f16_bits_to_f32(us[q]) * dav) * (float)du : 0.0f;
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
  const int W = g.gu_waves;               // waves holding pieces (the others hold +0)
  if (lane < DGU_ROWS) {
    wsum[wave][lane] = tg;
    wsum[wave][DGU_ROWS + lane] = tu;
  }
  __syncthreads();
  if (tid < 2 * DGU_ROWS) {               // the W wave sums, pairwise
    float t[kFuWaves];
#pragma unroll
    for (int w = 0; w < kFuWaves; w++) t[w] = wsum[min(w, W - 1)][tid];   // all reads in flight
#pragma unroll
    for (int w = 0; w < kFuWaves; w++) t[w] = w < W ? t[w] : 0.0f;
#pragma unroll
    for (int n = kFuWaves; n > 1; n >>= 1)
      if (n <= W) {
#pragma unroll
        for (int i = 0; i < n / 2; i++) t[i] = t[2 * i] + t[2 * i + 1];
      }
    val[tid] = t[0];
  }
  __syncthreads();
  if (tid < DGU_ROWS) {                   // h of the 32-group, its q8, published
    const float h = silu_p(val[tid]) * val[DGU_ROWS + tid];
    float amax = fabsf(h);
#pragma unroll
    for (int m = 1; m < BLK; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, BLK));
    const float d = amax / 127.0f;
    const int q = (d == 0.0f) ? 0 : (int)roundf(h / d);
    int sum = q;
#pragma unroll
    for (int m = 1; m < BLK; m <<= 1) sum += __shfl_xor(sum, m, BLK);
    const uint32_t q0 = (uint32_t)q & 0xffu;
    const uint32_t q1 = (uint32_t)__shfl(q, tid + 1, BLK) & 0xffu;
    const uint32_t q2 = (uint32_t)__shfl(q, tid + 2, BLK) & 0xffu;
    const uint32_t q3 = (uint32_t)__shfl(q, tid + 3, BLK) & 0xffu;
    uint64_t* dst = a.ll_qh + (size_t)(slot * ngrp + gx) * kFuQhWords;
    if ((tid & 3) == 0) ll_store(dst + tid / 4, tag, q0 | (q1 << 8) | (q2 << 16) | (q3 << 24));
    if (tid == 0) {
      ll_store(dst + 8, tag, __float_as_uint(d));
      ll_store(dst + 9, tag, (uint32_t)sum);
    }
    const size_t hi = (size_t)slot * I + i0 + tid;
    if (a.t_qh) a.t_qh[hi] = (int8_t)q;
    if (tid == 0 && a.t_dh) a.t_dh[hi / BLK] = d;
  }
}

// ---------------------------------------------------------------- down role
// LDS of a down unit: every slot's q8(h) (padded layout), scales, code sums,
// then the per-task row values [8][ns][NH].
__host__ __device__ inline size_t fu_dn_lds_bytes(int ns, int nbi, int NH) {
  return 4 * ((size_t)ns * act_row_dwords(nbi) + 2 * (size_t)ns * nbi + (size_t)kDtRows * ns * NH);
}

// A down unit: 8 output rows r0 .. r0+7 (a quarter of a 32-row group of the
// tile order).  Wave t = NH * sg + hh takes slots 4*sg .. 4*sg+3 and pieces
// hh * SPH .. +SPH-1 of the padded row (+0 leaves past I/32): lane L =
// 32*half + 8*gsub + rr holds slot 4*sg + gsub, row r0 + rr and block 2s +
// half of each piece s, so one load instruction reads 8 runs of 128
// contiguous bytes.  The tree: blocks 2s and 2s+1 (lanes L, L^32), then the
// pieces pairwise; with NH = 2 the two halves are the row's top subtrees,
// added before the combine.  Then the fixed-order combine.
template <int SPH, int FMT>
__device__ void fu_down(const DecodeArgs& a, const StackLayer& LW, uint64_t* lly, const FusedGeometry& g, int u,
                        const uint32_t* tag_s, uint8_t* dyn, bool& ok) {
  using TF = TileFmt<FMT>;
  __shared__ int ids_d[32];
  __shared__ float w_d[32];
  const int tid = threadIdx.x, lane = tid % 64, nt = blockDim.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int H = a.H, I = a.I, nbi = I / BLK, nsteps = I / 64;
  const int ns = a.k + (a.has_shared ? 1 : 0), ngrp = nbi;
  const int NH = g.dn_nh, SS = act_row_dwords(nbi);
  uint32_t* qh_l = reinterpret_cast<uint32_t*>(dyn);                     // ns * SS dwords
  float* dh_l = reinterpret_cast<float*>(qh_l + (size_t)ns * SS);         // ns * nbi
  int32_t* sh_l = reinterpret_cast<int32_t*>(dh_l + (size_t)ns * nbi);    // ns * nbi
  float* op_l = reinterpret_cast<float*>(sh_l + (size_t)ns * nbi);        // [8][ns][NH]
  // the four units of a 32-row group on one XCD (blocks are dealt to the 8
  // XCDs round robin and base_dn % 8 == 0): their pieces share scale lines
  const int r0 = (H % 256 == 0) ? 32 * (8 * (u / 32) + u % 8) + kDtRows * ((u / 8) % 4) : u * kDtRows;
  __syncthreads();                        // the tag
  const uint32_t ptag = *tag_s;           // this call's words carry it
  const uint32_t tag = ptag + (a.test_wait_fail ? kFuTestTag : 0u);   // waited for (test: a tag no word carries)
  // ids and weights
  if (tid < 2 * a.k) {
    uint32_t v[1];
    ok = ll_wait<1>(a.ll_route + tid, 1, 1, tag, v, a.spin_max) && ok;
    if (tid < a.k) ids_d[tid] = (int)v[0];
    else w_d[tid - a.k] = __uint_as_float(v[0]);
  }
  __syncthreads();
  // this wave's task and its weight pieces (in flight while q8(h) is awaited)
  const int ntask = ((ns + 3) / 4) * NH;
  const bool busy = wave < ntask;
  const int sg = wave / NH, hh = wave % NH;
  const int half = lane >> 5, gsub = (lane >> 3) & 3, rr = lane & 7;
  const int slot = 4 * sg + gsub;
  const bool live = busy && slot < ns;
  const int sl = live ? slot : ns - 1;    // lanes past the last slot mirror it (results unused)
  const size_t gbytes = (size_t)nsteps * TF::piece;                      // one 32-row group
  const int pl = 32 * half + (r0 % 32) + rr;                             // lane inside a piece
  const size_t G = (size_t)(r0 / 32);
  const int eid = min(max(ids_d[min(sl, a.k - 1)], 0), a.E - 1);
  const uint8_t* base = (sl < a.k) ? LW.t_down + ((size_t)eid * (H / 32) + G) * gbytes : LW.ts_down + G * gbytes;
  const int s0 = hh * SPH;
  TileCodes<FMT> wn[SPH];
  uint32_t wsc[SPH];
  if (busy) {
#pragma unroll
    for (int q = 0; q < SPH; q++)
      wn[q] = tile_codes<FMT>(base + (size_t)min(s0 + q, nsteps - 1) * TF::piece + TF::code * pl);
#pragma unroll
    for (int q = 0; q < SPH; q++)
      wsc[q] = *reinterpret_cast<const uint16_t*>(base + (size_t)min(s0 + q, nsteps - 1) * TF::piece + TF::scale + 2 * pl);
  }
  // every gate/up unit's indicator (its group's code-sum word), by one wave
  const int ng = ns * ngrp;
  if (wave == ntask % kFuWaves) {
    for (int i0 = 0; i0 < ng; i0 += 8 * 64) {
      uint32_t v[8];
      const int n = max(0, min(8, (ng - i0 - lane + 63) / 64));
      ok = ll_wait<8>(a.ll_qh + (size_t)(i0 + lane) * kFuQhWords + 9, (size_t)64 * kFuQhWords, n, tag, v, a.spin_max) && ok;
    }
  }
  __syncthreads();
  // every slot's q8(h) groups into LDS (each word checked again)
  for (int gi = tid; gi < ng; gi += nt) {
    uint32_t v[kFuQhWords];
    ok = ll_wait<kFuQhWords, true>(a.ll_qh + (size_t)gi * kFuQhWords, 1, kFuQhWords, tag, v, a.spin_max) && ok;
    const int s = gi / ngrp, b = gi % ngrp;
    uint4* dst = reinterpret_cast<uint4*>(qh_l + (size_t)s * SS + act_off(b));
    dst[0] = make_uint4(v[0], v[1], v[2], v[3]);
    dst[1] = make_uint4(v[4], v[5], v[6], v[7]);
    dh_l[gi] = __uint_as_float(v[8]);
    sh_l[gi] = (int32_t)v[9];
  }
  __syncthreads();
  if (busy) {
    const uint32_t* qs = qh_l + (size_t)sl * SS;
    float v[SPH];
#pragma unroll
    for (int q = 0; q < SPH; q++) {
      const int st = s0 + q;
      const int b = 2 * min(st, nsteps - 1) + half;
      const uint4* qp = reinterpret_cast<const uint4*>(qs + act_off(b));
      const uint4 a0 = qp[0], a1 = qp[1];
      const uint32_t av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const int32_t dot = tile_dot<FMT>(wn[q], av, sh_l[sl * nbi + b]);
      v[q] = st < nsteps ? (f16_bits_to_f32(wsc[q]) * dh_l[sl * nbi + b]) * (float)dot : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < SPH; q++) v[q] = v[q] + __shfl_xor(v[q], 32, 64);   // blocks 2s and 2s+1
    const float o = reg_tree<SPH>(v);
    if (live && half == 0) op_l[((size_t)rr * ns + slot) * NH + hh] = o;
  }
  __syncthreads();
  if (tid < kDtRows && r0 + tid < H) {    // every value into registers, then the fixed-order chain
    // every LDS read unconditional (indices clamped into the unit's values),
    // so all are in flight before the fixed-order chain
    const float* ov = op_l + (size_t)tid * ns * NH;
    float o0[kFuMaxSlots], o1[kFuMaxSlots], w[kFuMaxSlots];
#pragma unroll
    for (int s = 0; s < kFuMaxSlots; s++) {
      const int sc = min(s, ns - 1);
      o0[s] = ov[sc * NH];
      o1[s] = ov[sc * NH + NH - 1];
      w[s] = w_d[min(s, a.k - 1)];
    }
    auto row = [&](int s) { return NH == 2 ? o0[s] + o1[s] : o0[s]; };
    float acc = w[0] * row(0);
#pragma unroll
    for (int s = 1; s < kFuMaxSlots; s++)
      if (s < a.k) acc = acc + w[s] * row(s);
    if (a.has_shared) {
      float osh = row(0);
#pragma unroll
      for (int s = 1; s < kFuMaxSlots; s++) osh = s == a.k ? row(s) : osh;
      acc = acc + osh;
    }
    if (lly) ll_store(lly + r0 + tid, ptag, __float_as_uint(acc));   // (a stacked layer's y)
    else a.y[r0 + tid] = acc;
  }
}

// ---------------------------------------------------------------- kernel
// Block roles.  Kernels start on XCDs 0 and 1 about 2 us before the others
// (measured), so the router blocks, the head of the dependency chain, take
// blocks b with b % 8 < 2 of the first rspan = 8 * ceil(nR / 2) blocks; the
// other blocks of that span and the ones after it are the gate/up units, then
// the down units from base_dn (a multiple of 8).
template <int GSP, int DSP, int FMT>
__global__ void __launch_bounds__(kFuThreads, 2) decode_fused_kernel(DecodeArgs a, FusedGeometry g) {
  extern __shared__ __align__(16) uint8_t dyn[];
  __shared__ uint32_t tag_s;
  __shared__ float part[512], tmp[512];   // RMSNorm scale of the previous layer's y
  const int b = blockIdx.x;
  const StackLayer LW = {a.w_router, a.bias, a.t_gate, a.t_up, a.t_down, a.ts_gate, a.ts_up, a.ts_down};
  uint32_t* slots = reinterpret_cast<uint32_t*>(a.hdr + 1);
  if (threadIdx.x == 0) {                 // read by each role after its first barrier
    const uint32_t ep = __hip_atomic_load(slots + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    tag_s = ep + 1u == 0u ? 1u : ep + 1u;           // (tags are never 0)
  }
  bool ok = true;
  const int rspan = 8 * ((g.nR + 1) / 2);
  int gu = -1;
  if (b < rspan) {
    const int x = b % 8, r = 2 * (b / 8) + x;
    if (x < 2) {
      if (r < g.nR) fu_router(a, LW, a.norm_in, g, r, &tag_s, dyn, part, tmp, nullptr, 0u, nullptr, ok);
    } else {
      gu = 6 * (b / 8) + x - 2;
    }
  } else if (b < g.base_dn) {
    gu = 6 * (rspan / 8) + (b - rspan);
  } else if (b < g.base_dn + g.n_dn) {
    fu_down<DSP, FMT>(a, LW, nullptr, g, b - g.base_dn, &tag_s, dyn, ok);
  }
  if (gu >= 0 && gu < g.n_gu) fu_gateup<GSP, FMT>(a, LW, a.norm_in, g, gu, &tag_s, dyn, part, tmp, nullptr, 0u, nullptr, ok);
  if (!ok) fu_fail(a);
  // the next call's epoch, into this block's slots (read by no other block)
  __syncthreads();
  if (threadIdx.x == 0)
    for (int i = b; i < kFuSlots; i += g.nblocks)
      __hip_atomic_store(slots + i, tag_s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- stacked layers
// The stacked decode (x_{l+1} = RMSNorm(y_l)) in one launch: every block keeps
// its role of the one-launch step and runs it layer after layer.  Layer l's
// words carry tag ep + 1 + l (ep: the block's epoch slot), so words of the
// layer before never pass as this layer's.  A layer's y goes to the next
// layer as one tagged word per value (ll_y): the next layer's router blocks
// and gate/up units wait for all H of them, after issuing their own first
// weight loads (the router's), then take the RMSNorm of y themselves.  The
// last layer writes y.  One set of handoff words serves every layer: a
// layer's producers only publish after reading the previous layer's y, which
// is complete only after every reader of the previous layer's words is done.
// What the launch boundary cost between layers (the drain, the next
// kernel's start, the later start of XCDs 2-7) becomes one handoff.
template <int GSP, int DSP, int FMT>
__global__ void __launch_bounds__(kFuThreads, 4) decode_stack_kernel(DecodeArgs a0, FusedGeometry g, StackTable st) {
  extern __shared__ __align__(16) uint8_t dyn[];
  __shared__ uint32_t tag_s, ep_s;
  __shared__ float part[512], tmp[512];   // RMSNorm scale of the previous layer's y
  float* xl = reinterpret_cast<float*>(dyn + g.lds);     // [H] a stacked layer's x
  const int b = blockIdx.x;
  uint32_t* slots = reinterpret_cast<uint32_t*>(a0.hdr + 1);
  if (threadIdx.x == 0) ep_s = __hip_atomic_load(slots + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bool ok = true;
  const int rspan = 8 * ((g.nR + 1) / 2);
  int role = 0, idx = -1;                 // 1 router, 2 gate/up, 3 down
  if (b < rspan) {
    const int x = b % 8, r = 2 * (b / 8) + x;
    if (x < 2) {
      if (r < g.nR) { role = 1; idx = r; }
    } else {
      role = 2;
      idx = 6 * (b / 8) + x - 2;
    }
  } else if (b < g.base_dn) {
    role = 2;
    idx = 6 * (rspan / 8) + (b - rspan);
  } else if (b < g.base_dn + g.n_dn) {
    role = 3;
    idx = b - g.base_dn;
  }
  if (role == 2 && idx >= g.n_gu) role = 0;
  const uint32_t test = a0.test_wait_fail ? kFuTestTag : 0u;
  // one layer loop per role (a loop around all three roles kept every
  // role's loop-invariant values live at once and spilled)
#define MOEQ4_LAYER_LOOP(CALL)                                                          \
  for (int l = 0; l < st.n; l++) {                                                      \
    __syncthreads();                      /* done with the previous layer's tag, LDS */ \
    if (threadIdx.x == 0) tag_s = ep_s + 1u + (uint32_t)l;                              \
    const StackLayer& LW = st.l[l];                                                     \
    const int norm_in = l > 0 ? 1 : a0.norm_in;                                         \
    const uint64_t* llx = l > 0 ? a0.ll_y : nullptr;                                    \
    const uint32_t xtag = ep_s + (uint32_t)l + test;   /* the previous layer's words */ \
    (void)norm_in; (void)llx; (void)xtag;                                               \
    CALL;                                                                               \
  }
  if (role == 1) {
    MOEQ4_LAYER_LOOP(fu_router(a0, LW, norm_in, g, idx, &tag_s, dyn, part, tmp, llx, xtag, xl, ok))
  } else if (role == 2) {
    MOEQ4_LAYER_LOOP((fu_gateup<GSP, FMT>(a0, LW, norm_in, g, idx, &tag_s, dyn, part, tmp, llx, xtag, xl, ok)))
  } else if (role == 3) {
    MOEQ4_LAYER_LOOP((fu_down<DSP, FMT>(a0, LW, l + 1 < st.n ? a0.ll_y : nullptr, g, idx, &tag_s, dyn, ok)))
  }
#undef MOEQ4_LAYER_LOOP
  if (!ok) fu_fail(a0);
  // the next call's epoch (this call's last tag), into this block's slots
  __syncthreads();
  if (threadIdx.x == 0)
    for (int i = b; i < kFuSlots; i += g.nblocks)
      __hip_atomic_store(slots + i, ep_s + (uint32_t)st.n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- launch
FusedGeometry fused_geometry(int H, int I, int E, int k, int has_shared) {
  FusedGeometry g;
  memset(&g, 0, sizeof g);
  const int ns = k + (has_shared ? 1 : 0);
  if (H % 64 || I % 64 || H > 8192 || I > 2048 || E > 1024 || k > 32) return g;
  const int nc = H / BLK;
  int m = 1;
  while (m < nc) m <<= 1;
  // router blocks: EB experts x cpb chunks each, n_eg expert groups x n_cg
  // chunk groups, about 32 blocks (each a small share of W_r: the router is
  // the head of the dependency chain)
  const int EB = E < 16 ? E : 16 * ((E + 127) / 128);
  const int n_eg = (E + EB - 1) / EB;
  int cpb = 1;
  while (cpb < m && cpb < 64 && (m / (cpb * 2)) * n_eg >= 32 && cpb * 2 * EB <= kFuThreads) cpb <<= 1;
  g.cpb = cpb;
  g.eb = EB;
  g.n_eg = (E + EB - 1) / EB;
  g.n_cg = (nc + cpb - 1) / cpb;
  g.nR = g.n_eg * g.n_cg;
  const int mR = m / cpb;                 // subtree values per expert (power of two)
  int P = 1;                              // lanes per expert: at most 16 values per lane
  while (mR / P > 16) P <<= 1;
  while (P < mR && P < 64 && E * P * 2 <= kFuThreads) P <<= 1;
  g.P = P;
  g.L = mR / P;
  // gate/up: W = min(8, m/2) waves of SP = m / (2W) pieces
  const int W = m / 2 < kFuWaves ? m / 2 : kFuWaves;
  g.gu_waves = W;
  g.gu_sp = m / (2 * W);
  g.n_gu = I / DGU_ROWS * ns;
  // down: 8-row units, a wave per (4 slots, one of NH halves of the pieces)
  const int nbi = I / BLK;
  int md = 1;
  while (md < nbi) md <<= 1;
  const int sp = md / 2, groups = (ns + 3) / 4;
  g.dn_nh = (sp >= 2 && groups * 2 <= kFuWaves - 1) ? 2 : 1;
  g.dn_sp = sp / g.dn_nh;
  if (groups * g.dn_nh > kFuWaves - 1 || ns > kFuMaxSlots) return g;   // (one wave left to poll)
  g.n_dn = (H + kDtRows - 1) / kDtRows;
  const int rspan = 8 * ((g.nR + 1) / 2);
  const int gu_in_span = 6 * (rspan / 8);
  g.base_dn = (rspan + (g.n_gu > gu_in_span ? g.n_gu - gu_in_span : 0) + 7) / 8 * 8;
  g.nblocks = g.base_dn + g.n_dn;
  const size_t lr = 4 * ((size_t)cpb * BLK + (size_t)cpb * EB);
  const size_t lg = fu_gu_lds_bytes(nc, E);
  const size_t ld = fu_dn_lds_bytes(ns, nbi, g.dn_nh);
  g.lds = lr > lg ? lr : lg;
  g.lds = g.lds > ld ? g.lds : ld;
  if (g.lds > 48 * 1024 || g.nblocks > kFuSlots) return g;
  if (g.gu_sp > 8 || g.dn_sp > 8) return g;
  g.ok = 1;
  return g;
}

template <int FMT>
static const void* fused_kernel_ptr(int gsp, int dsph) {
#define MOEQ4_FK(G, D) reinterpret_cast<const void*>(&decode_fused_kernel<G, D, FMT>)
#define MOEQ4_FKROW(G) \
  switch (dsph) { case 1: return MOEQ4_FK(G, 1); case 2: return MOEQ4_FK(G, 2); case 4: return MOEQ4_FK(G, 4); default: return MOEQ4_FK(G, 8); }
  switch (gsp) {
    case 1: MOEQ4_FKROW(1);
    case 2: MOEQ4_FKROW(2);
    case 4: MOEQ4_FKROW(4);
    default: MOEQ4_FKROW(8);
  }
#undef MOEQ4_FKROW
#undef MOEQ4_FK
}

// Resident blocks of the fused kernel per CU (occupancy query, cached per
// kernel and LDS size) times the CU count: the grid must fit at once, since
// its blocks wait on one another.
static int fused_capacity(const void* fn, size_t lds) {
  struct Entry { const void* fn; size_t lds; int dev; int cap; };
  static Entry cache[64];
  static int n_cache = 0;
  static std::mutex mu;
  std::lock_guard<std::mutex> lock(mu);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  for (int i = 0; i < n_cache; i++)
    if (cache[i].fn == fn && cache[i].lds == lds && cache[i].dev == dev) return cache[i].cap;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kFuThreads, lds) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const int cap = per_cu * cus;
  if (n_cache < 64) cache[n_cache++] = {fn, lds, dev, cap};
  return cap;
}

template <int FMT>
static const void* stack_kernel_ptr(int gsp, int dsph) {
#define MOEQ4_SK(G, D) reinterpret_cast<const void*>(&decode_stack_kernel<G, D, FMT>)
#define MOEQ4_SKROW(G) \
  switch (dsph) { case 1: return MOEQ4_SK(G, 1); case 2: return MOEQ4_SK(G, 2); case 4: return MOEQ4_SK(G, 4); default: return MOEQ4_SK(G, 8); }
  switch (gsp) {
    case 1: MOEQ4_SKROW(1);
    case 2: MOEQ4_SKROW(2);
    case 4: MOEQ4_SKROW(4);
    default: MOEQ4_SKROW(8);
  }
#undef MOEQ4_SKROW
#undef MOEQ4_SK
}

bool fused_decode_available(const DecodeArgs& a) {
  if (!a.hdr || !a.t_gate || !a.t_up || !a.t_down) return false;
  if (a.has_shared && (!a.ts_gate || !a.ts_up || !a.ts_down)) return false;
  const FusedGeometry g = fused_geometry(a.H, a.I, a.E, a.k, a.has_shared);
  if (!g.ok) return false;
  const void* fn = a.wfmt == kQ8 ? fused_kernel_ptr<kQ8>(g.gu_sp, g.dn_sp) : fused_kernel_ptr<kQ4>(g.gu_sp, g.dn_sp);
  return g.nblocks <= fused_capacity(fn, g.lds);
}

template <int FMT>
static hipError_t launch_fused(const DecodeArgs& a, const FusedGeometry& g, hipStream_t stream) {
  const void* fn = fused_kernel_ptr<FMT>(g.gu_sp, g.dn_sp);
  DecodeArgs aa = a;
  FusedGeometry gg = g;
  void* args[] = {&aa, &gg};
  return hipLaunchKernel(fn, dim3(g.nblocks), dim3(kFuThreads), args, g.lds, stream);
}

bool stack_decode_available(const DecodeArgs& a) {
  if (!a.hdr || !a.ll_y || !a.t_gate || !a.t_up || !a.t_down) return false;
  if (a.has_shared && (!a.ts_gate || !a.ts_up || !a.ts_down)) return false;
  const FusedGeometry g = fused_geometry(a.H, a.I, a.E, a.k, a.has_shared);
  if (!g.ok) return false;
  const size_t lds = g.lds + 4 * (size_t)a.H;
  const void* fn = a.wfmt == kQ8 ? stack_kernel_ptr<kQ8>(g.gu_sp, g.dn_sp) : stack_kernel_ptr<kQ4>(g.gu_sp, g.dn_sp);
  return lds <= 64 * 1024 && g.nblocks <= fused_capacity(fn, lds);
}

hipError_t launch_decode_stack(const DecodeArgs& a, const StackTable& t, hipStream_t stream) {
  const FusedGeometry g = fused_geometry(a.H, a.I, a.E, a.k, a.has_shared);
  const void* fn = a.wfmt == kQ8 ? stack_kernel_ptr<kQ8>(g.gu_sp, g.dn_sp) : stack_kernel_ptr<kQ4>(g.gu_sp, g.dn_sp);
  DecodeArgs aa = a;
  FusedGeometry gg = g;
  StackTable tt = t;
  void* args[] = {&aa, &gg, &tt};
  hipError_t e = hipLaunchKernel(fn, dim3(g.nblocks), dim3(kFuThreads), args, g.lds + 4 * (size_t)a.H, stream);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_decode_fused(const DecodeArgs& a, hipStream_t stream) {
  const FusedGeometry g = fused_geometry(a.H, a.I, a.E, a.k, a.has_shared);
  hipError_t e = a.wfmt == kQ8 ? launch_fused<kQ8>(a, g, stream) : launch_fused<kQ4>(a, g, stream);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace moeq4
