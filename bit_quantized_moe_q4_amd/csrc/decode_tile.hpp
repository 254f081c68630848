// decode_tile.hpp -- the one-token decode's tile-order weight access and its
// top-k by rank, shared by the three-launch and the one-launch decode.
#pragma once
#include "w4a8.hpp"
#include "decode_common.hpp"

namespace moeq4 {

// Gate/up unit: 32 values of i (32 gate and 32 up rows).  Down unit of the
// tile-order kernels: 8 output rows.
constexpr int DGU_ROWS = 32;
constexpr int kDtRows = 8;

// Tile order per weight format (q4_tile / q8w_tile in moe_q4.h): bytes of a
// piece, bytes of a lane's block codes (at lane * code), scale offset.
template <int FMT> struct TileFmt;
template <> struct TileFmt<kQ4> { static constexpr int piece = 1152, code = 16, scale = 1024; };
template <> struct TileFmt<kQ8> { static constexpr int piece = 2176, code = 32, scale = 2048; };

// One lane's block of a piece: its code dwords (Q4_0 nibbles or Q8_0 codes).
template <int FMT>
struct TileCodes {
  uint32_t w[TileFmt<FMT>::code / 4];
};

template <int FMT>
__device__ __forceinline__ TileCodes<FMT> tile_codes(const uint8_t* p) {
  TileCodes<FMT> t;
#pragma unroll
  for (int h = 0; h < TileFmt<FMT>::code / 16; h++) {
    const uint4 v = *reinterpret_cast<const uint4*>(p + 16 * h);
    t.w[4 * h] = v.x; t.w[4 * h + 1] = v.y; t.w[4 * h + 2] = v.z; t.w[4 * h + 3] = v.w;
  }
  return t;
}

template <int FMT>
__device__ __forceinline__ int32_t tile_dot(const TileCodes<FMT>& t, const uint32_t (&av)[8], int32_t sa) {
  if constexpr (FMT == kQ4) return q4_block_dot(t.w, av, sa);
  else return q8_block_dot(t.w, av);
}

// Top-k by rank over E order keys in LDS (key[e] = rank_key(logit[e], e)):
// expert e's rank is the number of keys above its own, which for non-NaN
// logits picks the same experts in the same order as k rounds of "first
// maximum among the rest".  ids_l / vals_l [k] (LDS) receive the experts and
// their logits.  Called by every thread of the block (barriers inside); E <=
// 1024.
__device__ __forceinline__ void rank_topk(const uint64_t* key, const float* logit, int E, int k,
                                          int* ids_l, float* vals_l) {
  const int tid = threadIdx.x, nt = blockDim.x;
  // Rank pass.  A wave task is (64 experts, one range of Q equal key ranges):
  // every lane compares its expert's key against the range's keys, all lanes
  // reading the same key at once (an LDS broadcast, no bank conflicts).  The
  // Q partial counts of an expert are then summed by one thread.
  __shared__ int32_t rpart[1024];         // [Q][E]; Q * E <= max(E, 64 * waves) <= 1024
  const int nw = nt / 64, lane = tid % 64;
  const int nchunk = (E + 63) / 64;
  const int Q = nw / nchunk > 1 ? nw / nchunk : 1;
  const int span = ((E + Q - 1) / Q + 1) & ~1;          // even: 16-byte key pairs
  const ulonglong2* K2 = reinterpret_cast<const ulonglong2*>(key);
  for (int task = tid / 64; task < nchunk * Q; task += nw) {
    const int e = (task % nchunk) * 64 + lane, q = task / nchunk;
    const uint64_t ke = key[e < E ? e : 0];
    const int j0 = min(q * span, E), j1 = min(j0 + span, E);
    int rank = 0;
    int j = j0;                           // j0 is even
#pragma unroll 8
    for (; j + 2 <= j1; j += 2) {
      const ulonglong2 kk = K2[j >> 1];
      rank += (kk.x > ke) ? 1 : 0;
      rank += (kk.y > ke) ? 1 : 0;
    }
    if (j < j1) rank += (key[j] > ke) ? 1 : 0;
    if (e < E) rpart[q * E + e] = rank;
  }
  __syncthreads();
  for (int e = tid; e < E; e += nt) {
    int rank = 0;
    for (int q = 0; q < Q; q++) rank += rpart[q * E + e];
    if (rank < k) {
      ids_l[rank] = e;
      vals_l[rank] = logit[e];
    }
  }
  __syncthreads();
}

}  // namespace moeq4
