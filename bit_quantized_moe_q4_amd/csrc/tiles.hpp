// tiles.hpp -- expert-segment tiles of the grouped prefill GEMMs (bf16 and
// W4A8): which rows of which expert segment a block works on, found on the
// device from expert_offsets (no host round trip).
#pragma once
#include "device_math.hpp"

namespace moeq4 {

struct Tile {
  int valid;     // 0: no work for this block
  int rows;      // valid rows in the tile (1..BM)
  int pos0;      // row position of the tile's first row in h / o_perm
  int expert;    // routed expert, or -1 for the shared expert
  int m0;        // first row inside the expert segment (token index for shared)
};

// Balanced tiles: expert e's c_e rows are cut into ceil(c_e / FMAXR)
// near-equal tiles of a multiple of 32 rows, so a thin expert (c_e ~ T*k/E)
// is ONE tile and each of its weights is read once per column block.
// Tile mt, found by every wave on its own (registers only, no LDS): the
// shared expert's ceil(T / FMAXR) tiles come first (its dense M = T tiles
// are the largest units and their down work the longest chain), then
// expert e owns ceil(c_e / FMAXR) consecutive tile indices, experts in order.
// BAL = false: greedy tiles instead, FMAXR rows each but the segment's last
// (fewest 32-row groups per expert; for kernels that skip idle 32-row groups).
template <int FMAXR, bool BAL = true>
__device__ __forceinline__ Tile find_tile_bal(const int32_t* __restrict__ offsets, int E, int T,
                                              int k, int has_shared, int mt) {
  const int lane = threadIdx.x % 64;
  Tile t;
  t.valid = 0;
  t.rows = 0;
  t.pos0 = 0;
  t.expert = -1;
  t.m0 = 0;
  int c = -1, q = 0, seg0 = 0;
  // the shared expert's tiles, the largest units, come in a multiple of 8
  // once there are 8 or more (balanced: tiles are dealt to the 8 XCDs by
  // index, and 13 tiles at 2048 tokens gave five XCDs one heavy tile more)
  int n_sh = has_shared ? (T + FMAXR - 1) / FMAXR : 0;
  if (BAL && n_sh >= 8) n_sh = (n_sh + 7) / 8 * 8;
  if (mt < n_sh) {                        // (uniform per wave)
    c = T;
    q = mt;
  } else {
    const int mr = mt - n_sh;
    int carry = 0;
    for (int base = 0; base < E; base += 64) {
      const int e = base + lane;
      int ce = 0, o0 = 0;
      if (e < E) {
        o0 = offsets[e];
        ce = offsets[e + 1] - o0;
      }
      const int nt = (ce + FMAXR - 1) / FMAXR;
      int incl = nt;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
      }
      const unsigned long long hit = __ballot(carry + incl > mr);
      if (hit) {
        const int f = __builtin_ctzll(hit);
        t.expert = base + f;
        c = __shfl(ce, f, 64);
        seg0 = __shfl(o0, f, 64);          // the segment's start, already loaded
        q = mr - (carry + __shfl(incl, f, 64) - __shfl(nt, f, 64));
        break;
      }
      carry += __shfl(incl, 63, 64);
    }
    if (c < 0) return t;
  }
  const int nt = (c + FMAXR - 1) / FMAXR;
  if (q < 0 || q >= nt) return t;
  const int tr = BAL ? 32 * (((c + nt - 1) / nt + 31) / 32) : FMAXR;   // rows per tile, <= FMAXR
  t.m0 = q * tr;
  t.rows = min(tr, c - t.m0);
  if (t.rows <= 0) return t;
  t.valid = 1;
  t.pos0 = (t.expert >= 0) ? seg0 + t.m0 : T * k + t.m0;
  return t;
}

}  // namespace moeq4
