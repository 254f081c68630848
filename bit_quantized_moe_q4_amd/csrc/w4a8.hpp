// w4a8.hpp -- the W4A8 row program shared by the decode kernels and the
// exported test GEMV.
//
// "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU",
// technical summary, Methodology 1 / Key Contribution 2: the decode path is
// an integer kernel over 4-bit weights and 8-bit activations (pmaddubsw on
// the pages' SSSE3 host: unsigned bytes times signed bytes, pairwise added).
// Here one 32-block dot is 8 v_dot4_i32_i8 on the unsigned codes q (0..15)
// against the int8 activations, minus 8 * (sum of the activation codes) --
// the same offset form, exact in int32.  Per block the fp32 value is
// (d_w * d_a) * (float)dot; a row is the pairwise sum of its block values.
//
// The same program runs on Q8_0 weights (the 8-bit weights of "A Modern
// Multimodal Assistant on a 6 GB 2011 GPU", abstract; 34-byte blocks, signed
// codes): a block dot is 8 v_dot4_i32_i8 of the signed codes against the
// activations, with no offset term.  FMT selects the format: kQ4 or kQ8.
//
// Work split: a row of nb blocks (padded to the power of two m) is handled by
// LPR = m / BPL adjacent lanes, each owning BPL consecutive blocks; a lane
// sums its blocks pairwise, then a butterfly over the LPR lanes finishes the
// level-by-level tree.
#pragma once
#include "device_math.hpp"

namespace moeq4 {

constexpr int kQ4 = 0, kQ8 = 1;
template <int FMT> struct WFmt;
template <> struct WFmt<kQ4> { static constexpr int bytes = 18; };   // fp16 d + 16 nibble bytes
template <> struct WFmt<kQ8> { static constexpr int bytes = 34; };   // fp16 d + 32 int8 codes

// Activation operand of one 32-block: 8 dwords of int8 codes (elements 0..31),
// its scale and the sum of its codes.
struct ActBlock {
  uint32_t a[8];
  float d;
  int32_t s;
};

__device__ __forceinline__ int32_t q4_block_dot(const uint32_t nib[4], const uint32_t a[8],
                                                int32_t asum) {
  int32_t acc = 0;
#pragma unroll
  for (int n = 0; n < 4; n++) {
    acc = __builtin_amdgcn_sdot4((int)(nib[n] & 0x0f0f0f0fu), (int)a[n], acc, false);
    acc = __builtin_amdgcn_sdot4((int)((nib[n] >> 4) & 0x0f0f0f0fu), (int)a[4 + n], acc, false);
  }
  return acc - 8 * asum;
}

__device__ __forceinline__ int32_t q8_block_dot(const uint32_t q[8], const uint32_t a[8]) {
  int32_t acc = 0;
#pragma unroll
  for (int n = 0; n < 8; n++) acc = __builtin_amdgcn_sdot4((int)q[n], (int)a[n], acc, false);
  return acc;
}

// Bytes of block j (0-based inside a span that starts 4-byte aligned), taken
// from the span's dwords D: the fp16 scale bits and the 4 nibble dwords.
template <int J>
__device__ __forceinline__ void span_block(const uint32_t* D, uint32_t& scale, uint32_t nib[4]) {
  constexpr int o = 18 * J;               // byte offset of the block
  if constexpr ((J & 1) == 0) {           // o % 4 == 0: scale low half, nibbles at +2
    scale = D[o / 4] & 0xffffu;
#pragma unroll
    for (int n = 0; n < 4; n++) nib[n] = __builtin_amdgcn_alignbyte(D[o / 4 + n + 1], D[o / 4 + n], 2);
  } else {                                // o % 4 == 2: scale high half, nibbles aligned
    scale = D[(o - 2) / 4] >> 16;
#pragma unroll
    for (int n = 0; n < 4; n++) nib[n] = D[(o + 2) / 4 + n];
  }
}

// Q8_0 block j of a span: fp16 scale bits and the 8 code dwords (34-byte
// blocks: even j starts 4-byte aligned, odd j 2 bytes past a dword).
template <int J>
__device__ __forceinline__ void span_block8(const uint32_t* D, uint32_t& scale, uint32_t q[8]) {
  constexpr int o = 34 * J;
  if constexpr ((J & 1) == 0) {
    scale = D[o / 4] & 0xffffu;
#pragma unroll
    for (int n = 0; n < 8; n++) q[n] = __builtin_amdgcn_alignbyte(D[o / 4 + n + 1], D[o / 4 + n], 2);
  } else {
    scale = D[(o - 2) / 4] >> 16;
#pragma unroll
    for (int n = 0; n < 8; n++) q[n] = D[(o + 2) / 4 + n];
  }
}

// Value of block J of a register span: (d_w * d_a) * (float)dot.
template <int FMT, int J, typename ActFn>
__device__ __forceinline__ float span_value(const uint32_t* Dg, int b, ActFn act, int32_t* dots) {
  uint32_t sc;
  int32_t dot;
  const ActBlock A = act(b);
  if constexpr (FMT == kQ4) {
    uint32_t nib[4];
    span_block<J>(Dg, sc, nib);
    dot = q4_block_dot(nib, A.a, A.s);
  } else {
    uint32_t q[8];
    span_block8<J>(Dg, sc, q);
    dot = q8_block_dot(q, A.a);
  }
  if (dots) dots[b] = dot;
  const float s = f16_bits_to_f32(sc) * A.d;
  return s * (float)dot;
}

// Pairwise tree of BPL values in registers (BPL a power of two).
template <int BPL>
__device__ __forceinline__ float reg_tree(float (&v)[BPL]) {
#pragma unroll
  for (int w = BPL; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; i++) v[i] = v[2 * i] + v[2 * i + 1];
  return v[0];
}

// The FAST row program on a lane's span already in registers: D holds the
// bytes of blocks b0 .. b0+BPL-1 (BPL % 8 == 0; 8 blocks repeat every 36
// dwords for Q4_0, 68 for Q8_0) plus one spare dword.  Blocks >= nb are +0
// leaves.  dots (optional) receives dot_b at dots[b].
template <int BPL, int FMT, typename ActFn>
__device__ __forceinline__ float wxa8_regs(const uint32_t* D, int nb, int b0, ActFn act,
                                           int32_t* dots = nullptr) {
  static_assert(BPL % 8 == 0, "register spans hold whole groups of 8 blocks");
  constexpr int GD = 8 * WFmt<FMT>::bytes / 4;     // dwords per group of 8 blocks
  if (b0 >= nb) return 0.0f;              // a lane of padding leaves only
  float p[BPL];
#pragma unroll
  for (int g = 0; g < BPL / 8; g++) {
    const uint32_t* Dg = D + GD * g;
    const int bg = b0 + 8 * g;
    p[8 * g + 0] = span_value<FMT, 0>(Dg, bg + 0, act, dots);
    p[8 * g + 1] = span_value<FMT, 1>(Dg, bg + 1, act, dots);
    p[8 * g + 2] = span_value<FMT, 2>(Dg, bg + 2, act, dots);
    p[8 * g + 3] = span_value<FMT, 3>(Dg, bg + 3, act, dots);
    p[8 * g + 4] = span_value<FMT, 4>(Dg, bg + 4, act, dots);
    p[8 * g + 5] = span_value<FMT, 5>(Dg, bg + 5, act, dots);
    p[8 * g + 6] = span_value<FMT, 6>(Dg, bg + 6, act, dots);
    p[8 * g + 7] = span_value<FMT, 7>(Dg, bg + 7, act, dots);
  }
  return reg_tree<BPL>(p);
}

template <int BPL, typename ActFn>
__device__ __forceinline__ float w4a8_regs(const uint32_t* D, int nb, int b0, ActFn act,
                                           int32_t* dots = nullptr) {
  return wxa8_regs<BPL, kQ4>(D, nb, b0, act, dots);
}

// One lane's share of a row: blocks b = b0 .. b0+BPL-1 (blocks >= nb are +0
// leaves).  `row` points at the row's first block.  `act(b)` returns the
// activation block b.  FAST: the lane's span is 16-byte aligned and whole
// (BPL % 8 == 0, b0 + BPL <= nb); otherwise halfword loads per block.
// dots (optional) receives dot_b at dots[b] for valid b.
template <int BPL, bool FAST, int FMT, typename ActFn>
__device__ __forceinline__ float wxa8_lane(const uint8_t* __restrict__ row, int nb, int b0,
                                           ActFn act, int32_t* dots) {
  constexpr int QB = WFmt<FMT>::bytes;
  if constexpr (FAST) {
    if (b0 >= nb) return 0.0f;
    constexpr int NV = QB * BPL / 16;     // uint4 per span
    uint32_t D[4 * NV + 1];
    const uint4* src = reinterpret_cast<const uint4*>(row + (size_t)b0 * QB);
#pragma unroll
    for (int v = 0; v < NV; v++) {
      const uint4 t = src[v];
      D[4 * v] = t.x; D[4 * v + 1] = t.y; D[4 * v + 2] = t.z; D[4 * v + 3] = t.w;
    }
    D[4 * NV] = 0u;
    return wxa8_regs<BPL, FMT>(D, nb, b0, act, dots);
  } else {
    float p[BPL];
    const uint16_t* hw = reinterpret_cast<const uint16_t*>(row);
#pragma unroll
    for (int j = 0; j < BPL; j++) {
      const int b = b0 + j;
      p[j] = 0.0f;
      if (b < nb) {
        const uint16_t* q = hw + (size_t)b * (QB / 2);
        const uint32_t sc = q[0];
        const ActBlock A = act(b);
        int32_t dot;
        if constexpr (FMT == kQ4) {
          uint32_t nib[4];
#pragma unroll
          for (int n = 0; n < 4; n++) nib[n] = (uint32_t)q[1 + 2 * n] | ((uint32_t)q[2 + 2 * n] << 16);
          dot = q4_block_dot(nib, A.a, A.s);
        } else {
          uint32_t c[8];
#pragma unroll
          for (int n = 0; n < 8; n++) c[n] = (uint32_t)q[1 + 2 * n] | ((uint32_t)q[2 + 2 * n] << 16);
          dot = q8_block_dot(c, A.a);
        }
        if (dots) dots[b] = dot;
        const float s = f16_bits_to_f32(sc) * A.d;
        p[j] = s * (float)dot;
      }
    }
    return reg_tree<BPL>(p);
  }
}

template <int BPL, bool FAST, typename ActFn>
__device__ __forceinline__ float w4a8_lane(const uint8_t* __restrict__ row, int nb, int b0,
                                           ActFn act, int32_t* dots) {
  return wxa8_lane<BPL, FAST, kQ4>(row, nb, b0, act, dots);
}

// Geometry of the row program for a K-long row: m = next_pow2(K/32),
// BPL = blocks per lane, LPR = lanes per row (both powers of two).
struct RowSplit {
  int nb, m, bpl, lpr;
};
inline RowSplit row_split(int K, int max_lpr) {
  RowSplit r;
  r.nb = K / BLK;
  r.m = 1;
  while (r.m < r.nb) r.m <<= 1;
  r.bpl = r.m < 8 ? r.m : 8;
  while (r.m / r.bpl > max_lpr) r.bpl <<= 1;
  r.lpr = r.m / r.bpl;
  return r;
}

}  // namespace moeq4
