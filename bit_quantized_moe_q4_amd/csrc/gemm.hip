// gemm.hip -- batched prefill of the Q4_0 expert FFN: grouped 4-bit GEMMs.
//
// "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU",
// technical summary, Methodology 1 (the prompt's MoE part is a grouped 4-bit
// GEMM over the tokens routed to each expert), Methodology 4 (one pass over
// the whole prompt maximises the GEMM batch) and Results (the structural
// bottleneck is the thin-M GEMM: ~T*k/E rows per expert).  The pages' kernel
// ran on a GPU without matrix units; here the contraction runs on gfx950's
// bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32 accumulation.
//
// Kernels:
//   gateup   per (expert tile of <=BM rows, 128 columns of I): G = X W_g^T and
//            U = X W_u^T, epilogue h = silu(G) * U -> bf16, rows in segment order
//   down     per (expert tile, 128 columns of H): O = h W_d^T -> bf16 rows in
//            segment order (routed) or fp32 straight into y (shared expert)
//   combine  y[t] += sum_s w[t,s] * O[inv_perm[t*k+s]]
//
// Work split inside a block: 4 waves, each owns 32 output columns and every
// row of the tile (BM/32 MFMA subtiles), so each weight is dequantised once
// per block.  Activation rows (gathered through perm) are staged in LDS per
// K-step of 256 (8 Q4 blocks).  K inside a step is permuted, identically for
// both operands (a dot product does not depend on the order of its terms):
// MFMA instruction i (0..15) takes, in lane half g, elements 8*(i%4)..+8 of
// block 4g + i/4 -- so lane (n, g) needs exactly blocks 4g..4g+3 of weight
// row n, one contiguous 72-byte run of whole 18-byte blocks, and reads its
// activations at step offset 128g + 8i.
//
// Tiles are found on the device from expert_offsets (no host round trip):
// expert e has ceil(c_e / BM) tiles, in expert order, then the shared expert's
// ceil(T / BM) tiles; blocks beyond the last tile exit.
#include "launch.hpp"
#include "device_math.hpp"
#include "w4a8.hpp"

namespace moeq4 {

typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int GKB = 256;          // K elements per step (8 Q4 blocks)
constexpr int GLDA = GKB + 8;     // LDS row stride in bf16 elements (16-byte pad)
constexpr int GBN = 128;          // output columns per block (4 waves x 32)
constexpr int GMaxE = 1024;

struct Tile {
  int valid;     // 0: no work for this block
  int rows;      // valid rows in the tile (1..BM)
  int pos0;      // row position of the tile's first row in h / o_perm
  int expert;    // routed expert, or -1 for the shared expert
  int m0;        // first row inside the expert segment (token index for shared)
};

// pref[e] = tiles of experts < e (pref[E] = routed total), computed by wave 0.
template <int BM>
__device__ __forceinline__ Tile find_tile(const int32_t* __restrict__ offsets, int E, int T, int k,
                                          int has_shared, int mt, int32_t* pref) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    int carry = 0;
    if (tid == 0) pref[0] = 0;
    for (int base = 0; base < E; base += 64) {
      const int e = base + tid;
      int c = 0;
      if (e < E) c = (offsets[e + 1] - offsets[e] + BM - 1) / BM;
      int incl = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (tid >= d) incl += o;
      }
      if (e < E) pref[e + 1] = carry + incl;
      carry += __shfl(incl, 63, 64);
    }
  }
  __syncthreads();
  Tile t;
  t.valid = 0;
  t.rows = 0;
  t.pos0 = 0;
  t.expert = -1;
  t.m0 = 0;
  const int routed = pref[E];
  if (mt < routed) {
    int lo = 0, hi = E - 1;                 // last e with pref[e] <= mt
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pref[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int q = mt - pref[e];
    const int c = offsets[e + 1] - offsets[e];
    t.valid = 1;
    t.expert = e;
    t.m0 = q * BM;
    t.rows = min(BM, c - t.m0);
    t.pos0 = offsets[e] + t.m0;
  } else if (has_shared) {
    const int q = mt - routed;
    if (q * BM < T) {
      t.valid = 1;
      t.expert = -1;
      t.m0 = q * BM;
      t.rows = min(BM, T - t.m0);
      t.pos0 = T * k + t.m0;
    }
  }
  return t;
}

// Token of the tile's first row: padding rows of a tile read this valid row.
__device__ __forceinline__ int tok_fill(const PrefillArgs& a, const Tile& t) {
  return (t.expert >= 0) ? min(max(a.perm[t.pos0] / a.k, 0), a.T - 1) : t.m0;
}

// 8 bf16 weights of element group Q (0..3) of block J of a lane's run of
// whole blocks.  Group 0: elements 0..7 (low nibbles of bytes 0..7), 1: 8..15
// (low nibbles of bytes 8..15), 2: 16..23 (high nibbles of bytes 0..7),
// 3: 24..31.  Each value (q - 8) * d is exact in fp32 and rounded once to
// bf16.  A high nibble is read in place as the byte 16q and scaled by d/16
// (exact: a power-of-two step).  The nibble mask goes through an opaque
// v_and_b32 so that each byte converts with one v_cvt_f32_ubyte{0..3}.
__device__ __forceinline__ uint32_t opaque_and(uint32_t w, uint32_t m) {
  uint32_t r;
  asm volatile("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(w), "v"(m));
  return r;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  const bf16x2_t b = __builtin_convertvector(v, bf16x2_t);   // round to nearest even
  return __builtin_bit_cast(uint32_t, b);
}

template <int J, int Q>
__device__ __forceinline__ bf16x8_t dequant8(const uint32_t* D) {
  uint32_t sc, nib[4];
  span_block<J>(D, sc, nib);
  const float d = f16_bits_to_f32(sc);
  const float off = -8.0f * d;
  const float mul = (Q >> 1) ? d * 0.0625f : d;
  const uint32_t mask = (Q >> 1) ? 0xf0f0f0f0u : 0x0f0f0f0fu;
  const uint32_t v0 = opaque_and(nib[2 * (Q & 1)], mask);
  const uint32_t v1 = opaque_and(nib[2 * (Q & 1) + 1], mask);
  float f[8];
#pragma unroll
  for (int b = 0; b < 4; b++) {
    f[b] = __builtin_fmaf((float)((v0 >> (8 * b)) & 0xffu), mul, off);
    f[4 + b] = __builtin_fmaf((float)((v1 >> (8 * b)) & 0xffu), mul, off);
  }
  uint32_t w[4];
#pragma unroll
  for (int p = 0; p < 4; p++) w[p] = pack_bf16x2(f[2 * p], f[2 * p + 1]);
  return __builtin_bit_cast(bf16x8_t, w);
}

// Load a lane's run of blocks 4g..4g+3 of one weight row for one K-step into
// 18 dwords.  nv = number of valid blocks (0..4); 8-byte loads when the run is
// whole and aligned, halfword loads otherwise (missing blocks read as zero).
__device__ __forceinline__ void load_run(const uint8_t* __restrict__ p, int nv, bool vec,
                                         uint32_t (&D)[18]) {
  if (vec && nv == 4) {
    const uint2* s = reinterpret_cast<const uint2*>(p);
#pragma unroll
    for (int v = 0; v < 9; v++) {
      const uint2 t = s[v];
      D[2 * v] = t.x;
      D[2 * v + 1] = t.y;
    }
  } else {
    const uint16_t* h = reinterpret_cast<const uint16_t*>(p);
#pragma unroll
    for (int v = 0; v < 18; v++) {
      const int j = (2 * v) / 9;          // block of the low halfword
      const uint32_t lo = (j < nv) ? h[2 * v] : 0u;
      const uint32_t hi = ((2 * v + 1) / 9 < nv) ? h[2 * v + 1] : 0u;
      D[v] = lo | (hi << 16);
    }
  }
}

template <int J, int Q, int MT>
__device__ __forceinline__ void mma_step_one(const uint16_t* As, int ln, int g, int i, int ms,
                                             bool bvalid, const bf16x8_t& b0, const bf16x8_t* b1,
                                             f32x16_t (&acc0)[MT], f32x16_t (*acc1)[MT]) {
#pragma unroll
  for (int sub = 0; sub < MT; sub++) {
    if (sub < ms) {
      bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(As + (32 * sub + ln) * GLDA + 128 * g + 8 * i);
      if (!bvalid) av = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      acc0[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b0, acc0[sub], 0, 0, 0);
      if (b1) (*acc1)[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, *b1, (*acc1)[sub], 0, 0, 0);
    }
  }
}

// One K-step of MFMAs for one lane: 16 instructions per subtile per matrix.
template <int MT, bool TWO>
__device__ __forceinline__ void mma_step(const uint16_t* As, int ln, int g, int ms, int nv,
                                         const uint32_t (&D0)[18], const uint32_t (&D1)[18],
                                         f32x16_t (&acc0)[MT], f32x16_t (&acc1)[MT]) {
#define MOEQ4_I(J, Q)                                                                      \
  {                                                                                        \
    const bool bv = (J) < nv;                                                              \
    bf16x8_t b0 = dequant8<J, Q>(D0);                                                      \
    if (!bv) b0 = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};                                        \
    if (TWO) {                                                                             \
      bf16x8_t b1 = dequant8<J, Q>(D1);                                                    \
      if (!bv) b1 = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};                                      \
      mma_step_one<J, Q, MT>(As, ln, g, 4 * (J) + (Q), ms, bv, b0, &b1, acc0, &acc1);      \
    } else {                                                                               \
      mma_step_one<J, Q, MT>(As, ln, g, 4 * (J) + (Q), ms, bv, b0, nullptr, acc0, nullptr); \
    }                                                                                      \
  }
  MOEQ4_I(0, 0) MOEQ4_I(0, 1) MOEQ4_I(0, 2) MOEQ4_I(0, 3)
  MOEQ4_I(1, 0) MOEQ4_I(1, 1) MOEQ4_I(1, 2) MOEQ4_I(1, 3)
  MOEQ4_I(2, 0) MOEQ4_I(2, 1) MOEQ4_I(2, 2) MOEQ4_I(2, 3)
  MOEQ4_I(3, 0) MOEQ4_I(3, 1) MOEQ4_I(3, 2) MOEQ4_I(3, 3)
#undef MOEQ4_I
}

// Stage the activation tile of one K-step: rows r < rows, 16-byte chunks
// c < 4*nblk of source row src(r) (bf16 [.. ][K]).
template <int BM, typename RowFn>
__device__ __forceinline__ void stage_a(uint16_t* As, int rows, int nblk, int kofs, RowFn src) {
  const int nchunk = 4 * nblk;
  for (int idx = threadIdx.x; idx < BM * 32; idx += blockDim.x) {
    const int r = idx / 32, c = idx % 32;
    if (r < rows && c < nchunk) {
      const uint4 v = *reinterpret_cast<const uint4*>(src(r) + kofs + 8 * c);
      *reinterpret_cast<uint4*>(As + r * GLDA + 8 * c) = v;
    }
  }
}

// ---------------------------------------------------------------- gate/up
template <int MT>
__global__ void __launch_bounds__(256, 2) gateup_kernel(PrefillArgs a, int vec_b) {
  constexpr int BM = 32 * MT;
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * GLDA];
  __shared__ int32_t pref[GMaxE + 1];
  __shared__ int32_t tok[BM];
  const Tile t = find_tile<BM>(a.offsets, a.E, a.T, a.k, a.has_shared, blockIdx.y, pref);
  if (!t.valid) return;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, g = lane / 32;
  const int H = a.H, I = a.I, nb = H / BLK;
  for (int r = tid; r < BM; r += blockDim.x)
    tok[r] = (r < t.rows) ? ((t.expert >= 0) ? min(max(a.perm[t.pos0 + r] / a.k, 0), a.T - 1)
                                             : t.m0 + r)
                          : 0;
  const int ncol0 = blockIdx.x * GBN + wave * 32;
  const bool live = ncol0 < I;
  const int n = ncol0 + ln;
  const size_t rb = (size_t)nb * Q4B;
  const uint8_t* rowg = (t.expert >= 0) ? a.w_gate + ((size_t)t.expert * I + n) * rb : a.s_gate + (size_t)n * rb;
  const uint8_t* rowu = (t.expert >= 0) ? a.w_up + ((size_t)t.expert * I + n) * rb : a.s_up + (size_t)n * rb;
  const int ms = (t.rows + 31) / 32;

  f32x16_t accg[MT], accu[MT];
#pragma unroll
  for (int s = 0; s < MT; s++)
#pragma unroll
    for (int r = 0; r < 16; r++) { accg[s][r] = 0.0f; accu[s][r] = 0.0f; }

  const int nsteps = (nb + 7) / 8;
  for (int s = 0; s < nsteps; s++) {
    const int nblk = min(8, nb - 8 * s);
    __syncthreads();
    stage_a<BM>(As, t.rows, nblk, GKB * s, [&](int r) { return a.x + (size_t)tok[r] * H; });
    int nv = nblk - 4 * g;
    nv = nv < 0 ? 0 : (nv > 4 ? 4 : nv);
    uint32_t Dg[18], Du[18];
    if (live) {
      const size_t ofs = (size_t)(8 * s + 4 * g) * Q4B;
      load_run(rowg + ofs, nv, vec_b, Dg);
      load_run(rowu + ofs, nv, vec_b, Du);
    }
    __syncthreads();
    if (live) mma_step<MT, true>(As, ln, g, ms, nv, Dg, Du, accg, accu);
  }
  if (!live) return;
  // epilogue: D row = 8*(r/4) + 4*g + r%4 of each 32-row subtile, column n
#pragma unroll
  for (int sub = 0; sub < MT; sub++) {
    if (sub >= ms) break;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int row = 32 * sub + 8 * (r / 4) + 4 * g + (r % 4);
      if (row < t.rows) {
        const float gv = accg[sub][r], uv = accu[sub][r];
        const float hv = gv / (1.0f + __expf(-gv)) * uv;
        a.h[(size_t)(t.pos0 + row) * I + n] = f32_to_bf16_bits(hv);
      }
    }
  }
}

// ---------------------------------------------------------------- down
template <int MT>
__global__ void __launch_bounds__(256, 2) down_kernel(PrefillArgs a, int vec_b) {
  constexpr int BM = 32 * MT;
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * GLDA];
  __shared__ int32_t pref[GMaxE + 1];
  const Tile t = find_tile<BM>(a.offsets, a.E, a.T, a.k, a.has_shared, blockIdx.y, pref);
  if (!t.valid) return;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, g = lane / 32;
  const int H = a.H, I = a.I, nb = I / BLK;
  const int ncol0 = blockIdx.x * GBN + wave * 32;
  const bool live = ncol0 < H;
  const int n = ncol0 + ln;
  const size_t rb = (size_t)nb * Q4B;
  const uint8_t* rowd = (t.expert >= 0) ? a.w_down + ((size_t)t.expert * H + n) * rb : a.s_down + (size_t)n * rb;
  const int ms = (t.rows + 31) / 32;

  f32x16_t acc[MT], dummy[MT];
#pragma unroll
  for (int s = 0; s < MT; s++)
#pragma unroll
    for (int r = 0; r < 16; r++) { acc[s][r] = 0.0f; dummy[s][r] = 0.0f; }

  const int nsteps = (nb + 7) / 8;
  for (int s = 0; s < nsteps; s++) {
    const int nblk = min(8, nb - 8 * s);
    __syncthreads();
    stage_a<BM>(As, t.rows, nblk, GKB * s, [&](int r) { return a.h + (size_t)(t.pos0 + r) * I; });
    int nv = nblk - 4 * g;
    nv = nv < 0 ? 0 : (nv > 4 ? 4 : nv);
    uint32_t Dd[18];
    if (live) load_run(rowd + (size_t)(8 * s + 4 * g) * Q4B, nv, vec_b, Dd);
    __syncthreads();
    if (live) mma_step<MT, false>(As, ln, g, ms, nv, Dd, Dd, acc, dummy);
  }
  if (!live) return;
#pragma unroll
  for (int sub = 0; sub < MT; sub++) {
    if (sub >= ms) break;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int row = 32 * sub + 8 * (r / 4) + 4 * g + (r % 4);
      if (row < t.rows) {
        if (t.expert >= 0)
          a.o_perm[(size_t)(t.pos0 + row) * H + n] = f32_to_bf16_bits(acc[sub][r]);
        else
          a.y[(size_t)(t.m0 + row) * H + n] = acc[sub][r];
      }
    }
  }
}

// ---------------------------------------------------------------- fast path
// Shapes with K a multiple of 128 (whole 4-block steps) and 4-byte aligned
// weight rows.
//
// Tiles: expert e's c_e rows are cut into ceil(c_e / 160) near-equal tiles of
// a multiple of 32 rows, so a thin expert (c_e ~ T*k/E) is ONE tile and each
// of its weights is dequantised once per block of columns, not once per
// fixed-size piece (the thin-M cost the pages identify).
//
// Block: 8 waves, each computing two 32-column MFMA operands per activation
// fragment -- gate and up for the same 32 columns of I (gate/up kernel), or
// two 32-column groups of H (down kernel) -- so one 1 KB LDS read of A feeds
// two MFMAs.  gate/up blocks cover 256 columns of I, down blocks 512 of H;
// the 8 waves share one activation tile.
//
// Software pipeline, one K-step ahead, everything through LDS with direct
// global->LDS loads (no register staging):
//   - activations: the next step's tile [rows][16 chunks of 16 B] into the
//     other of two buffers; chunk c of row m sits at slot c ^ (m & 15), so
//     the 32 rows a wave reads for one MFMA hit distinct banks;
//   - weights: each wave's next-step bytes of its 32 (or 2x32) weight rows,
//     as 12-byte chunks of the rows' 72-byte step pieces (4 whole blocks), so
//     each 64-lane load touches a few cache lines instead of one line per
//     lane; the wave copies the current step's pieces into registers first,
//     then reuses its LDS region for the next step's;
// while the current step's MFMAs run.  Raw barriers (no memory fence) keep
// the prefetch in flight across them; each wave waits for its own loads of a
// buffer before the barrier that publishes it.
// K order inside a step: MFMA instruction i (0..7) takes, in lane half g,
// elements 8*(i%4)..+8 of block 2g + i/4 -- lane (n, g) reads blocks
// 2g, 2g+1 of weight row n and activations at step offset 64g + 8i.
constexpr int FMAXS = 5;                 // max 32-row subtiles per tile
constexpr int FMAXR = 32 * FMAXS;        // max rows per tile

// Tile mt, found by every wave on its own (registers only, no LDS):
// expert e owns ceil(c_e / FMAXR) consecutive tile indices, experts in
// order, then the shared expert's tiles.
__device__ __forceinline__ Tile find_tile_bal(const int32_t* __restrict__ offsets, int E, int T,
                                              int k, int has_shared, int mt) {
  const int lane = threadIdx.x % 64;
  Tile t;
  t.valid = 0;
  t.rows = 0;
  t.pos0 = 0;
  t.expert = -1;
  t.m0 = 0;
  int carry = 0, c = -1, q = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    int ce = 0;
    if (e < E) ce = offsets[e + 1] - offsets[e];
    const int nt = (ce + FMAXR - 1) / FMAXR;
    int incl = nt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    const unsigned long long hit = __ballot(carry + incl > mt);
    if (hit) {
      const int f = __builtin_ctzll(hit);
      t.expert = base + f;
      c = __shfl(ce, f, 64);
      q = mt - (carry + __shfl(incl, f, 64) - __shfl(nt, f, 64));
      break;
    }
    carry += __shfl(incl, 63, 64);
  }
  if (c < 0) {
    if (!has_shared) return t;
    c = T;
    q = mt - carry;
  }
  const int nt = (c + FMAXR - 1) / FMAXR;
  if (q < 0 || q >= nt) return t;
  const int tr = 32 * (((c + nt - 1) / nt + 31) / 32);   // rows per tile, <= FMAXR
  t.m0 = q * tr;
  t.rows = min(tr, c - t.m0);
  if (t.rows <= 0) return t;
  t.valid = 1;
  t.pos0 = (t.expert >= 0) ? offsets[t.expert] + t.m0 : T * k + t.m0;
  return t;
}

__device__ __forceinline__ void lds_load16(const void* g, uint16_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  // s_waitcnt vmcnt(N), expcnt/lgkmcnt untouched (gfx9 encoding)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void load_run2(const uint8_t* __restrict__ p, uint32_t (&D)[9]) {
  const uint32_t* s = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
  for (int v = 0; v < 9; v++) D[v] = s[v];
}

__device__ __forceinline__ void lds_load12(const void* g, uint32_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 12, 0, 0);
}

// One K-step: 8 k-slices x MS subtiles x 2 operands (weights in D0, D1).
template <int MS>
__device__ __forceinline__ void mma_step128(const uint16_t* As, const uint32_t (&D0)[9],
                                            const uint32_t (&D1)[9], int ln, int g,
                                            f32x16_t (&acc0)[FMAXS], f32x16_t (&acc1)[FMAXS]) {
  const int x = ln & 15;
  const uint16_t* base = As + ln * 128;
#define MOEQ4_F(J, Q)                                                                      \
  {                                                                                        \
    const bf16x8_t b0 = dequant8<J, Q>(D0);                                                \
    const bf16x8_t b1 = dequant8<J, Q>(D1);                                                \
    const int ofs = 8 * ((8 * g + 4 * (J) + (Q)) ^ x);                                     \
    _Pragma("unroll") for (int sub = 0; sub < MS; sub++) {                                 \
      const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(base + sub * 32 * 128 + ofs); \
      acc0[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b0, acc0[sub], 0, 0, 0);     \
      acc1[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b1, acc1[sub], 0, 0, 0);     \
    }                                                                                      \
  }
  MOEQ4_F(0, 0) MOEQ4_F(0, 1) MOEQ4_F(0, 2) MOEQ4_F(0, 3)
  MOEQ4_F(1, 0) MOEQ4_F(1, 1) MOEQ4_F(1, 2) MOEQ4_F(1, 3)
#undef MOEQ4_F
}

constexpr int FWAVES = 8;
// 12-byte direct loads land at a 16-byte lane stride: one operand's 32 rows
// x 6 chunks take 192 x 16 B of LDS
constexpr int FBOP = 192 * 4;            // dwords per operand region
constexpr int FBW = 2 * FBOP;            // dwords per wave

// LDS of one block: two activation buffers of FMAXR rows x 256 B (80 KB) and
// one weight region per wave (8 x 6 KB).
struct FastSmem {
  uint16_t a0[FMAXR * 128];
  uint16_t a1[FMAXR * 128];
  uint32_t b[FWAVES * FBW];
};

// Lane (n, g)'s 36 weight bytes of a step: row n's chunks 3g..3g+2.
__device__ __forceinline__ void read_piece(const uint32_t* op, int n, int g, uint32_t (&D)[9]) {
#pragma unroll
  for (int j = 0; j < 3; j++) {
    const uint32_t* c = op + 4 * (6 * n + 3 * g + j);
    D[3 * j] = c[0];
    D[3 * j + 1] = c[1];
    D[3 * j + 2] = c[2];
  }
}

template <int MS, bool GATEUP>
__device__ __forceinline__ void fast_tile(const PrefillArgs& a, const Tile& t, FastSmem& sm) {
  constexpr int NA = MS;                       // activation 1 KB loads per wave per step
  constexpr int NB = 6;                        // weight 12-byte-chunk loads per wave per step
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, g = lane / 32;
  const int H = a.H, I = a.I;
  const int N = GATEUP ? I : H, K = GATEUP ? H : I;
  const int nb = K / BLK;
  // gate/up: 32 columns per wave; down: 64 columns per wave (two groups)
  const int ncol0 = GATEUP ? blockIdx.x * 256 + wave * 32 : blockIdx.x * 512 + wave * 64;
  const bool live0 = ncol0 < N;
  const bool live1 = GATEUP ? live0 : (ncol0 + 32 < N);
  const int c0 = min(ncol0, N - 32);           // dead groups load valid rows and store nothing
  const int c1 = GATEUP ? c0 : min(ncol0 + 32, N - 32);
  const size_t rb = (size_t)nb * Q4B;
  const uint8_t *rows0, *rows1;                // first weight row of each 32-row operand
  if (GATEUP) {
    rows0 = (t.expert >= 0) ? a.w_gate + ((size_t)t.expert * I + c0) * rb : a.s_gate + (size_t)c0 * rb;
    rows1 = (t.expert >= 0) ? a.w_up + ((size_t)t.expert * I + c0) * rb : a.s_up + (size_t)c0 * rb;
  } else {
    const uint8_t* wd = (t.expert >= 0) ? a.w_down + (size_t)t.expert * H * rb : a.s_down;
    rows0 = wd + (size_t)c0 * rb;
    rows1 = wd + (size_t)c1 * rb;
  }
  // weight loads: a row's 72 bytes of the step are six 12-byte chunks; wave-
  // load v covers chunks 64v..64v+63 of the operand's 32 rows
  uint32_t boff[3];
#pragma unroll
  for (int v = 0; v < 3; v++) {
    const int d = 64 * v + lane;
    boff[v] = (uint32_t)(d / 6) * (uint32_t)rb + 12u * (uint32_t)(d % 6);
  }
  // activation loads: 4 rows per 1 KB wave-load
  const uint16_t* abase = GATEUP ? a.x : a.h + (size_t)t.pos0 * I;
  uint32_t src[NA];
#pragma unroll
  for (int q = 0; q < NA; q++) {
    const int jj = wave + FWAVES * q;
    const int m = min(4 * jj + (lane >> 4), t.rows - 1);   // padding rows repeat the last row
    const int c = ((lane & 15) ^ ((4 * jj + (lane >> 4)) & 15));
    uint32_t rowel;
    if (GATEUP) {
      const int tk = (t.expert >= 0) ? a.perm[t.pos0 + m] / a.k : t.m0 + m;
      rowel = (uint32_t)min(max(tk, 0), a.T - 1) * (uint32_t)H;
    } else {
      rowel = (uint32_t)m * (uint32_t)I;
    }
    src[q] = rowel + 8u * (uint32_t)c;
  }
  uint32_t* bw = sm.b + wave * FBW;
  auto issue_a = [&](int s, uint16_t* abuf) {
#pragma unroll
    for (int q = 0; q < NA; q++) lds_load16(abase + src[q] + 128 * s, abuf + (wave + FWAVES * q) * 512);
  };
  auto issue_b = [&](int s) {
    const size_t ko = (size_t)s * 72;
#pragma unroll
    for (int v = 0; v < 3; v++) lds_load12(rows0 + ko + boff[v], bw + 256 * v);
#pragma unroll
    for (int v = 0; v < 3; v++) lds_load12(rows1 + ko + boff[v], bw + FBOP + 256 * v);
  };
  // step s: A(s) and B(s) landed; copy B(s) to registers, refill with B(s+1)
  auto take_b = [&](int s, int nsteps, uint32_t (&D0)[9], uint32_t (&D1)[9]) {
    read_piece(bw, ln, g, D0);
    read_piece(bw + FBOP, ln, g, D1);
    if (s + 1 < nsteps) {
      __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0): the piece reads are done
      issue_b(s + 1);
    }
  };

  f32x16_t acc0[FMAXS], acc1[FMAXS];
#pragma unroll
  for (int q = 0; q < FMAXS; q++)
#pragma unroll
    for (int r = 0; r < 16; r++) { acc0[q][r] = 0.0f; acc1[q][r] = 0.0f; }

  const int nsteps = nb / 4;
  uint32_t D0[9], D1[9];
  issue_b(0);
  issue_a(0, sm.a0);
  // per step s: [barrier] issue A(s+1); wait (everything but A(s+1));
  // [barrier]; take B(s) and issue B(s+1); MFMAs of step s.
  // Pairs of steps use buffer 0 then buffer 1; a single loop exit keeps the
  // accumulators in place.
  const int npairs = nsteps / 2;
  for (int pi = 0; pi < npairs; pi++) {
    const int s = 2 * pi;
    __builtin_amdgcn_s_barrier();               // buffer 1 free (step s-1 done everywhere)
    issue_a(s + 1, sm.a1);
    wait_vm<NA>();                              // own A(s), B(s) complete
    __builtin_amdgcn_s_barrier();               // step s tile complete everywhere
    take_b(s, nsteps, D0, D1);
    mma_step128<MS>(sm.a0, D0, D1, ln, g, acc0, acc1);
    __builtin_amdgcn_s_barrier();
    if (s + 2 < nsteps) {
      issue_a(s + 2, sm.a0);
      wait_vm<NA>();
    } else {
      wait_vm<0>();
    }
    __builtin_amdgcn_s_barrier();
    take_b(s + 1, nsteps, D0, D1);
    mma_step128<MS>(sm.a1, D0, D1, ln, g, acc0, acc1);
  }
  if (nsteps & 1) {                             // last step in buffer 0
    wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    take_b(nsteps - 1, nsteps, D0, D1);
    mma_step128<MS>(sm.a0, D0, D1, ln, g, acc0, acc1);
  }
  const int n0 = c0 + ln, n1 = c1 + ln;
#pragma unroll
  for (int sub = 0; sub < MS; sub++)
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int rr = 32 * sub + 8 * (r / 4) + 4 * g + (r % 4);
      if (rr >= t.rows) continue;
      if (GATEUP) {
        if (!live0) continue;
        const float gv = acc0[sub][r], uv = acc1[sub][r];
        const float hv = __fdividef(gv, 1.0f + __expf(-gv)) * uv;
        a.h[(size_t)(t.pos0 + rr) * I + n0] = f32_to_bf16_bits(hv);
      } else if (t.expert >= 0) {
        if (live0) a.o_perm[(size_t)(t.pos0 + rr) * H + n0] = f32_to_bf16_bits(acc0[sub][r]);
        if (live1) a.o_perm[(size_t)(t.pos0 + rr) * H + n1] = f32_to_bf16_bits(acc1[sub][r]);
      } else {
        if (live0) a.y[(size_t)(t.m0 + rr) * H + n0] = acc0[sub][r];
        if (live1) a.y[(size_t)(t.m0 + rr) * H + n1] = acc1[sub][r];
      }
    }
}

template <bool GATEUP>
__global__ void __launch_bounds__(512, 2) gemm_fast_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) FastSmem sm;
  const Tile t = find_tile_bal(a.offsets, a.E, a.T, a.k, a.has_shared, blockIdx.y);
  if (!t.valid) return;
  const int ms = (t.rows + 31) / 32;
  switch (ms) {
    case 1: fast_tile<1, GATEUP>(a, t, sm); break;
    case 2: fast_tile<2, GATEUP>(a, t, sm); break;
    case 3: fast_tile<3, GATEUP>(a, t, sm); break;
    case 4: fast_tile<4, GATEUP>(a, t, sm); break;
    default: fast_tile<5, GATEUP>(a, t, sm); break;
  }
}

// ---------------------------------------------------------------- combine
__global__ void __launch_bounds__(256) combine_kernel(PrefillArgs a) {
  const int H = a.H, k = a.k;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = H / 8;
  if (idx >= (int64_t)a.T * per_row) return;
  const int t = (int)(idx / per_row), c = (int)(idx % per_row) * 8;
  float acc[8];
  float* yr = a.y + (size_t)t * H + c;
  if (a.has_shared) {
    const float4 u0 = *reinterpret_cast<const float4*>(yr);
    const float4 u1 = *reinterpret_cast<const float4*>(yr + 4);
    acc[0] = u0.x; acc[1] = u0.y; acc[2] = u0.z; acc[3] = u0.w;
    acc[4] = u1.x; acc[5] = u1.y; acc[6] = u1.z; acc[7] = u1.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = 0.0f;
  }
  for (int s = 0; s < k; s++) {
    const int p = min(max(a.inv_perm[(size_t)t * k + s], 0), a.T * k - 1);
    const float w = a.topk_w[(size_t)t * k + s];
    const uint4 v = *reinterpret_cast<const uint4*>(a.o_perm + (size_t)p * H + c);
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      acc[2 * i] += w * bf16_bits_to_f32(q[i] & 0xffffu);
      acc[2 * i + 1] += w * bf16_bits_to_f32(q[i] >> 16);
    }
  }
  *reinterpret_cast<float4*>(yr) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(yr + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// ---------------------------------------------------------------- launch
hipError_t launch_prefill(const PrefillArgs& a, int stages, hipStream_t stream) {
  constexpr int MT = 4, BM = 32 * MT;
  const int64_t assignments = (int64_t)a.T * a.k;
  const int mtiles = (int)(assignments / BM) + a.E + (a.has_shared ? (a.T + BM - 1) / BM : 0);
  const int ftiles = (int)(assignments / FMAXR) + a.E + (a.has_shared ? (a.T + FMAXR - 1) / FMAXR : 0);
  const int vec_g = ((a.H / BLK) % 4 == 0) && (((uintptr_t)a.w_gate | (uintptr_t)a.w_up) % 8 == 0) &&
                    (!a.has_shared || (((uintptr_t)a.s_gate | (uintptr_t)a.s_up) % 8 == 0));
  const int vec_d = ((a.I / BLK) % 4 == 0) && ((uintptr_t)a.w_down % 8 == 0) &&
                    (!a.has_shared || ((uintptr_t)a.s_down % 8 == 0));
  const bool fast_g = (a.H / BLK) % 4 == 0 && ((uintptr_t)a.x % 16 == 0) &&
                      (((uintptr_t)a.w_gate | (uintptr_t)a.w_up) % 4 == 0) &&
                      (!a.has_shared || (((uintptr_t)a.s_gate | (uintptr_t)a.s_up) % 4 == 0));
  const bool fast_d = (a.I / BLK) % 4 == 0 && ((uintptr_t)a.h % 16 == 0) &&
                      ((uintptr_t)a.w_down % 4 == 0) && (!a.has_shared || ((uintptr_t)a.s_down % 4 == 0));
  hipError_t err = hipSuccess;
  if (stages & 1) {
    if (fast_g)
      hipLaunchKernelGGL((gemm_fast_kernel<true>), dim3((a.I + 255) / 256, ftiles), dim3(512), 0,
                         stream, a);
    else
      hipLaunchKernelGGL((gateup_kernel<MT>), dim3((a.I + GBN - 1) / GBN, mtiles), dim3(256), 0,
                         stream, a, vec_g);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (stages & 2) {
    if (fast_d)
      hipLaunchKernelGGL((gemm_fast_kernel<false>), dim3((a.H + 511) / 512, ftiles), dim3(512), 0,
                         stream, a);
    else
      hipLaunchKernelGGL((down_kernel<MT>), dim3((a.H + GBN - 1) / GBN, mtiles), dim3(256), 0,
                         stream, a, vec_d);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (stages & 4) {
    const int64_t n = (int64_t)a.T * (a.H / 8);
    hipLaunchKernelGGL(combine_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, stream, a);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace moeq4
