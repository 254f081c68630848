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
//   gateup/down (generic, any K a multiple of 32): per (expert tile of <= 128
//            rows, 128 columns), 4 waves each owning 32 output columns and
//            every row of the tile, activation rows staged in LDS per K-step
//            of 256; one launch per projection.
//   g2 unit (K a multiple of 64): 4-wave blocks, two per CU, balanced
//            tiles of <= 160 rows, K-steps of 64, direct global->LDS
//            activation loads double buffered, weights one step ahead in
//            registers, column blocks of a tile on one XCD.  Run as
//            gemm_ffn (gate/up units, then down units that wait per tile,
//            in one launch) or as gemm_g2 (one projection, for single stages).
//   combine  y[t] += sum_s w[t,s] * O[inv_perm[t*k+s]]
// Epilogues: gate/up writes h = silu(G) * U in bf16 (rows in segment order);
// down writes each routed row's output in bf16 (segment order) and the shared
// expert's output in fp32 straight into y.
//
// Dequantisation: each weight value (q - 8) * d is exact in fp32 (a 4-bit
// integer times an 11-bit significand) and is rounded once to bf16, in
// registers, once per weight per block.  K inside a step is permuted
// identically for both operands (a dot product does not depend on the order
// of its terms), so the 8 bf16 values a lane feeds one MFMA are one element
// group of one Q4 block.
//
// Tiles are found on the device from expert_offsets (no host round trip).
#include "launch.hpp"
#include "device_math.hpp"
#include "w4a8.hpp"
#include "tiles.hpp"

namespace moeq4 {

typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int GKB = 256;          // K elements per step (8 Q4 blocks)
constexpr int GLDA = GKB + 8;     // LDS row stride in bf16 elements (16-byte pad)
constexpr int GBN = 128;          // output columns per block (4 waves x 32)
constexpr int GMaxE = 1024;


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
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(w), "v"(m));
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

// ---------------------------------------------------------------- balanced tiles
// Expert e's c_e rows are cut into ceil(c_e / 160) near-equal tiles of a
// multiple of 32 rows, so a thin expert (c_e ~ T*k/E) is ONE tile and each of
// its weights is dequantised once per column block, not once per fixed-size
// piece (the thin-M cost the pages identify).
constexpr int FMAXS = 5;                 // max 32-row subtiles per tile
constexpr int FMAXR = 32 * FMAXS;        // max rows per tile
static_assert(FMAXR == kPrefillTileRows, "tile rows shared with the workspace bound");

__device__ __forceinline__ void lds_load16(const void* g, uint16_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  // s_waitcnt vmcnt(N), expcnt/lgkmcnt untouched (gfx9 encoding)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------- two blocks per CU
// Shapes with K a multiple of 64, weights in the tile order of q4_tile.
//
// Block: 4 waves and 40 KB of LDS, so two blocks share a CU and one block's
// barrier and load waits are covered by the other's MFMAs.  A block owns one
// tile (<= 160 rows of one expert segment, found as in find_tile_bal) and a
// column block: gate/up 128 columns of I (wave w: gate and up rows
// 32w..32w+31, two MFMA operands per activation fragment), down 256 columns
// of H (wave w: two groups of 32 columns).
//
// K-step 64 = two Q4 blocks.  Lane (n, g) owns block g of the step of weight
// row n: MFMA slice i (0..3) takes, in lane half g, elements 8i..8i+7 of that
// block (the same permutation of K on both operands).  In tile order a step of
// 32 rows is one 1152-byte piece: the lane reads its 16 nibble bytes at 16 *
// lane and its scale at 1024 + 2 * lane, one step ahead into registers, so a
// wave's weight loads cover 9 whole cache lines (row-major blocks would put
// every lane on a line of its own).
//
// Activations: the step's [rows][64] bf16 tile lands in LDS by direct
// global->LDS loads, double buffered; 16-byte chunk cc of row m sits at slot
// cc ^ (m & 7) ^ ((m >> 3) & 1), so the rows a fragment read touches in one
// LDS cycle fall in distinct banks for 32 or 64 banks.  One barrier per step.
//
// Column blocks of a tile are placed on one XCD (blocks are dealt to the 8
// XCDs round robin): block b serves tile 8 * ((b / 8) / NCB) + b % 8 and
// column block (b / 8) % NCB, so a tile's activation rows are fetched into
// that XCD's L2 once.
constexpr int G2W = 4;                  // waves per block
constexpr int G2S = FMAXS;              // max 32-row subtiles per tile
constexpr int G2R = 32 * G2S;           // max rows per tile
constexpr int G2K = 64;                 // K per step

struct G2Smem {
  uint16_t a[2][G2R * G2K];
  // the fused launch's wait result, read by every wave after a barrier (kept
  // in the tile's LDS object: a second __shared__ object made the compiler
  // wait for every load in flight, the next step's included, before each
  // fragment read of the step loop)
  int gave_up;
};

__device__ __forceinline__ int g2_slot(int cc, int m) { return cc ^ (m & 7) ^ ((m >> 3) & 1); }

#if defined(__HIP_DEVICE_COMPILE__)   // buffer descriptors exist only in the device pass
typedef uint32_t g2_u32x4 __attribute__((ext_vector_type(4)));

// Step s of the lane's weights from a group's pieces: nibble dwords D[0..3]
// at vn = 16 * lane, the fp16 scale bits in D[4] at 1024 + 2 * lane.
__device__ __forceinline__ void g2_load_w(__amdgpu_buffer_rsrc_t r, uint32_t vn, int s, uint32_t (&D)[5]) {
  const g2_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, vn, 1152 * s, 0);
  D[0] = v.x;
  D[1] = v.y;
  D[2] = v.z;
  D[3] = v.w;
  D[4] = __builtin_amdgcn_raw_buffer_load_b16(r, 1024u + (vn >> 3), 1152 * s, 0);
}

#endif

// 8 bf16 weights of element group Q of the lane's block: scale d, nibble
// dwords nib[0..3] (byte j of the 16 holds element j low, j+16 high).
// A byte holding one nibble q, read as an OCP fp8 e4m3 value, is exactly
// q * 2^-9 (q < 8: the subnormals m * 2^-9; q >= 8: (8 + m) * 2^-9), so one
// v_cvt_pk_f32_fp8 turns two nibbles into fp32 (a high nibble is shifted
// down first).  Then (q - 8) * d = fma(q * 2^-9, d * 2^9, -8 d), exact in
// fp32, rounded once to bf16: the same bits as a byte-by-byte conversion,
// in 19 VALU instructions per 8 weights instead of 22.
template <int Q>
__device__ __forceinline__ bf16x8_t g2_deq(const uint32_t* nib, float d) {
  const float off = -8.0f * d;
  const float mul = d * 512.0f;
  const uint32_t w0 = nib[2 * (Q & 1)], w1 = nib[2 * (Q & 1) + 1];
  const uint32_t v0 = ((Q >> 1) ? (w0 >> 4) : w0) & 0x0f0f0f0fu;
  const uint32_t v1 = ((Q >> 1) ? (w1 >> 4) : w1) & 0x0f0f0f0fu;
  const f32x2_t p[4] = {__builtin_amdgcn_cvt_pk_f32_fp8((int)v0, false), __builtin_amdgcn_cvt_pk_f32_fp8((int)v0, true),
                        __builtin_amdgcn_cvt_pk_f32_fp8((int)v1, false), __builtin_amdgcn_cvt_pk_f32_fp8((int)v1, true)};
  float f[8];
#pragma unroll
  for (int b = 0; b < 4; b++) {
    f[2 * b] = __builtin_fmaf(p[b].x, mul, off);
    f[2 * b + 1] = __builtin_fmaf(p[b].y, mul, off);
  }
  uint32_t w[4];
#pragma unroll
  for (int p = 0; p < 4; p++) w[p] = pack_bf16x2(f[2 * p], f[2 * p + 1]);
  return __builtin_bit_cast(bf16x8_t, w);
}

// Scheduling groups for one slice: each MFMA is followed by its share of the
// next slice's dequantisation VALU, and every second one by a fragment read.
template <int MS>
__device__ __forceinline__ void g2_interleave() {
#pragma unroll
  for (int j = 0; j < 2 * MS; j++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, (40 + 2 * MS - 1) / (2 * MS), 0);  // VALU
    if (j & 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);            // DS read
  }
}

__device__ __forceinline__ void g2_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int MS, bool GATEUP>
__device__ __forceinline__ void g2_tile(const PrefillArgs& a, const Tile& t, int cb, G2Smem& sm) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int tid = threadIdx.x, lane = tid % 64, ln = lane % 32, g = lane / 32;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int H = a.H, I = a.I;
  const int N = GATEUP ? I : H, K = GATEUP ? H : I;
  const int nsteps = K / G2K;
  const size_t rb = (size_t)(K / BLK) * Q4B;
  const int col0 = GATEUP ? cb * 128 + wave * 32 : cb * 256 + wave * 64;
  const int col1 = GATEUP ? col0 : col0 + 32;
  const bool live0 = col0 < N, live1 = col1 < N;
  const int c0 = min(col0, N - 32), c1 = min(col1, N - 32);   // dead groups load valid rows
  const uint8_t *w0, *w1;
  // a 32-row group keeps its row-major byte range in tile order
  if (GATEUP) {
    w0 = (t.expert >= 0) ? a.t_gate + ((size_t)t.expert * I + c0) * rb : a.ts_gate + (size_t)c0 * rb;
    w1 = (t.expert >= 0) ? a.t_up + ((size_t)t.expert * I + c0) * rb : a.ts_up + (size_t)c0 * rb;
  } else {
    const uint8_t* wd = (t.expert >= 0) ? a.t_down + (size_t)t.expert * H * rb : a.ts_down;
    w0 = wd + (size_t)c0 * rb;
    w1 = wd + (size_t)c1 * rb;
  }
  // Raw buffer resources: the wave's two 32-row groups (their tile-order
  // pieces) and the activation rows.  The per-step offset is a scalar, so the
  // loop computes no addresses; an offset past num_records would read zeros.
  const __amdgpu_buffer_rsrc_t rw0 = uniform_buffer_rsrc(w0, (uint32_t)(32 * rb));
  const __amdgpu_buffer_rsrc_t rw1 = uniform_buffer_rsrc(w1, (uint32_t)(32 * rb));
  const uint32_t vn = 16u * (uint32_t)lane;                   // the lane's nibbles in a piece (scale: 1024 + 2 * lane)

  // activation rows: wave-load j = wave + 4q covers tile rows 8j..8j+7
  const uint16_t* abase = GATEUP ? a.x : a.h + (size_t)t.pos0 * I;
  const __amdgpu_buffer_rsrc_t ra =
      uniform_buffer_rsrc(abase, GATEUP ? (uint32_t)a.T * (uint32_t)H * 2u : (uint32_t)t.rows * (uint32_t)I * 2u);
  uint32_t voff[MS];                                          // byte offset of the lane's 16-byte chunk, step 0
#pragma unroll
  for (int q = 0; q < MS; q++) {
    const int r = 8 * (wave + G2W * q) + lane / 8;            // LDS row
    const int m = min(r, t.rows - 1);                         // padding rows repeat the last row
    uint32_t rowel;
    if (GATEUP) {
      const int tk = (t.expert >= 0) ? a.perm[t.pos0 + m] / a.k : t.m0 + m;
      rowel = (uint32_t)min(max(tk, 0), a.T - 1) * (uint32_t)H;
    } else {
      rowel = (uint32_t)m * (uint32_t)I;
    }
    voff[q] = 2u * (rowel + 8u * (uint32_t)g2_slot(lane & 7, r));
  }
  auto issue_a = [&](int s, uint16_t* buf) {
#pragma unroll
    for (int q = 0; q < MS; q++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(buf + (wave + G2W * q) * 512),
                                               16, voff[q], 2 * G2K * s, 0, 0);
  };

  f32x16_t acc0[MS], acc1[MS];
#pragma unroll
  for (int q = 0; q < MS; q++)
#pragma unroll
    for (int r = 0; r < 16; r++) { acc0[q][r] = 0.0f; acc1[q][r] = 0.0f; }

  // weights of step s land in W[s & 1]: the loop is unrolled by two so that
  // each register set has a fixed role and nothing is copied
  uint32_t W[2][2][5];
  issue_a(0, sm.a[0]);
  g2_load_w(rw0, vn, 0, W[0][0]);
  g2_load_w(rw1, vn, 0, W[0][1]);
  // fragment read offsets (elements) inside a buffer, per slice i: row 32*sub + ln
  int aofs[4];
#pragma unroll
  for (int i = 0; i < 4; i++) aofs[i] = ln * G2K + 8 * g2_slot(4 * g + i, ln);

  for (int s0 = 0; s0 < nsteps; s0 += 2) {
#pragma unroll
  for (int P = 0; P < 2; P++) {
    const int s = s0 + P;
    if (P == 1 && s >= nsteps) break;
    uint16_t* cur = sm.a[P];
    wait_vm<0>();                                // own A(s) and W(s) landed (issued a step ago)
    g2_barrier();                                // everyone's A(s) landed; step s-1 done
    const uint32_t* n0 = W[P][0];
    const uint32_t* n1 = W[P][1];
    const float d0 = f16_bits_to_f32(n0[4]);
    const float d1 = f16_bits_to_f32(n1[4]);
    // next step's loads; the last step fetches its own data again (in bounds,
    // unused) so the body stays one branch-free block
    const int sn = min(s + 1, nsteps - 1);
    issue_a(sn, sm.a[P ^ 1]);
    g2_load_w(rw0, vn, sn, W[P ^ 1][0]);
    g2_load_w(rw1, vn, sn, W[P ^ 1][1]);
    bf16x8_t b0 = g2_deq<0>(n0, d0), b1 = g2_deq<0>(n1, d1);
    bf16x8_t avs[MS];
#pragma unroll
    for (int sub = 0; sub < MS; sub++) avs[sub] = *reinterpret_cast<const bf16x8_t*>(cur + sub * 32 * G2K + aofs[0]);
    __builtin_amdgcn_sched_barrier(0);
    // slice Q's MFMAs with slice Q+1's dequantisation and fragment reads
    // interleaved between them: a wave issues in order, so VALU work only
    // runs under its own MFMAs when it sits between them in the stream
#define MOEQ4_G2(Q)                                                                            \
  {                                                                                            \
    bf16x8_t c0, c1;                                                                           \
    _Pragma("unroll") for (int sub = 0; sub < MS; sub++) {                                     \
      acc0[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(avs[sub], b0, acc0[sub], 0, 0, 0);   \
      acc1[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(avs[sub], b1, acc1[sub], 0, 0, 0);   \
      if (Q < 3) avs[sub] = *reinterpret_cast<const bf16x8_t*>(cur + sub * 32 * G2K + aofs[(Q + 1) & 3]); \
    }                                                                                          \
    if (Q < 3) {                                                                               \
      c0 = g2_deq<(Q + 1) & 3>(n0, d0);                                                        \
      c1 = g2_deq<(Q + 1) & 3>(n1, d1);                                                        \
      g2_interleave<MS>();                                                                     \
      b0 = c0;                                                                                 \
      b1 = c1;                                                                                 \
    }                                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                         \
  }
    MOEQ4_G2(0) MOEQ4_G2(1) MOEQ4_G2(2) MOEQ4_G2(3)
#undef MOEQ4_G2
  }
  }
  wait_vm<0>();                                  // the repeated last fetch has landed in LDS
  // Stores through a buffer descriptor over the tile's output rows (h, o_perm
  // or, for the shared expert, y): a row past t.rows lies past the
  // descriptor's end and its store is dropped, so the padding rows need no
  // test, and each store adds one wave-uniform row offset to the lane's
  // offset instead of forming a 64-bit address.  (Per-element 64-bit
  // addresses and row tests made the epilogue of a down unit about a third
  // of its time.)  Pairs of values are rounded to bf16 by one conversion.
  const int Nout = GATEUP ? I : H;
  // (wave-uniform values made visibly so: scalar row strides and branches)
  const int routed = __builtin_amdgcn_readfirstlane(t.expert >= 0 ? 1 : 0);
  const int l0 = __builtin_amdgcn_readfirstlane(live0 ? 1 : 0), l1 = __builtin_amdgcn_readfirstlane(live1 ? 1 : 0);
  const int esz = (!GATEUP && !routed) ? 4 : 2;
  const void* obase = GATEUP ? static_cast<const void*>(a.h + (size_t)t.pos0 * I)
                    : routed ? static_cast<const void*>(a.o_perm + (size_t)t.pos0 * H)
                             : static_cast<const void*>(a.y + (size_t)t.m0 * H);
  const __amdgpu_buffer_rsrc_t ro = uniform_buffer_rsrc(obase, (uint32_t)t.rows * (uint32_t)Nout * (uint32_t)esz);
  const uint32_t rstride = __builtin_amdgcn_readfirstlane((uint32_t)(Nout * esz));   // bytes per output row
  const uint32_t vb0 = (uint32_t)((4 * g * Nout + c0 + ln) * esz);
  const uint32_t vb1 = (uint32_t)((4 * g * Nout + c1 + ln) * esz);
  auto off = [&](uint32_t vb, int sub, int r) { return vb + (uint32_t)(32 * sub + 8 * (r / 4) + (r % 4)) * rstride; };
  if (GATEUP) {
    if (l0) {
#pragma unroll
      for (int sub = 0; sub < MS; sub++)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float hv[2];
#pragma unroll
          for (int i = 0; i < 2; i++) {
            const float gv = acc0[sub][r + i], uv = acc1[sub][r + i];
            hv[i] = __fdividef(gv, 1.0f + __expf(-gv)) * uv;
          }
          const uint32_t hb = bf16x2_bits(hv[0], hv[1]);
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)hb, ro, off(vb0, sub, r), 0, 0);
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(hb >> 16), ro, off(vb0, sub, r + 1), 0, 0);
        }
    }
  } else if (routed) {
    if (l0 && l1) {
#pragma unroll
      for (int sub = 0; sub < MS; sub++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const uint32_t ob = bf16x2_bits(acc0[sub][r], acc1[sub][r]);
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)ob, ro, off(vb0, sub, r), 0, 0);
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(ob >> 16), ro, off(vb1, sub, r), 0, 0);
        }
    } else if (l0) {
#pragma unroll
      for (int sub = 0; sub < MS; sub++)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const uint32_t ob = bf16x2_bits(acc0[sub][r], acc0[sub][r + 1]);
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)ob, ro, off(vb0, sub, r), 0, 0);
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(ob >> 16), ro, off(vb0, sub, r + 1), 0, 0);
        }
    }
  } else {
#pragma unroll
    for (int sub = 0; sub < MS; sub++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        if (l0) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc0[sub][r]), ro, off(vb0, sub, r), 0, 0);
        if (l1) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc1[sub][r]), ro, off(vb1, sub, r), 0, 0);
      }
  }
#endif
}

template <bool GATEUP>
__global__ void __launch_bounds__(256, 2) gemm_g2_kernel(PrefillArgs a, int ncb) {
  __shared__ __attribute__((aligned(16))) G2Smem sm;
  const int b = blockIdx.x, q = b / 8;
  const int tile = 8 * (q / ncb) + b % 8, cb = q % ncb;
  const Tile t = find_tile_bal<FMAXR>(a.offsets, a.E, a.T, a.k, a.has_shared, tile);
  if (!t.valid) return;
  switch ((t.rows + 31) / 32) {
    case 1: g2_tile<1, GATEUP>(a, t, cb, sm); break;
    case 2: g2_tile<2, GATEUP>(a, t, cb, sm); break;
    case 3: g2_tile<3, GATEUP>(a, t, cb, sm); break;
    case 4: g2_tile<4, GATEUP>(a, t, cb, sm); break;
    default: g2_tile<5, GATEUP>(a, t, cb, sm); break;
  }
}

// ---------------------------------------------------------------- fused gate/up -> down
// One launch for both grouped GEMMs.  Blocks [0, n_gu) are the gate/up units
// of g2 (tile, column block), the rest the down units, mapped the same way,
// so a tile's gate/up and down units run on the same XCD.  A down unit starts
// once all ncb_gu gate/up units of its tile have written their h rows: each
// gate/up unit ends with an agent-scope release increment of tile_done[tile],
// and the down unit's thread 0 polls it and takes an acquire fence.  Down
// work thus fills the CUs that the last gate/up units leave idle, and the
// other way round.  The wait ends: every gate/up block has a lower index than
// every down block, so it is dispatched first, and it waits on nothing.  The
// poll is bounded all the same (spin_max polls); a down unit whose wait gives
// up stores nothing and counts itself in tile_done[n_tiles], which the host
// reads back (moe_q4_prefill_status).  tile_done, that count included, is
// zeroed by a fill launch just before.
constexpr int kTileSpinMax = 1 << 22;

__global__ void __launch_bounds__(256) fill_zero_kernel(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ void __launch_bounds__(256, 2) gemm_ffn_kernel(PrefillArgs a, int ncb_gu, int ncb_dn, int n_gu,
                                                          int n_tiles, int need, int spin_max) {
  __shared__ __attribute__((aligned(16))) G2Smem sm;
  const bool gu = (int)blockIdx.x < n_gu;
  const int b = gu ? (int)blockIdx.x : (int)blockIdx.x - n_gu;   // n_gu % 8 == 0: same XCD mapping
  const int ncb = gu ? ncb_gu : ncb_dn;
  const int q = b / 8;
  const int tile = 8 * (q / ncb) + b % 8, cb = q % ncb;
  const Tile t = find_tile_bal<FMAXR>(a.offsets, a.E, a.T, a.k, a.has_shared, tile);
  if (!t.valid) return;
  const int S = (t.rows + 31) / 32;
  if (gu) {
    // gate/up waves issue ahead of a down unit sharing the CU: the last
    // gate/up units gate the down units of their tiles
    __builtin_amdgcn_s_setprio(2);
    switch (S) {
      case 1: g2_tile<1, true>(a, t, cb, sm); break;
      case 2: g2_tile<2, true>(a, t, cb, sm); break;
      case 3: g2_tile<3, true>(a, t, cb, sm); break;
      case 4: g2_tile<4, true>(a, t, cb, sm); break;
      default: g2_tile<5, true>(a, t, cb, sm); break;
    }
    __syncthreads();                      // every wave's h stores are complete
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(a.tile_done + tile, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (threadIdx.x == 0) {
    int n = __hip_atomic_load(a.tile_done + tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int it = 0; n < need && it < spin_max; it++) {
      __builtin_amdgcn_s_sleep(8);
      n = __hip_atomic_load(a.tile_done + tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    sm.gave_up = n < need;
    if (n < need) __hip_atomic_fetch_add(a.tile_done + n_tiles, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (sm.gave_up) return;                 // h of this tile may be incomplete: store nothing
  switch (S) {
    case 1: g2_tile<1, false>(a, t, cb, sm); break;
    case 2: g2_tile<2, false>(a, t, cb, sm); break;
    case 3: g2_tile<3, false>(a, t, cb, sm); break;
    case 4: g2_tile<4, false>(a, t, cb, sm); break;
    default: g2_tile<5, false>(a, t, cb, sm); break;
  }
}

// ---------------------------------------------------------------- combine
// Up to KU slots per token with every load issued before the first sum:
// the k indices and weights, then the k expert-output rows.  Sum order:
// y = (((shared + w_0 o_0) + w_1 o_1) + ...), slots in order.
template <int KU>
__global__ void __launch_bounds__(256) combine_kernel(PrefillArgs a) {
  const int H = a.H, k = a.k;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = H / 8;
  if (idx >= (int64_t)a.T * per_row) return;
  const int t = (int)(idx / per_row), c = (int)(idx % per_row) * 8;
  int p[KU];
  float w[KU];
#pragma unroll
  for (int s = 0; s < KU; s++) {
    p[s] = 0;
    w[s] = 0.0f;
    if (s < k) {
      p[s] = min(max(a.inv_perm[(size_t)t * k + s], 0), a.T * k - 1);
      w[s] = a.topk_w[(size_t)t * k + s];
    }
  }
  uint4 v[KU];
#pragma unroll
  for (int s = 0; s < KU; s++)
    if (s < k) v[s] = *reinterpret_cast<const uint4*>(a.o_perm + (size_t)p[s] * H + c);
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
#pragma unroll
  for (int s = 0; s < KU; s++) {
    if (s < k) {
      const uint32_t q[4] = {v[s].x, v[s].y, v[s].z, v[s].w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        acc[2 * i] += w[s] * bf16_bits_to_f32(q[i] & 0xffffu);
        acc[2 * i + 1] += w[s] * bf16_bits_to_f32(q[i] >> 16);
      }
    }
  }
  *reinterpret_cast<float4*>(yr) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(yr + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// ---------------------------------------------------------------- launch
// Kernel choice: with tile-order weights (H and I multiples of 64) gate/up and
// down together take the fused launch and a single projection gemm_g2; the
// generic kernels cover row-major weights and any shape with K a multiple of
// 32.
hipError_t launch_prefill(const PrefillArgs& a, int stages, hipStream_t stream) {
  constexpr int MT = 4, BM = 32 * MT;
  const int64_t assignments = (int64_t)a.T * a.k;
  const int mtiles = (int)(assignments / BM) + a.E + (a.has_shared ? (a.T + BM - 1) / BM : 0);
  // upper bound of the balanced tile count (find_tile_bal)
  const int btiles = (int)prefill_tile_bound(a.T, a.k, a.E, a.has_shared);
  const int vec_g = ((a.H / BLK) % 4 == 0) && (((uintptr_t)a.w_gate | (uintptr_t)a.w_up) % 8 == 0) &&
                    (!a.has_shared || (((uintptr_t)a.s_gate | (uintptr_t)a.s_up) % 8 == 0));
  const int vec_d = ((a.I / BLK) % 4 == 0) && ((uintptr_t)a.w_down % 8 == 0) &&
                    (!a.has_shared || ((uintptr_t)a.s_down % 8 == 0));
  const bool tiled = a.t_gate && a.t_up && a.t_down && (!a.has_shared || (a.ts_gate && a.ts_up && a.ts_down));
  // (g2 addresses x through one buffer descriptor of T*H*2 bytes, a 32-bit
  // count: larger batches take the generic kernels)
  const bool g2_g = tiled && a.H % G2K == 0 && ((uintptr_t)a.x % 16 == 0) &&
                    (uint64_t)a.T * (uint64_t)a.H * 2u <= 0xffffffffull;
  const bool g2_d = tiled && a.I % G2K == 0 && ((uintptr_t)a.h % 16 == 0);
  const int g2_groups = (btiles + 7) / 8;
  hipError_t err = hipSuccess;
  if ((stages & 3) == 3 && g2_g && g2_d && a.tile_done) {
    const int ncb_gu = (a.I + 127) / 128, ncb_dn = (a.H + 255) / 256;
    const int n_gu = g2_groups * 8 * ncb_gu, n_dn = g2_groups * 8 * ncb_dn;
    // (a test of the failure path asks for one gate/up unit more than a tile
    // has, with a short spin: every wait then gives up)
    const int need = ncb_gu + (a.test_wait_fail ? 1 : 0);
    const int spin = a.test_wait_fail ? 16 : kTileSpinMax;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((btiles + 1 + 255) / 256), dim3(256), 0, stream, a.tile_done,
                       btiles + 1);
    hipLaunchKernelGGL(gemm_ffn_kernel, dim3(n_gu + n_dn), dim3(256), 0, stream, a, ncb_gu, ncb_dn, n_gu,
                       btiles, need, spin);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    stages &= ~3;
  }
  if (stages & 1) {
    if (g2_g) {
      const int ncb = (a.I + 127) / 128;
      hipLaunchKernelGGL((gemm_g2_kernel<true>), dim3(g2_groups * 8 * ncb), dim3(256), 0, stream, a, ncb);
    } else {
      hipLaunchKernelGGL((gateup_kernel<MT>), dim3((a.I + GBN - 1) / GBN, mtiles), dim3(256), 0,
                         stream, a, vec_g);
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (stages & 2) {
    if (g2_d) {
      const int ncb = (a.H + 255) / 256;
      hipLaunchKernelGGL((gemm_g2_kernel<false>), dim3(g2_groups * 8 * ncb), dim3(256), 0, stream, a, ncb);
    } else {
      hipLaunchKernelGGL((down_kernel<MT>), dim3((a.H + GBN - 1) / GBN, mtiles), dim3(256), 0,
                         stream, a, vec_d);
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (stages & 4) {
    const int64_t n = (int64_t)a.T * (a.H / 8);
    const dim3 grid((uint32_t)((n + 255) / 256));
    if (a.k <= 8) hipLaunchKernelGGL(combine_kernel<8>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(combine_kernel<32>, grid, dim3(256), 0, stream, a);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace moeq4
