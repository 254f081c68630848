// w4a8_prefill.hip -- the batched prefill of the Q4_0 expert FFN with 8-bit
// activations on int8 MFMA (the W4A8 form of the grouped GEMM).
//
// "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU",
// technical summary, Methodology 1 (prefill is a grouped 4-bit GEMM over the
// tokens routed to each expert; decode is a W4A8 integer kernel) and
// Methodology 2 (group-wise 4-bit weights, 8-bit activations).  This is the
// prefill GEMM in the W4A8 form: tokens quantised per 32-block to int8 (the
// program of q8_quantize), gate/up as int8 block dots, h = silu(g) * u
// quantised to int8 again, down the same way, then the weighted combine.
//
// One v_mfma_i32_32x32x32_i8 spans K = 32, exactly one Q4_0 block, and yields
// that block's int32 dots for 32 tokens x 32 weight rows.  Each dot is then
// rescaled on its own and accumulated with ONE fused multiply-add:
// acc = fma(d_w * d_a, (float)dot, acc) -- a tolerance path, so no pinned
// summation order (the one-token decode keeps that).  The rescale is the cost:
// three VALU instructions per output per block against one MFMA per 32 x 32
// outputs, so the kernel is bound by VALU issue, not by the matrix cores.
//
// Weight codes enter the MFMA as signed bytes 16 * (q - 8): a nibble moved to
// a byte's high half and its top bit flipped ((b & 0xf0) ^ 0x80 is 16q - 128
// as a signed byte), so no -8 * (sum of codes) correction is needed; the
// factor 16 goes into d_w / 16 (exact).  K order inside a block: MFMA lane
// half h takes elements 16h .. 16h+15 on both operands -- the low nibbles of
// the block's 16 code bytes for h = 0, the high nibbles for h = 1, and
// activation bytes 16h .. 16h+15.
//
// Kernels (all on the caller's stream):
//   q8x   x bf16 [T][H] -> codes [T][H] int8, scales [T][H/32] fp32
//   gate/up   unit = one wave: (tile of <= 32 rows of one expert segment,
//         32 columns of I), gate and up of the 32 columns;
//         h = silu(g) * u and its q8 (the unit holds whole 32-groups of I)
//   down  unit = one wave: (tile, 64 columns of H), two groups of 32
//         columns; routed rows -> bf16 expert outputs in segment order, the
//         shared expert -> y
//   combine  (gemm.hip) y[t] += sum_s w[t,s] * O[inv_perm[t*k+s]]
// Tiles are greedy 32-row groups of a segment (an expert of c rows costs
// ceil(c/32) units per column block, no idle rows past the last group).
// Blocks are dealt to the 8 XCDs round robin; each aligned group of eight
// consecutive tiles runs on one XCD with all its column blocks, so an
// expert's weight columns are mostly fetched into one XCD's L2 (groups of
// four split most ~128-row experts over two XCDs: 1.2x the HBM reads at the
// same speed).  One-wave units schedule finer than the four-wave units of
// 128-row tiles that came before (342 -> 405 TOPS for gate/up + down at 2048
// tokens, same bits).
#include "launch.hpp"
#include "device_math.hpp"
#include "tiles.hpp"

namespace moeq4 {

typedef int w8v4 __attribute__((ext_vector_type(4)));
typedef int w8v16 __attribute__((ext_vector_type(16)));

constexpr int kW8Rows = 32;            // rows per tile, greedy tiles
constexpr int kW8Threads = 64;         // one wave per unit
constexpr int kW8Group = 8;            // consecutive tiles dealt to one XCD
constexpr int kW8WavesPerSimd = 4;     // occupancy asked of the compiler: at most 128 VGPRs
constexpr int kW8DnCols = 64;          // columns of H per down unit
static_assert(kW8Threads == 2 * kW8Rows, "the scale staging takes two threads per tile row");

// Block b -> (tile, column block cb) out of ncb: tiles 8G*m + G*x .. + G-1
// (G = kW8Group) run on XCD slot x = b % 8, the G tiles of a column block
// next to each other in dispatch order.
__device__ __forceinline__ void w8_unit(int b, int ncb, int& tile, int& cb) {
  const int x = b % 8, q = b / 8;
  tile = 8 * kW8Group * (q / (kW8Group * ncb)) + kW8Group * x + q % kW8Group;
  cb = (q / kW8Group) % ncb;
}

// ---------------------------------------------------------------- q8 of x
// 8 threads per 32-block, 4 elements each: d = amax / 127, q = round(x / d)
// (round half away from zero), the program of q8_quantize on the bf16 values
// widened to fp32.
__global__ void __launch_bounds__(256) w8_q8x_kernel(const uint16_t* __restrict__ x, int64_t nblk,
                                                     int8_t* __restrict__ q, float* __restrict__ d) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = t / 8;
  const int s = (int)(t % 8);
  const bool in = b < nblk;
  const int64_t bc = in ? b : nblk - 1;   // (the block's 8 threads stay together for the shuffles)
  const uint2 raw = *reinterpret_cast<const uint2*>(x + bc * 32 + 4 * s);
  float v[4] = {bf16_bits_to_f32(raw.x & 0xffffu), bf16_bits_to_f32(raw.x >> 16),
                bf16_bits_to_f32(raw.y & 0xffffu), bf16_bits_to_f32(raw.y >> 16)};
  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 8));
  const float dd = amax / 127.0f;
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int qi = (dd == 0.0f) ? 0 : (int)roundf(v[i] / dd);
    packed |= ((uint32_t)qi & 0xffu) << (8 * i);
  }
  if (in) {
    *reinterpret_cast<uint32_t*>(q + b * 32 + 4 * s) = packed;
    if (s == 0) d[b] = dd;
  }
}

// ---------------------------------------------------------------- operands
// Signed MFMA weight bytes 16 * (q - 8) of a block's 16 code bytes: lane half
// h = 0 the low nibbles, h = 1 the high ones.
__device__ __forceinline__ w8v4 w8_weights(uint4 raw, int shl) {
  w8v4 o;
  o.x = (int)(((raw.x << shl) & 0xf0f0f0f0u) ^ 0x80808080u);
  o.y = (int)(((raw.y << shl) & 0xf0f0f0f0u) ^ 0x80808080u);
  o.z = (int)(((raw.z << shl) & 0xf0f0f0f0u) ^ 0x80808080u);
  o.w = (int)(((raw.w << shl) & 0xf0f0f0f0u) ^ 0x80808080u);
  return o;
}

__device__ __forceinline__ w8v4 w8_as_v4(uint4 v) {
  w8v4 o;
  o.x = (int)v.x; o.y = (int)v.y; o.z = (int)v.z; o.w = (int)v.w;
  return o;
}

// One block's dots for the wave's 32 x 32 tile, accumulated: output register
// r of lane l is row 8*(r/4) + 4*(l/32) + r%4 of the wave's rows and column
// l%32; dw is the lane's column's weight scale / 16, da4[q] the activation
// scales of its rows 8q + 4h .. +3.
__device__ __forceinline__ void w8_accumulate(float (&acc)[16], const w8v16& dot, float dw, const float4 (&da4)[4]) {
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const float dv[4] = {da4[q].x, da4[q].y, da4[q].z, da4[q].w};
#pragma unroll
    for (int p = 0; p < 4; p++) acc[4 * q + p] = __builtin_fmaf(dw * dv[p], (float)dot[4 * q + p], acc[4 * q + p]);
  }
}

// ---------------------------------------------------------------- gate/up
// LDS: activation scales of the tile's rows [nb][kW8Rows], the q8(h) codes
// [32][32] for the coalesced store, the tile rows' tokens.
template <bool DOTS>
__global__ void __launch_bounds__(kW8Threads) __attribute__((amdgpu_waves_per_eu(DOTS ? 1 : kW8WavesPerSimd))) w8_gateup_kernel(W4A8PrefillArgs a, int32_t* __restrict__ gate_dots) {
  extern __shared__ __align__(16) uint8_t dyn[];
  const int H = a.H, I = a.I, nb = H / BLK, nsteps = H / 64, ncb = I / 32;
  float* da_l = reinterpret_cast<float*>(dyn);                              // [nb][kW8Rows]
  uint8_t* qo_l = dyn + (size_t)nb * kW8Rows * 4;                           // [32][32]
  int* tok_l = reinterpret_cast<int*>(qo_l + 1024);                         // [kW8Rows]
  int tile, cb;
  w8_unit(blockIdx.x, ncb, tile, cb);
  const Tile t = find_tile_bal<kW8Rows, false>(a.offsets, a.E, a.T, a.k, a.has_shared, tile);
  if (!t.valid) return;
  const int tid = threadIdx.x, lane = tid % 64;
  // token of each tile row (rows past the tile repeat its first row)
  if (tid < kW8Rows) {
    const int r = tid < t.rows ? tid : 0;
    tok_l[tid] = t.expert >= 0 ? min(max(a.perm[t.pos0 + r] / a.k, 0), a.T - 1) : t.m0 + r;
  }
  __syncthreads();
  {                                                          // da_l[bb][row], 4 independent loads per round
    const int row = tid % kW8Rows, b0 = tid / kW8Rows;       // (two threads per row: 2 blocks per round)
    const float* src = a.dx + (size_t)tok_l[row] * nb;
    for (int bb = b0; bb < nb; bb += 8) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; u++) v[u] = src[min(bb + 2 * u, nb - 1)];
#pragma unroll
      for (int u = 0; u < 4; u++)
        if (bb + 2 * u < nb) da_l[(bb + 2 * u) * kW8Rows + row] = v[u];
    }
  }
  const int n = lane % 32, h = lane / 32, shl = 4 * (1 - h);
  const int8_t* arow = a.qx + (size_t)tok_l[n] * H + 16 * h;   // the lane's A row (token)
  const size_t gbytes = (size_t)nsteps * 1152;              // one 32-row group of a matrix
  const uint8_t* gw = (t.expert >= 0 ? a.t_gate + ((size_t)t.expert * ncb + cb) * gbytes : a.ts_gate + cb * gbytes);
  const uint8_t* uw = (t.expert >= 0 ? a.t_up + ((size_t)t.expert * ncb + cb) * gbytes : a.ts_up + cb * gbytes);
  __syncthreads();
  float accg[16], accu[16];
#pragma unroll
  for (int r = 0; r < 16; r++) accg[r] = accu[r] = 0.0f;
  const w8v16 zero = {};
  const float* da_w = da_l + 4 * h;                         // + bb * kW8Rows + 8 q
  // operands of a step (blocks 2s, 2s+1), one step ahead in registers
  auto load = [&](int s, uint4 (&A)[2], uint4 (&G)[2], uint4 (&U)[2], uint32_t (&sg)[2], uint32_t (&su)[2]) {
    const uint8_t* gp = gw + (size_t)s * 1152;
    const uint8_t* up = uw + (size_t)s * 1152;
#pragma unroll
    for (int j = 0; j < 2; j++) {
      A[j] = *reinterpret_cast<const uint4*>(arow + 64 * s + 32 * j);
      G[j] = *reinterpret_cast<const uint4*>(gp + 16 * (32 * j + n));
      U[j] = *reinterpret_cast<const uint4*>(up + 16 * (32 * j + n));
      sg[j] = *reinterpret_cast<const uint16_t*>(gp + 1024 + 2 * (32 * j + n));
      su[j] = *reinterpret_cast<const uint16_t*>(up + 1024 + 2 * (32 * j + n));
    }
  };
  auto compute = [&](int s, const uint4 (&A)[2], const uint4 (&G)[2], const uint4 (&U)[2], const uint32_t (&sg)[2],
                     const uint32_t (&su)[2]) {
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int bb = 2 * s + j;
      const w8v4 av = w8_as_v4(A[j]);
      const w8v16 dg = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, w8_weights(G[j], shl), zero, 0, 0, 0);
      const w8v16 du = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, w8_weights(U[j], shl), zero, 0, 0, 0);
      float4 da4[4];
#pragma unroll
      for (int q = 0; q < 4; q++) da4[q] = *reinterpret_cast<const float4*>(da_w + bb * kW8Rows + 8 * q);
      const float dwg = f16_bits_to_f32(sg[j]) * 0.0625f, dwu = f16_bits_to_f32(su[j]) * 0.0625f;
      w8_accumulate(accg, dg, dwg, da4);
      w8_accumulate(accu, du, dwu, da4);
      if (DOTS) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int row = 8 * (r / 4) + 4 * h + (r % 4);
          if (row < t.rows)
            gate_dots[((size_t)(t.pos0 + row) * I + 32 * cb + n) * nb + bb] = dg[r] >> 4;
        }
      }
    }
  };
  // the next step's operands are loaded while this step computes (the last
  // step re-reads its own, unused)
  uint4 A[2], G[2], U[2];
  uint32_t sg[2], su[2];
  load(0, A, G, U, sg, su);
  for (int s = 0; s < nsteps; s++) {
    uint4 An[2], Gn[2], Un[2];
    uint32_t sgn[2], sun[2];
    load(min(s + 1, nsteps - 1), An, Gn, Un, sgn, sun);
    compute(s, A, G, U, sg, su);
#pragma unroll
    for (int j = 0; j < 2; j++) {
      A[j] = An[j]; G[j] = Gn[j]; U[j] = Un[j]; sg[j] = sgn[j]; su[j] = sun[j];
    }
  }
  // h = silu(g) * u, then q8 of each row's 32 values (lanes of one half hold
  // a row's 32 columns): amax by a butterfly over the half, d = amax / 127,
  // q = round(h / d)
  uint8_t* qw = qo_l;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const float g = accg[r], u = accu[r];
    const float hv = g / (1.0f + __expf(-g)) * u;
    float amax = fabsf(hv);
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 32));
    const float d = amax / 127.0f;
    const int qv = (d == 0.0f) ? 0 : (int)roundf(hv / d);
    const int row = 8 * (r / 4) + 4 * h + (r % 4);          // the row inside the tile
    qw[32 * row + n] = (uint8_t)qv;
    if (n == 0 && row < t.rows) a.dh[(size_t)(t.pos0 + row) * ncb + cb] = d;
  }
  __syncthreads();
  {                                                          // 32 rows x 32 bytes: 16 bytes per lane
    const int row = lane / 2;
    if (row < t.rows)
      *reinterpret_cast<uint4*>(a.qh + (size_t)(t.pos0 + row) * I + 32 * cb + 16 * (lane % 2)) =
          *reinterpret_cast<const uint4*>(qw + 32 * row + 16 * (lane % 2));
  }
}

// ---------------------------------------------------------------- down
// LDS: q8(h) scales of the tile's rows [I/32][kW8Rows].
__global__ void __launch_bounds__(kW8Threads) __attribute__((amdgpu_waves_per_eu(kW8WavesPerSimd))) w8_down_kernel(W4A8PrefillArgs a) {
  extern __shared__ __align__(16) uint8_t dyn[];
  const int H = a.H, I = a.I, nb = I / BLK, nsteps = I / 64, ncb = H / kW8DnCols;
  float* da_l = reinterpret_cast<float*>(dyn);                              // [nb][kW8Rows]
  int tile, cb;
  w8_unit(blockIdx.x, ncb, tile, cb);
  const Tile t = find_tile_bal<kW8Rows, false>(a.offsets, a.E, a.T, a.k, a.has_shared, tile);
  if (!t.valid) return;
  const int tid = threadIdx.x, lane = tid % 64;
  {                                                          // da_l[bb][row], 4 independent loads per round
    const int row = tid % kW8Rows, b0 = tid / kW8Rows;
    const float* src = a.dh + (size_t)(t.pos0 + (row < t.rows ? row : 0)) * nb;
    for (int bb = b0; bb < nb; bb += 8) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; u++) v[u] = src[min(bb + 2 * u, nb - 1)];
#pragma unroll
      for (int u = 0; u < 4; u++)
        if (bb + 2 * u < nb) da_l[(bb + 2 * u) * kW8Rows + row] = v[u];
    }
  }
  const int n = lane % 32, h = lane / 32, shl = 4 * (1 - h);
  const int8_t* arow = a.qh + (size_t)(t.pos0 + (n < t.rows ? n : 0)) * I + 16 * h;   // the lane's A row
  const size_t gbytes = (size_t)nsteps * 1152;
  const int G0 = 2 * cb;                                     // the unit's two 32-column groups of H
  const uint8_t* w0 = (t.expert >= 0 ? a.t_down + ((size_t)t.expert * (H / 32) + G0) * gbytes : a.ts_down + G0 * gbytes);
  const uint8_t* w1 = w0 + gbytes;
  __syncthreads();
  float acc0[16], acc1[16];
#pragma unroll
  for (int r = 0; r < 16; r++) acc0[r] = acc1[r] = 0.0f;
  const w8v16 zero = {};
  const float* da_w = da_l + 4 * h;
  auto load = [&](int s, uint4 (&A)[2], uint4 (&B0)[2], uint4 (&B1)[2], uint32_t (&s0)[2], uint32_t (&s1)[2]) {
    const uint8_t* p0 = w0 + (size_t)s * 1152;
    const uint8_t* p1 = w1 + (size_t)s * 1152;
#pragma unroll
    for (int j = 0; j < 2; j++) {
      A[j] = *reinterpret_cast<const uint4*>(arow + 64 * s + 32 * j);
      B0[j] = *reinterpret_cast<const uint4*>(p0 + 16 * (32 * j + n));
      B1[j] = *reinterpret_cast<const uint4*>(p1 + 16 * (32 * j + n));
      s0[j] = *reinterpret_cast<const uint16_t*>(p0 + 1024 + 2 * (32 * j + n));
      s1[j] = *reinterpret_cast<const uint16_t*>(p1 + 1024 + 2 * (32 * j + n));
    }
  };
  auto compute = [&](int s, const uint4 (&A)[2], const uint4 (&B0)[2], const uint4 (&B1)[2], const uint32_t (&s0)[2],
                     const uint32_t (&s1)[2]) {
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int bb = 2 * s + j;
      const w8v4 av = w8_as_v4(A[j]);
      const w8v16 d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, w8_weights(B0[j], shl), zero, 0, 0, 0);
      const w8v16 d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, w8_weights(B1[j], shl), zero, 0, 0, 0);
      float4 da4[4];
#pragma unroll
      for (int q = 0; q < 4; q++) da4[q] = *reinterpret_cast<const float4*>(da_w + bb * kW8Rows + 8 * q);
      w8_accumulate(acc0, d0, f16_bits_to_f32(s0[j]) * 0.0625f, da4);
      w8_accumulate(acc1, d1, f16_bits_to_f32(s1[j]) * 0.0625f, da4);
    }
  };
  uint4 A[2], B0[2], B1[2];
  uint32_t s0[2], s1[2];
  load(0, A, B0, B1, s0, s1);
  for (int s = 0; s < nsteps; s++) {
    uint4 An[2], B0n[2], B1n[2];
    uint32_t s0n[2], s1n[2];
    load(min(s + 1, nsteps - 1), An, B0n, B1n, s0n, s1n);
    compute(s, A, B0, B1, s0, s1);
#pragma unroll
    for (int j = 0; j < 2; j++) {
      A[j] = An[j]; B0[j] = B0n[j]; B1[j] = B1n[j]; s0[j] = s0n[j]; s1[j] = s1n[j];
    }
  }
#if defined(__HIP_DEVICE_COMPILE__)   // (buffer descriptors exist only in the device pass)
  // Stores through a descriptor over the tile's output rows (o_perm, or y for
  // the shared expert): rows past t.rows fall past its end and are dropped,
  // and each store adds a scalar row offset to the lane's offset.
  const int routed = __builtin_amdgcn_readfirstlane(t.expert >= 0 ? 1 : 0);
  const int esz = routed ? 2 : 4;
  const void* obase = routed ? static_cast<const void*>(a.o_perm + (size_t)t.pos0 * H)
                             : static_cast<const void*>(a.y + (size_t)t.m0 * H);
  const __amdgpu_buffer_rsrc_t ro = uniform_buffer_rsrc(obase, (uint32_t)t.rows * (uint32_t)H * (uint32_t)esz);
  const uint32_t rstride = __builtin_amdgcn_readfirstlane((uint32_t)(H * esz));
  const uint32_t vb0 = (uint32_t)((4 * h * H + kW8DnCols * cb + n) * esz), vb1 = vb0 + 32u * (uint32_t)esz;
  if (routed) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const uint32_t ro_r = (uint32_t)(8 * (r / 4) + (r % 4)) * rstride;
      const uint32_t ob = bf16x2_bits(acc0[r], acc1[r]);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)ob, ro, vb0 + ro_r, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(ob >> 16), ro, vb1 + ro_r, 0, 0);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const uint32_t ro_r = (uint32_t)(8 * (r / 4) + (r % 4)) * rstride;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc0[r]), ro, vb0 + ro_r, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc1[r]), ro, vb1 + ro_r, 0, 0);
    }
  }
#endif
}

// ---------------------------------------------------------------- launch
int64_t w4a8_prefill_tile_bound(int64_t T, int k, int E, int has_shared) {
  // sum over experts of ceil(c_e / kW8Rows) <= T k / kW8Rows + E
  return T * k / kW8Rows + E + (has_shared ? (T + kW8Rows - 1) / kW8Rows : 0);
}

hipError_t launch_prefill_w4a8(const W4A8PrefillArgs& a, int32_t* gate_dots, int stages, hipStream_t stream) {
  // w8_unit covers tiles [0, 8 * kW8Group * supers)
  const int supers = (int)((w4a8_prefill_tile_bound(a.T, a.k, a.E, a.has_shared) + 8 * kW8Group - 1) / (8 * kW8Group));
  const int ncb_gu = a.I / 32, ncb_dn = a.H / kW8DnCols;
  hipError_t err = hipSuccess;
  if (stages & 1) {                      // q8(x), then gate/up + SwiGLU + q8(h)
    const int64_t nblk = (int64_t)a.T * (a.H / BLK);
    hipLaunchKernelGGL(w8_q8x_kernel, dim3((unsigned)((nblk * 8 + 255) / 256)), dim3(256), 0, stream, a.x, nblk,
                       a.qx, a.dx);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const size_t lds_gu = (size_t)(a.H / BLK) * kW8Rows * 4 + 1024 + kW8Rows * 4;
    if (gate_dots)
      hipLaunchKernelGGL(w8_gateup_kernel<true>, dim3(supers * 8 * kW8Group * ncb_gu), dim3(kW8Threads), lds_gu, stream, a, gate_dots);
    else
      hipLaunchKernelGGL(w8_gateup_kernel<false>, dim3(supers * 8 * kW8Group * ncb_gu), dim3(kW8Threads), lds_gu, stream, a, gate_dots);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (stages & 2) {
    const size_t lds_dn = (size_t)(a.I / BLK) * kW8Rows * 4;
    hipLaunchKernelGGL(w8_down_kernel, dim3(supers * 8 * kW8Group * ncb_dn), dim3(kW8Threads), lds_dn, stream, a);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace moeq4
