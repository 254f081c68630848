// launch.hpp -- host-side launchers of the HIP kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moeq4 {

hipError_t launch_q4_pack(const float* w, int64_t rows, int64_t K, void* packed,
                          hipStream_t stream);
hipError_t launch_q8w_pack(const float* w, int64_t rows, int64_t K, void* packed, hipStream_t stream);
hipError_t launch_q4_tile(const void* q4, int64_t rows, int64_t K, void* tiled, hipStream_t stream);
hipError_t launch_q8w_tile(const void* q8, int64_t rows, int64_t K, void* tiled, hipStream_t stream);
// W4A8 row program for M tokens on int8 MFMA (weights in q4_tile order).
size_t w4a8_gemm_lds_bytes(int K);
hipError_t launch_w4a8_gemm(const uint8_t* Wt, int N, int K, const int8_t* qa, const float* da, int M,
                            int32_t* dots, float* out, hipStream_t stream);
hipError_t launch_q8_quantize(const float* x, int64_t rows, int64_t K, int8_t* q, float* d,
                              hipStream_t stream);

// Router split geometry: the chunk tree (nc = H/32 leaves padded to the power
// of two m) is cut into nsplit aligned subtrees of cw leaves each.
struct RouterSplit {
  int nc, m, cw, nsplit;
};
RouterSplit prefill_router_split(int H);

// Prefill routing.
hipError_t launch_router_partials(const void* x, int x_bf16, int T, int H, const float* w_router,
                                  int E, const RouterSplit& sp, float* partials,
                                  hipStream_t stream);
hipError_t launch_topk_hist(const float* partials, const RouterSplit& sp, const float* bias,
                            int T, int E, int k, float* logits_out, int32_t* ids, float* w,
                            int32_t* counts_w, int32_t* rank, hipStream_t stream);
hipError_t launch_route_colscan(int32_t* counts_w, int n_tiles, int E, int32_t* tot, hipStream_t stream);
// tot == nullptr: T == 0, offsets all zero
hipError_t launch_route_scatter(const int32_t* ids, const int32_t* rank, const int32_t* base_w,
                                const int32_t* tot, int T, int k, int E, int32_t* offsets, int32_t* perm,
                                int32_t* inv_perm, hipStream_t stream);
constexpr int kTopkTokensPerBlock = 16;   // tokens (= waves) per top-k block

// Matrix-core rate probes (probe.hip): kind 0 bf16 32x32x16, 1 int8
// 32x32x32, 2 fp32 32x32x1 (two blocks); MFMA instructions a launch issues.
int64_t probe_mfma_count(int kind, int blocks, int iters);
hipError_t launch_probe_mfma(int kind, int blocks, int iters, float* out, hipStream_t stream);

// Prefill expert FFN.
struct PrefillArgs {
  const uint16_t* x;        // [T][H] bf16
  int T, H, I, E, k, has_shared;
  const int32_t* perm;      // [T*k]
  const int32_t* offsets;   // [E+1]
  const int32_t* inv_perm;  // [T*k]
  const float* topk_w;      // [T][k]
  const uint8_t* w_gate;    // [E][I][H/32*18]
  const uint8_t* w_up;
  const uint8_t* w_down;    // [E][H][I/32*18]
  const uint8_t* s_gate;
  const uint8_t* s_up;
  const uint8_t* s_down;
  const uint8_t* t_gate;    // the same matrices in q4_tile order, or all NULL
  const uint8_t* t_up;
  const uint8_t* t_down;
  const uint8_t* ts_gate;
  const uint8_t* ts_up;
  const uint8_t* ts_down;
  uint16_t* h;              // [(T*k + T*S)][I] bf16
  uint16_t* o_perm;         // [T*k][H] bf16
  float* y;                 // [T][H] fp32
  int32_t* tile_done;       // [prefill_tile_bound + 1] gate/up units finished per tile (fused
                            // launch), then the count of down units whose wait gave up
  int test_wait_fail;       // test only: make every wait of the fused launch give up
};
hipError_t launch_prefill(const PrefillArgs& a, int stages, hipStream_t stream);

// The W4A8 form of the batched prefill (w4a8_prefill.hip): int8 MFMA block
// dots over 8-bit tokens and 8-bit h, one fp32 FMA per block dot.
struct W4A8PrefillArgs {
  const uint16_t* x;        // [T][H] bf16
  int T, H, I, E, k, has_shared;
  const int32_t* perm;      // [T*k]
  const int32_t* offsets;   // [E+1]
  const uint8_t* t_gate;    // tile-order matrices (q4_tile)
  const uint8_t* t_up;
  const uint8_t* t_down;
  const uint8_t* ts_gate;
  const uint8_t* ts_up;
  const uint8_t* ts_down;
  int8_t* qx;               // [T][H]        q8 codes of x
  float* dx;                // [T][H/32]     their scales
  int8_t* qh;               // [T*k + T*S][I] q8 codes of h, segment order (shared rows last)
  float* dh;                // [T*k + T*S][I/32]
  uint16_t* o_perm;         // [T*k][H] bf16 routed expert outputs, segment order
  float* y;                 // [T][H]
};
int64_t w4a8_prefill_tile_bound(int64_t T, int k, int E, int has_shared);
// stages: 1 = q8(x) + gate/up, 2 = down (the combine is the bf16 form's)
hipError_t launch_prefill_w4a8(const W4A8PrefillArgs& a, int32_t* gate_dots, int stages, hipStream_t stream);

// Rows per tile of the grouped GEMMs (an expert segment of c rows is cut into
// ceil(c / kPrefillTileRows) tiles) and an upper bound of the tile count.
constexpr int kPrefillTileRows = 160;
inline int64_t prefill_tile_bound(int64_t T, int k, int E, int has_shared) {
  // (+ 7: the shared expert's tile count is rounded up to a multiple of 8)
  return T * k / kPrefillTileRows + E + (has_shared ? (T + kPrefillTileRows - 1) / kPrefillTileRows + 7 : 0);
}

// Decode.
struct DecodeArgs {
  int wfmt;                 // weight format: 0 Q4_0, 1 Q8_0
  int norm_in;              // 1: x is the previous layer's y, RMSNorm-ed on the fly
  float norm_eps;
  const float* x;           // [H]
  float* y;                 // [H]
  int H, I, E, k, has_shared;
  const float* w_router;
  const float* bias;
  const uint8_t* w_gate;
  const uint8_t* w_up;
  const uint8_t* w_down;
  const uint8_t* s_gate;
  const uint8_t* s_up;
  const uint8_t* s_down;
  // tile-order copies (of the layer's weight format), or NULL: the gate/up
  // and down launches then read these instead of the row-major blocks
  const uint8_t* t_gate;
  const uint8_t* t_up;
  const uint8_t* ts_gate;
  const uint8_t* ts_up;
  const uint8_t* t_down;
  const uint8_t* ts_down;
  // workspace pieces (no initialisation needed: every piece is written
  // before it is read within one call)
  float* partials;          // [H/32][E] router chunk chains
  int32_t* ids;             // [k]
  float* w;                 // [k]
  int8_t* qx;               // [H]         (16-byte aligned)
  float* dx;                // [H/32]
  int32_t* sx;              // [H/32] sum of the int8 codes of each block
  int8_t* qh;               // [k+S][I]    (16-byte aligned)
  float* dh;                // [(k+S) I/32]
  int32_t* sh;              // [(k+S) I/32]
  // the one-launch decode's handoff words (workspace; see decode_fused.hip)
  uint64_t* hdr;            // [0] low 32 bits: waits that gave up; then kFuSlots uint32 epoch slots
  uint64_t* ll_leaf;        // [n_cg][E] router subtree values
  uint64_t* ll_route;       // [2k] ids, then weights
  uint64_t* ll_qh;          // [(k+S) * I/32][10] q8(h) groups: 8 code dwords, d, code sum
  uint64_t* ll_y;           // [H] the stacked decode's y of a layer that is not the last, or NULL
  int spin_max;             // polls of one wait before it gives up
  int test_wait_fail;       // test only: every wait looks for a tag no word carries
  // optional trace
  float* t_logits;
  int32_t* t_ids;
  float* t_w;
  int8_t* t_qx;
  float* t_dx;
  int8_t* t_qh;
  float* t_dh;
};
// Launch shapes of the three decode kernels.  The down kernel stages every
// slot's q8(h) in LDS when that fits in kDecodeLdsMax bytes (dn_act_lds),
// else it reads the activation blocks from the workspace in memory.
constexpr size_t kDecodeLdsMax = 64 * 1024;
struct DecodeGeometry {
  int router_threads;
  int gu_lpr, gu_bpl, gu_fast, gu_threads, gu_parts;
  size_t gu_lds;
  int gt_sp, gt_threads, gt_parts;   // tile-order gate/up (gt_sp 0: not available)
  int dn_lpr, dn_bpl, dn_fast, dn_rows, dn_threads, dn_act_lds;
  size_t dn_lds;
  int dt_sp, dt_threads;             // tile-order down (dt_sp 0: not available)
  size_t dt_lds;
};
DecodeGeometry decode_geometry(int H, int I, int E, int k, int has_shared);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// The one-launch decode (decode_fused.hip): block roles, their counts and
// split parameters; ok = 0 when the shape is not covered (the three-launch
// path then runs).
constexpr int kFuSlots = 2048;            // epoch slots = the largest one-launch grid
constexpr size_t kFuHeaderBytes = 8 + 4 * kFuSlots;
struct FusedGeometry {
  int ok;
  int cpb, eb, n_eg, n_cg, nR;   // router: chunks and experts per block, expert and chunk groups, blocks
  int P, L;                 // logit tree: lanes per expert, subtree values per lane
  int gu_waves, gu_sp, n_gu;
  int dn_nh, dn_sp, n_dn;    // down: step halves per row, pieces per lane and task, units
  int base_dn, nblocks;
  size_t lds;
};
FusedGeometry fused_geometry(int H, int I, int E, int k, int has_shared);
// true if the layer (tile-order copies, shape) and the GPU's resident block
// count allow the one-launch decode with the given workspace words
bool fused_decode_available(const DecodeArgs& a);
hipError_t launch_decode_fused(const DecodeArgs& a, hipStream_t stream);

// The stacked decode in one launch per run of up to kStackMaxLayers layers of
// one shape (the table travels in the kernel arguments).
constexpr int kStackMaxLayers = 40;
struct StackLayer {
  const float* w_router;
  const float* bias;
  const uint8_t* t_gate;
  const uint8_t* t_up;
  const uint8_t* t_down;
  const uint8_t* ts_gate;
  const uint8_t* ts_up;
  const uint8_t* ts_down;
};
struct StackTable {
  int n;
  StackLayer l[kStackMaxLayers];
};
// true if the one-launch step is available for the shape of `a` with the
// stacked kernel's extra LDS (the layer's x)
bool stack_decode_available(const DecodeArgs& a);
// a: layer 0's arguments with x, y, norm_in, norm_eps of the run and ll_y;
// the layers' pointers come from t
hipError_t launch_decode_stack(const DecodeArgs& a, const StackTable& t, hipStream_t stream);

// Batched decode: M <= kDecodeBatchMax tokens, each through the single-token
// program; the selected experts' weights are read once per call.
constexpr int kDecodeBatchMax = 32;
constexpr size_t kDecodeBatchLds = 40 * 1024;   // LDS budget of the batched gate/up and down blocks
struct DecodeBatchArgs {
  int wfmt;                 // weight format: 0 Q4_0, 1 Q8_0
  const float* x;           // [M][H]
  float* y;                 // [M][H]
  int M, H, I, E, k, has_shared;
  const float* w_router;
  const float* bias;
  const uint8_t* w_gate;
  const uint8_t* w_up;
  const uint8_t* w_down;
  const uint8_t* s_gate;
  const uint8_t* s_up;
  const uint8_t* s_down;
  // the same matrices in tile order (q4_tile / q8w_tile), or NULL: read in
  // place of the row-major ones when given
  const uint8_t* t_gate;
  const uint8_t* t_up;
  const uint8_t* t_down;
  const uint8_t* ts_gate;
  const uint8_t* ts_up;
  const uint8_t* ts_down;
  // workspace
  float* partials;          // [M][H/32][E] router leaves
  int8_t* qx;               // [M][H]
  float* dx;                // [M][H/32]
  int32_t* sx;              // [M][H/32]
  int32_t* ids;             // [M][k]
  float* w;                 // [M][k]
  int8_t* qh;               // [M*k + M*S][I] q8(h) per pair t*k+s (shared expert: M*k + t)
  float* dh;                // [M*k + M*S][I/32]
  int32_t* sh;              // [M*k + M*S][I/32]
  float* o;                 // [M*k + M*S][H] expert outputs per pair
  int32_t* t_ids;           // optional copies of ids / w, or NULL
  float* t_w;
};
struct DecodeBatchGeometry {
  int router_threads;
  int route_parts, route_threads;
  size_t route_lds;
  int gu_lpr, gu_bpl, gu_fast, gu_threads, gu_tb;
  size_t gu_lds;
  int dn_lpr, dn_bpl, dn_fast, dn_rows, dn_threads, dn_tb;
  size_t dn_lds;
};
DecodeBatchGeometry decode_batch_geometry(int M, int H, int I, int E, int k, int has_shared);
hipError_t launch_decode_batch(const DecodeBatchArgs& a, hipStream_t stream);

hipError_t launch_w4a8_gemv(const uint8_t* W, int N, int K, const int8_t* qa, const float* da,
                            int32_t* dots, float* out, hipStream_t stream);

hipError_t launch_rmsnorm(const float* y, int T, int H, float eps, float* out_f32,
                          uint16_t* out_bf16, hipStream_t stream);

}  // namespace moeq4
