// abi.cpp -- the extern "C" entry points of libmoe_q4.so (declared and
// documented in include/moe_q4.h): argument checks, workspace layout and the
// launch sequence of each call.  No device memory is allocated here.
#include "moe_q4.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "launch.hpp"

// Scratch of moe_q4_decode_noalloc: one array on every GPU the library runs
// on, held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: host code uses only the address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[MOE_Q4_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MOE_Q4_EHIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxDim = 16384;

int check_layer(const moe_q4_layer* L) {
  if (!L) return fail(MOE_Q4_EINVAL, "layer is NULL");
  if (L->hidden <= 0 || L->hidden % 32 || L->hidden > kMaxDim)
    return fail(MOE_Q4_EINVAL, "hidden=%d must be a positive multiple of 32 <= %d", L->hidden, kMaxDim);
  if (L->inter <= 0 || L->inter % 32 || L->inter > kMaxDim)
    return fail(MOE_Q4_EINVAL, "inter=%d must be a positive multiple of 32 <= %d", L->inter, kMaxDim);
  if (L->n_experts < 1 || L->n_experts > kMaxExperts)
    return fail(MOE_Q4_EINVAL, "n_experts=%d must be in [1, %d]", L->n_experts, kMaxExperts);
  if (L->top_k < 1 || L->top_k > L->n_experts || L->top_k > kMaxTopK)
    return fail(MOE_Q4_EINVAL, "top_k=%d must be in [1, min(n_experts, %d)]", L->top_k, kMaxTopK);
  if (L->has_shared != 0 && L->has_shared != 1)
    return fail(MOE_Q4_EINVAL, "has_shared=%d must be 0 or 1", L->has_shared);
  if (!L->w_router) return fail(MOE_Q4_EINVAL, "w_router must be non-NULL");
  // the row-major matrices: all given, or (a tile-only layer) all NULL
  const bool rm_any = L->w_gate || L->w_up || L->w_down || L->s_gate || L->s_up || L->s_down;
  if (rm_any) {
    if (!L->w_gate || !L->w_up || !L->w_down)
      return fail(MOE_Q4_EINVAL, "w_gate, w_up and w_down are given together or not at all");
    if (L->has_shared && (!L->s_gate || !L->s_up || !L->s_down))
      return fail(MOE_Q4_EINVAL, "has_shared=1 needs s_gate, s_up and s_down");
    if (!L->has_shared && (L->s_gate || L->s_up || L->s_down))
      return fail(MOE_Q4_EINVAL, "s_gate, s_up and s_down are given only with has_shared=1");
  }
  if (!aligned(L->w_router, 16) || !aligned(L->w_gate, 16) || !aligned(L->w_up, 16) ||
      !aligned(L->w_down, 16) || (L->router_bias && !aligned(L->router_bias, 4)))
    return fail(MOE_Q4_EINVAL, "layer pointers must be 16-byte aligned (router_bias 4-byte)");
  if (L->has_shared && (!aligned(L->s_gate, 16) || !aligned(L->s_up, 16) || !aligned(L->s_down, 16)))
    return fail(MOE_Q4_EINVAL, "shared expert pointers must be 16-byte aligned");
  if (L->weight_format != MOE_Q4_WEIGHTS_Q4_0 && L->weight_format != MOE_Q4_WEIGHTS_Q8_0)
    return fail(MOE_Q4_EINVAL, "weight_format=%d must be MOE_Q4_WEIGHTS_Q4_0 or _Q8_0", L->weight_format);
  const bool any_t = L->t_gate || L->t_up || L->t_down || L->ts_gate || L->ts_up || L->ts_down;
  if (any_t) {
    const bool routed = L->t_gate && L->t_up && L->t_down;
    const bool shared = L->has_shared ? (L->ts_gate && L->ts_up && L->ts_down)
                                      : !(L->ts_gate || L->ts_up || L->ts_down);
    if (!routed || !shared)
      return fail(MOE_Q4_EINVAL, "tile-order matrices: t_gate, t_up, t_down (and ts_* exactly when has_shared) "
                                 "are given together or not at all");
    if (L->hidden % 64 || L->inter % 64)
      return fail(MOE_Q4_EINVAL, "tile-order matrices need hidden and inter multiples of 64 (H=%d I=%d)",
                  L->hidden, L->inter);
    if (!aligned(L->t_gate, 16) || !aligned(L->t_up, 16) || !aligned(L->t_down, 16) ||
        (L->has_shared && (!aligned(L->ts_gate, 16) || !aligned(L->ts_up, 16) || !aligned(L->ts_down, 16))))
      return fail(MOE_Q4_EINVAL, "tile-order matrices must be 16-byte aligned");
  }
  if (!rm_any) {
    // tile-only: every decode form must have its tile-order kernels for the
    // shape (the one-launch step falls back to the three-launch kernels)
    if (!any_t) return fail(MOE_Q4_EINVAL, "the layer needs its row-major matrices or their tile-order copies");
    const moeq4::DecodeGeometry g =
        moeq4::decode_geometry(L->hidden, L->inter, L->n_experts, L->top_k, L->has_shared);
    if (g.gt_sp <= 0 || g.dt_sp <= 0)
      return fail(MOE_Q4_EINVAL, "a layer without row-major matrices needs a shape the tile-order decode kernels "
                                 "cover (H=%d I=%d E=%d k=%d)", L->hidden, L->inter, L->n_experts, L->top_k);
  }
  return MOE_Q4_OK;
}

bool tile_only(const moe_q4_layer* L) { return !L->w_gate; }

struct RouteWs {
  size_t partials, counts, rank, tot, total;
};
RouteWs route_ws(const moe_q4_layer* L, int32_t T, const moeq4::RouterSplit& sp) {
  RouteWs w;
  const size_t tiles = ((size_t)T + moeq4::kTopkTokensPerBlock - 1) / moeq4::kTopkTokensPerBlock;
  w.partials = 0;
  w.counts = w.partials + up256((size_t)sp.nsplit * T * L->n_experts * sizeof(float));
  w.rank = w.counts + up256(tiles * L->n_experts * sizeof(int32_t));
  w.tot = w.rank + up256((size_t)T * L->top_k * sizeof(int32_t));
  w.total = w.tot + up256((size_t)L->n_experts * sizeof(int32_t));
  return w;
}

// Prefill workspace, one size for both forms.  bf16 form: h, the routed
// expert outputs (o), the fused launch's tile counters.  W4A8 form: the same
// o, then q8(h) codes and scales, then q8(x) codes and scales.
struct PrefillWs {
  size_t h, o, tile_done, qh, dh, qx, dx, total;
};
PrefillWs prefill_ws(const moe_q4_layer* L, int32_t T) {
  PrefillWs w;
  const size_t rows = (size_t)T * L->top_k + (L->has_shared ? (size_t)T : 0);
  const size_t H = L->hidden, I = L->inter;
  w.h = 0;
  w.o = w.h + up256(rows * I * 2);
  w.tile_done = w.o + up256((size_t)T * L->top_k * H * 2);
  // per-tile counters of the fused launch, then the count of waits that gave up
  const size_t bf16_total =
      w.tile_done + up256(((size_t)moeq4::prefill_tile_bound(T, L->top_k, L->n_experts, L->has_shared) + 1) * 4);
  w.qh = w.tile_done;
  w.dh = w.qh + up256(rows * I);
  w.qx = w.dh + up256(rows * (I / 32) * 4);
  w.dx = w.qx + up256((size_t)T * H);
  const size_t w4a8_total = w.dx + up256((size_t)T * (H / 32) * 4);
  w.total = bf16_total > w4a8_total ? bf16_total : w4a8_total;
  return w;
}

// Decode workspace: a header (the one-launch decode's failure count and epoch
// slots), the one-launch path's handoff words, then the three-launch path's
// pieces.
struct DecodeWs {
  size_t hdr, ll_leaf, ll_route, ll_qh, partials, ids, w, qx, dx, sx, qh, dh, sh, total;
};
DecodeWs decode_ws(const moe_q4_layer* L) {
  DecodeWs w;
  const size_t ns = (size_t)L->top_k + (L->has_shared ? 1 : 0);
  const size_t H = L->hidden, I = L->inter;
  const moeq4::FusedGeometry fg = moeq4::fused_geometry(L->hidden, L->inter, L->n_experts, L->top_k, L->has_shared);
  w.hdr = 0;
  w.ll_leaf = up256(moeq4::kFuHeaderBytes);
  w.ll_route = w.ll_leaf + (fg.ok ? up256((size_t)fg.n_cg * L->n_experts * 8) : 0);
  w.ll_qh = w.ll_route + (fg.ok ? up256((size_t)L->top_k * 2 * 8) : 0);
  w.partials = w.ll_qh + (fg.ok ? up256(ns * I / 32 * 10 * 8) : 0);
  w.ids = w.partials + up256(H / 32 * (size_t)L->n_experts * 4);
  w.w = w.ids + up256((size_t)L->top_k * 4);
  w.qx = w.w + up256((size_t)L->top_k * 4);
  w.dx = w.qx + up256(H);
  w.sx = w.dx + up256(H / 32 * 4);
  w.qh = w.sx + up256(H / 32 * 4);
  w.dh = w.qh + up256(ns * I);
  w.sh = w.dh + up256(ns * I / 32 * 4);
  w.total = w.sh + up256(ns * I / 32 * 4);
  return w;
}

struct DecodeBatchWs {
  size_t partials, qx, dx, sx, ids, w, qh, dh, sh, o, total;
};
DecodeBatchWs decode_batch_ws(const moe_q4_layer* L, int32_t M) {
  DecodeBatchWs w;
  const size_t m = (size_t)M, k = (size_t)L->top_k, E = (size_t)L->n_experts;
  const size_t H = L->hidden, I = L->inter, nc = H / 32;
  const size_t np = m * k + (L->has_shared ? m : 0);
  // after the one-token layout, which M <= 2 uses on the same workspace
  w.partials = decode_ws(L).total;
  w.qx = w.partials + up256(m * nc * E * 4);
  w.dx = w.qx + up256(m * H);
  w.sx = w.dx + up256(m * nc * 4);
  w.ids = w.sx + up256(m * nc * 4);
  w.w = w.ids + up256(m * k * 4);
  w.qh = w.w + up256(m * k * 4);
  w.dh = w.qh + up256(np * I);
  w.sh = w.dh + up256(np * I / 32 * 4);
  w.o = w.sh + up256(np * I / 32 * 4);
  w.total = w.o + up256(np * H * 4);
  return w;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return MOE_Q4_OK;
  if (!ws) return fail(MOE_Q4_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(ws, 256)) return fail(MOE_Q4_EWORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(MOE_Q4_EWORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return MOE_Q4_OK;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

// The decode arguments of layer L with workspace ws laid out by decode_ws;
// the caller sets x, y, the trace and the norm fields.
moeq4::DecodeArgs decode_args(const moe_q4_layer* L, void* ws) {
  const DecodeWs W = decode_ws(L);
  moeq4::DecodeArgs a;
  memset(&a, 0, sizeof a);
  a.H = L->hidden;
  a.I = L->inter;
  a.E = L->n_experts;
  a.k = L->top_k;
  a.has_shared = L->has_shared;
  a.wfmt = L->weight_format;
  a.w_router = L->w_router;
  a.bias = L->router_bias;
  a.w_gate = static_cast<const uint8_t*>(L->w_gate);
  a.w_up = static_cast<const uint8_t*>(L->w_up);
  a.w_down = static_cast<const uint8_t*>(L->w_down);
  a.s_gate = static_cast<const uint8_t*>(L->s_gate);
  a.s_up = static_cast<const uint8_t*>(L->s_up);
  a.s_down = static_cast<const uint8_t*>(L->s_down);
  a.t_gate = static_cast<const uint8_t*>(L->t_gate);
  a.t_up = static_cast<const uint8_t*>(L->t_up);
  a.ts_gate = static_cast<const uint8_t*>(L->ts_gate);
  a.ts_up = static_cast<const uint8_t*>(L->ts_up);
  a.t_down = static_cast<const uint8_t*>(L->t_down);
  a.ts_down = static_cast<const uint8_t*>(L->ts_down);
  a.partials = at<float>(ws, W.partials);
  a.ids = at<int32_t>(ws, W.ids);
  a.w = at<float>(ws, W.w);
  a.qx = at<int8_t>(ws, W.qx);
  a.dx = at<float>(ws, W.dx);
  a.sx = at<int32_t>(ws, W.sx);
  a.qh = at<int8_t>(ws, W.qh);
  a.dh = at<float>(ws, W.dh);
  a.sh = at<int32_t>(ws, W.sh);
  a.hdr = at<uint64_t>(ws, W.hdr);
  a.ll_leaf = at<uint64_t>(ws, W.ll_leaf);
  a.ll_route = at<uint64_t>(ws, W.ll_route);
  a.ll_qh = at<uint64_t>(ws, W.ll_qh);
  return a;
}

// One decode step: the one-launch kernel when the layer and the GPU allow it
// (tile-order copies, covered shape, grid resident at once), else the three
// launches.  Both give the same y bit for bit.
std::atomic<int> g_test_decode_wait_fail{0};

hipError_t decode_step(const moeq4::DecodeArgs& a, hipStream_t stream) {
  if (moeq4::fused_decode_available(a)) {
    moeq4::DecodeArgs b = a;
    b.test_wait_fail = g_test_decode_wait_fail.load();
    b.spin_max = b.test_wait_fail ? 16 : (1 << 20);
    return moeq4::launch_decode_fused(b, stream);
  }
  return moeq4::launch_decode(a, stream);
}

// Device address of `scratch` on each device, looked up once per device with
// that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int noalloc_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_Q4_EINVAL, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "moe_q4_decode_noalloc: hipGetSymbolAddress(scratch)");
    if (!p || !aligned(p, 256)) return fail(MOE_Q4_EHIP, "moe_q4_decode_noalloc: scratch at %p is not 256-byte aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_Q4_OK;
}

}  // namespace

extern "C" {

const char* moe_q4_last_error(void) { return g_err; }

size_t q4_packed_bytes(int64_t rows, int64_t K) {
  if (rows < 0 || K <= 0 || K % 32) return 0;
  return (size_t)rows * (size_t)(K / 32) * 18;
}

int q4_pack(const float* w, int64_t rows, int64_t K, void* packed, hipStream_t stream) {
  if (rows < 0 || K <= 0 || K % 32) return fail(MOE_Q4_EINVAL, "q4_pack: rows=%lld K=%lld (K %% 32 == 0)", (long long)rows, (long long)K);
  if (rows == 0) return MOE_Q4_OK;
  if (!w || !packed) return fail(MOE_Q4_EINVAL, "q4_pack: NULL pointer");
  if (!aligned(w, 16) || !aligned(packed, 2)) return fail(MOE_Q4_EINVAL, "q4_pack: w must be 16-byte and packed 2-byte aligned");
  if (rows * (K / 32) > ((int64_t)1 << 40)) return fail(MOE_Q4_EINVAL, "q4_pack: too many blocks");
  hipError_t e = moeq4::launch_q4_pack(w, rows, K, packed, stream);
  return e == hipSuccess ? MOE_Q4_OK : hip_fail(e, "q4_pack");
}

size_t q8w_packed_bytes(int64_t rows, int64_t K) {
  if (rows < 0 || K <= 0 || K % 32) return 0;
  return (size_t)rows * (size_t)(K / 32) * 34;
}

int q8w_pack(const float* w, int64_t rows, int64_t K, void* packed, hipStream_t stream) {
  if (rows < 0 || K <= 0 || K % 32) return fail(MOE_Q4_EINVAL, "q8w_pack: rows=%lld K=%lld (K %% 32 == 0)", (long long)rows, (long long)K);
  if (rows == 0) return MOE_Q4_OK;
  if (!w || !packed) return fail(MOE_Q4_EINVAL, "q8w_pack: NULL pointer");
  if (!aligned(w, 16) || !aligned(packed, 2)) return fail(MOE_Q4_EINVAL, "q8w_pack: w must be 16-byte and packed 2-byte aligned");
  if (rows * (K / 32) > ((int64_t)1 << 40)) return fail(MOE_Q4_EINVAL, "q8w_pack: too many blocks");
  hipError_t e = moeq4::launch_q8w_pack(w, rows, K, packed, stream);
  return e == hipSuccess ? MOE_Q4_OK : hip_fail(e, "q8w_pack");
}

int q4_tile(const void* q4, int64_t rows, int64_t K, void* tiled, hipStream_t stream) {
  if (rows < 0 || rows % 32 || K <= 0 || K % 64)
    return fail(MOE_Q4_EINVAL, "q4_tile: rows=%lld K=%lld (rows %% 32 == 0, K %% 64 == 0)", (long long)rows, (long long)K);
  if (rows == 0) return MOE_Q4_OK;
  if (!q4 || !tiled) return fail(MOE_Q4_EINVAL, "q4_tile: NULL pointer");
  if (!aligned(q4, 2) || !aligned(tiled, 16)) return fail(MOE_Q4_EINVAL, "q4_tile: q4 must be 2-byte and tiled 16-byte aligned");
  if (rows * (K / 32) > ((int64_t)1 << 40)) return fail(MOE_Q4_EINVAL, "q4_tile: too many blocks");
  const size_t bytes = (size_t)rows * (size_t)(K / 32) * 18;
  const uintptr_t a0 = (uintptr_t)q4, b0 = (uintptr_t)tiled;
  if (a0 < b0 + bytes && b0 < a0 + bytes) return fail(MOE_Q4_EINVAL, "q4_tile: q4 and tiled overlap");
  hipError_t e = moeq4::launch_q4_tile(q4, rows, K, tiled, stream);
  return e == hipSuccess ? MOE_Q4_OK : hip_fail(e, "q4_tile");
}

int q8w_tile(const void* q8, int64_t rows, int64_t K, void* tiled, hipStream_t stream) {
  if (rows < 0 || rows % 32 || K <= 0 || K % 64)
    return fail(MOE_Q4_EINVAL, "q8w_tile: rows=%lld K=%lld (rows %% 32 == 0, K %% 64 == 0)", (long long)rows, (long long)K);
  if (rows == 0) return MOE_Q4_OK;
  if (!q8 || !tiled) return fail(MOE_Q4_EINVAL, "q8w_tile: NULL pointer");
  if (!aligned(q8, 2) || !aligned(tiled, 16)) return fail(MOE_Q4_EINVAL, "q8w_tile: q8 must be 2-byte and tiled 16-byte aligned");
  if (rows * (K / 32) > ((int64_t)1 << 40)) return fail(MOE_Q4_EINVAL, "q8w_tile: too many blocks");
  const size_t bytes = (size_t)rows * (size_t)(K / 32) * 34;
  const uintptr_t a0 = (uintptr_t)q8, b0 = (uintptr_t)tiled;
  if (a0 < b0 + bytes && b0 < a0 + bytes) return fail(MOE_Q4_EINVAL, "q8w_tile: q8 and tiled overlap");
  hipError_t e = moeq4::launch_q8w_tile(q8, rows, K, tiled, stream);
  return e == hipSuccess ? MOE_Q4_OK : hip_fail(e, "q8w_tile");
}

int q8_quantize(const float* x, int64_t rows, int64_t K, int8_t* q, float* d, hipStream_t stream) {
  if (rows < 0 || K <= 0 || K % 32) return fail(MOE_Q4_EINVAL, "q8_quantize: rows=%lld K=%lld (K %% 32 == 0)", (long long)rows, (long long)K);
  if (rows == 0) return MOE_Q4_OK;
  if (!x || !q || !d) return fail(MOE_Q4_EINVAL, "q8_quantize: NULL pointer");
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(d, 4)) return fail(MOE_Q4_EINVAL, "q8_quantize: x and q must be 16-byte aligned");
  hipError_t e = moeq4::launch_q8_quantize(x, rows, K, q, d, stream);
  return e == hipSuccess ? MOE_Q4_OK : hip_fail(e, "q8_quantize");
}

size_t moe_q4_route_workspace_bytes(const moe_q4_layer* L, int32_t T) {
  if (check_layer(L) != MOE_Q4_OK || T < 0) return 0;
  return route_ws(L, T, moeq4::prefill_router_split(L->hidden)).total;
}

int moe_q4_route(const moe_q4_layer* L, const void* x, int32_t x_dtype, int32_t T,
                 const moe_q4_routing* out, float* logits, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (T < 0) return fail(MOE_Q4_EINVAL, "moe_q4_route: T=%d < 0", T);
  if (x_dtype != MOE_Q4_F32 && x_dtype != MOE_Q4_BF16) return fail(MOE_Q4_EINVAL, "moe_q4_route: bad x_dtype %d", x_dtype);
  if ((int64_t)T * L->top_k > 0x7fffffff) return fail(MOE_Q4_EINVAL, "moe_q4_route: T*k exceeds int32");
  if (!out) return fail(MOE_Q4_EINVAL, "moe_q4_route: routing is NULL");
  if (T == 0) {
    // only the offsets have content: all zero (the scan over no tiles)
    if (!out->expert_offsets) return fail(MOE_Q4_EINVAL, "moe_q4_route: expert_offsets is NULL");
    hipError_t e = moeq4::launch_route_scatter(nullptr, nullptr, nullptr, nullptr, 0, L->top_k, L->n_experts,
                                               out->expert_offsets, nullptr, nullptr, stream);
    return e == hipSuccess ? MOE_Q4_OK : hip_fail(e, "moe_q4_route");
  }
  if (!x || !out->topk_ids || !out->topk_w || !out->expert_offsets || !out->perm || !out->inv_perm)
    return fail(MOE_Q4_EINVAL, "moe_q4_route: NULL pointer");
  if (!aligned(x, 16)) return fail(MOE_Q4_EINVAL, "moe_q4_route: x must be 16-byte aligned");
  const moeq4::RouterSplit sp = moeq4::prefill_router_split(L->hidden);
  const RouteWs W = route_ws(L, T, sp);
  rc = check_ws(ws, ws_bytes, W.total);
  if (rc) return rc;
  float* partials = at<float>(ws, W.partials);
  int32_t* counts = at<int32_t>(ws, W.counts);
  int32_t* rank = at<int32_t>(ws, W.rank);
  const int E = L->n_experts, k = L->top_k;
  hipError_t e = moeq4::launch_router_partials(x, x_dtype == MOE_Q4_BF16, T, L->hidden, L->w_router, E, sp,
                                               partials, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_q4_route/router");
  e = moeq4::launch_topk_hist(partials, sp, L->router_bias, T, E, k, logits, out->topk_ids, out->topk_w,
                              counts, rank, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_q4_route/topk");
  const int tiles = (T + moeq4::kTopkTokensPerBlock - 1) / moeq4::kTopkTokensPerBlock;
  int32_t* tot = at<int32_t>(ws, W.tot);
  e = moeq4::launch_route_colscan(counts, tiles, E, tot, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_q4_route/scan");
  e = moeq4::launch_route_scatter(out->topk_ids, rank, counts, tot, T, k, E, out->expert_offsets, out->perm,
                                  out->inv_perm, stream);
  if (e != hipSuccess) return hip_fail(e, "moe_q4_route/scatter");
  return MOE_Q4_OK;
}

size_t moe_q4_prefill_workspace_bytes(const moe_q4_layer* L, int32_t T) {
  if (check_layer(L) != MOE_Q4_OK || T < 0) return 0;
  return prefill_ws(L, T).total;
}

int moe_q4_prefill(const moe_q4_layer* L, const uint16_t* x_bf16, int32_t T,
                   const moe_q4_routing* routing, float* y, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
  return moe_q4_prefill_stage(L, x_bf16, T, routing, y, ws, ws_bytes, MOE_Q4_STAGE_ALL, stream);
}

int moe_q4_prefill_stage(const moe_q4_layer* L, const uint16_t* x_bf16, int32_t T,
                         const moe_q4_routing* routing, float* y, void* ws, size_t ws_bytes,
                         int32_t stages, hipStream_t stream) {
  const int test_wait_fail = (stages & MOE_Q4_STAGE_TEST_WAIT_FAIL) != 0;
  stages &= ~MOE_Q4_STAGE_TEST_WAIT_FAIL;
  if (stages <= 0 || stages > MOE_Q4_STAGE_ALL)
    return fail(MOE_Q4_EINVAL, "moe_q4_prefill_stage: stages=%d must be a non-empty mask of 1|2|4 (| 16)", stages);
  int rc = check_layer(L);
  if (rc) return rc;
  if (T < 0) return fail(MOE_Q4_EINVAL, "moe_q4_prefill: T=%d < 0", T);
  if ((int64_t)T * L->top_k > 0x7fffffff) return fail(MOE_Q4_EINVAL, "moe_q4_prefill: T*k exceeds int32");
  if (L->weight_format != MOE_Q4_WEIGHTS_Q4_0)
    return fail(MOE_Q4_EINVAL, "moe_q4_prefill: the grouped GEMM takes Q4_0 weights (weight_format=%d)", L->weight_format);
  if (T == 0) return MOE_Q4_OK;
  if (!x_bf16 || !routing || !y || !routing->topk_w || !routing->expert_offsets || !routing->perm ||
      !routing->inv_perm)
    return fail(MOE_Q4_EINVAL, "moe_q4_prefill: NULL pointer");
  if (!aligned(x_bf16, 16) || !aligned(y, 16)) return fail(MOE_Q4_EINVAL, "moe_q4_prefill: x_bf16 and y must be 16-byte aligned");
  // (the tile-order kernels address x through one 32-bit byte range; larger
  // batches take the generic kernels, which read the row-major matrices)
  if (tile_only(L) && (uint64_t)T * (uint64_t)L->hidden * 2u > 0xffffffffull)
    return fail(MOE_Q4_EINVAL, "moe_q4_prefill: T=%d too large for a layer without row-major matrices "
                               "(T * hidden * 2 must fit 32 bits)", T);
  const PrefillWs W = prefill_ws(L, T);
  rc = check_ws(ws, ws_bytes, W.total);
  if (rc) return rc;
  moeq4::PrefillArgs a;
  a.x = x_bf16;
  a.T = T;
  a.H = L->hidden;
  a.I = L->inter;
  a.E = L->n_experts;
  a.k = L->top_k;
  a.has_shared = L->has_shared;
  a.perm = routing->perm;
  a.offsets = routing->expert_offsets;
  a.inv_perm = routing->inv_perm;
  a.topk_w = routing->topk_w;
  a.w_gate = static_cast<const uint8_t*>(L->w_gate);
  a.w_up = static_cast<const uint8_t*>(L->w_up);
  a.w_down = static_cast<const uint8_t*>(L->w_down);
  a.s_gate = static_cast<const uint8_t*>(L->s_gate);
  a.s_up = static_cast<const uint8_t*>(L->s_up);
  a.s_down = static_cast<const uint8_t*>(L->s_down);
  a.t_gate = static_cast<const uint8_t*>(L->t_gate);
  a.t_up = static_cast<const uint8_t*>(L->t_up);
  a.t_down = static_cast<const uint8_t*>(L->t_down);
  a.ts_gate = static_cast<const uint8_t*>(L->ts_gate);
  a.ts_up = static_cast<const uint8_t*>(L->ts_up);
  a.ts_down = static_cast<const uint8_t*>(L->ts_down);
  a.h = at<uint16_t>(ws, W.h);
  a.o_perm = at<uint16_t>(ws, W.o);
  a.tile_done = at<int32_t>(ws, W.tile_done);
  a.test_wait_fail = test_wait_fail;
  a.y = y;
  hipError_t e = moeq4::launch_prefill(a, stages, stream);
  return e == hipSuccess ? MOE_Q4_OK : hip_fail(e, "moe_q4_prefill");
}

int moe_q4_prefill_w4a8(const moe_q4_layer* L, const uint16_t* x_bf16, int32_t T, const moe_q4_routing* routing,
                        float* y, int32_t* gate_dots, void* ws, size_t ws_bytes, hipStream_t stream) {
  return moe_q4_prefill_w4a8_stage(L, x_bf16, T, routing, y, gate_dots, ws, ws_bytes, MOE_Q4_STAGE_ALL, stream);
}

int moe_q4_prefill_w4a8_stage(const moe_q4_layer* L, const uint16_t* x_bf16, int32_t T,
                              const moe_q4_routing* routing, float* y, int32_t* gate_dots, void* ws,
                              size_t ws_bytes, int32_t stages, hipStream_t stream) {
  if (stages & ~MOE_Q4_STAGE_ALL || !stages)
    return fail(MOE_Q4_EINVAL, "moe_q4_prefill_w4a8_stage: stages=%d (a nonzero mask of GATEUP, DOWN, COMBINE)",
                stages);
  int rc = check_layer(L);
  if (rc) return rc;
  if (T < 0) return fail(MOE_Q4_EINVAL, "moe_q4_prefill_w4a8: T=%d < 0", T);
  if ((int64_t)T * L->top_k > 0x7fffffff) return fail(MOE_Q4_EINVAL, "moe_q4_prefill_w4a8: T*k exceeds int32");
  if (L->weight_format != MOE_Q4_WEIGHTS_Q4_0)
    return fail(MOE_Q4_EINVAL, "moe_q4_prefill_w4a8: Q4_0 weights only (weight_format=%d)", L->weight_format);
  if (!L->t_gate) return fail(MOE_Q4_EINVAL, "moe_q4_prefill_w4a8: needs the tile-order copies (q4_tile)");
  if (L->hidden > 4096 || L->inter > 4096)
    return fail(MOE_Q4_EINVAL, "moe_q4_prefill_w4a8: hidden=%d inter=%d (each <= 4096)", L->hidden, L->inter);
  if (T == 0) return MOE_Q4_OK;
  if (!x_bf16 || !routing || !y || !routing->topk_w || !routing->expert_offsets || !routing->perm ||
      !routing->inv_perm)
    return fail(MOE_Q4_EINVAL, "moe_q4_prefill_w4a8: NULL pointer");
  if (!aligned(x_bf16, 16) || !aligned(y, 16) || !aligned(gate_dots, 4))
    return fail(MOE_Q4_EINVAL, "moe_q4_prefill_w4a8: x_bf16 and y 16-byte, gate_dots 4-byte aligned");
  const PrefillWs W = prefill_ws(L, T);
  rc = check_ws(ws, ws_bytes, W.total);
  if (rc) return rc;
  moeq4::W4A8PrefillArgs a;
  memset(&a, 0, sizeof a);
  a.x = x_bf16;
  a.T = T;
  a.H = L->hidden;
  a.I = L->inter;
  a.E = L->n_experts;
  a.k = L->top_k;
  a.has_shared = L->has_shared;
  a.perm = routing->perm;
  a.offsets = routing->expert_offsets;
  a.t_gate = static_cast<const uint8_t*>(L->t_gate);
  a.t_up = static_cast<const uint8_t*>(L->t_up);
  a.t_down = static_cast<const uint8_t*>(L->t_down);
  a.ts_gate = static_cast<const uint8_t*>(L->ts_gate);
  a.ts_up = static_cast<const uint8_t*>(L->ts_up);
  a.ts_down = static_cast<const uint8_t*>(L->ts_down);
  a.qx = at<int8_t>(ws, W.qx);
  a.dx = at<float>(ws, W.dx);
  a.qh = at<int8_t>(ws, W.qh);
  a.dh = at<float>(ws, W.dh);
  a.o_perm = at<uint16_t>(ws, W.o);
  a.y = y;
  hipError_t e = hipSuccess;
  if (stages & (MOE_Q4_STAGE_GATEUP | MOE_Q4_STAGE_DOWN)) {
    e = moeq4::launch_prefill_w4a8(a, gate_dots, stages & 3, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_q4_prefill_w4a8");
  }
  if (!(stages & MOE_Q4_STAGE_COMBINE)) return MOE_Q4_OK;
  // the weighted combine of the routed outputs into y (the bf16 form's)
  moeq4::PrefillArgs c;
  memset(&c, 0, sizeof c);
  c.x = x_bf16;
  c.T = T;
  c.H = L->hidden;
  c.I = L->inter;
  c.E = L->n_experts;
  c.k = L->top_k;
  c.has_shared = L->has_shared;
  c.perm = routing->perm;
  c.offsets = routing->expert_offsets;
  c.inv_perm = routing->inv_perm;
  c.topk_w = routing->topk_w;
  c.o_perm = a.o_perm;
  c.y = y;
  e = moeq4::launch_prefill(c, MOE_Q4_STAGE_COMBINE, stream);
  return e == hipSuccess ? MOE_Q4_OK : hip_fail(e, "moe_q4_prefill_w4a8/combine");
}

int moe_q4_check_layer(const moe_q4_layer* L) { return check_layer(L); }

int moe_q4_prefill_status(const moe_q4_layer* L, int32_t T, const void* ws, size_t ws_bytes,
                          int32_t* failed_waits, hipStream_t stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (T < 0 || !failed_waits) return fail(MOE_Q4_EINVAL, "moe_q4_prefill_status: T=%d, failed_waits=%p", T,
                                          (void*)failed_waits);
  *failed_waits = 0;
  if (T == 0) return MOE_Q4_OK;
  const PrefillWs W = prefill_ws(L, T);
  rc = check_ws(const_cast<void*>(ws), ws_bytes, W.total);
  if (rc) return rc;
  const size_t n_tiles = (size_t)moeq4::prefill_tile_bound(T, L->top_k, L->n_experts, L->has_shared);
  const char* src = static_cast<const char*>(ws) + W.tile_done + n_tiles * 4;
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, src, 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "moe_q4_prefill_status");
  *failed_waits = v;
  return MOE_Q4_OK;
}

// Batches of up to this many tokens run the one-token program token by
// token (3 launches each): faster than the batched kernels' 5 launches there
// (1 token: 17.4 against 34.9 us; 2: 34.8 against 39.0 us at the decode
// layer's shape), and the same results by construction.
constexpr int32_t kDecodeBatchPerToken = 2;

size_t moe_q4_decode_batch_workspace_bytes(const moe_q4_layer* L, int32_t M) {
  if (check_layer(L) != MOE_Q4_OK || M < 0 || M > moeq4::kDecodeBatchMax) return 0;
  if (M == 0) return 0;
  if (M <= kDecodeBatchPerToken) return decode_ws(L).total;
  return decode_batch_ws(L, M).total;
}

int moe_q4_decode_batch(const moe_q4_layer* L, const float* x, int32_t M, float* y, int32_t* ids_out,
                        float* w_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (M < 0 || M > moeq4::kDecodeBatchMax)
    return fail(MOE_Q4_EINVAL, "moe_q4_decode_batch: M=%d must be in [0, %d]", M, moeq4::kDecodeBatchMax);
  if (L->hidden > 32 * 512) return fail(MOE_Q4_EINVAL, "moe_q4_decode_batch: hidden=%d > 16384", L->hidden);
  if (M == 0) return MOE_Q4_OK;
  if (!x || !y) return fail(MOE_Q4_EINVAL, "moe_q4_decode_batch: NULL pointer");
  if (!aligned(x, 16) || !aligned(y, 4)) return fail(MOE_Q4_EINVAL, "moe_q4_decode_batch: x must be 16-byte aligned");
  if (M <= kDecodeBatchPerToken) {
    rc = check_ws(ws, ws_bytes, decode_ws(L).total);
    if (rc) return rc;
    const size_t H = (size_t)L->hidden, k = (size_t)L->top_k;
    for (int32_t t = 0; t < M; t++) {     // one stream: the calls reuse the workspace in order
      moeq4::DecodeArgs a = decode_args(L, ws);
      a.x = x + t * H;
      a.y = y + t * H;
      a.t_ids = ids_out ? ids_out + t * k : nullptr;
      a.t_w = w_out ? w_out + t * k : nullptr;
      hipError_t e = decode_step(a, stream);
      if (e != hipSuccess) return hip_fail(e, "moe_q4_decode_batch");
    }
    return MOE_Q4_OK;
  }
  const DecodeBatchWs W = decode_batch_ws(L, M);
  rc = check_ws(ws, ws_bytes, W.total);
  if (rc) return rc;
  moeq4::DecodeBatchArgs a;
  memset(&a, 0, sizeof a);
  a.x = x;
  a.y = y;
  a.M = M;
  a.H = L->hidden;
  a.I = L->inter;
  a.E = L->n_experts;
  a.k = L->top_k;
  a.has_shared = L->has_shared;
  a.wfmt = L->weight_format;
  a.w_router = L->w_router;
  a.bias = L->router_bias;
  a.w_gate = static_cast<const uint8_t*>(L->w_gate);
  a.w_up = static_cast<const uint8_t*>(L->w_up);
  a.w_down = static_cast<const uint8_t*>(L->w_down);
  a.s_gate = static_cast<const uint8_t*>(L->s_gate);
  a.s_up = static_cast<const uint8_t*>(L->s_up);
  a.s_down = static_cast<const uint8_t*>(L->s_down);
  a.t_gate = static_cast<const uint8_t*>(L->t_gate);
  a.t_up = static_cast<const uint8_t*>(L->t_up);
  a.t_down = static_cast<const uint8_t*>(L->t_down);
  a.ts_gate = static_cast<const uint8_t*>(L->ts_gate);
  a.ts_up = static_cast<const uint8_t*>(L->ts_up);
  a.ts_down = static_cast<const uint8_t*>(L->ts_down);
  a.partials = at<float>(ws, W.partials);
  a.qx = at<int8_t>(ws, W.qx);
  a.dx = at<float>(ws, W.dx);
  a.sx = at<int32_t>(ws, W.sx);
  a.ids = at<int32_t>(ws, W.ids);
  a.w = at<float>(ws, W.w);
  a.qh = at<int8_t>(ws, W.qh);
  a.dh = at<float>(ws, W.dh);
  a.sh = at<int32_t>(ws, W.sh);
  a.o = at<float>(ws, W.o);
  a.t_ids = ids_out;
  a.t_w = w_out;
  hipError_t e = moeq4::launch_decode_batch(a, stream);
  return e == hipSuccess ? MOE_Q4_OK : hip_fail(e, "moe_q4_decode_batch");
}

size_t moe_q4_decode_workspace_bytes(const moe_q4_layer* L) {
  if (check_layer(L) != MOE_Q4_OK) return 0;
  return decode_ws(L).total;
}

int moe_q4_decode(const moe_q4_layer* L, const float* x, float* y, const moe_q4_decode_trace* tr,
                  void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (!x || !y) return fail(MOE_Q4_EINVAL, "moe_q4_decode: NULL pointer");
  if (!aligned(x, 16) || !aligned(y, 4)) return fail(MOE_Q4_EINVAL, "moe_q4_decode: x must be 16-byte aligned");
  const DecodeWs W = decode_ws(L);
  rc = check_ws(ws, ws_bytes, W.total);
  if (rc) return rc;
  if (tr && ((tr->qx && !aligned(tr->qx, 16)) || (tr->qh && !aligned(tr->qh, 16))))
    return fail(MOE_Q4_EINVAL, "moe_q4_decode: trace qx and qh must be 16-byte aligned");
  moeq4::DecodeArgs a = decode_args(L, ws);
  a.x = x;
  a.y = y;
  if (tr) {
    a.t_logits = tr->logits;
    a.t_ids = tr->ids;
    a.t_w = tr->w;
    a.t_qx = tr->qx;
    a.t_dx = tr->dx;
    a.t_qh = tr->qh;
    a.t_dh = tr->dh;
  }
  hipError_t e = decode_step(a, stream);
  return e == hipSuccess ? MOE_Q4_OK : hip_fail(e, "moe_q4_decode");
}

int moe_q4_decode_noalloc(const moe_q4_layer* L, const float* x, float* y, hipStream_t stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (!x || !y) return fail(MOE_Q4_EINVAL, "moe_q4_decode_noalloc: NULL pointer");
  if (!aligned(x, 16) || !aligned(y, 4)) return fail(MOE_Q4_EINVAL, "moe_q4_decode_noalloc: x must be 16-byte aligned");
  const size_t need = decode_ws(L).total;
  if (need > (size_t)MOE_Q4_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_Q4_EWORKSPACE,
                "moe_q4_decode_noalloc: this layer needs %zu bytes of scratch, the fixed array holds %zu "
                "(use moe_q4_decode with a workspace)", need, (size_t)MOE_Q4_NOALLOC_SCRATCH_BYTES);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "moe_q4_decode_noalloc: hipGetDevice");
  if (stream) {
    int sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return hip_fail(e, "moe_q4_decode_noalloc: hipStreamGetDevice");
    if (sdev != dev)
      return fail(MOE_Q4_EINVAL, "moe_q4_decode_noalloc: the stream belongs to device %d, the current device is %d",
                  sdev, dev);
  }
  void* ws = nullptr;
  rc = noalloc_scratch(dev, &ws);
  if (rc) return rc;
  // the three decode kernels write every scratch piece before reading it, so
  // nothing needs clearing between calls
  moeq4::DecodeArgs a = decode_args(L, ws);
  a.x = x;
  a.y = y;
  e = moeq4::launch_decode(a, stream);
  return e == hipSuccess ? MOE_Q4_OK : hip_fail(e, "moe_q4_decode_noalloc");
}

void moe_q4_test_decode_wait_fail(int32_t on) { g_test_decode_wait_fail.store(on ? 1 : 0); }

int moe_q4_decode_status(const moe_q4_layer* L, const void* ws, size_t ws_bytes, int32_t* failed_waits,
                         hipStream_t stream) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (!failed_waits) return fail(MOE_Q4_EINVAL, "moe_q4_decode_status: failed_waits is NULL");
  rc = check_ws(const_cast<void*>(ws), ws_bytes, decode_ws(L).total);
  if (rc) return rc;
  uint32_t* word = reinterpret_cast<uint32_t*>(const_cast<void*>(ws));
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, word, 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e == hipSuccess && v != 0) {
    e = hipMemsetAsync(word, 0, 4, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
  }
  if (e != hipSuccess) return hip_fail(e, "moe_q4_decode_status");
  *failed_waits = (int32_t)v;
  return MOE_Q4_OK;
}

size_t moe_q4_decode_stack_workspace_bytes(const moe_q4_layer* layers, int32_t n_layers) {
  if (!layers || n_layers < 0) return 0;
  size_t need = 0;
  for (int32_t l = 0; l < n_layers; l++) {
    if (check_layer(&layers[l]) != MOE_Q4_OK) return 0;
    const size_t w = decode_ws(&layers[l]).total;
    need = w > need ? w : need;
  }
  // two y buffers between runs of layers, then the tagged words of a layer's y
  return need + (n_layers > 0 ? 2 * up256((size_t)layers[0].hidden * 4) + up256((size_t)layers[0].hidden * 8) : 0);
}

// Layers that one stacked launch can run together: one shape, one weight
// format, tile-order copies.
static bool same_stack_shape(const moe_q4_layer* a, const moe_q4_layer* b) {
  return a->hidden == b->hidden && a->inter == b->inter && a->n_experts == b->n_experts && a->top_k == b->top_k &&
         a->has_shared == b->has_shared && a->weight_format == b->weight_format && b->t_gate && b->t_up &&
         b->t_down && (!b->has_shared || (b->ts_gate && b->ts_up && b->ts_down));
}

int moe_q4_decode_stack(const moe_q4_layer* layers, int32_t n_layers, const float* x, float* y,
                        float eps, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (n_layers < 0) return fail(MOE_Q4_EINVAL, "moe_q4_decode_stack: n_layers=%d < 0", n_layers);
  if (n_layers == 0) return MOE_Q4_OK;
  if (!layers || !x || !y) return fail(MOE_Q4_EINVAL, "moe_q4_decode_stack: NULL pointer");
  if (!(eps >= 0.0f)) return fail(MOE_Q4_EINVAL, "moe_q4_decode_stack: eps must be >= 0");
  size_t dws = 0;
  for (int32_t l = 0; l < n_layers; l++) {
    int rc = check_layer(&layers[l]);
    if (rc) return rc;
    if (layers[l].hidden != layers[0].hidden)
      return fail(MOE_Q4_EINVAL, "moe_q4_decode_stack: layer %d has hidden=%d, layer 0 %d", l,
                  layers[l].hidden, layers[0].hidden);
    const size_t w = decode_ws(&layers[l]).total;
    dws = w > dws ? w : dws;
  }
  if (!aligned(x, 16) || !aligned(y, 4)) return fail(MOE_Q4_EINVAL, "moe_q4_decode_stack: x must be 16-byte aligned");
  const size_t H = (size_t)layers[0].hidden;
  const size_t need = dws + 2 * up256(H * 4) + up256(H * 8);
  int rc = check_ws(ws, ws_bytes, need);
  if (rc) return rc;
  float* ybuf[2] = {at<float>(ws, dws), at<float>(ws, dws + up256(H * 4))};
  // one launch per run of up to kStackMaxLayers layers when every layer has
  // the first one's shape and the one-launch step is available for it
  bool same = true;
  for (int32_t l = 0; l < n_layers; l++) same = same && same_stack_shape(&layers[0], &layers[l]);
  if (same) {
    moeq4::DecodeArgs a = decode_args(&layers[0], ws);
    a.ll_y = at<uint64_t>(ws, dws + 2 * up256(H * 4));
    a.test_wait_fail = g_test_decode_wait_fail.load();
    // (a normal wait ends within microseconds; a shorter bound than one
    // step's keeps a broken stack from waiting out 40 layers of bounds)
    a.spin_max = a.test_wait_fail ? 16 : (1 << 16);
    a.norm_eps = eps;
    if (moeq4::stack_decode_available(a)) {
      int run = 0;
      for (int32_t c0 = 0; c0 < n_layers; c0 += moeq4::kStackMaxLayers, run++) {
        const int32_t n = n_layers - c0 < moeq4::kStackMaxLayers ? n_layers - c0 : moeq4::kStackMaxLayers;
        moeq4::StackTable t;
        memset(&t, 0, sizeof t);
        t.n = n;
        for (int32_t i = 0; i < n; i++) {
          const moe_q4_layer* L = &layers[c0 + i];
          t.l[i] = {L->w_router, L->router_bias, static_cast<const uint8_t*>(L->t_gate),
                    static_cast<const uint8_t*>(L->t_up), static_cast<const uint8_t*>(L->t_down),
                    static_cast<const uint8_t*>(L->ts_gate), static_cast<const uint8_t*>(L->ts_up),
                    static_cast<const uint8_t*>(L->ts_down)};
        }
        a.norm_in = c0 > 0;
        a.x = c0 == 0 ? x : ybuf[(run - 1) & 1];
        a.y = c0 + n == n_layers ? y : ybuf[run & 1];
        hipError_t e = moeq4::launch_decode_stack(a, t, stream);
        if (e != hipSuccess) return hip_fail(e, "moe_q4_decode_stack");
      }
      return MOE_Q4_OK;
    }
  }
  for (int32_t l = 0; l < n_layers; l++) {
    const moe_q4_layer* L = &layers[l];
    moeq4::DecodeArgs a = decode_args(L, ws);
    a.norm_in = l > 0;
    a.norm_eps = eps;
    a.x = l == 0 ? x : ybuf[(l - 1) & 1];
    a.y = l == n_layers - 1 ? y : ybuf[l & 1];
    hipError_t e = decode_step(a, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_q4_decode_stack");
  }
  return MOE_Q4_OK;
}

int moe_q4_w4a8_gemv(const void* W, int32_t N, int32_t K, const int8_t* qa, const float* da,
                     int32_t* dots, float* out, hipStream_t stream) {
  if (N < 0 || K <= 0 || K % 32 || K > kMaxDim)
    return fail(MOE_Q4_EINVAL, "moe_q4_w4a8_gemv: N=%d K=%d (K a multiple of 32 <= %d)", N, K, kMaxDim);
  if (N == 0) return MOE_Q4_OK;
  if (!W || !qa || !da || !out) return fail(MOE_Q4_EINVAL, "moe_q4_w4a8_gemv: NULL pointer");
  if (!aligned(W, 2) || !aligned(qa, 4) || !aligned(da, 4))
    return fail(MOE_Q4_EINVAL, "moe_q4_w4a8_gemv: W 2-byte, qa/da 4-byte alignment");
  hipError_t e = moeq4::launch_w4a8_gemv(static_cast<const uint8_t*>(W), N, K, qa, da, dots, out, stream);
  return e == hipSuccess ? MOE_Q4_OK : hip_fail(e, "moe_q4_w4a8_gemv");
}

int moe_q4_w4a8_gemm(const void* Wt, int32_t N, int32_t K, const int8_t* qa, const float* da, int32_t M,
                     int32_t* dots, float* out, hipStream_t stream) {
  if (N < 0 || N % 32 || N / 32 > 65535 || K < 64 || K % 64 || K > 4096 || M < 0)
    return fail(MOE_Q4_EINVAL,
                "moe_q4_w4a8_gemm: N=%d K=%d M=%d (N %% 32 == 0, N <= 2097120, K %% 64 == 0, 64 <= K <= 4096)",
                N, K, M);
  if (N == 0 || M == 0) return MOE_Q4_OK;
  if (!Wt || !qa || !da || !out) return fail(MOE_Q4_EINVAL, "moe_q4_w4a8_gemm: NULL pointer");
  if (!aligned(Wt, 16) || !aligned(qa, 16) || !aligned(da, 4) || !aligned(out, 4) || !aligned(dots, 4))
    return fail(MOE_Q4_EINVAL, "moe_q4_w4a8_gemm: Wt and qa 16-byte, da, dots and out 4-byte alignment");
  hipError_t e = moeq4::launch_w4a8_gemm(static_cast<const uint8_t*>(Wt), N, K, qa, da, M, dots, out, stream);
  return e == hipSuccess ? MOE_Q4_OK : hip_fail(e, "moe_q4_w4a8_gemm");
}

int moe_q4_probe_mfma(int32_t kind, int32_t blocks, int32_t iters, float* out, int64_t* ops, hipStream_t stream) {
  if (kind < 0 || kind > 2 || blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 22) || !out || !ops)
    return fail(MOE_Q4_EINVAL, "moe_q4_probe_mfma: kind=%d (0..2) blocks=%d (1..65536) iters=%d (1..2^22), "
                               "out and ops non-NULL", kind, blocks, iters);
  static const int64_t kOpsPerMfma[3] = {32 * 32 * 16 * 2, 32 * 32 * 32 * 2, 2 * 32 * 32 * 1 * 2};
  *ops = moeq4::probe_mfma_count(kind, blocks, iters) * kOpsPerMfma[kind];
  const hipError_t e = moeq4::launch_probe_mfma(kind, blocks, iters, out, stream);
  return e == hipSuccess ? MOE_Q4_OK : hip_fail(e, "moe_q4_probe_mfma");
}

int moe_q4_rmsnorm(const float* y, int32_t T, int32_t H, float eps, float* out_f32,
                   uint16_t* out_bf16, hipStream_t stream) {
  if (T < 0 || H <= 0 || H % 32 || H > kMaxDim)
    return fail(MOE_Q4_EINVAL, "moe_q4_rmsnorm: T=%d H=%d (H a multiple of 32 <= %d)", T, H, kMaxDim);
  if (T == 0) return MOE_Q4_OK;
  if (!y || (!out_f32 && !out_bf16)) return fail(MOE_Q4_EINVAL, "moe_q4_rmsnorm: NULL pointer");
  if (!aligned(y, 16)) return fail(MOE_Q4_EINVAL, "moe_q4_rmsnorm: y must be 16-byte aligned");
  hipError_t e = moeq4::launch_rmsnorm(y, T, H, eps, out_f32, out_bf16, stream);
  return e == hipSuccess ? MOE_Q4_OK : hip_fail(e, "moe_q4_rmsnorm");
}

}  // extern "C"
