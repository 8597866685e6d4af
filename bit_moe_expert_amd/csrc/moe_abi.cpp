// C ABI of libmoe_int4.so: argument validation (before any HIP call), workspace layout and the
// stage sequence of each entry point. The kernels live in route.hip, gemv.hip, gemm.hip,
// dequant.hip and vocab_topk.hip.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "kernels.h"
#include "moe_int4.h"

namespace moe {
namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_dims(const moe_dims* dm, int32_t T) {
  if (!dm) return fail(MOE_EINVAL, "dims is NULL");
  if (T < 0) return fail(MOE_EINVAL, "T = %d is negative", T);
  if (T > 65536) return fail(MOE_EUNSUPPORTED, "T = %d exceeds 65536", T);
  if (dm->group_size != 64) return fail(MOE_EUNSUPPORTED, "group_size = %d, only 64 is supported", dm->group_size);
  if (dm->d_model < 64 || dm->d_model > 16384 || dm->d_model % 64)
    return fail(MOE_EUNSUPPORTED, "d_model = %d must be a multiple of 64 in [64, 16384]", dm->d_model);
  if (dm->n_experts < 1 || dm->n_experts > 1024)
    return fail(MOE_EUNSUPPORTED, "n_experts = %d must be in [1, 1024]", dm->n_experts);
  if (dm->top_k < 1 || dm->top_k > 16 || dm->top_k > dm->n_experts)
    return fail(MOE_EUNSUPPORTED, "top_k = %d must be in [1, min(n_experts, 16)]", dm->top_k);
  if (dm->d_ff < 64 || dm->d_ff > 8192 || dm->d_ff % 64)
    return fail(MOE_EUNSUPPORTED, "d_ff = %d must be a multiple of 64 in [64, 8192]", dm->d_ff);
  if (dm->d_ff_shared < 0 || dm->d_ff_shared > 8192 || dm->d_ff_shared % 64)
    return fail(MOE_EUNSUPPORTED, "d_ff_shared = %d must be 0 or a multiple of 64 up to 8192", dm->d_ff_shared);
  if (dm->code_bits != 0 && dm->code_bits != 2 && dm->code_bits != 3 && dm->code_bits != 4)
    return fail(MOE_EUNSUPPORTED, "code_bits = %d must be 4 (or 0), 3 or 2", dm->code_bits);
  return MOE_OK;
}

int bits_of(const moe_dims& dm) { return dm.code_bits == 0 ? 4 : dm.code_bits; }

// 16-byte loads of 4- and 2-bit codes, 12-byte (dword-aligned) loads of 3-bit codes
size_t code_align(int bits) { return bits == 3 ? 4 : 16; }

int32_t max_tiles_of(const moe_dims& dm, int32_t T) {
  const int64_t P = (int64_t)T * dm.top_k;
  const int64_t t = std::min<int64_t>(dm.n_experts, P) + P / kTileRows + (dm.d_ff_shared ? (T + kTileRows - 1) / kTileRows : 0);
  return (int32_t)t;
}

// Calls of up to kGemvMaxT tokens route through chunk partials (one per token) ...
bool small_call(int32_t T) { return T >= 1 && T <= kGemvMaxT; }

// ... and, when a token's h fits the down kernel, run the expert FFN on the GEMV path.
bool gemv_path(const moe_dims& dm, int32_t T) {
  return small_call(T) && dm.top_k * dm.d_ff + dm.d_ff_shared <= kGemvMaxH && dm.d_ff <= kGemvMaxFF &&
         dm.d_ff_shared <= kGemvMaxFF;
}

struct Layout {
  size_t parts, logits, ids, w, counts, offsets, sorted, inv_pos, tiles, n_tiles, meta_hist, xp, xsum, h, hs, hsum,
      hsum_sh, y_rows, y_exp, total;
};

Layout layout_of(const moe_dims& dm, int32_t T) {
  Layout L;
  const size_t P = (size_t)T * dm.top_k, E = dm.n_experts, d = dm.d_model;
  size_t o = 0;
  L.parts = o;
  o += up((size_t)std::min<int32_t>(T, kGemvMaxT) * (d / 64) * E * 4);
  L.logits = o;
  o += up((size_t)T * E * 4);
  L.ids = o;
  o += up(P * 4);
  L.w = o;
  o += up(P * 4);
  L.counts = o;
  o += up(E * 4);
  L.offsets = o;
  o += up((E + 1) * 4);
  L.sorted = o;
  o += up(P * 4);
  L.inv_pos = o;
  o += up(P * 4);
  L.tiles = o;
  o += up((size_t)max_tiles_of(dm, T) * 12);
  L.n_tiles = o;
  o += up(4);
  L.meta_hist = o;
  o += up((size_t)meta_slices(P) * E * 4);
  L.xp = o;
  o += up((size_t)T * d * 2);
  L.xsum = o;
  o += up((size_t)T * (d / 64) * 4);
  L.h = o;
  o += up(P * dm.d_ff * 2);
  L.hs = o;
  o += up((size_t)T * dm.d_ff_shared * 2);
  L.hsum = o;
  o += up(P * (dm.d_ff / 64) * 4);
  L.hsum_sh = o;
  o += up((size_t)T * (dm.d_ff_shared / 64) * 4);
  L.y_rows = o;
  o += up((P + T) * d * 2);
  L.y_exp = o;
  o += up((P + T) * (d / 32));
  L.total = o;
  return L;
}

int check_q4(const moe_q4& q, const char* what, int bits) {
  if (!q.codes || !q.scales || !q.biases) return fail(MOE_EINVAL, "%s: NULL codes/scales/biases", what);
  if (!aligned(q.codes, code_align(bits)))
    return fail(MOE_EINVAL, "%s: codes not %zu-byte aligned", what, code_align(bits));
  if (!aligned(q.scales, 4) || !aligned(q.biases, 4)) return fail(MOE_EINVAL, "%s: scales/biases not 4-byte aligned", what);
  return MOE_OK;
}

int check_ffn(const moe_ffn_q4* f, const char* what, int bits) {
  if (!f) return fail(MOE_EINVAL, "%s weights are NULL", what);
  char buf[64];
  const char* names[3] = {"gate", "up", "down"};
  const moe_q4* qs[3] = {&f->gate, &f->up, &f->down};
  for (int i = 0; i < 3; ++i) {
    snprintf(buf, sizeof(buf), "%s.%s", what, names[i]);
    if (int rc = check_q4(*qs[i], buf, bits)) return rc;
  }
  return MOE_OK;
}

int check_routing(const moe_routing* r) {
  if (!r) return fail(MOE_EINVAL, "routing is NULL");
  const void* ps[8] = {r->topk_ids, r->topk_w, r->counts, r->offsets, r->sorted_token, r->inv_pos, r->tiles, r->n_tiles};
  for (const void* p : ps)
    if (!p || !aligned(p, 4)) return fail(MOE_EINVAL, "routing array NULL or not 4-byte aligned");
  return MOE_OK;
}

int check_ws(const moe_dims& dm, int32_t T, void* ws, size_t ws_bytes) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(MOE_EINVAL, "workspace not 256-byte aligned");
  const size_t need = layout_of(dm, T).total;
  if (ws_bytes < need) return fail(MOE_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  return MOE_OK;
}

enum Stage {
  kRouterDecode,      // chunk partials of the logits (+ shared expert gate/up when its weights are set)
  kDecodeTopk,        // partials -> top-k (moe_route at T <= kGemvMaxT)
  kRouterPrefill,     // logits for T >= 2
  kTopkPrefill,       // logits -> top-k for T >= 2
  kMeta,              // histogram, scan, scatter, block map
  kGemvGateupTopk,    // GEMV gate/up of the routed slots, top-k fused in
  kGemvGateup,        // GEMV gate/up from given routing, shared slot included
  kGemvDown,          // GEMV down + weighted combine + shared
  kGemmGateup,
  kGemmDown,
  kCombine,
  kPairX              // x in pair order for the grouped GEMM (moe_expert_ffn; the layer does it in kMeta)
};
const char* kStageNames[] = {"router_decode", "decode_topk", "router_prefill", "topk_prefill", "route_meta", "gemv_gateup_topk",
                             "gemv_gateup", "gemv_down_combine", "gateup_gemm", "down_gemm", "combine",
                             "pair_x"};

int layer_stages(const moe_dims& dm, int32_t T, Stage* out) {
  int n = 0;
  if (gemv_path(dm, T)) {
    out[n++] = kRouterDecode;
    out[n++] = kGemvGateupTopk;
    out[n++] = kGemvDown;
    return n;
  }
  if (small_call(T)) {
    out[n++] = kRouterDecode;
    out[n++] = kDecodeTopk;
  } else {
    out[n++] = kRouterPrefill;
    out[n++] = kTopkPrefill;
  }
  out[n++] = kMeta;
  out[n++] = kGemmGateup;
  out[n++] = kGemmDown;
  out[n++] = kCombine;
  return n;
}

int run_stage(Stage s, const Ctx& c0) {
  Ctx c = c0;
  hipError_t e = hipSuccess;
  switch (s) {
    case kRouterDecode: e = launch_router_decode(c); break;
    case kDecodeTopk: e = launch_decode_topk(c); break;
    case kRouterPrefill: e = launch_router_prefill(c); break;
    case kTopkPrefill: e = launch_topk_prefill(c); break;
    case kMeta: e = launch_route_meta(c); break;
    case kGemvGateupTopk: e = launch_gemv_gateup(c, true); break;
    case kGemvGateup: e = launch_gemv_gateup(c, false); break;
    case kGemvDown: e = launch_gemv_down_combine(c); break;
    case kGemmGateup: e = launch_gateup_gemm(c); break;
    case kGemmDown: e = launch_down_gemm(c); break;
    case kCombine: e = launch_combine(c); break;
    case kPairX: e = launch_pair_x(c); break;
  }
  if (e != hipSuccess) return fail(MOE_EHIP, "launch of %s failed: %s", kStageNames[s], hipGetErrorString(e));
  return MOE_OK;
}

void fill_ctx(Ctx& c, const moe_dims& dm, int32_t T, void* ws, hipStream_t stream) {
  const Layout L = layout_of(dm, T);
  char* b = static_cast<char*>(ws);
  c.d = dm.d_model;
  c.E = dm.n_experts;
  c.k = dm.top_k;
  c.I = dm.d_ff;
  c.Is = dm.d_ff_shared;
  c.bits = bits_of(dm);
  c.T = T;
  c.P = T * dm.top_k;
  c.max_tiles = max_tiles_of(dm, T);
  c.router_parts = reinterpret_cast<float*>(b + L.parts);
  c.logits = reinterpret_cast<float*>(b + L.logits);
  c.xp = reinterpret_cast<uint16_t*>(b + L.xp);
  c.xsum = reinterpret_cast<float*>(b + L.xsum);
  c.hsum = reinterpret_cast<float*>(b + L.hsum);
  c.hsum_sh = reinterpret_cast<float*>(b + L.hsum_sh);
  c.pair_in_meta = false;
  c.h = reinterpret_cast<uint16_t*>(b + L.h);
  c.hs = reinterpret_cast<uint16_t*>(b + L.hs);
  c.y_rows = reinterpret_cast<uint16_t*>(b + L.y_rows);
  c.y_exp = reinterpret_cast<uint8_t*>(b + L.y_exp);
  c.r.topk_ids = reinterpret_cast<int32_t*>(b + L.ids);
  c.r.topk_w = reinterpret_cast<float*>(b + L.w);
  c.r.counts = reinterpret_cast<int32_t*>(b + L.counts);
  c.r.offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  c.r.sorted_token = reinterpret_cast<int32_t*>(b + L.sorted);
  c.r.inv_pos = reinterpret_cast<int32_t*>(b + L.inv_pos);
  c.r.tiles = reinterpret_cast<int32_t*>(b + L.tiles);
  c.r.n_tiles = reinterpret_cast<int32_t*>(b + L.n_tiles);
  c.meta_hist = reinterpret_cast<int32_t*>(b + L.meta_hist);
  c.stream = stream;
  c.x = nullptr;
  c.w_router = nullptr;
  c.logit_bias = nullptr;
  c.y = nullptr;
  c.dbg_g = nullptr;
  c.dbg_u = nullptr;
  c.dbg_y = nullptr;
  memset(&c.routed, 0, sizeof(c.routed));
  memset(&c.shared, 0, sizeof(c.shared));
}

int check_layer_args(const moe_dims* dims, int32_t T, const uint16_t* x, const float* w_router, bool need_router,
                     const moe_ffn_q4* routed, const moe_ffn_q4* shared, const uint16_t* y, void* ws, size_t ws_bytes) {
  if (int rc = check_dims(dims, T)) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !aligned(x, 16)) return fail(MOE_EINVAL, "x NULL or not 16-byte aligned");
  if (need_router && (!w_router || !aligned(w_router, 16)))
    return fail(MOE_EINVAL, "w_router NULL or not 16-byte aligned");
  const int bits = bits_of(*dims);
  if (int rc = check_ffn(routed, "routed", bits)) return rc;
  if (dims->d_ff_shared > 0) {
    if (int rc = check_ffn(shared, "shared", bits)) return rc;
  } else if (shared) {
    return fail(MOE_EINVAL, "shared weights given but d_ff_shared == 0");
  }
  if (!y || !aligned(y, 16)) return fail(MOE_EINVAL, "y NULL or not 16-byte aligned");
  if ((const void*)y == (const void*)x) return fail(MOE_EINVAL, "y aliases x");
  return check_ws(*dims, T, ws, ws_bytes);
}

int layer_ctx(Ctx& c, const moe_dims* dims, int32_t T, const uint16_t* x, const float* w_router,
              const float* logit_bias, const moe_ffn_q4* routed, const moe_ffn_q4* shared, uint16_t* y, void* ws,
              void* stream) {
  fill_ctx(c, *dims, T, ws, static_cast<hipStream_t>(stream));
  c.x = x;
  c.w_router = w_router;
  c.logit_bias = logit_bias;
  c.routed = *routed;
  if (shared) c.shared = *shared;
  c.y = y;
  c.pair_in_meta = true;  // the layer's metadata launch pairs x for its GEMMs
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int32_t moe_max_tiles(const moe_dims* dims, int32_t T) {
  if (check_dims(dims, T)) return -1;
  return max_tiles_of(*dims, T);
}

size_t moe_workspace_bytes(const moe_dims* dims, int32_t T) {
  if (check_dims(dims, T)) return 0;
  return layout_of(*dims, T).total;
}

int moe_route(const moe_dims* dims, int32_t T, const uint16_t* x, const float* w_router, const float* logit_bias,
              const moe_routing* out, void* ws, size_t ws_bytes, void* stream) {
  if (int rc = check_dims(dims, T)) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !aligned(x, 16)) return fail(MOE_EINVAL, "x NULL or not 16-byte aligned");
  if (!w_router || !aligned(w_router, 16)) return fail(MOE_EINVAL, "w_router NULL or not 16-byte aligned");
  if (logit_bias && !aligned(logit_bias, 4)) return fail(MOE_EINVAL, "logit_bias not 4-byte aligned");
  if (int rc = check_routing(out)) return rc;
  if (int rc = check_ws(*dims, T, ws, ws_bytes)) return rc;
  if (T == 0) return MOE_OK;
  Ctx c;
  fill_ctx(c, *dims, T, ws, static_cast<hipStream_t>(stream));
  c.x = x;
  c.w_router = w_router;
  c.logit_bias = logit_bias;
  c.r = *out;
  if (small_call(T)) {
    if (int rc = run_stage(kRouterDecode, c)) return rc;
    if (int rc = run_stage(kDecodeTopk, c)) return rc;
  } else {
    if (int rc = run_stage(kRouterPrefill, c)) return rc;
    if (int rc = run_stage(kTopkPrefill, c)) return rc;
  }
  return run_stage(kMeta, c);
}

int moe_expert_ffn(const moe_dims* dims, int32_t T, const uint16_t* x, const moe_routing* routing,
                   const moe_ffn_q4* routed, const moe_ffn_q4* shared, uint16_t* y, void* ws, size_t ws_bytes,
                   void* stream) {
  if (int rc = check_dims(dims, T)) return rc;
  if (T == 0) return MOE_OK;
  if (int rc = check_routing(routing)) return rc;
  if (int rc = check_layer_args(dims, T, x, nullptr, false, routed, shared, y, ws, ws_bytes)) return rc;
  if (T == 0) return MOE_OK;
  Ctx c;
  layer_ctx(c, dims, T, x, nullptr, nullptr, routed, shared, y, ws, stream);
  c.r = *routing;
  if (gemv_path(*dims, T)) {
    if (int rc = run_stage(kGemvGateup, c)) return rc;
    return run_stage(kGemvDown, c);
  }
  if (int rc = run_stage(kPairX, c)) return rc;
  if (int rc = run_stage(kGemmGateup, c)) return rc;
  if (int rc = run_stage(kGemmDown, c)) return rc;
  return run_stage(kCombine, c);
}

int moe_forward_layer(const moe_dims* dims, int32_t T, const uint16_t* x, const float* w_router,
                      const float* logit_bias, const moe_ffn_q4* routed, const moe_ffn_q4* shared, uint16_t* y,
                      void* ws, size_t ws_bytes, void* stream) {
  if (int rc = check_layer_args(dims, T, x, w_router, true, routed, shared, y, ws, ws_bytes)) return rc;
  if (logit_bias && !aligned(logit_bias, 4)) return fail(MOE_EINVAL, "logit_bias not 4-byte aligned");
  if (T == 0) return MOE_OK;
  Ctx c;
  layer_ctx(c, dims, T, x, w_router, logit_bias, routed, shared, y, ws, stream);
  Stage st[8];
  const int n = layer_stages(*dims, T, st);
  for (int i = 0; i < n; ++i)
    if (int rc = run_stage(st[i], c)) return rc;
  return MOE_OK;
}

int moe_forward_layer_noalloc(const moe_dims* dims, int32_t T, const uint16_t* x, const float* w_router,
                              const float* logit_bias, const moe_ffn_q4* routed, const moe_ffn_q4* shared, uint16_t* y,
                              void* stream) {
  if (int rc = check_dims(dims, T)) return rc;
  if (T == 0) return MOE_OK;
  const size_t need = layout_of(*dims, T).total;
  if (need > kScratchBytes)
    return fail(MOE_EWORKSPACE, "T = %d needs %zu bytes of workspace; the fixed scratch holds %zu", T, need,
                kScratchBytes);
  // every other argument is checked against a stand-in workspace address (never dereferenced)
  void* fake_ws = reinterpret_cast<void*>((uintptr_t)256);
  if (int rc = check_layer_args(dims, T, x, w_router, true, routed, shared, y, fake_ws, need)) return rc;
  if (logit_bias && !aligned(logit_bias, 4)) return fail(MOE_EINVAL, "logit_bias not 4-byte aligned");
  void* ws = nullptr;
  const hipError_t e = scratch_device_ptr(&ws);
  if (e != hipSuccess) return fail(MOE_EHIP, "scratch address lookup failed: %s", hipGetErrorString(e));
  return moe_forward_layer(dims, T, x, w_router, logit_bias, routed, shared, y, ws, kScratchBytes, stream);
}

int32_t moe_num_stages(const moe_dims* dims, int32_t T) {
  if (check_dims(dims, T) || T == 0) return 0;
  Stage st[8];
  return layer_stages(*dims, T, st);
}

const char* moe_stage_name(const moe_dims* dims, int32_t T, int32_t stage) {
  if (check_dims(dims, T) || T == 0) return nullptr;
  Stage st[8];
  const int n = layer_stages(*dims, T, st);
  if (stage < 0 || stage >= n) return nullptr;
  return kStageNames[st[stage]];
}

int moe_launch_stage(int32_t stage, const moe_dims* dims, int32_t T, const uint16_t* x, const float* w_router,
                     const float* logit_bias, const moe_ffn_q4* routed, const moe_ffn_q4* shared, uint16_t* y,
                     void* ws, size_t ws_bytes, void* stream) {
  if (int rc = check_layer_args(dims, T, x, w_router, true, routed, shared, y, ws, ws_bytes)) return rc;
  if (T == 0) return fail(MOE_EINVAL, "no stages at T = 0");
  if (logit_bias && !aligned(logit_bias, 4)) return fail(MOE_EINVAL, "logit_bias not 4-byte aligned");
  Stage st[8];
  const int n = layer_stages(*dims, T, st);
  if (stage < 0 || stage >= n) return fail(MOE_EINVAL, "stage %d out of range [0, %d)", stage, n);
  Ctx c;
  layer_ctx(c, dims, T, x, w_router, logit_bias, routed, shared, y, ws, stream);
  return run_stage(st[stage], c);
}

int moe_debug_dequant_bits(const moe_q4* w, int64_t rows, int32_t in_dim, int32_t bits, uint16_t* out_bf16,
                           void* stream) {
  if (bits != 2 && bits != 3 && bits != 4) return fail(MOE_EUNSUPPORTED, "bits = %d must be 4, 3 or 2", bits);
  if (!w) return fail(MOE_EINVAL, "weights are NULL");
  if (int rc = check_q4(*w, "weights", bits)) return rc;
  if (!out_bf16 || !aligned(out_bf16, 16)) return fail(MOE_EINVAL, "out NULL or not 16-byte aligned");
  if (rows < 0) return fail(MOE_EINVAL, "rows < 0");
  if (in_dim < 64 || in_dim % 64) return fail(MOE_EUNSUPPORTED, "in_dim = %d must be a positive multiple of 64", in_dim);
  if (rows == 0) return MOE_OK;
  if (rows * (in_dim / 64) > (int64_t)1 << 38) return fail(MOE_EUNSUPPORTED, "too many rows");
  hipError_t e = launch_dequant(*w, rows, in_dim, bits, out_bf16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MOE_EHIP, "launch of dequant failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

int moe_debug_dequant(const moe_q4* w, int64_t rows, int32_t in_dim, uint16_t* out_bf16, void* stream) {
  return moe_debug_dequant_bits(w, rows, in_dim, 4, out_bf16, stream);
}

int moe_debug_router_logits(const moe_dims* dims, int32_t T, const uint16_t* x, const float* w_router,
                            const float* logit_bias, float* out, void* stream) {
  if (int rc = check_dims(dims, T)) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !aligned(x, 16)) return fail(MOE_EINVAL, "x NULL or not 16-byte aligned");
  if (!w_router || !aligned(w_router, 16)) return fail(MOE_EINVAL, "w_router NULL or not 16-byte aligned");
  if (logit_bias && !aligned(logit_bias, 4)) return fail(MOE_EINVAL, "logit_bias not 4-byte aligned");
  if (!out || !aligned(out, 16)) return fail(MOE_EINVAL, "out NULL or not 16-byte aligned");
  Ctx c{};  // the router kernel reads only the fields set below
  c.T = T;
  c.d = dims->d_model;
  c.E = dims->n_experts;
  c.x = x;
  c.w_router = w_router;
  c.logit_bias = logit_bias;
  c.logits = out;
  c.stream = static_cast<hipStream_t>(stream);
  const hipError_t e = launch_router_prefill(c);
  if (e != hipSuccess) return fail(MOE_EHIP, "launch of router_prefill failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

int moe_debug_grouped_gemm(const moe_dims* dims, int32_t T, int32_t which, const uint16_t* a,
                           const moe_routing* routing, const moe_ffn_q4* routed, const moe_ffn_q4* shared, float* out,
                           float* out2, void* ws, size_t ws_bytes, void* stream) {
  if (int rc = check_dims(dims, T)) return rc;
  if (which != 0 && which != 1) return fail(MOE_EINVAL, "which = %d must be 0 (gate/up) or 1 (down)", which);
  if (T == 0) return MOE_OK;
  if (int rc = check_routing(routing)) return rc;
  // x (which = 0) or h (which = 1) stands in for x in the argument checks
  if (int rc = check_layer_args(dims, T, a, nullptr, false, routed, shared, reinterpret_cast<const uint16_t*>(out),
                                ws, ws_bytes))
    return rc;
  if (!out || !aligned(out, 16) || (which == 0 && (!out2 || !aligned(out2, 16))))
    return fail(MOE_EINVAL, "output NULL or not 16-byte aligned");
  Ctx c;
  layer_ctx(c, dims, T, a, nullptr, nullptr, routed, shared, nullptr, ws, stream);
  c.r = *routing;
  hipError_t e;
  if (which == 0) {
    c.dbg_g = out;
    c.dbg_u = out2;
    if (int rc = run_stage(kPairX, c)) return rc;
    return run_stage(kGemmGateup, c);
  }
  e = launch_pair_rows(a, c.h, c.hsum, c.P, c.I, c.stream);
  if (e == hipSuccess && c.Is) e = launch_pair_rows(a + (size_t)c.P * c.I, c.hs, c.hsum_sh, c.T, c.Is, c.stream);
  if (e != hipSuccess) return fail(MOE_EHIP, "launch of pair_rows failed: %s", hipGetErrorString(e));
  c.dbg_y = out;
  return run_stage(kGemmDown, c);
}

size_t moe_vocab_topk_workspace_bytes(int32_t R, int32_t V, int32_t K) {
  if (R < 0 || V < 1 || K < 1 || K > kVocabMaxK || K > V) return 0;
  const int64_t nch = ((int64_t)V + vocab_chunk(K) - 1) / vocab_chunk(K);
  if (nch > kVocabMaxChunks) return 0;
  return up((size_t)std::max<int32_t>(R, 1) * (size_t)nch * 4);
}

int moe_vocab_topk_stage(int32_t stage, int32_t R, int32_t V, int32_t K, const float* logits, int32_t* ids,
                         float* vals, void* ws, size_t ws_bytes, void* stream) {
  if (stage < -1 || stage > 1) return fail(MOE_EINVAL, "stage %d is not 0 or 1", stage);
  if (R < 0) return fail(MOE_EINVAL, "R = %d is negative", R);
  if (V < 1 || K < 1 || K > V) return fail(MOE_EUNSUPPORTED, "need 1 <= K <= V (K = %d, V = %d)", K, V);
  if (K > kVocabMaxK) return fail(MOE_EUNSUPPORTED, "K = %d exceeds %d", K, kVocabMaxK);
  const size_t need = moe_vocab_topk_workspace_bytes(R, V, K);
  if (need == 0)
    return fail(MOE_EUNSUPPORTED, "V = %d exceeds %d chunks of %d", V, kVocabMaxChunks, vocab_chunk(K));
  if (R == 0) return MOE_OK;
  if (!logits || !aligned(logits, 4)) return fail(MOE_EINVAL, "logits NULL or not 4-byte aligned");
  if (!ids || !aligned(ids, 4) || !vals || !aligned(vals, 4))
    return fail(MOE_EINVAL, "ids/vals NULL or not 4-byte aligned");
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(MOE_EINVAL, "workspace not 256-byte aligned");
  if (ws_bytes < need) return fail(MOE_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  const hipError_t e = launch_vocab_topk(R, V, K, logits, static_cast<uint32_t*>(ws), ids, vals,
                                         static_cast<hipStream_t>(stream), stage);
  if (e != hipSuccess) return fail(MOE_EHIP, "launch of the top-K kernels failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

int moe_vocab_topk(int32_t R, int32_t V, int32_t K, const float* logits, int32_t* ids, float* vals, void* ws,
                   size_t ws_bytes, void* stream) {
  return moe_vocab_topk_stage(-1, R, V, K, logits, ids, vals, ws, ws_bytes, stream);
}

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: dimensions outside the supported limits";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: HIP launch failed";
    default: return "unknown moe_status";
  }
}

const char* moe_last_error(void) { return g_err; }

}  // extern "C"
