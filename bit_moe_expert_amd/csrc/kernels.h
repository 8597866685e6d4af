// Host-side launch interface of the gfx950 kernels (internal to libmoe_int4.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_int4.h"

namespace moe {

// Everything one layer call needs, resolved to device pointers by the C-ABI layer.
struct Ctx {
  int d, E, k, I, Is, T, P, max_tiles;
  int bits;  // bits per expert weight code: 4, 3 or 2
  const uint16_t* x;
  const float* w_router;
  const float* logit_bias;
  moe_ffn_q4 routed;
  moe_ffn_q4 shared;  // all-null when Is == 0
  moe_routing r;      // routing arrays (caller's or carved from the workspace)
  int32_t* meta_hist;     // [slices][E] per-slice expert counts (sliced routing metadata only)
  float* router_parts;    // [T][E][d/64] router chunk partials (GEMV path, T <= kGemvMaxT)
  float* logits;          // [T][E] router logits (T >= 2)
  uint16_t* xp;           // [T][d] bf16: x with each 8-input chunk in pair order (grouped GEMM operand)
  float* xsum;            // [T][d/64] fp32 group sums of x (written with xp)
  float* hsum;            // [P][I/64] fp32 group sums of h (grouped GEMM path)
  float* hsum_sh;         // [T][Is/64] fp32 group sums of the shared expert's h
  bool pair_in_meta;      // the routing-metadata launch also writes xp
  uint16_t* h;            // [P][I] bf16, grouped order (slot order at T == 1); pair order on the GEMM path
  uint16_t* hs;           // [T][Is] bf16
  uint16_t* y_rows;       // [P + T][d] fp16 bits, grouped order, shared rows last; each (row, 32-column
                          // segment) holds the values times 2^-e ...
  uint8_t* y_exp;         // [P + T][d/32] ... with the segment's e here
  uint16_t* y;            // [T][d] bf16
  float* dbg_g;           // when set, the gate/up GEMM writes fp32 g and u ([P][I] then [T][Is]) instead of h
  float* dbg_u;
  float* dbg_y;           // when set, the down GEMM writes its fp32 rows ([P + T][d]) here instead
  hipStream_t stream;
};

// router chunk partials of T <= kGemvMaxT tokens
hipError_t launch_router_decode(const Ctx& c);
hipError_t launch_decode_topk(const Ctx& c);
hipError_t launch_router_prefill(const Ctx& c);  // logits [T][E]
hipError_t launch_topk_prefill(const Ctx& c);    // logits -> topk_ids, topk_w
hipError_t launch_route_meta(const Ctx& c);  // + xp, xsum from x in extra blocks when c.pair_in_meta
hipError_t launch_pair_x(const Ctx& c);      // xp, xsum from x
// bf16 rows of K inputs (K a multiple of 64) in pair order, dst from src, with their group sums
// sums [nrows][K/64] (fp32, inputs of a group added in ascending order)
hipError_t launch_pair_rows(const uint16_t* src, uint16_t* dst, float* sums, int64_t nrows, int K, hipStream_t stream);
// fused_topk: take the top-k from the router partials in every block, plus the shared expert's
// rows in blocks of their own when its weights are set; otherwise read topk_ids and compute the
// shared slot after each token's routed slots
hipError_t launch_gemv_gateup(const Ctx& c, bool fused_topk);
hipError_t launch_gemv_down_combine(const Ctx& c);
hipError_t launch_gateup_gemm(const Ctx& c);
hipError_t launch_down_gemm(const Ctx& c);
hipError_t launch_combine(const Ctx& c);
// Exact top-K of logit rows (vocab_topk.hip): chunk size C for a given K (K * C = 32768 keys at
// most in LDS), the largest K and V supported, and the launch (cmax: [R][ceil(V / C)] keys).
constexpr int kVocabMaxK = 128;
constexpr int kVocabMaxChunks = 8192;
inline int vocab_chunk(int K) { return K <= 32 ? 1024 : K <= 64 ? 512 : 256; }
// stage: -1 both kernels, 0 the chunk maxima only, 1 the selection only
hipError_t launch_vocab_topk(int R, int V, int K, const float* logits, uint32_t* cmax, int32_t* ids, float* vals,
                             hipStream_t stream, int stage);
hipError_t launch_dequant(const moe_q4& w, int64_t rows, int in_dim, int bits, uint16_t* out, hipStream_t stream);

// The fixed device scratch of moe_forward_layer_noalloc (noalloc.hip): its size, and its address on
// the current device (looked up once per device).
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
hipError_t scratch_device_ptr(void** out);

// Block-map tile height (rows of one expert group per tile).
constexpr int kTileRows = 32;

// Routing metadata of more than kMetaSlicedFrom pairs (T k) runs in three launches over at most
// kMetaMaxSlices slices of a whole number of 1024-pair spans; smaller calls take one launch.
constexpr int kMetaSlicedFrom = 32768;
constexpr int kMetaMaxSlices = 256;
inline bool meta_sliced(int64_t P) { return P > kMetaSlicedFrom; }
inline int meta_slice_span(int64_t P) {
  const int64_t per = (P + kMetaMaxSlices - 1) / kMetaMaxSlices;
  return (int)((per + 1023) / 1024 * 1024);
}
inline int meta_slices(int64_t P) { return meta_sliced(P) ? (int)((P + meta_slice_span(P) - 1) / meta_slice_span(P)) : 0; }

// Calls of up to kGemvMaxT tokens take the GEMV path (one token per wave, no grouping).
constexpr int kGemvMaxT = 32;
// The GEMV path's down kernel keeps a token's selected experts' h in LDS: (k*I + Is) bf16 values.
constexpr int kGemvMaxH = 28672;
// ... and its down kernel keeps two 16-lane rounds of 32-input pieces per row in registers.
constexpr int kGemvMaxFF = 1024;

}  // namespace moe
