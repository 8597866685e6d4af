/*
 * moe_int4.h -- C ABI of the routed mixture-of-experts FFN over groupwise-affine 4-bit
 * weights, for AMD MI355X (gfx950). Library: libmoe_int4.so.
 *
 * The problem, as the pages state it:
 *   - activations x [T][d] in bf16; a router that scores every expert and keeps the top k,
 *     plus one always-on shared expert that sees every token
 *     ("Perplexity's Lily Beats MLX-LM on MacBook M5. Because It Only Runs One Model.",
 *     section "Why Qwen3.6-35B-A3B is a weird workload"; "Perplexity builds a custom engine
 *     for Qwen on M5 Macs");
 *   - expert weights stored as 4-bit codes with one bf16 scale and one bf16 bias per group
 *     of 64 weights (same blog, section "Prefill: keep routing on the GPU, dequantize in
 *     flight");
 *   - routing (histogram, prefix scan, scatter, block map) kept on the GPU with no CPU round
 *     trip, a grouped GEMM for prefill with the weights dequantised tile by tile in on-chip
 *     memory, and a bandwidth-bound GEMV for batch-1 decode with the expert input projections
 *     fused with the gate activation and the output projection fused with the routing
 *     scores and the shared expert (same blog, sections "Prefill: ..." and "Decode: minimize
 *     bytes per token").
 *
 * Conventions shared by every entry point:
 *   - Pointers. Every array argument is a DEVICE pointer, owned by the caller. The library
 *     allocates nothing and keeps no pointer after it returns. x, codes, w_router and y must
 *     be 16-byte aligned; scales, biases and all int32/fp32 routing arrays 4-byte aligned;
 *     the workspace 256-byte aligned. y must not alias x.
 *   - Streams. `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue
 *     work on it: no host synchronisation, no device-to-host copy, no printing. Results are
 *     valid when the stream reaches that point; inputs must stay alive until then.
 *   - Errors. Each call returns a moe_status. Arguments are checked before any HIP call, so
 *     a rejected call has enqueued nothing. Nothing throws or aborts across the ABI.
 *     moe_last_error() gives a per-thread message for the last failure. Asynchronous device
 *     faults surface at the caller's next synchronisation, as for any HIP launch.
 *   - Determinism. The same inputs give bit-identical outputs on every call (atomics are
 *     used only for integer counts, never for floating-point sums).
 *   - Workspace. `ws` is device scratch of at least moe_workspace_bytes() bytes; its contents
 *     on entry do not matter.
 *   - Concurrency. No global mutable state. Calls on different streams with different
 *     workspaces may overlap; calls sharing one workspace must be ordered by the caller.
 *   - T = 0 is a no-op that returns MOE_OK once the dims are valid (pointers are not checked).
 *
 * Data layouts (row-major):
 *   x          [T][d]                 bf16 bits (uint16)
 *   w_router   [d][E]                 fp32
 *   logit_bias [E]                    fp32, or NULL; added to the router logits before the
 *                                     top-k choice and before the softmax
 *   moe_q4     codes  [n][out][in/2]  uint8, two 4-bit codes per byte, the even input index
 *                                     in the low nibble; with b = code_bits of 3 or 2,
 *                     [n][out][in*b/8] each row's codes form a little-endian bit stream
 *                                     (code c at bits [b*c, b*c + b), bit j of the stream is
 *                                     bit j % 8 of byte j / 8; for b = 4 this is the nibble
 *                                     order above)
 *              scales [n][out][in/64] bf16 bits; biases likewise
 *              weight = scale * code + bias (code in 0..2^b-1), groups run along the input
 *              codes 16-byte aligned (b = 4), 4-byte (b = 3) or 8-byte (b = 2)
 *   routed     gate, up: n = E, out = d_ff, in = d;  down: n = E, out = d, in = d_ff
 *   shared     the same with n = 1 and d_ff_shared (NULL when d_ff_shared == 0)
 *   y          [T][d]                 bf16 bits
 *
 * Limits (else MOE_EUNSUPPORTED): group_size == 64; d, d_ff, d_ff_shared multiples of 64
 * (d_ff_shared may be 0); 64 <= d <= 16384; d_ff, d_ff_shared <= 8192; 1 <= E <= 1024;
 * 1 <= k <= min(E, 16); 0 <= T <= 65536.
 */
#ifndef MOE_INT4_H
#define MOE_INT4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* null or misaligned pointer, negative size, missing shared weights */
  MOE_EUNSUPPORTED = 2,  /* dimensions outside the limits above */
  MOE_EWORKSPACE = 3,    /* workspace smaller than moe_workspace_bytes() */
  MOE_EHIP = 4           /* a HIP launch failed; see moe_last_error() */
} moe_status;

typedef struct {
  int32_t d_model;      /* d */
  int32_t n_experts;    /* E, routed experts */
  int32_t top_k;        /* k, experts per token */
  int32_t d_ff;         /* I, routed expert intermediate size */
  int32_t d_ff_shared;  /* I_s, shared expert intermediate size; 0 = no shared expert */
  int32_t group_size;   /* quantisation group along the input dimension; must be 64 */
  int32_t code_bits;    /* bits per expert weight code: 4 (0 also means 4), or the 3- and 2-bit variant
                           ("Squeezing a 26B diffusion LLM onto a Mac", "The physics ceiling: why 300+
                           tok/s is blocked", which names 2-3 bit experts as the lever that cuts the
                           streamed bytes); every width runs on both the GEMV and the grouped-GEMM
                           path */
} moe_dims;

/* One projection of every expert (n matrices [out][in]). */
typedef struct {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* biases;
} moe_q4;

/* The three projections of a SwiGLU expert FFN: h = silu(x Wg^T) * (x Wu^T); y = h Wd^T. */
typedef struct {
  moe_q4 gate, up, down;
} moe_ffn_q4;

/*
 * Routing of one call, written by moe_route and read by moe_expert_ffn (device arrays).
 *   topk_ids [T][k]  int32  the k chosen experts of each token, best first; equal logits go
 *                           to the lower expert index
 *   topk_w   [T][k]  fp32   softmax over the k chosen logits (gate weights, sum 1)
 *   counts   [E]     int32  pairs routed to each expert (histogram); sum = T*k
 *   offsets  [E+1]   int32  exclusive prefix sum of counts; offsets[E] = T*k
 *   sorted_token [T*k] int32 token of each grouped row; rows of one expert are contiguous
 *                           (offsets[e] .. offsets[e+1]) and in ascending token order
 *   inv_pos  [T][k]  int32  grouped row of pair (t, j)
 *   tiles    [moe_max_tiles()][3] int32  block map: (expert, first grouped row, rows);
 *                           each non-empty group in ascending expert order is cut into
 *                           tiles of at most 32 rows; the shared expert's T rows follow
 *                           as grouped rows T*k .. T*k+T-1 tagged with expert index E
 *   n_tiles  [1]     int32  number of valid tiles (stays on the device)
 */
typedef struct {
  int32_t* topk_ids;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_token;
  int32_t* inv_pos;
  int32_t* tiles;
  int32_t* n_tiles;
} moe_routing;

/* Host-only, pure. Upper bound on the block map's length for T tokens:
 * min(E, T*k) + floor(T*k / 32) + (shared ? ceil(T / 32) : 0). Returns -1 on bad dims. */
int32_t moe_max_tiles(const moe_dims* dims, int32_t T);

/* Host-only, pure. Bytes of workspace every entry point below needs for T tokens (the same
 * figure serves all of them). Returns 0 on bad dims. */
size_t moe_workspace_bytes(const moe_dims* dims, int32_t T);

/*
 * Router, top-k and routing metadata (steps on the GPU, no host sync). The router scores every
 * expert and keeps the top k ("Perplexity's Lily Beats MLX-LM on MacBook M5. Because It Only Runs
 * One Model.", section "Why Qwen3.6-35B-A3B is a weird workload"); the grouped rows need a
 * histogram, prefix scan, scatter and block map after every top-k selection, kept on the GPU with
 * no CPU round trip (same blog, section "Prefill: keep routing on the GPU, dequantize in flight").
 *   logits[t][e] = sum_i x[t][i] * w_router[i][e] (+ logit_bias[e]), in fp32 in a fixed order:
 *   the input dimension is cut into chunks of 64, each chunk reduced by an fma chain in
 *   ascending i, the chunk partials added in ascending order, the bias added last;
 *   then top-k, gate weights, histogram, prefix scan, stable scatter and block map.
 * Writes every array of `out`. `ws` as sized by moe_workspace_bytes.
 */
int moe_route(const moe_dims* dims, int32_t T, const uint16_t* x, const float* w_router,
              const float* logit_bias, const moe_routing* out, void* ws, size_t ws_bytes,
              void* stream);

/*
 * Expert FFN of routed tokens given their routing (as written by moe_route). Prefill is a grouped
 * GEMM that reconstructs the 4-bit weights tile by tile in on-chip memory with fp32 accumulation
 * and bf16 output, never expanding them in memory; batch-1 decode is a bandwidth-bound GEMV
 * ("Perplexity's Lily Beats MLX-LM on MacBook M5. Because It Only Runs One Model.", sections
 * "Prefill and decode are different problems", "Prefill: keep routing on the GPU, dequantize in
 * flight" and "Decode: minimize bytes per token"; codes of 3 and 2 bits: "Squeezing a 26B
 * diffusion LLM onto a Mac", section "The physics ceiling: why 300+ tok/s is blocked").
 *   y[t] = bf16( sum_j topk_w[t][j] * FFN_{topk_ids[t][j]}(x[t]) + FFN_shared(x[t]) ),
 *   FFN_e(x) = h Wd_e^T with h = bf16( silu(x Wg_e^T) * (x Wu_e^T) ), each weight taken as
 *   scale * code + bias inside the dot products (never expanded in memory), fp32 accumulation.
 * Calls of 1..32 tokens run the GEMV path (uses topk_ids and topk_w only) when
 * top_k * d_ff + d_ff_shared <= 28672 and d_ff, d_ff_shared <= 1024; other calls run the grouped
 * GEMM path (uses every routing array). `shared` must be NULL iff d_ff_shared == 0.
 */
int moe_expert_ffn(const moe_dims* dims, int32_t T, const uint16_t* x, const moe_routing* routing,
                   const moe_ffn_q4* routed, const moe_ffn_q4* shared, uint16_t* y, void* ws,
                   size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): moe_forward_layer with the workspace taken from a fixed device
 * array inside the library instead of `ws`. The array holds MOE_NOALLOC_SCRATCH_BYTES bytes on each
 * GPU the library runs on (the current device at the call) and lives until the process ends; calls
 * whose moe_workspace_bytes(dims, T) exceeds it return MOE_EWORKSPACE. The first call on a device
 * looks the array's address up (hipGetSymbolAddress); no call allocates or frees memory. All calls
 * on one GPU share the array: calls that may overlap on one GPU (unordered streams) race on it and
 * must be ordered by the caller. Otherwise as moe_forward_layer. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_layer_noalloc(const moe_dims* dims, int32_t T, const uint16_t* x, const float* w_router,
                              const float* logit_bias, const moe_ffn_q4* routed, const moe_ffn_q4* shared,
                              uint16_t* y, void* stream);

/* The whole routed MoE FFN layer: top-k of the routed experts plus the shared expert, weighted by
 * the renormalised gate scores ("Perplexity's Lily Beats MLX-LM on MacBook M5. Because It Only
 * Runs One Model.", section "Why Qwen3.6-35B-A3B is a weird workload"; "Perplexity builds a custom
 * engine for Qwen on M5 Macs"), as moe_route followed by moe_expert_ffn, with the routing arrays
 * carved from `ws`. On the GEMV path the block-map steps are skipped (it does not read them), the
 * top-k is taken inside the gate/up kernel, and only topk_ids/topk_w of the carved routing are
 * written. */
int moe_forward_layer(const moe_dims* dims, int32_t T, const uint16_t* x, const float* w_router,
                      const float* logit_bias, const moe_ffn_q4* routed, const moe_ffn_q4* shared,
                      uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/* Check export: dequantise `rows` rows of length in_dim (rows counts all matrices) to bf16
 * bits out_bf16 [rows][in_dim]: w = bf16(fp32(scale * code + bias)), round to nearest even.
 * moe_debug_dequant_bits takes codes of `bits` = 4, 3 or 2 bits (layout above); it reads them
 * with the GEMV kernels' own unpacking. */
int moe_debug_dequant(const moe_q4* w, int64_t rows, int32_t in_dim, uint16_t* out_bf16, void* stream);
int moe_debug_dequant_bits(const moe_q4* w, int64_t rows, int32_t in_dim, int32_t bits, uint16_t* out_bf16,
                           void* stream);

/* Check export of the router (test use): out = logits [T][E] fp32 of T >= 1 tokens, in the fixed
 * order of moe_route (chunks of 64 inputs, each an fma chain in ascending i from +0, the chunk
 * partials added in ascending order, then logit_bias), computed by the router kernel of calls of
 * more than 32 tokens whatever T, so its logits can be compared bit for bit (the router scores every
 * expert: "Perplexity's Lily Beats MLX-LM on MacBook M5. Because It Only Runs One Model.", section
 * "Why Qwen3.6-35B-A3B is a weird workload"). Only d_model and n_experts of `dims` matter beyond
 * validation. x and w_router 16-byte aligned, out 16-byte aligned; same status codes as moe_route. */
int moe_debug_router_logits(const moe_dims* dims, int32_t T, const uint16_t* x, const float* w_router,
                            const float* logit_bias, float* out, void* stream);

/* Check export of the grouped GEMMs (test use): runs one of the two grouped-GEMM kernels over the
 * block map of `routing` (as written by moe_route for these dims and T), with the same unpacking of
 * the codes, LDS stages and scale/bias slots as moe_expert_ffn's grouped path (codes of any width
 * dims->code_bits allows), and writes its fp32 results before any activation or rounding (the layer
 * itself keeps the down rows as fp16 with one power-of-two exponent per 32 columns):
 *   which = 0: a = x [T][d] bf16; out = g, out2 = u, each [T*k][d_ff] fp32 in grouped row order
 *              followed by [T][d_ff_shared] for the shared expert: g = x Wg^T, u = x Wu^T.
 *   which = 1: a = h, [T*k][d_ff] bf16 in grouped row order followed by [T][d_ff_shared];
 *              out = [T*k + T][d] fp32 rows h Wd^T (shared rows last; [T*k][d] without a shared
 *              expert); out2 unused (may be NULL).
 * The products are those of the expert FFN in "Perplexity's Lily Beats MLX-LM on MacBook M5. Because
 * It Only Runs One Model.", section "Prefill: keep routing on the GPU, dequantize in flight". `ws`
 * as sized by moe_workspace_bytes; same validation and status codes as moe_expert_ffn. */
int moe_debug_grouped_gemm(const moe_dims* dims, int32_t T, int32_t which, const uint16_t* a,
                           const moe_routing* routing, const moe_ffn_q4* routed, const moe_ffn_q4* shared, float* out,
                           float* out2, void* ws, size_t ws_bytes, void* stream);

/* Profiling: moe_forward_layer runs moe_num_stages() kernels in sequence for this T; stage s
 * is named moe_stage_name(). moe_launch_stage enqueues stage s alone (same arguments as
 * moe_forward_layer); its inputs are what the earlier stages left in `ws`, so run
 * moe_forward_layer once on that workspace first. For per-kernel timing only. */
int32_t moe_num_stages(const moe_dims* dims, int32_t T);
const char* moe_stage_name(const moe_dims* dims, int32_t T, int32_t stage);
int moe_launch_stage(int32_t stage, const moe_dims* dims, int32_t T, const uint16_t* x,
                     const float* w_router, const float* logit_bias, const moe_ffn_q4* routed,
                     const moe_ffn_q4* shared, uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/*
 * Exact top-K of each row of a logit matrix, the candidates a sampler over a large vocabulary
 * needs ("Squeezing a 26B diffusion LLM onto a Mac", section "The optimizations that worked",
 * the hierarchical exact top-K): for every row r < R of logits [R][V] (fp32, row-major),
 *   ids[r][j], vals[r][j] = index and value of the j-th entry of the row in the order
 *   (value descending, index ascending), j < K.
 * The row is reduced to chunk maxima, the K chunks with the largest maxima are kept, and the
 * top K is taken among their entries; the result equals the full sort's (no approximation).
 * -0 and +0 compare equal; rows must hold no NaN.
 * Limits: 1 <= K <= 128, K <= V, and V <= 8192 * C with C = 1024 for K <= 32, 512 for K <= 64,
 * 256 above (so V <= 4,194,304 at K = 64); otherwise MOE_EUNSUPPORTED. R = 0 is a no-op.
 * Pointers are device pointers, 4-byte aligned (logits 16-byte aligned with V % 4 == 0 gives
 * the fastest loads); ids [R][K] int32 and vals [R][K] fp32 must not overlap logits. ws holds
 * moe_vocab_topk_workspace_bytes(R, V, K) bytes, 256-byte aligned, contents irrelevant.
 * Enqueues two kernels on `stream`; no host synchronisation.
 */
size_t moe_vocab_topk_workspace_bytes(int32_t R, int32_t V, int32_t K);  /* 0 if unsupported */
int moe_vocab_topk(int32_t R, int32_t V, int32_t K, const float* logits, int32_t* ids, float* vals, void* ws,
                   size_t ws_bytes, void* stream);
/* Profiling: moe_vocab_topk's kernels one at a time, with its arguments and checks. Stage 0
 * writes the chunk maxima into ws; stage 1 selects from the chunk maxima ws already holds (run
 * stage 0 or moe_vocab_topk on that ws first). For per-kernel timing only. */
int moe_vocab_topk_stage(int32_t stage, int32_t R, int32_t V, int32_t K, const float* logits, int32_t* ids,
                         float* vals, void* ws, size_t ws_bytes, void* stream);

const char* moe_status_str(int status);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_INT4_H */
