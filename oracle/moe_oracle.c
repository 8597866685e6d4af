/*
 * CPU oracle for the routed mixture-of-experts FFN over groupwise-affine 4-bit weights.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg may load this file's library. The GPU library never includes, links
 * or calls it, and this file includes nothing from the GPU library.
 *
 * It is deliberately plain and slow: loops written in the order of the definitions below,
 * double precision wherever the method leaves the precision open, and a rounding to bf16
 * or fp32 only where the method's data types force one. Built with -ffp-contract=off and
 * without fast-math, so every `a * b + c` below is two IEEE roundings unless fma() is named.
 *
 * Pages cited (title, then section):
 *   [LILY-BLOG]  "Perplexity's Lily Beats MLX-LM on MacBook M5. Because It Only Runs One Model."
 *   [LILY-NEWS]  "Perplexity builds a custom engine for Qwen on M5 Macs"
 *   [LILY-FEED]  "Perplexity Open Sources Lily: A Rust + Metal Inference Engine for Qwen3.6-35B-A3B
 *                 on Apple Silicon"
 *   [DIFFGEMMA]  "Squeezing a 26B diffusion LLM onto a Mac"
 *
 * What is computed, per layer call with T tokens (x: [T][d] bf16):
 *   1. router logits, fp32, in one fixed summation order (reading: the pages do not give the
 *      order; a fixed one makes the top-k choice unique) -- [LILY-BLOG "Why Qwen3.6-35B-A3B is
 *      a weird workload"]: a router scores every expert and picks 8 of 256;
 *   2. top-k by (logit descending, expert index ascending) and a softmax over the k picked
 *      logits (the renormalised gate weights) -- same section;
 *   3. histogram, prefix scan, scatter and block map of the token-expert pairs --
 *      [LILY-BLOG "Prefill: keep routing on the GPU, dequantize in flight"];
 *   4. dequantisation w = scale * q + bias per group of 64 along the input dimension, rounded
 *      to bf16 because the matrix units take bf16 operands -- same section, and
 *      [LILY-NEWS] on the scale and bias that reconstruct each 4-bit value;
 *   5. per grouped row, the SwiGLU expert FFN h = silu(x Wg^T) * (x Wu^T), h rounded to bf16
 *      (the grouped GEMM writes bf16), then y_row = h Wd^T -- same section, and [LILY-BLOG
 *      "Decode: minimize bytes per token"] (expert input projections fused with the gate
 *      activation);
 *   6. the always-on shared expert on every token, ungated, added with weight 1 --
 *      [LILY-NEWS] and [LILY-BLOG "Why Qwen3.6-35B-A3B is a weird workload"];
 *   7. the weighted gather back to token order y[t] = sum_j w[t][j] * y_row(pair t,j) + shared,
 *      rounded to bf16 -- [LILY-BLOG "Decode: minimize bytes per token"] (expert output
 *      projection fused with the routing scores and the shared expert).
 *
 *   8. (separate workload) the exact top-K of each row of a logit matrix, by (value descending,
 *      index ascending) -- [DIFFGEMMA "The optimizations that worked"], whose hierarchical
 *      chunk-max selection reaches exactly this set; the oracle is the plain definition, a full
 *      sort of the row.
 *
 * Parity pins: every function here is checked by the CPU tests against closed forms,
 * exhaustive identities or brute force (see the tests named test_oracle_*.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_GROUP 64
#define ORC_TILE_ROWS 32

typedef struct {
  const uint8_t* codes;    /* [n_mat][out][in * bits / 8]: each row a little-endian bit stream */
  const uint16_t* scales;  /* [n_mat][out][in/64] bf16 bits */
  const uint16_t* biases;  /* [n_mat][out][in/64] bf16 bits */
  int32_t bits;            /* bits per code: 4 (also when 0), 3 or 2 */
} orc_q4;

typedef struct {
  orc_q4 gate, up, down;   /* gate, up: out = I, in = d; down: out = d, in = I */
} orc_ffn;

/* ---------------------------------------------------------------- number formats */

static double orc_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round an fp32 value to the nearest bf16, ties to even (the IEEE default rounding). */
static uint16_t orc_round_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
  uint32_t upper = u >> 16, lower = u & 0xffffu;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

void oracle_round_bf16(int64_t n, const float* in, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_round_bf16(in[i]);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------- 1. router logits
 * logits[t][e] = sum_i x[t][i] * Wr[i][e] (+ bias[e]), x widened exactly from bf16.
 * Summation order (reading): the input dimension is cut into consecutive chunks of 64; each
 * chunk's partial is a chain of fused multiply-adds over ascending i starting from +0; the
 * chunk partials are then added in ascending chunk order to an accumulator starting at +0;
 * the bias, when given, is added last. All in fp32. */
int oracle_router_logits(int32_t T, int32_t d, int32_t E, const uint16_t* x, const float* w_router,
                         const float* bias, float* logits) {
  if (d % ORC_GROUP) return 1;
#pragma omp parallel for schedule(static)
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      float acc = 0.0f;
      for (int32_t c = 0; c < d / ORC_GROUP; ++c) {
        float part = 0.0f;
        for (int32_t i = c * ORC_GROUP; i < (c + 1) * ORC_GROUP; ++i)
          part = fmaf((float)orc_bf16_value(x[(int64_t)t * d + i]), w_router[(int64_t)i * E + e], part);
        acc = acc + part;
      }
      if (bias) acc = acc + bias[e];
      logits[(int64_t)t * E + e] = acc;
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- 2. top-k and gate weights
 * Slot j holds the j-th best expert under the order (logit descending, index ascending), so
 * equal logits go to the lower expert index. Gate weights: softmax over the k selected logits
 * (equal to a softmax over all experts renormalised over the selected ones), in double and
 * then rounded to fp32. */
int oracle_topk_softmax(int32_t T, int32_t E, int32_t k, const float* logits, int32_t* ids, float* w) {
  if (k < 1 || k > E) return 1;
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  double* ex = (double*)malloc(sizeof(double) * (size_t)k);
  for (int32_t t = 0; t < T; ++t) {
    const float* l = logits + (int64_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
      taken[best] = 1;
      ids[(int64_t)t * k + j] = best;
    }
    double top = (double)l[ids[(int64_t)t * k]];
    double sum = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      ex[j] = exp((double)l[ids[(int64_t)t * k + j]] - top);
      sum += ex[j];
    }
    for (int32_t j = 0; j < k; ++j) w[(int64_t)t * k + j] = (float)(ex[j] / sum);
  }
  free(ex);
  free(taken);
  return 0;
}

/* ---------------------------------------------------------------- 3. routing metadata
 * Pair p = t*k + j (token-major). counts[e] = number of pairs routed to e (histogram);
 * offsets = exclusive prefix sum, offsets[E] = T*k (scan); the scatter is a stable counting
 * sort of pairs by expert, so rows of one expert keep ascending token order (reading: the
 * pages do not fix the order inside a group); sorted_token[row] = token of that grouped row,
 * inv_pos[t][j] = grouped row of pair (t, j).
 * Block map (reading; the pages say that block size follows each expert's load and that 32-row
 * tiles beat 16-row ones): each non-empty group, in ascending expert order, is cut into
 * consecutive tiles of at most 32 rows; then, when a shared expert exists, its T rows (grouped
 * rows T*k .. T*k+T-1, token order) are cut the same way and tagged with expert index E. A tile
 * is (expert, first grouped row, rows). */
int oracle_route_meta(int32_t T, int32_t E, int32_t k, int32_t has_shared, const int32_t* ids,
                      int32_t* counts, int32_t* offsets, int32_t* sorted_token, int32_t* inv_pos,
                      int32_t* tiles, int32_t tiles_cap, int32_t* n_tiles) {
  if (E < 1 || k < 1 || T < 0) return 1;
  const int64_t P = (int64_t)T * k;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < P; ++p) {
    if (ids[p] < 0 || ids[p] >= E) return 1;
    counts[ids[p]] += 1;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* cursor = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = ids[(int64_t)t * k + j];
      int32_t row = offsets[e] + cursor[e]++;
      sorted_token[row] = t;
      inv_pos[(int64_t)t * k + j] = row;
    }
  }
  free(cursor);
  int32_t n = 0;
  for (int32_t e = 0; e < E; ++e) {
    for (int32_t r = 0; r < counts[e]; r += ORC_TILE_ROWS) {
      if (n >= tiles_cap) return 2;
      tiles[3 * n + 0] = e;
      tiles[3 * n + 1] = offsets[e] + r;
      tiles[3 * n + 2] = counts[e] - r < ORC_TILE_ROWS ? counts[e] - r : ORC_TILE_ROWS;
      ++n;
    }
  }
  if (has_shared) {
    for (int32_t r = 0; r < T; r += ORC_TILE_ROWS) {
      if (n >= tiles_cap) return 2;
      tiles[3 * n + 0] = E;
      tiles[3 * n + 1] = (int32_t)P + r;
      tiles[3 * n + 2] = T - r < ORC_TILE_ROWS ? T - r : ORC_TILE_ROWS;
      ++n;
    }
  }
  *n_tiles = n;
  return 0;
}

/* ---------------------------------------------------------------- 4. dequantisation
 * Group g of row r covers inputs 64g .. 64g+63 and has one bf16 scale s and one bf16 bias b.
 * With 4-bit codes, input c of row r has code q = (byte >> (4 * (c & 1))) & 15 of byte c/2 (two
 * codes per byte, the even input in the low nibble -- reading). In general a row's codes form a
 * little-endian bit stream: code c occupies bits [bits * c, bits * c + bits) of the row's bytes
 * (bit j of the stream is bit j % 8 of byte j / 8), which for 4 bits is the nibble order above
 * (reading for 2- and 3-bit codes, a variant [DIFFGEMMA "The physics ceiling: why 300+ tok/s is
 * blocked"] names but does not define). The weight is w = s * q + b evaluated in fp32 (s * q is
 * exact in fp32, so this is one rounding) and then rounded to bf16, the operand type of the
 * matrix units. */
static uint16_t orc_dequant_one(const orc_q4* m, int64_t row, int32_t in_dim, int32_t c) {
  const int32_t bits = m->bits ? m->bits : 4;
  const int64_t row_bytes = (int64_t)in_dim * bits / 8;
  const uint8_t* rp = m->codes + row * row_bytes;
  const int64_t bit = (int64_t)c * bits;
  uint32_t two = rp[bit / 8];
  if (bit / 8 + 1 < row_bytes) two |= (uint32_t)rp[bit / 8 + 1] << 8;
  const uint32_t q = (two >> (bit % 8)) & ((1u << bits) - 1u);
  int64_t gi = row * (in_dim / ORC_GROUP) + c / ORC_GROUP;
  float s = (float)orc_bf16_value(m->scales[gi]);
  float b = (float)orc_bf16_value(m->biases[gi]);
  float w32 = s * (float)q + b;
  return orc_round_bf16(w32);
}

/* rows counts rows over all matrices (n_mat * out); out_bf16 is [rows][in_dim]. */
int oracle_dequant_bits(int64_t rows, int32_t in_dim, int32_t bits, const uint8_t* codes, const uint16_t* scales,
                        const uint16_t* biases, uint16_t* out_bf16) {
  if (in_dim % ORC_GROUP || (bits != 2 && bits != 3 && bits != 4)) return 1;
  orc_q4 m = {codes, scales, biases, bits};
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int32_t c = 0; c < in_dim; ++c) out_bf16[r * in_dim + c] = orc_dequant_one(&m, r, in_dim, c);
  return 0;
}

int oracle_dequant(int64_t rows, int32_t in_dim, const uint8_t* codes, const uint16_t* scales,
                   const uint16_t* biases, uint16_t* out_bf16) {
  return oracle_dequant_bits(rows, in_dim, 4, codes, scales, biases, out_bf16);
}

/* Dequantise matrix `mat` ([out][in]) of a projection into doubles (values are bf16). */
static void orc_dequant_matrix(const orc_q4* m, int32_t mat, int32_t out_dim, int32_t in_dim, double* dst) {
#pragma omp parallel for schedule(static)
  for (int32_t o = 0; o < out_dim; ++o) {
    int64_t row = (int64_t)mat * out_dim + o;
    for (int32_t c = 0; c < in_dim; ++c)
      dst[(int64_t)o * in_dim + c] = orc_bf16_value(orc_dequant_one(m, row, in_dim, c));
  }
}

/* ---------------------------------------------------------------- 5. one expert row
 * g_i = sum_c x_c Wg[i][c], u_i = sum_c x_c Wu[i][c] (double, ascending c);
 * a_i = silu(g_i) * u_i with silu(z) = z / (1 + e^-z); h_i = bf16(fp32(a_i));
 * y_o = sum_i h_i Wd[o][i] (double, ascending i). */
static void orc_ffn_row(int32_t d, int32_t I, const uint16_t* x_row, const double* Wg, const double* Wu,
                        const double* Wd, double* h, double* y_row, uint16_t* h_bits) {
  for (int32_t i = 0; i < I; ++i) {
    double g = 0.0, u = 0.0;
    for (int32_t c = 0; c < d; ++c) {
      double xc = orc_bf16_value(x_row[c]);
      g += xc * Wg[(int64_t)i * d + c];
      u += xc * Wu[(int64_t)i * d + c];
    }
    double a = (g / (1.0 + exp(-g))) * u;
    uint16_t hb = orc_round_bf16((float)a);
    h[i] = orc_bf16_value(hb);
    if (h_bits) h_bits[i] = hb;
  }
  for (int32_t o = 0; o < d; ++o) {
    double acc = 0.0;
    for (int32_t i = 0; i < I; ++i) acc += h[i] * Wd[(int64_t)o * I + i];
    y_row[o] = acc;
  }
}

/* ---------------------------------------------------------------- 5a. the two grouped products alone
 * The two products of step 5 over the grouped rows, before the activation and before any rounding
 * of their results, so that a grouped GEMM can be checked stage by stage:
 *   gate/up: g[r][i] = sum_c x[tok(r)][c] * Wg_e(r)[i][c] and u[r][i] likewise with Wu, in double,
 *            c ascending; grouped row r < P = T*k belongs to the routed expert e(r) whose group
 *            [offsets[e], offsets[e+1]) holds it and to token tok(r) = sorted_token[r]; rows
 *            P .. P+T-1 are the shared expert's, token r - P. Outputs [P][I] then [T][Is].
 *   down:    y[r][o] = sum_i h[r][i] * Wd_e(r)[o][i], in double, i ascending, for given bf16 h
 *            laid out [P][I] then [T][Is]; output [P + T][d] (shared rows only when Is > 0).
 * The weights are the bf16 dequantised values of step 4. */
static int orc_offsets_ok(int32_t E, int64_t P, const int32_t* offsets) {
  if (offsets[0] != 0 || offsets[E] != P) return 0;
  for (int32_t e = 0; e < E; ++e)
    if (offsets[e + 1] < offsets[e]) return 0;
  return 1;
}

int oracle_gateup_preact(int32_t T, int32_t d, int32_t E, int32_t k, int32_t I, int32_t Is, const uint16_t* x,
                         const orc_ffn* routed, const orc_ffn* shared, const int32_t* offsets,
                         const int32_t* sorted_token, double* g, double* u) {
  if (d % ORC_GROUP || I % ORC_GROUP || Is % ORC_GROUP || k < 1 || k > E) return 1;
  if ((Is > 0) != (shared != NULL)) return 1;
  const int64_t P = (int64_t)T * k;
  if (!orc_offsets_ok(E, P, offsets)) return 1;
  const int32_t Imax = I > Is ? I : Is;
  double* Wg = (double*)malloc(sizeof(double) * (size_t)Imax * d);
  double* Wu = (double*)malloc(sizeof(double) * (size_t)Imax * d);
  for (int32_t e = 0; e <= E; ++e) {
    const int sh = (e == E);
    if (sh && Is == 0) break;
    const int64_t r0 = sh ? P : offsets[e], r1 = sh ? P + T : offsets[e + 1];
    if (r0 == r1) continue;
    const int32_t Ie = sh ? Is : I;
    orc_dequant_matrix(sh ? &shared->gate : &routed->gate, sh ? 0 : e, Ie, d, Wg);
    orc_dequant_matrix(sh ? &shared->up : &routed->up, sh ? 0 : e, Ie, d, Wu);
    double* go = sh ? g + P * I : g;
    double* uo = sh ? u + P * I : u;
#pragma omp parallel for schedule(static)
    for (int64_t r = r0; r < r1; ++r) {
      const int64_t t = sh ? r - P : sorted_token[r];
      const int64_t orow = sh ? r - P : r;
      for (int32_t i = 0; i < Ie; ++i) {
        double gs = 0.0, us = 0.0;
        for (int32_t c = 0; c < d; ++c) {
          const double xc = orc_bf16_value(x[t * d + c]);
          gs += xc * Wg[(int64_t)i * d + c];
          us += xc * Wu[(int64_t)i * d + c];
        }
        go[orow * Ie + i] = gs;
        uo[orow * Ie + i] = us;
      }
    }
  }
  free(Wg);
  free(Wu);
  return 0;
}

int oracle_down_rows(int32_t T, int32_t d, int32_t E, int32_t k, int32_t I, int32_t Is, const uint16_t* h,
                     const orc_ffn* routed, const orc_ffn* shared, const int32_t* offsets, double* y) {
  if (d % ORC_GROUP || I % ORC_GROUP || Is % ORC_GROUP || k < 1 || k > E) return 1;
  if ((Is > 0) != (shared != NULL)) return 1;
  const int64_t P = (int64_t)T * k;
  if (!orc_offsets_ok(E, P, offsets)) return 1;
  const int32_t Imax = I > Is ? I : Is;
  double* Wd = (double*)malloc(sizeof(double) * (size_t)Imax * d);
  for (int32_t e = 0; e <= E; ++e) {
    const int sh = (e == E);
    if (sh && Is == 0) break;
    const int64_t r0 = sh ? P : offsets[e], r1 = sh ? P + T : offsets[e + 1];
    if (r0 == r1) continue;
    const int32_t Ie = sh ? Is : I;
    orc_dequant_matrix(sh ? &shared->down : &routed->down, sh ? 0 : e, d, Ie, Wd);
    const uint16_t* hb = sh ? h + P * I : h;
#pragma omp parallel for schedule(static)
    for (int64_t r = r0; r < r1; ++r) {
      const int64_t hrow = sh ? r - P : r;
      for (int32_t o = 0; o < d; ++o) {
        double acc = 0.0;
        for (int32_t i = 0; i < Ie; ++i) acc += orc_bf16_value(hb[hrow * Ie + i]) * Wd[(int64_t)o * Ie + i];
        y[r * d + o] = acc;
      }
    }
  }
  free(Wd);
  return 0;
}

/* ---------------------------------------------------------------- 7. combine
 * y[t] = bf16(fp32(sum_j w[t][j] * y_pair(t,j) + y_shared(t))), j ascending, in double. */
static uint16_t orc_combine_one(int32_t k, const float* w_t, const double* const* rows, const double* shared_row,
                                int32_t o) {
  double acc = 0.0;
  for (int32_t j = 0; j < k; ++j) acc += (double)w_t[j] * rows[j][o];
  if (shared_row) acc += shared_row[o];
  return orc_round_bf16((float)acc);
}

/* ---------------------------------------------------------------- whole layer, grouped
 * Runs steps 1-7 on all T tokens. Optional outputs (NULL to skip): logits [T][E], ids/w [T][k],
 * counts [E], offsets [E+1], sorted_token [T*k], inv_pos [T*k], tiles [3*tiles_cap], n_tiles,
 * h_bits [T*k][I] (grouped order) and h_shared_bits [T][Is]. */
int oracle_forward_layer(int32_t T, int32_t d, int32_t E, int32_t k, int32_t I, int32_t Is, const uint16_t* x,
                         const float* w_router, const float* bias, const orc_ffn* routed, const orc_ffn* shared,
                         uint16_t* y, float* logits_out, int32_t* ids_out, float* w_out, int32_t* counts_out,
                         int32_t* offsets_out, int32_t* sorted_out, int32_t* inv_pos_out, int32_t* tiles_out,
                         int32_t tiles_cap, int32_t* n_tiles_out, uint16_t* h_bits, uint16_t* h_shared_bits) {
  if (d % ORC_GROUP || I % ORC_GROUP || Is % ORC_GROUP || k < 1 || k > E || k > 64) return 1;
  if ((Is > 0) != (shared != NULL)) return 1;
  const int64_t P = (int64_t)T * k;
  float* logits = (float*)malloc(sizeof(float) * (size_t)((int64_t)T * E + 1));
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)(P + 1));
  float* w = (float*)malloc(sizeof(float) * (size_t)(P + 1));
  int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t* sorted_token = (int32_t*)malloc(sizeof(int32_t) * (size_t)(P + 1));
  int32_t* inv_pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)(P + 1));
  int32_t cap = (int32_t)(E + P / ORC_TILE_ROWS + T / ORC_TILE_ROWS + 2);
  int32_t* tiles = (int32_t*)malloc(sizeof(int32_t) * 3 * (size_t)cap);
  int32_t n_tiles = 0;
  int rc = oracle_router_logits(T, d, E, x, w_router, bias, logits);
  if (!rc) rc = oracle_topk_softmax(T, E, k, logits, ids, w);
  if (!rc) rc = oracle_route_meta(T, E, k, Is > 0, ids, counts, offsets, sorted_token, inv_pos, tiles, cap, &n_tiles);
  double* y_rows = NULL;
  double* y_shared = NULL;
  if (!rc) {
    y_rows = (double*)malloc(sizeof(double) * (size_t)(P * d + 1));
    int32_t Imax = I > Is ? I : Is;
    double* Wg = (double*)malloc(sizeof(double) * (size_t)Imax * d);
    double* Wu = (double*)malloc(sizeof(double) * (size_t)Imax * d);
    double* Wd = (double*)malloc(sizeof(double) * (size_t)Imax * d);
    for (int32_t e = 0; e < E; ++e) {
      if (counts[e] == 0) continue; /* empty experts are never read */
      orc_dequant_matrix(&routed->gate, e, I, d, Wg);
      orc_dequant_matrix(&routed->up, e, I, d, Wu);
      orc_dequant_matrix(&routed->down, e, d, I, Wd);
#pragma omp parallel
      {
        double* h = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
        for (int32_t r = offsets[e]; r < offsets[e + 1]; ++r)
          orc_ffn_row(d, I, x + (int64_t)sorted_token[r] * d, Wg, Wu, Wd, h, y_rows + (int64_t)r * d,
                      h_bits ? h_bits + (int64_t)r * I : NULL);
        free(h);
      }
    }
    if (Is > 0) {
      y_shared = (double*)malloc(sizeof(double) * (size_t)((int64_t)T * d + 1));
      orc_dequant_matrix(&shared->gate, 0, Is, d, Wg);
      orc_dequant_matrix(&shared->up, 0, Is, d, Wu);
      orc_dequant_matrix(&shared->down, 0, d, Is, Wd);
#pragma omp parallel
      {
        double* h = (double*)malloc(sizeof(double) * (size_t)Is);
#pragma omp for schedule(dynamic, 1)
        for (int32_t t = 0; t < T; ++t)
          orc_ffn_row(d, Is, x + (int64_t)t * d, Wg, Wu, Wd, h, y_shared + (int64_t)t * d,
                      h_shared_bits ? h_shared_bits + (int64_t)t * Is : NULL);
        free(h);
      }
    }
    free(Wg);
    free(Wu);
    free(Wd);
#pragma omp parallel for schedule(static)
    for (int32_t t = 0; t < T; ++t) {
      const double* rows[64];
      for (int32_t j = 0; j < k; ++j) rows[j] = y_rows + (int64_t)inv_pos[(int64_t)t * k + j] * d;
      for (int32_t o = 0; o < d; ++o)
        y[(int64_t)t * d + o] = orc_combine_one(k, w + (int64_t)t * k, rows, y_shared ? y_shared + (int64_t)t * d : NULL, o);
    }
  }
  if (!rc) {
    if (logits_out) memcpy(logits_out, logits, sizeof(float) * (size_t)((int64_t)T * E));
    if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)P);
    if (w_out) memcpy(w_out, w, sizeof(float) * (size_t)P);
    if (counts_out) memcpy(counts_out, counts, sizeof(int32_t) * (size_t)E);
    if (offsets_out) memcpy(offsets_out, offsets, sizeof(int32_t) * (size_t)(E + 1));
    if (sorted_out) memcpy(sorted_out, sorted_token, sizeof(int32_t) * (size_t)P);
    if (inv_pos_out) memcpy(inv_pos_out, inv_pos, sizeof(int32_t) * (size_t)P);
    if (tiles_out) {
      if (n_tiles > tiles_cap) rc = 2;
      else memcpy(tiles_out, tiles, sizeof(int32_t) * 3 * (size_t)n_tiles);
    }
    if (n_tiles_out) *n_tiles_out = n_tiles;
  }
  free(y_rows);
  free(y_shared);
  free(logits);
  free(ids);
  free(w);
  free(counts);
  free(offsets);
  free(sorted_token);
  free(inv_pos);
  free(tiles);
  return rc;
}

/* ---------------------------------------------------------------- selected tokens only
 * The same output for a list of tokens, evaluated token by token (no grouping): for each
 * listed token, its logits, top-k and weights, then each selected expert's FFN row and the
 * shared expert's, combined as in step 7. Routing is per token, so this equals the grouped
 * result row for row; it lets large workloads be checked on a sample of tokens. */
int oracle_forward_tokens(int32_t T, int32_t d, int32_t E, int32_t k, int32_t I, int32_t Is, const uint16_t* x,
                          const float* w_router, const float* bias, const orc_ffn* routed, const orc_ffn* shared,
                          int32_t n_sel, const int32_t* sel, uint16_t* y_sel, int32_t* ids_sel, float* w_sel) {
  if (d % ORC_GROUP || I % ORC_GROUP || Is % ORC_GROUP || k < 1 || k > E || k > 64) return 1;
  if ((Is > 0) != (shared != NULL)) return 1;
  for (int32_t s = 0; s < n_sel; ++s)
    if (sel[s] < 0 || sel[s] >= T) return 1;
  int rc = 0;
  int32_t Imax = I > Is ? I : Is;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : rc)
  for (int32_t s = 0; s < n_sel; ++s) {
    const int32_t t = sel[s];
    const uint16_t* xr = x + (int64_t)t * d;
    float* lg = (float*)malloc(sizeof(float) * (size_t)E);
    int32_t ids[64];
    float w[64];
    rc |= oracle_router_logits(1, d, E, xr, w_router, bias, lg);
    rc |= oracle_topk_softmax(1, E, k, lg, ids, w);
    double* Wg = (double*)malloc(sizeof(double) * (size_t)Imax * d);
    double* Wu = (double*)malloc(sizeof(double) * (size_t)Imax * d);
    double* Wd = (double*)malloc(sizeof(double) * (size_t)Imax * d);
    double* h = (double*)malloc(sizeof(double) * (size_t)Imax);
    double* yr = (double*)malloc(sizeof(double) * (size_t)(k + 1) * d);
    const double* rows[64];
    for (int32_t j = 0; j < k; ++j) {
      const int32_t e = ids[j];
      for (int32_t i = 0; i < I; ++i)
        for (int32_t c = 0; c < d; ++c) {
          Wg[(int64_t)i * d + c] = orc_bf16_value(orc_dequant_one(&routed->gate, (int64_t)e * I + i, d, c));
          Wu[(int64_t)i * d + c] = orc_bf16_value(orc_dequant_one(&routed->up, (int64_t)e * I + i, d, c));
        }
      for (int32_t o = 0; o < d; ++o)
        for (int32_t i = 0; i < I; ++i)
          Wd[(int64_t)o * I + i] = orc_bf16_value(orc_dequant_one(&routed->down, (int64_t)e * d + o, I, i));
      orc_ffn_row(d, I, xr, Wg, Wu, Wd, h, yr + (int64_t)j * d, NULL);
      rows[j] = yr + (int64_t)j * d;
    }
    const double* shared_row = NULL;
    if (Is > 0) {
      for (int32_t i = 0; i < Is; ++i)
        for (int32_t c = 0; c < d; ++c) {
          Wg[(int64_t)i * d + c] = orc_bf16_value(orc_dequant_one(&shared->gate, i, d, c));
          Wu[(int64_t)i * d + c] = orc_bf16_value(orc_dequant_one(&shared->up, i, d, c));
        }
      for (int32_t o = 0; o < d; ++o)
        for (int32_t i = 0; i < Is; ++i)
          Wd[(int64_t)o * Is + i] = orc_bf16_value(orc_dequant_one(&shared->down, o, Is, i));
      orc_ffn_row(d, Is, xr, Wg, Wu, Wd, h, yr + (int64_t)k * d, NULL);
      shared_row = yr + (int64_t)k * d;
    }
    for (int32_t o = 0; o < d; ++o) y_sel[(int64_t)s * d + o] = orc_combine_one(k, w, rows, shared_row, o);
    if (ids_sel) memcpy(ids_sel + (int64_t)s * k, ids, sizeof(int32_t) * (size_t)k);
    if (w_sel) memcpy(w_sel + (int64_t)s * k, w, sizeof(float) * (size_t)k);
    free(lg);
    free(Wg);
    free(Wu);
    free(Wd);
    free(h);
    free(yr);
  }
  return rc;
}

/* ---------------------------------------------------------------- 8. exact top-K of logit rows
 * [DIFFGEMMA "The optimizations that worked"]: a sampler needs only the K largest logits of a
 * position; the pages reach them through chunk maxima and state that the result is exactly
 * the global top-K. Definition used here: sort the row by (value descending, index ascending)
 * and keep the first K; ids[r][j] and vals[r][j] are the j-th entry. -0 and +0 compare equal
 * (so the lower index comes first). Rows must hold no NaN (reading: the pages' logits are
 * finite). */
static const float* orc_sort_row;
static int orc_cmp_desc(const void* a, const void* b) {
  const int32_t i = *(const int32_t*)a, j = *(const int32_t*)b;
  const float x = orc_sort_row[i], y = orc_sort_row[j];
  if (x > y) return -1;
  if (x < y) return 1;
  return (i > j) - (i < j);
}

int oracle_vocab_topk(int32_t R, int32_t V, int32_t K, const float* logits, int32_t* ids, float* vals) {
  if (R < 0 || V < 1 || K < 1 || K > V) return 1;
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)V);
  if (!idx) return 2;
  /* qsort takes no context argument, so rows are sorted one after another */
  for (int32_t r = 0; r < R; ++r) {
    const float* row = logits + (int64_t)r * V;
    for (int32_t i = 0; i < V; ++i) idx[i] = i;
    orc_sort_row = row;
    qsort(idx, (size_t)V, sizeof(int32_t), orc_cmp_desc);
    for (int32_t j = 0; j < K; ++j) {
      ids[(int64_t)r * K + j] = idx[j];
      vals[(int64_t)r * K + j] = row[idx[j]];
    }
  }
  free(idx);
  return 0;
}
