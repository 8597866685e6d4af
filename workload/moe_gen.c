/*
 * Seeded, counter-based input generator for the routed int4 MoE layer workloads.
 *
 * This module only draws random inputs. It holds none of the method's arithmetic
 * (no routing, no dequantisation, no FFN), so it may serve both the CPU oracle and
 * the GPU library without coupling them.
 *
 * Definition (so a reader can re-implement it):
 *   - mix64 is the SplitMix64 finaliser (Steele, Lea, Flood, "Fast splittable
 *     pseudorandom number generators", OOPSLA 2014; constants as published there).
 *   - A stream is identified by a 64-bit key; its word n (n = 0, 1, ...) is
 *     mix64(key + (n + 1) * 0x9E3779B97F4A7C15), i.e. SplitMix64's output sequence
 *     started from state `key`. Any element can therefore be produced on its own.
 *   - The key of (seed, layer, tensor) is
 *     k0 = mix64(seed + G); k1 = mix64(k0 ^ (layer + 1) * C1); key = mix64(k1 ^ (tensor + 1) * C2).
 *   - Byte b of a stream is byte (b mod 8) (little-endian) of word b / 8.
 *   - Uniform u = (word >> 11) * 2^-53 in [0, 1).
 *   - Normal element n uses words 2n and 2n+1 (Box-Muller, cosine branch only):
 *     z = sqrt(-2 ln(1 - u1)) * cos(2 pi u2), computed in double with the C library.
 *   - A value v is stored as fp32 by a C cast (round to nearest even), and as bf16
 *     by rounding that fp32 to the nearest bf16, ties to even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL
#define C_LAYER 0xD1B54A32D192ED03ULL
#define C_TENSOR 0x8CB92BA72F3D8DD7ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t word_at(uint64_t key, uint64_t n) { return mix64(key + (n + 1) * GOLDEN); }

static inline double uniform_of(uint64_t r) { return (double)(r >> 11) * 0x1.0p-53; }

static inline double normal_at(uint64_t key, uint64_t n) {
  double u1 = uniform_of(word_at(key, 2 * n));
  double u2 = uniform_of(word_at(key, 2 * n + 1));
  return sqrt(-2.0 * log(1.0 - u1)) * cos(6.283185307179586 * u2);
}

static inline uint16_t gen_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline float gen_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint64_t gen_stream_key(uint64_t seed, uint64_t layer, uint64_t tensor) {
  uint64_t k = mix64(seed + GOLDEN);
  k = mix64(k ^ ((layer + 1) * C_LAYER));
  return mix64(k ^ ((tensor + 1) * C_TENSOR));
}

uint64_t gen_word(uint64_t key, uint64_t n) { return word_at(key, n); }

/* n random bytes starting at stream byte `start`. */
void gen_bytes(uint64_t key, uint64_t start, int64_t n, uint8_t* out) {
  int64_t head = (int64_t)((8 - (start & 7)) & 7);
  if (head > n) head = n;
  for (int64_t i = 0; i < head; ++i) {
    uint64_t b = start + (uint64_t)i;
    out[i] = (uint8_t)(word_at(key, b >> 3) >> (8 * (b & 7)));
  }
  int64_t nw = (n - head) / 8;
  uint64_t w0 = (start + (uint64_t)head) >> 3;
#pragma omp parallel for schedule(static)
  for (int64_t w = 0; w < nw; ++w) {
    uint64_t r = word_at(key, w0 + (uint64_t)w);
    memcpy(out + head + 8 * w, &r, 8); /* little-endian host */
  }
  for (int64_t i = head + 8 * nw; i < n; ++i) {
    uint64_t b = start + (uint64_t)i;
    out[i] = (uint8_t)(word_at(key, b >> 3) >> (8 * (b & 7)));
  }
}

/* n normals N(0, sigma^2) starting at element `start`, stored as bf16 bits. */
void gen_normal_bf16(uint64_t key, uint64_t start, int64_t n, double sigma, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = gen_f32_to_bf16((float)(sigma * normal_at(key, start + (uint64_t)i)));
}

/* n normals N(0, sigma^2) starting at element `start`, stored as fp32. */
void gen_normal_f32(uint64_t key, uint64_t start, int64_t n, double sigma, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(sigma * normal_at(key, start + (uint64_t)i));
}

/* Quantisation scales bf16(|N(0, sigma^2)|) and biases bf16(-8 * scale) (the product by -8
 * is exact, so the bias is exactly -8 times the stored scale). */
void gen_scale_bias_bf16(uint64_t key, uint64_t start, int64_t n, double sigma, uint16_t* scales,
                         uint16_t* biases) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint16_t s = gen_f32_to_bf16((float)fabs(sigma * normal_at(key, start + (uint64_t)i)));
    scales[i] = s;
    biases[i] = gen_f32_to_bf16(-8.0f * gen_bf16_to_f32(s));
  }
}

/* Zipf-like additive logit bias: bias[e] = (float)(alpha * ln(1 / rank[e])); rank[e] = e + 1
 * when `rank` is NULL. */
void gen_zipf_bias(int32_t n_experts, double alpha, const int32_t* rank, float* out) {
  for (int32_t e = 0; e < n_experts; ++e) {
    double r = rank ? (double)rank[e] : (double)(e + 1);
    out[e] = (float)(alpha * log(1.0 / r));
  }
}
