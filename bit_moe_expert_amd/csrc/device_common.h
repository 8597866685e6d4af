// Device helpers shared by the gfx950 kernels of the routed int4 MoE FFN.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_int4.h"

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kGroup = 64;      // quantisation group along the input dimension
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (low half = a), hardware round-to-nearest-even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float a) { return (uint16_t)(pack_bf16x2(a, 0.0f) & 0xffffu); }

// Two fp32 -> packed fp16 pair (low half = a), round-to-nearest-even; and the way back.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  f32x2_t v = {a, b};
  h2 r = __builtin_convertvector(v, h2);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float f16lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// A constant the compiler must hold in a VGPR: gfx9 VOP3 encodings take no literal, so
// (t & mask) | magic with plain constants becomes an AND and an OR; with both in registers it is
// one v_and_or_b32. The value is loop-invariant and the asm has no side effects, so it is
// materialised once.
__device__ __forceinline__ uint32_t opaque_v(uint32_t c) {
  asm("" : "+v"(c));
  return c;
}

// "128 + q" as bf16: 0x4300 is 128.0 and its 7 mantissa bits hold q exactly. From a word of
// 8 codes, pair n (n = 0..3) holds inputs (n, n + 4) of the word: a shift and one v_and_or_b32.
__device__ __forceinline__ uint32_t magic_pair(uint32_t w, int n) {
  return ((w >> (4 * n)) & opaque_v(0x000F000Fu)) | opaque_v(0x43004300u);
}

// All four magic_pair(w, n), n = 0..3, in 7 operations: the low and high nibbles of every byte
// (lo = inputs 0, 2, 4, 6 and hi = inputs 1, 3, 5, 7, one per byte), then byte permutes that
// put each code under a 0x43 high byte: pair (n, n + 4) takes bytes (0, 2) of lo or hi for
// n = 0, 1 and bytes (1, 3) for n = 2, 3.
__device__ __forceinline__ void magic_pairs4(uint32_t w, uint32_t p[4]) {
  const uint32_t lo = w & 0x0F0F0F0Fu;
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  p[0] = __builtin_amdgcn_perm(0x43434343u, lo, 0x04020400u);
  p[1] = __builtin_amdgcn_perm(0x43434343u, hi, 0x04020400u);
  p[2] = __builtin_amdgcn_perm(0x43434343u, lo, 0x04030401u);
  p[3] = __builtin_amdgcn_perm(0x43434343u, hi, 0x04030401u);
}

// The 32 weight codes of one 32-input segment: a row's codes are a little-endian bit stream of
// BITS bits per code, so the segment occupies 4 * BITS bytes at p (16-, 12- or 8-byte loads);
// load_code_words returns those words (unused ones zero). The load and the unpack (seg_pairs)
// are separate so that the unpack can wait until the codes are used.
template <int BITS>
__device__ __forceinline__ uint4 load_code_words(const uint8_t* p) {
  if (BITS == 4) return *reinterpret_cast<const uint4*>(p);
  if (BITS == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_uint4(w.x, w.y, 0u, 0u);
  }
  const uint3 w = *reinterpret_cast<const uint3*>(p);
  return make_uint4(w.x, w.y, w.z, 0u);
}

// Which inputs of the segment magic pair k of seg_pairs<BITS> holds: (pair_input(k),
// pair_input(k) + pair_gap). 4-bit pairs take inputs (n, n + 4) of each 8-input word; 3- and
// 2-bit pairs take inputs (i, i + 8) of each 16-input half.
template <int BITS>
__host__ __device__ constexpr int pair_gap() {
  return BITS == 4 ? 4 : 8;
}
template <int BITS>
__host__ __device__ constexpr int pair_input(int k) {
  return BITS == 4 ? 8 * (k / 4) + k % 4 : 16 * (k / 8) + k % 8;
}

// The segment's 16 "128 + q" magic pairs straight from its code words, in pair_input order.
//  4 bits: magic_pairs4 per word (7 operations per 8 codes).
//  2 bits: a word holds the 16 codes of one half, code c at bits 2c; shifted right by 2r, codes
//          r and r + 8 sit at bits 0 and 16, codes 4 + r and 12 + r at bits 8 and 24, so each
//          pair is one v_and_or_b32 (15 operations per 16 codes).
//  3 bits: a half's 16 codes span 6 bytes and codes i, i + 8 lie 24 bits apart, so a byte
//          permute that puts stream bits [8a, 8a + 16) and [8a + 24, 8a + 40) in the low and
//          high halves of a dword leaves both codes at the same offset in their halves; one
//          shift and one v_and_or_b32 then give the pair (a = 0 serves i = 0..4, a = 1 serves
//          i = 5..7; 17 operations per 16 codes).
template <int BITS>
__device__ __forceinline__ void seg_pairs(const uint4& w, uint32_t p[16]) {
  if (BITS == 4) {
    magic_pairs4(w.x, p);
    magic_pairs4(w.y, p + 4);
    magic_pairs4(w.z, p + 8);
    magic_pairs4(w.w, p + 12);
  } else if (BITS == 2) {
    const uint32_t m = opaque_v(0x00030003u), g = opaque_v(0x43004300u);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t t = (h ? w.y : w.x) >> (2 * r);
        p[8 * h + r] = (t & m) | g;
        p[8 * h + 4 + r] = ((t >> 8) & m) | g;
      }
  } else {
    const uint32_t m = opaque_v(0x00070007u), g = opaque_v(0x43004300u);
    // half 0: stream bytes (0, 1, 3, 4) and (1, 2, 4, 5) of words x, y;
    // half 1: stream bytes (6, 7, 9, 10) and (7, 8, 10, 11) of words y, z.
    const uint32_t t[4] = {__builtin_amdgcn_perm(w.y, w.x, 0x04030100u), __builtin_amdgcn_perm(w.y, w.x, 0x05040201u),
                           __builtin_amdgcn_perm(w.z, w.y, 0x06050302u), __builtin_amdgcn_perm(w.z, w.y, 0x07060403u)};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t u = i < 5 ? t[2 * h] >> (3 * i) : t[2 * h + 1] >> (3 * i - 8);
        p[8 * h + i] = (u & m) | g;
      }
  }
}

// Re-pair 8 bf16 values (4 dwords in natural order) to match magic_pair: pair n = (v[n], v[n+4]).
// The result holds the inputs of the chunk in "pair order": 0, 4, 1, 5, 2, 6, 3, 7.
__device__ __forceinline__ void repair8(const uint32_t v[4], uint32_t p[4]) {
  p[0] = __builtin_amdgcn_perm(v[2], v[0], 0x05040100u);
  p[1] = __builtin_amdgcn_perm(v[2], v[0], 0x07060302u);
  p[2] = __builtin_amdgcn_perm(v[3], v[1], 0x05040100u);
  p[3] = __builtin_amdgcn_perm(v[3], v[1], 0x07060302u);
}

// Position of input i in pair order: within its chunk of 8, input j goes to 2j (j < 4) or
// 2(j - 4) + 1 (j >= 4).
__device__ __forceinline__ int pair_pos(int i) {
  const int j = i & 7;
  return (i & ~7) | (j < 4 ? 2 * j : 2 * j - 7);
}

// fp32 += a.lo * b.lo + a.hi * b.hi over bf16 pairs.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// silu(g) * u = g / (1 + e^-g) * u, with the hardware exponential and reciprocal (about 1 ulp
// each; the division's correctly rounded sequence costs an order of magnitude more).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Sum over the wave, the same value in every lane: DPP within rows of 16 lanes (swap
// neighbours, swap pairs, rotate by 4, rotate by 8), then the four row sums of lanes 0, 16, 32
// and 48 in that order.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// A value from another lane of the quad (quad_perm CTRL), every lane written (no old value kept).
template <int CTRL>
__device__ __forceinline__ float quad_swap(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x124>(v);
  v += dpp_f32<0x128>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return ((r0 + r1) + r2) + r3;
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63u; }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const uint32_t l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Order-preserving 32-bit key of a logit: a larger logit gives a larger key; -0 is first turned
// into +0 so that equal logits give equal keys. Key 0 means "empty" (no finite logit maps to 0).
__device__ __forceinline__ uint32_t topk_key(float v) {
  uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Max of a 32-bit value over the wave, returned uniform: DPP steps within each row of 16 lanes
// (swap neighbours, swap pairs, rotate by 4, rotate by 8) leave the row maximum in every lane;
// the four row maxima are then read as scalars.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm 1,0,3,2
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm 2,3,0,1
  v = max(v, dpp_u32<0x124>(v));  // row_ror 4
  v = max(v, dpp_u32<0x128>(v));  // row_ror 8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// One wave: top-k of logits lg[0..E) (E <= 64 * SLOTS, k <= 16) by (logit desc, index asc),
// then the softmax over the chosen logits. Lane l holds experts l + 64 s. Each round takes the
// largest key over the wave, then the lowest expert index holding it (ballots over the slots in
// ascending order, lowest lane first). Lane j < k writes slot j. Call with a whole wave.
template <int SLOTS>
__device__ __forceinline__ void wave_topk_softmax_n(const float* lg, int E, int k, int32_t* ids_out, float* w_out) {
  const int lane = (int)lane_id();
  uint32_t key[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int e = lane + 64 * s;
    key[s] = e < E ? topk_key(lg[e]) : 0u;
  }
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t loc = key[0];
#pragma unroll
    for (int s = 1; s < SLOTS; ++s) loc = max(loc, key[s]);
    const uint32_t best = wave_max_u32(loc);
    int win = -1;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) {
      const uint64_t m = __ballot(key[s] == best);
      if (win < 0 && m != 0) win = 64 * s + (int)__builtin_ctzll(m);
    }
#pragma unroll
    for (int s = 0; s < SLOTS; ++s)
      if (lane + 64 * s == win) key[s] = 0u;
    if (lane == j) my_e = win;
  }
  const float my_l = lane < k ? lg[my_e] : 0.0f;
  const float top = __shfl(my_l, 0, 64);
  const float ex = lane < k ? expf(my_l - top) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    ids_out[lane] = my_e;
    w_out[lane] = ex / sum;
  }
}

// Min of a 32-bit value over the wave, returned uniform (as wave_max_u32).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<0xB1>(v));
  v = min(v, dpp_u32<0x4E>(v));
  v = min(v, dpp_u32<0x124>(v));
  v = min(v, dpp_u32<0x128>(v));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return min(min(r0, r1), min(r2, r3));
}

// wave_topk_softmax with each lane's keys sorted first: a lane's SLOTS experts are ordered by
// (key desc, index asc) once, and every round reduces only the lanes' heads. The largest head
// is the next pick; when several lanes' heads hold it (an exact tie), the lowest expert among
// them wins. The winning lane then moves to its next key.
template <int SLOTS>
__device__ __forceinline__ void wave_topk_softmax_sorted(const float* lg, int E, int k, int32_t* ids_out,
                                                         float* w_out) {
  const int lane = (int)lane_id();
  uint32_t key[SLOTS];
  int idx[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    idx[s] = lane + 64 * s;
    key[s] = idx[s] < E ? topk_key(lg[idx[s]]) : 0u;
  }
  // insertion sort by key desc; idx ascends with s, so a strict comparison keeps equal keys
  // in index order
#pragma unroll
  for (int a = 1; a < SLOTS; ++a)
#pragma unroll
    for (int b = a; b > 0; --b) {
      const bool sw = key[b] > key[b - 1];
      const uint32_t tk = key[b];
      const int ti = idx[b];
      key[b] = sw ? key[b - 1] : key[b];
      idx[b] = sw ? idx[b - 1] : idx[b];
      key[b - 1] = sw ? tk : key[b - 1];
      idx[b - 1] = sw ? ti : idx[b - 1];
    }
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t best = wave_max_u32(key[0]);
    const uint64_t m = __ballot(key[0] == best);
    int wl;
    if (__builtin_popcountll(m) == 1) {
      wl = (int)__builtin_ctzll(m);
    } else {
      const uint32_t lo = wave_min_u32(key[0] == best ? (uint32_t)idx[0] : 0xFFFFFFFFu);
      wl = (int)__builtin_ctzll(__ballot(key[0] == best && (uint32_t)idx[0] == lo));
    }
    const int e = __builtin_amdgcn_readlane(idx[0], wl);
    if (lane == wl) {
#pragma unroll
      for (int s = 0; s + 1 < SLOTS; ++s) {
        key[s] = key[s + 1];
        idx[s] = idx[s + 1];
      }
      key[SLOTS - 1] = 0u;
    }
    if (lane == j) my_e = e;
  }
  const float my_l = lane < k ? lg[my_e] : 0.0f;
  const float top = __shfl(my_l, 0, 64);
  const float ex = lane < k ? expf(my_l - top) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    ids_out[lane] = my_e;
    w_out[lane] = ex / sum;
  }
}

__device__ __forceinline__ void wave_topk_softmax(const float* lg, int E, int k, int32_t* ids_out, float* w_out) {
  if (E <= 64)
    wave_topk_softmax_sorted<1>(lg, E, k, ids_out, w_out);
  else if (E <= 128)
    wave_topk_softmax_sorted<2>(lg, E, k, ids_out, w_out);
  else if (E <= 256)
    wave_topk_softmax_sorted<4>(lg, E, k, ids_out, w_out);
  else
    wave_topk_softmax_n<16>(lg, E, k, ids_out, w_out);
}

// Router logits of one token from its chunk partials parts[e][c] (c = 0 .. nchunks-1, each
// expert's partials contiguous): the partials are added in ascending chunk order to +0, then the
// bias. Threads of the block take experts tid, tid + blockDim.x, ...; results go to lg[e]. A
// thread issues every load of a 32-chunk batch (16-byte loads when nchunks % 4 == 0) before
// the adds.
__device__ __forceinline__ void sum_chunk_partials(const float* __restrict__ parts, const float* __restrict__ bias,
                                                   int nchunks, int E, float* lg) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const float* pe = parts + (size_t)e * nchunks;
    float acc = 0.0f;
    if ((nchunks & 31) == 0) {  // whole batches: straight-line loads, then the adds
      for (int cb = 0; cb < nchunks; cb += 32) {
        f32x4_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = reinterpret_cast<const f32x4_t*>(pe + cb)[q];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc = (((acc + v[q].x) + v[q].y) + v[q].z) + v[q].w;
      }
    } else if ((nchunks & 3) == 0) {
      for (int cb = 0; cb < nchunks; cb += 32) {
        f32x4_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          v[q] = cb + 4 * q < nchunks ? reinterpret_cast<const f32x4_t*>(pe + cb)[q] : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (cb + 4 * q < nchunks) acc = (((acc + v[q].x) + v[q].y) + v[q].z) + v[q].w;
      }
    } else {
      for (int cb = 0; cb < nchunks; cb += 32) {
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = cb + i < nchunks ? pe[cb + i] : 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i)
          if (cb + i < nchunks) acc = acc + v[i];
      }
    }
    if (bias) acc = acc + bias[e];
    lg[e] = acc;
  }
}

}  // namespace moe
