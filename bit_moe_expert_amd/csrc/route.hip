// Router, top-k and routing metadata on the GPU (no host round trip).
//
// The method keeps histogram, prefix scan, scatter and block map inside one GPU submission
// ("Perplexity's Lily Beats MLX-LM on MacBook M5. Because It Only Runs One Model.", section
// "Prefill: keep routing on the GPU, dequantize in flight"); the router scores every expert
// and keeps the top k (same page, "Why Qwen3.6-35B-A3B is a weird workload").
//
// Logit order (fixed so the top-k choice is unique): the input dimension is cut into chunks of
// 64; a chunk partial is an fp32 fma chain over ascending inputs from +0; partials are added in
// ascending chunk order to a +0 accumulator; the bias is added last.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------------------------
// Top-k of T <= kGemvMaxT tokens for moe_route: block t adds token t's router chunk partials in
// chunk order and takes the top-k. (moe_forward_layer fuses this step into its gate/up kernel.)
__global__ __launch_bounds__(256) void k_decode_topk(int d, int E, int k, const float* __restrict__ parts,
                                                     const float* __restrict__ bias, int32_t* __restrict__ ids,
                                                     float* __restrict__ w) {
  __shared__ float s_lg[kMaxExperts];
  const int t = blockIdx.x, nchunks = d / kGroup;
  sum_chunk_partials(parts + (size_t)t * nchunks * E, bias, nchunks, E, s_lg);
  __syncthreads();
  if (threadIdx.x < 64) wave_topk_softmax(s_lg, E, k, ids + (size_t)t * k, w + (size_t)t * k);
}

hipError_t launch_decode_topk(const Ctx& c) {
  hipLaunchKernelGGL(k_decode_topk, dim3(c.T), dim3(256), 0, c.stream, c.d, c.E, c.k, c.router_parts, c.logit_bias,
                     c.r.topk_ids, c.r.topk_w);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Prefill (T >= 2) logits: a block owns TOK tokens x EB experts (EB = 64 or 32). The block
// stages the tokens' inputs in LDS as fp32 [token][input]; its 16 waves take the 64-input chunks
// w, w + 16, ...: a wave holds the chunk's 64 router values of its lanes' experts in registers and
// runs one fma chain per (token, expert) over ascending inputs (on the matrix cores, below), so each
// router value feeds TOK chains. With EB = 32 the two halves of a wave hold the same 32 experts for
// different tokens, so 8 tokens per block keep a whole wave busy. The chunk partials meet in LDS
// and one thread per (token, expert) adds them in chunk order, then the bias. 16384 / TOK inputs
// are staged per pass (64 KB in every case; larger d in passes). More tokens per block mean fewer
// router loads per fma but fewer blocks: the launch takes 16 tokens x 64 experts when that still
// gives 256 blocks, else 8 x 64 when that does, else 8 x 32 (small calls, where the block count is
// what matters: the same blocks as 4 x 64, each reading half the router bytes). The (token block,
// expert block) items are dealt to the 8 XCDs (block b runs on XCD b % 8) in contiguous ranges of
// expert-block-major order, so each XCD's L2 fetches the router columns of only the expert blocks
// it works on instead of the whole matrix.
// Loads run ahead of their use: a wave's first router values go out with the first inputs, each
// router value of the wave's next chunk is loaded into its register right after its last use in
// the current chunk, and the next pass's inputs are loaded into registers while the current pass
// computes. The arithmetic and its order are those of one chunk at a time.
constexpr int kRpWaves = 16;

template <int TOK, int EB>
__global__ __launch_bounds__(1024) void k_router_prefill(int T, int d, int E, const uint16_t* __restrict__ x,
                                                         const float* __restrict__ wr, const float* __restrict__ bias,
                                                         float* __restrict__ logits) {
  constexpr int kMaxD = 16384 / TOK;          // inputs staged per pass
  constexpr int kMaxChunks = kMaxD / kGroup;  // a multiple of kRpWaves
  constexpr int kNV = TOK * kMaxD / 1024;     // staged values per thread and pass
  constexpr int kTG = 256 / EB;               // tokens per MFMA: 4 (EB = 64) or 8 (EB = 32)
  constexpr int kNG = TOK / kTG;              // MFMAs per input
  static_assert((EB == 64 || EB == 32) && TOK % kTG == 0 && TOK <= 16 && kMaxChunks % kRpWaves == 0, "block shape");
  // [token][input], each row 16 bytes longer so the rows one MFMA operand read touches start in
  // different banks
  __shared__ __attribute__((aligned(16))) float s_x[TOK][kMaxD + 4];
  __shared__ float s_parts[kMaxChunks][TOK][EB];  // 64 KB (EB = 64) or 32 KB
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nbx = (T + TOK - 1) / TOK, total = nbx * ((E + EB - 1) / EB);
  const int per = (total + 7) / 8;  // items per XCD
  const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (item >= total) return;
  const int by = item / nbx, bx = item - by * nbx;  // expert block, token block
  const int t0 = bx * TOK;
  const int e = by * EB + (lane & (EB - 1));
  const int ec = e < E ? e : E - 1;  // experts past E compute a copy that is never stored
  // lane L's tokens: kTG g + tl + (L & 3) in the A operand of group g, and kTG g + tl + r in its
  // output register r (with EB = 32 the upper half of the wave takes the group's last 4 tokens)
  const int tl = 4 * (lane / EB);
  const int nchunks = d / kGroup;
  const int s_tok = tid / EB, s_e = by * EB + (tid & (EB - 1));  // sum phase: threads 0 .. TOK EB - 1
  // inputs p*64 .. p*64 + nin of the tokens into registers: value q of a thread is (token, input)
  // = divmod(tid + 1024 q, kMaxD), so consecutive threads load consecutive inputs of one token
  uint16_t v[kNV];
  const auto load_x = [&](int p) __attribute__((always_inline)) {
    const int nin = min(kMaxChunks, nchunks - p) * kGroup;
#pragma unroll
    for (int q = 0; q < kNV; ++q) {
      const int f = tid + 1024 * q, tk = f / kMaxD, i = f % kMaxD;
      const int ic = i < nin ? i : 0;
      const int t = min(t0 + tk, T - 1);
      v[q] = x[(size_t)t * d + (size_t)p * kGroup + ic];
    }
  };
  float wv[kGroup];  // router values of the wave's current chunk
  const auto wcol = [&](int c) __attribute__((always_inline)) { return wr + (size_t)c * kGroup * E + ec; };
  const auto load_w = [&](int c) __attribute__((always_inline)) {
    const float* wp = wcol(c);
#pragma unroll
    for (int i = 0; i < kGroup; ++i) wv[i] = wp[(size_t)i * E];
  };
  load_x(0);
  if (wave < nchunks) load_w(wave);
  float acc = 0.0f;
  for (int p = 0; p < nchunks; p += kMaxChunks) {
    const int npass = min(kMaxChunks, nchunks - p);
    const int nin = npass * kGroup;
#pragma unroll
    for (int q = 0; q < kNV; ++q) {
      const int f = tid + 1024 * q, tk = f / kMaxD, i = f % kMaxD;
      if (i < nin) s_x[tk][i] = bf16_to_f32(v[q]);
    }
    // (a barrier waits for all of the thread's loads, so the next pass's inputs go out after it)
    __syncthreads();
    if (p + kMaxChunks < nchunks) load_x(p + kMaxChunks);
    for (int cc = wave; cc < npass; cc += kRpWaves) {
      const int cn = p + cc + kRpWaves;  // the wave's next chunk (this pass or the next)
      const float* wn = wcol(min(cn, nchunks - 1));
      // The chains run on the matrix cores: v_mfma_f32_4x4x1_16b_f32 is 16 independent 4 x 4 outer
      // products with K = 1, and each of its outputs is one a * b + c rounded once, as fmaf (checked
      // bit for bit on gfx950 against fmaf chains, subnormal results and signed zeros included). Lane
      // L = 4 blk + j gives B = its expert's router value and A = the value of its A token; register
      // r of lane L then accumulates the lane's r-th output token for expert e. One MFMA per input
      // and group of kTG tokens replaces kTG fmas per expert, and the chain keeps its order:
      // ascending inputs from +0.
      f32x4_t pr[kNG];
#pragma unroll
      for (int g = 0; g < kNG; ++g) pr[g] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      // two copies of the chunk, with and without the next chunk's loads (a per-value condition
      // would keep both values of every register alive)
      const auto chunk = [&](auto refill) __attribute__((always_inline)) {
#pragma unroll
        for (int i4 = 0; i4 < kGroup / 4; ++i4) {
          float4 xa[kNG];  // inputs 4 i4 .. 4 i4 + 3 of the lane's A token of each group
#pragma unroll
          for (int g = 0; g < kNG; ++g)
            xa[g] = *reinterpret_cast<const float4*>(&s_x[kTG * g + tl + (lane & 3)][cc * kGroup + 4 * i4]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i = 4 * i4 + q;
#pragma unroll
            for (int g = 0; g < kNG; ++g) {
              const float xv = q == 0 ? xa[g].x : q == 1 ? xa[g].y : q == 2 ? xa[g].z : xa[g].w;
              pr[g] = __builtin_amdgcn_mfma_f32_4x4x1f32(xv, wv[i], pr[g], 0, 0, 0);
            }
            if constexpr (decltype(refill)::value) wv[i] = wn[(size_t)i * E];
          }
        }
      };
      if (cn < nchunks)
        chunk(std::true_type{});
      else
        chunk(std::false_type{});
#pragma unroll
      for (int g = 0; g < kNG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_parts[cc][kTG * g + tl + r][lane & (EB - 1)] = pr[g][r];
    }
    __syncthreads();
    if (tid < TOK * EB)
      for (int cc = 0; cc < npass; ++cc) acc = acc + s_parts[cc][s_tok][tid & (EB - 1)];
    __syncthreads();
  }
  if (tid < TOK * EB && t0 + s_tok < T && s_e < E) {
    float v = acc;
    if (bias) v = v + bias[s_e];
    logits[(size_t)(t0 + s_tok) * E + s_e] = v;
  }
}

hipError_t launch_router_prefill(const Ctx& c) {
  // one block per (token block, expert block) item, the grid rounded up to whole rounds of 8 XCDs
  const auto items = [&](int tok, int eb) { return ((c.T + tok - 1) / tok) * ((c.E + eb - 1) / eb); };
  const auto grid = [&](int tok, int eb) { return dim3((unsigned)(8 * ((items(tok, eb) + 7) / 8))); };
  if (items(16, 64) >= 256) {
    hipLaunchKernelGGL((k_router_prefill<16, 64>), grid(16, 64), dim3(1024), 0, c.stream, c.T, c.d, c.E, c.x,
                       c.w_router, c.logit_bias, c.logits);
  } else if (items(8, 64) >= 256) {
    hipLaunchKernelGGL((k_router_prefill<8, 64>), grid(8, 64), dim3(1024), 0, c.stream, c.T, c.d, c.E, c.x,
                       c.w_router, c.logit_bias, c.logits);
  } else {
    hipLaunchKernelGGL((k_router_prefill<8, 32>), grid(8, 32), dim3(1024), 0, c.stream, c.T, c.d, c.E, c.x,
                       c.w_router, c.logit_bias, c.logits);
  }
  return hipGetLastError();
}

// Top-k and gate weights of T tokens from their logits, one wave per token.
__global__ __launch_bounds__(256) void k_topk_prefill(int T, int E, int k, const float* __restrict__ logits,
                                                      int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ float s_lg[4][kMaxExperts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  for (int e = lane; e < E; e += 64) s_lg[wave][e] = logits[(size_t)t * E + e];
  __builtin_amdgcn_wave_barrier();
  wave_topk_softmax(s_lg[wave], E, k, ids + (size_t)t * k, w + (size_t)t * k);
}

hipError_t launch_topk_prefill(const Ctx& c) {
  hipLaunchKernelGGL(k_topk_prefill, dim3((c.T + 3) / 4), dim3(256), 0, c.stream, c.T, c.E, c.k, c.logits,
                     c.r.topk_ids, c.r.topk_w);
  return hipGetLastError();
}

// x in pair order for the grouped GEMM's A operand, with its group sums: each 16-byte chunk of 8
// inputs is rewritten as inputs 0, 4, 1, 5, 2, 6, 3, 7, the order of the weight pairs its matrix
// cores multiply (so the GEMM reads rows without re-pairing them for every column block), and
// sums[row][g] = the sum of the row's inputs 64 g .. 64 g + 63 in fp32, the factor of the bias
// term of group g: each chunk's 8 inputs in ascending order, then the 8 chunks of the group pairwise
// (chunks 2c and 2c + 1, then pairs of those, then the two halves) across the 8 lanes that hold
// them. Rows hold K inputs (a multiple of 64); thread i of `nthreads` takes chunks i, i + nthreads,
// ... of the whole [rows][K] array (nthreads a multiple of 64, so a group's chunks meet in one wave).
__device__ __forceinline__ void pair_groups(const uint4* __restrict__ x, uint4* __restrict__ xp, float* __restrict__ sums,
                                            int64_t nchunks, int64_t i, int64_t nthreads) {
  for (int64_t base = i & ~(int64_t)63; base < nchunks; base += nthreads, i += nthreads) {
    const bool ok = i < nchunks;
    const uint4 v = ok ? x[i] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t p[4];
    repair8(w, p);
    if (ok) xp[i] = make_uint4(p[0], p[1], p[2], p[3]);
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = (acc + bf16lo(w[q])) + bf16hi(w[q]);
    acc += dpp_f32<0xB1>(acc);    // chunks (2c, 2c + 1): lane i ^ 1
    acc += dpp_f32<0x4E>(acc);    // pairs of pairs: lane i ^ 2
    acc += __shfl_xor(acc, 4, 64);  // the two halves of each 8-lane group: lane i ^ 4
    if (ok && (i & 7) == 0) sums[i >> 3] = acc;
  }
}

constexpr int kPairBlocks = 256;  // blocks that pair x (beside the metadata blocks, or alone)

__global__ __launch_bounds__(256) void k_pair_rows(const uint4* __restrict__ x, uint4* __restrict__ xp,
                                                   float* __restrict__ sums, int64_t nchunks) {
  pair_groups(x, xp, sums, nchunks, (int64_t)blockIdx.x * 256 + threadIdx.x, (int64_t)gridDim.x * 256);
}

static int pair_blocks(int64_t nchunks, int threads) {
  return (int)std::min<int64_t>(kPairBlocks, (nchunks + threads - 1) / threads);
}

hipError_t launch_pair_rows(const uint16_t* src, uint16_t* dst, float* sums, int64_t nrows, int K,
                            hipStream_t stream) {
  const int64_t nchunks = nrows * (K / 8);
  if (nchunks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pair_rows, dim3(pair_blocks(nchunks, 256)), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst), sums, nchunks);
  return hipGetLastError();
}

hipError_t launch_pair_x(const Ctx& c) { return launch_pair_rows(c.x, c.xp, c.xsum, c.T, c.d, c.stream); }

// ---------------------------------------------------------------------------------------------
// Histogram, prefix scan, stable scatter and block map over several 1024-thread blocks.
// Block b ranks the pairs of its slice [b span, (b + 1) span):
//   - counts are LDS atomic adds, one per pair (exact integers, whatever the order of the adds);
//   - a block scan over experts gives offsets; the first row of expert e for wave w of block b is
//     offsets[e] + (pairs of e before the block) + (pairs of e in waves 0 .. w - 1 of the block);
//   - within a wave, the lanes holding the same expert find each other with one ballot per bit of
//     the expert id, and a lane's rank among its peers is the popcount of its lower peers, so the
//     rows of an expert follow pair order, i.e. ascending token.
// Two ways to get the pairs of each expert before a slice:
//   - up to kMetaSlicedFrom pairs, one launch: every block counts all T k pairs (and those before
//     its slice) itself, so no block waits for another; block 0 also writes counts, offsets and
//     the block map;
//   - beyond that, the repeated count would grow with the square of T k, so three launches: each
//     slice's histogram; per-expert exclusive prefixes of the histograms over the slices (in
//     place) and the counts; then, in every slice block, offsets from a block scan of the counts
//     and the ranks of its slice (block 0 also writes offsets and the block map).
// The block map: each non-empty group in ascending expert order cut into consecutive tiles of at
// most kTileRows rows, then the shared expert's T rows. Blocks past the metadata blocks of the
// (last) launch pair x for the grouped GEMM (they need nothing from the others).
constexpr int kMetaWaves = 16;
constexpr int kMetaSpan = 1024;  // pairs ranked per metadata block (single launch)
constexpr int kMetaBatch = 8;    // 64-pair batches whose ids a wave loads together when counting

__device__ __forceinline__ int block_excl_scan(int v, int* s_wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int t = lane < (int)(blockDim.x >> 6) ? s_wsum[lane] : 0;
    int ti = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(ti, o, 64);
      if (lane >= o) ti += n;
    }
    if (lane < (int)(blockDim.x >> 6)) s_wsum[lane] = ti - t;
    if (lane == 63) s_wsum[16] = ti;
  }
  __syncthreads();
  const int r = s_wsum[wave] + incl - v;
  *total = s_wsum[16];
  __syncthreads();
  return r;
}

// The lanes of the wave (valid ones only) holding the same expert id as this lane.
__device__ __forceinline__ uint64_t peer_mask(int e, bool valid, int nbits) {
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(valid && bit);
    peers &= bit ? bb : ~bb;
  }
  return valid ? peers : 0ull;
}

__device__ __forceinline__ int expert_bits(int E) { return E > 1 ? 32 - __clz(E - 1) : 0; }

// This wave's part of the slice [b_begin, b_end): pairs [w_begin, w_end), 64-aligned lengths.
__device__ __forceinline__ void wave_part(int b_begin, int b_end, int& w_begin, int& w_end) {
  const int span = b_end - b_begin;
  const int wspan = (((span + kMetaWaves - 1) / kMetaWaves) + 63) & ~63;
  w_begin = min(b_end, b_begin + (int)(threadIdx.x >> 6) * wspan);
  w_end = min(b_end, w_begin + wspan);
}

// Pairs of each expert in this wave's part, into s_tab[wave][.] (zeroed by the caller); the ids of
// kMetaBatch 64-pair batches are loaded before any is counted.
__device__ __forceinline__ void wave_counts(const int32_t* __restrict__ ids, int E, int w_begin, int w_end,
                                            int* s_row) {
  const int lane = threadIdx.x & 63;
  for (int base = w_begin; base < w_end; base += 64 * kMetaBatch) {
    int ev[kMetaBatch];
#pragma unroll
    for (int i = 0; i < kMetaBatch; ++i) {
      const int p = base + 64 * i + lane;
      ev[i] = p < w_end ? ids[p] : -1;
    }
#pragma unroll
    for (int i = 0; i < kMetaBatch; ++i)
      if ((unsigned)ev[i] < (unsigned)E) atomicAdd(&s_row[ev[i]], 1);
  }
}

// Thread e (< E) turns the per-wave counts of expert e into each wave's first row of e, from the
// slice's first row `first` of e.
__device__ __forceinline__ void wave_cursors(int E, int first, int (*s_tab)[kMaxExperts]) {
  const int tid = threadIdx.x;
  if (tid < E) {
    int run = first;
#pragma unroll
    for (int w2 = 0; w2 < kMetaWaves; ++w2) {
      const int c = s_tab[w2][tid];
      s_tab[w2][tid] = run;
      run += c;
    }
  }
}

// Stable ranks of this wave's part: a lane's row is the wave's cursor plus the number of its lower
// peers; the lowest peer then advances the cursor. The next batch's ids are loaded before the
// current batch is ranked. The token index comes from an fp32 reciprocal with a one-step
// correction (exact for p < 2^21).
__device__ __forceinline__ void wave_ranks(const int32_t* __restrict__ ids, int E, int k, int w_begin, int w_end,
                                           int* s_row, int32_t* __restrict__ sorted_token,
                                           int32_t* __restrict__ inv_pos) {
  const int lane = threadIdx.x & 63, nbits = expert_bits(E);
  const float inv_k = 1.0f / (float)k;
  int e_next = w_begin + lane < w_end ? ids[w_begin + lane] : -1;
  for (int base = w_begin; base < w_end; base += 64) {
    const int p = base + lane;
    const int e = e_next;
    e_next = p + 64 < w_end ? ids[p + 64] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    int tq = (int)((float)p * inv_k);
    const int r = p - tq * k;
    tq += r >= k ? 1 : (r < 0 ? -1 : 0);
    const uint64_t peers = peer_mask(e, valid, nbits);
    int pos = 0;
    if (valid) pos = s_row[e] + __popcll(peers & lanemask_lt());
    __builtin_amdgcn_wave_barrier();
    if (valid && (peers & lanemask_lt()) == 0) s_row[e] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      sorted_token[pos] = tq;
      inv_pos[p] = pos;
    }
  }
}

// counts (when given), offsets and the block map, by one block whose thread e (< E) holds
// cnt = counts[e] and off = offsets[e]; total = T k.
__device__ __forceinline__ void write_block_map(int T, int E, int P, int has_shared, int cnt, int off, int total,
                                                int* s_wsum, int32_t* __restrict__ counts,
                                                int32_t* __restrict__ offsets, int32_t* __restrict__ tiles,
                                                int32_t* __restrict__ n_tiles) {
  const int tid = threadIdx.x;
  if (tid < E) {
    if (counts) counts[tid] = cnt;
    offsets[tid] = off;
  }
  if (tid == 0) offsets[E] = total;
  const int nt = tid < E ? (cnt + kTileRows - 1) / kTileRows : 0;
  int n_routed = 0;
  const int tfirst = block_excl_scan(nt, s_wsum, &n_routed);
  for (int j = 0; j < nt; ++j) {
    int32_t* tl = tiles + 3 * (size_t)(tfirst + j);
    tl[0] = tid;
    tl[1] = off + j * kTileRows;
    tl[2] = min(kTileRows, cnt - j * kTileRows);
  }
  const int n_shared = has_shared ? (T + kTileRows - 1) / kTileRows : 0;
  for (int j = tid; j < n_shared; j += 1024) {
    int32_t* tl = tiles + 3 * (size_t)(n_routed + j);
    tl[0] = E;
    tl[1] = P + j * kTileRows;
    tl[2] = min(kTileRows, T - j * kTileRows);
  }
  if (tid == 0) *n_tiles = n_routed + n_shared;
}

__global__ __launch_bounds__(1024) void k_route_meta(int T, int E, int k, int has_shared, int n_meta,
                                                     const int32_t* __restrict__ ids, int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_token,
                                                     int32_t* __restrict__ inv_pos, int32_t* __restrict__ tiles,
                                                     int32_t* __restrict__ n_tiles, const uint4* __restrict__ x,
                                                     uint4* __restrict__ xp, float* __restrict__ xsum, int64_t nchunks) {
  __shared__ int s_all[kMaxExperts];                 // pairs of each expert
  __shared__ int s_before[kMaxExperts];              // pairs of each expert before this block's slice
  __shared__ int s_tab[kMetaWaves][kMaxExperts];     // per-wave counts of the slice, then cursors
  __shared__ int s_wsum[17];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if ((int)blockIdx.x >= n_meta) {
    pair_groups(x, xp, xsum, nchunks, (int64_t)(blockIdx.x - n_meta) * 1024 + tid,
                (int64_t)(gridDim.x - n_meta) * 1024);
    return;
  }
  const int P = T * k;
  const int b_begin = min(P, (int)blockIdx.x * kMetaSpan), b_end = min(P, b_begin + kMetaSpan);
  for (int e = tid; e < E; e += 1024) {
    s_all[e] = 0;
    s_before[e] = 0;
#pragma unroll
    for (int w2 = 0; w2 < kMetaWaves; ++w2) s_tab[w2][e] = 0;
  }
  __syncthreads();
  // 1. counts of all pairs and of the pairs before the slice (every block, every pair): a wave
  //    takes 64-pair batches wave, wave + 16, ... and loads kMetaBatch of them before counting any
  for (int base0 = wave * 64; base0 < P; base0 += 64 * kMetaWaves * kMetaBatch) {
    int ev[kMetaBatch];
#pragma unroll
    for (int i = 0; i < kMetaBatch; ++i) {
      const int p = base0 + 64 * kMetaWaves * i + lane;
      ev[i] = p < P ? ids[p] : -1;
    }
#pragma unroll
    for (int i = 0; i < kMetaBatch; ++i) {
      const int p = base0 + 64 * kMetaWaves * i + lane;
      const int e = ev[i];
      if ((unsigned)e < (unsigned)E) {
        atomicAdd(&s_all[e], 1);
        if (p < b_begin) atomicAdd(&s_before[e], 1);
      }
    }
  }
  // 2. per-wave counts of this block's slice
  int w_begin, w_end;
  wave_part(b_begin, b_end, w_begin, w_end);
  wave_counts(ids, E, w_begin, w_end, s_tab[wave]);
  __syncthreads();
  // 3. offsets, then each wave's first row in every group; block 0 writes the map
  const int cnt = tid < E ? s_all[tid] : 0;
  int total = 0;
  const int off = block_excl_scan(cnt, s_wsum, &total);
  wave_cursors(E, off + (tid < E ? s_before[tid] : 0), s_tab);
  if (blockIdx.x == 0) write_block_map(T, E, P, has_shared, cnt, off, total, s_wsum, counts, offsets, tiles, n_tiles);
  __syncthreads();
  // 4. stable ranks of the slice
  wave_ranks(ids, E, k, w_begin, w_end, s_tab[wave], sorted_token, inv_pos);
}

// Sliced metadata, launch 1: hist[s][e] = pairs of expert e in slice s.
__global__ __launch_bounds__(1024) void k_meta_hist(int P, int E, int span, const int32_t* __restrict__ ids,
                                                    int32_t* __restrict__ hist) {
  __shared__ int s_cnt[kMaxExperts];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) s_cnt[e] = 0;
  __syncthreads();
  const int b_begin = min(P, (int)blockIdx.x * span), b_end = min(P, b_begin + span);
  for (int p0 = b_begin; p0 < b_end; p0 += 1024 * kMetaBatch) {
    int ev[kMetaBatch];
#pragma unroll
    for (int i = 0; i < kMetaBatch; ++i) {
      const int p = p0 + 1024 * i + tid;
      ev[i] = p < b_end ? ids[p] : -1;
    }
#pragma unroll
    for (int i = 0; i < kMetaBatch; ++i)
      if ((unsigned)ev[i] < (unsigned)E) atomicAdd(&s_cnt[ev[i]], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 1024) hist[(size_t)blockIdx.x * E + e] = s_cnt[e];
}

// Sliced metadata, launch 2: block b takes experts 64 b .. 64 b + 63 (lane = expert); wave w takes
// the w-th run of kScanRun consecutive slices. hist[.][e] becomes its exclusive prefix over the
// slices and counts[e] the total.
constexpr int kScanRun = kMetaMaxSlices / kMetaWaves;
__global__ __launch_bounds__(1024) void k_meta_scan(int E, int n_slices, int32_t* __restrict__ hist,
                                                    int32_t* __restrict__ counts) {
  __shared__ int s_run[kMetaWaves][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = (int)blockIdx.x * 64 + lane, s0 = wave * kScanRun;
  int c[kScanRun], sum = 0;
#pragma unroll
  for (int i = 0; i < kScanRun; ++i) c[i] = (e < E && s0 + i < n_slices) ? hist[(size_t)(s0 + i) * E + e] : 0;
#pragma unroll
  for (int i = 0; i < kScanRun; ++i) sum += c[i];
  s_run[wave][lane] = sum;
  __syncthreads();
  int run = 0;
#pragma unroll
  for (int w2 = 0; w2 < kMetaWaves; ++w2) run += w2 < wave ? s_run[w2][lane] : 0;
  if (e < E) {
#pragma unroll
    for (int i = 0; i < kScanRun; ++i)
      if (s0 + i < n_slices) {
        hist[(size_t)(s0 + i) * E + e] = run;
        run += c[i];
      }
    if (wave == kMetaWaves - 1) counts[e] = run;
  }
}

// Sliced metadata, launch 3: every slice block scans counts into offsets (block 0 also writes
// offsets and the block map) and ranks its slice from offsets[e] + hist[b][e]. Blocks past the
// slices pair x for the grouped GEMM.
__global__ __launch_bounds__(1024) void k_meta_rank(int T, int E, int k, int has_shared, int span, int n_slices,
                                                    const int32_t* __restrict__ ids,
                                                    const int32_t* __restrict__ hist,
                                                    const int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_token,
                                                    int32_t* __restrict__ inv_pos, int32_t* __restrict__ tiles,
                                                    int32_t* __restrict__ n_tiles, const uint4* __restrict__ x,
                                                    uint4* __restrict__ xp, float* __restrict__ xsum, int64_t nchunks) {
  __shared__ int s_tab[kMetaWaves][kMaxExperts];
  __shared__ int s_wsum[17];
  const int tid = threadIdx.x, wave = tid >> 6;
  if ((int)blockIdx.x >= n_slices) {
    pair_groups(x, xp, xsum, nchunks, (int64_t)(blockIdx.x - n_slices) * 1024 + tid,
                (int64_t)(gridDim.x - n_slices) * 1024);
    return;
  }
  const int P = T * k;
  for (int e = tid; e < E; e += 1024) {
#pragma unroll
    for (int w2 = 0; w2 < kMetaWaves; ++w2) s_tab[w2][e] = 0;
  }
  const int cnt = tid < E ? counts[tid] : 0;
  const int before = tid < E ? hist[(size_t)blockIdx.x * E + tid] : 0;
  __syncthreads();
  const int b_begin = min(P, (int)blockIdx.x * span), b_end = min(P, b_begin + span);
  int w_begin, w_end;
  wave_part(b_begin, b_end, w_begin, w_end);
  wave_counts(ids, E, w_begin, w_end, s_tab[wave]);
  int total = 0;
  const int off = block_excl_scan(cnt, s_wsum, &total);  // its barriers also end the counting
  wave_cursors(E, off + before, s_tab);
  if (blockIdx.x == 0) write_block_map(T, E, P, has_shared, cnt, off, total, s_wsum, nullptr, offsets, tiles, n_tiles);
  __syncthreads();
  wave_ranks(ids, E, k, w_begin, w_end, s_tab[wave], sorted_token, inv_pos);
}

hipError_t launch_route_meta(const Ctx& c) {
  const int64_t nchunks = c.pair_in_meta ? (int64_t)c.T * c.d / 8 : 0;
  const int pair = nchunks ? pair_blocks(nchunks, 1024) : 0;
  const int has_shared = c.Is > 0 ? 1 : 0;
  const uint4* x = reinterpret_cast<const uint4*>(c.x);
  uint4* xp = reinterpret_cast<uint4*>(c.xp);
  if (!meta_sliced(c.P)) {
    const int n_meta = std::max(1, (c.P + kMetaSpan - 1) / kMetaSpan);
    hipLaunchKernelGGL(k_route_meta, dim3(n_meta + pair), dim3(1024), 0, c.stream, c.T, c.E, c.k, has_shared, n_meta,
                       c.r.topk_ids, c.r.counts, c.r.offsets, c.r.sorted_token, c.r.inv_pos, c.r.tiles, c.r.n_tiles, x,
                       xp, c.xsum, nchunks);
    return hipGetLastError();
  }
  const int span = meta_slice_span(c.P), n_slices = meta_slices(c.P);
  hipLaunchKernelGGL(k_meta_hist, dim3(n_slices), dim3(1024), 0, c.stream, c.P, c.E, span, c.r.topk_ids, c.meta_hist);
  hipLaunchKernelGGL(k_meta_scan, dim3((c.E + 63) / 64), dim3(1024), 0, c.stream, c.E, n_slices, c.meta_hist,
                     c.r.counts);
  hipLaunchKernelGGL(k_meta_rank, dim3(n_slices + pair), dim3(1024), 0, c.stream, c.T, c.E, c.k, has_shared, span,
                     n_slices, c.r.topk_ids, c.meta_hist, c.r.counts, c.r.offsets, c.r.sorted_token, c.r.inv_pos,
                     c.r.tiles, c.r.n_tiles, x, xp, c.xsum, nchunks);
  return hipGetLastError();
}

}  // namespace moe
