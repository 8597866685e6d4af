// Exact top-K of each row of a logit matrix, by (value descending, index ascending), the way a
// sampler over a large vocabulary needs it ("Squeezing a 26B diffusion LLM onto a Mac", section
// "The optimizations that worked", hierarchical exact top-K): the row is cut into chunks, the K
// chunks with the largest maxima are kept, and the top K is taken among their entries only. A
// value of the global top K has fewer than K chunk maxima above it, so its chunk is kept; among
// chunks with equal maxima the lower one is kept first, since the tied entries it displaces come
// earlier in the order. The result is the exact top K, not an approximation.
//
// Two kernels:
//   k_chunk_max   streams the logits once (the HBM-bound part): one wave per chunk of C entries,
//                 16-byte loads, writing each chunk's largest order-preserving key.
//   k_topk_rows   one 1024-thread block per row: a radix select over the row's chunk keys picks
//                 K chunks; their K * C entries are loaded into LDS as keys and a second radix
//                 select picks the K entries; a rank count orders them. Only K / (V / C) of the
//                 row is read a second time.
// Radix select: four passes over 8-bit digits from the top, each a histogram of the entries that
// still match the chosen prefix (per-wave LDS histograms, then summed), which leaves the K-th
// largest key tau, how many entries lie above it, and how many equal it. When more entries equal
// tau than are still needed, the needed ones are those of lowest index, found by a radix select
// over the inverted indices of the tied entries.
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;

// Order-preserving key of a logit (larger logit, larger key; -0 and +0 equal; never 0 for a
// non-NaN value, so 0 marks an empty slot).
__device__ __forceinline__ uint32_t logit_key(float v) { return topk_key(v); }

// ---------------------------------------------------------------------------------------------
// cmax[r][c] = largest key of row r's entries [c * C, min(V, (c + 1) * C)). A wave takes one
// chunk; lane l takes entries 4l .. 4l + 3 of each 256-entry segment (VEC: one 16-byte load).
template <bool VEC>
__global__ __launch_bounds__(256) void k_chunk_max(int V, int C, int nch, const float* __restrict__ logits,
                                                   uint32_t* __restrict__ cmax) {
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int r = blockIdx.y;
  if (c >= nch) return;
  const float* row = logits + (size_t)r * V;
  const int base = c * C;
  uint32_t m = 0u;
  constexpr int kSegMax = 4;  // C <= 1024
  float4 v[kSegMax];
#pragma unroll
  for (int s = 0; s < kSegMax; ++s) {
    const int i = base + s * 256 + 4 * lane;
    if (VEC) {
      v[s] = (s * 256 < C && i < V) ? *reinterpret_cast<const float4*>(row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      const bool in = s * 256 < C;
      v[s].x = in && i < V ? row[i] : 0.f;
      v[s].y = in && i + 1 < V ? row[i + 1] : 0.f;
      v[s].z = in && i + 2 < V ? row[i + 2] : 0.f;
      v[s].w = in && i + 3 < V ? row[i + 3] : 0.f;
    }
  }
#pragma unroll
  for (int s = 0; s < kSegMax; ++s) {
    const int i = base + s * 256 + 4 * lane;
    if (s * 256 >= C) break;
    // entries past V (VEC: only whole float4s past V, since V % 4 == 0) do not count
    if (i < V) m = max(m, logit_key(v[s].x));
    if (i + 1 < V) m = max(m, logit_key(v[s].y));
    if (i + 2 < V) m = max(m, logit_key(v[s].z));
    if (i + 3 < V) m = max(m, logit_key(v[s].w));
  }
  m = wave_max_u32(m);
  if (lane == 0) cmax[(size_t)r * nch + c] = m;
}

// ---------------------------------------------------------------------------------------------
// Block-wide radix select among the participating entries i < n (part(i) true) by the 32-bit
// value val(i): the result is the K-th largest value tau, `above` = how many participating
// values exceed it, and `eq` = how many equal it. K must not exceed the number of participants.
struct Sel {
  uint32_t tau;
  int above, eq;
};

template <class Part, class Val>
__device__ __forceinline__ Sel radix_select(int n, int K, Part part, Val val, uint32_t* s_hist /* kTkWaves x 256 */,
                                            int* s_ctl /* 4 ints */) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint32_t prefix = 0u, mask = 0u;
  int rem = K;  // how many are still to be taken at or below the current prefix
  int eq = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < kTkWaves * 256; i += kTkThreads) s_hist[i] = 0u;
    __syncthreads();
    uint32_t* h = s_hist + wave * 256;
    for (int i = tid; i < n; i += kTkThreads)
      if (part(i)) {
        const uint32_t v = val(i);
        if ((v & mask) == prefix) atomicAdd(&h[(v >> shift) & 255u], 1u);
      }
    __syncthreads();
    // the per-wave histograms summed into wave 0's
    for (int b = tid; b < 256; b += kTkThreads) {
      uint32_t t = 0u;
      for (int w = 0; w < kTkWaves; ++w) t += s_hist[w * 256 + b];
      s_hist[b] = t;
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds digits 4l .. 4l + 3; find the digit where the count from the top reaches rem
      uint32_t hb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) hb[q] = s_hist[4 * lane + q];
      const int mine = (int)(hb[0] + hb[1] + hb[2] + hb[3]);
      int incl = mine;  // sum over lanes >= this one
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_down(incl, off, 64);
        if (lane + off < 64) incl += t;
      }
      const int excl = incl - mine;
      if (excl < rem && rem <= incl) {
        int cum = excl;
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          if (cum + (int)hb[q] >= rem) {
            s_ctl[0] = 4 * lane + q;
            s_ctl[1] = cum;  // participants above this digit
            s_ctl[2] = (int)hb[q];
            break;
          }
          cum += (int)hb[q];
        }
      }
    }
    __syncthreads();
    const uint32_t digit = (uint32_t)s_ctl[0];
    rem -= s_ctl[1];
    eq = s_ctl[2];
    prefix |= digit << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  Sel s;
  s.tau = prefix;
  s.above = K - rem;
  s.eq = eq;
  return s;
}

// Appends i to out[0 .. K) (slot from the counter s_ctl[3]; never past K).
__device__ __forceinline__ void append(int* out, int K, int* s_ctl, int i) {
  const int slot = atomicAdd(&s_ctl[3], 1);
  if (slot < K) out[slot] = i;
}

// Positions of the K selected participants (value desc, then lower index(i) first) appended to
// out[0 .. K) in no particular order.
template <class Part, class Val, class Idx>
__device__ __forceinline__ void select_k(int n, int K, Part part, Val val, Idx index, int* out, uint32_t* s_hist,
                                         int* s_ctl) {
  const int tid = threadIdx.x;
  const Sel s = radix_select(n, K, part, val, s_hist, s_ctl);
  const int need = K - s.above;  // entries equal to tau to take
  if (tid == 0) s_ctl[3] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kTkThreads)
    if (part(i) && val(i) > s.tau) append(out, K, s_ctl, i);
  if (s.eq == need) {
    for (int i = tid; i < n; i += kTkThreads)
      if (part(i) && val(i) == s.tau) append(out, K, s_ctl, i);
    __syncthreads();
    return;
  }
  __syncthreads();
  // ties at tau: the `need` tied entries of lowest index (indices are distinct, so the select
  // over inverted indices leaves no tie of its own)
  auto tied = [&](int i) { return part(i) && val(i) == s.tau; };
  auto inv = [&](int i) { return ~(uint32_t)index(i); };
  const Sel t = radix_select(n, need, tied, inv, s_hist, s_ctl);
  for (int i = tid; i < n; i += kTkThreads)
    if (tied(i) && inv(i) >= t.tau) append(out, K, s_ctl, i);
  __syncthreads();
}

// One block per row. LDS (static, about 146 KB of gfx950's 160 KB): the keys, first of the
// row's chunk maxima and then of the chosen chunks' entries (max(nch, K * C) <= kTkMaxKeys);
// the K chosen chunks; the K chosen positions; per-wave histograms; control words.
constexpr int kTkMaxKeys = 32768;
constexpr int kTkMaxK = 128;

__global__ __launch_bounds__(kTkThreads) void k_topk_rows(int V, int K, int C, int nch, const float* __restrict__ logits,
                                                          const uint32_t* __restrict__ cmax, int32_t* __restrict__ ids,
                                                          float* __restrict__ vals) {
  __shared__ uint32_t s_key[kTkMaxKeys];
  __shared__ int s_chunk[kTkMaxK];
  __shared__ int s_pos[kTkMaxK];
  __shared__ uint32_t s_hist[kTkWaves * 256];
  __shared__ int s_ctl[4];
  const int tid = threadIdx.x, r = blockIdx.x;
  const float* row = logits + (size_t)r * V;

  // 1. the K chunks with the largest maxima (lower chunk first on equal maxima); all of them
  //    when there are no more than K
  const int nsel = min(K, nch);
  for (int i = tid; i < nch; i += kTkThreads) s_key[i] = cmax[(size_t)r * nch + i];
  __syncthreads();
  if (nch <= K) {
    for (int i = tid; i < nch; i += kTkThreads) s_chunk[i] = i;
    __syncthreads();
  } else {
    auto all = [](int) { return true; };
    auto ck = [&](int i) { return s_key[i]; };
    auto cid = [](int i) { return i; };
    select_k(nch, K, all, ck, cid, s_chunk, s_hist, s_ctl);
  }
  // 2. their entries as keys: slot q holds chunk s_chunk[q]; entries past V are empty (key 0)
  const int ncand = nsel * C;
  for (int p = tid; p < ncand; p += kTkThreads) {
    const int q = p / C, o = p - q * C;
    const int i = min(max(s_chunk[q], 0), nch - 1) * C + o;
    s_key[p] = i < V ? logit_key(row[i]) : 0u;
  }
  __syncthreads();
  // 3. the K entries among them (empty slots never take part)
  auto live = [&](int p) { return s_key[p] != 0u; };
  auto key = [&](int p) { return s_key[p]; };
  auto idx = [&](int p) {
    const int q = p / C;
    return min(max(s_chunk[q], 0), nch - 1) * C + (p - q * C);
  };
  select_k(ncand, K, live, key, idx, s_pos, s_hist, s_ctl);
  // 4. order: rank of each chosen entry among the K by (key desc, index asc)
  // (positions and indices are clamped to their ranges, so a selection that went wrong could
  // only give wrong answers, never an access outside the buffers)
  auto pos = [&](int j) { return min(max(s_pos[j], 0), ncand - 1); };
  if (tid < K) {
    const int p = pos(tid);
    const uint32_t kp = s_key[p];
    const int ip = idx(p);
    int rank = 0;
    for (int j = 0; j < K; ++j) {
      const int pj = pos(j);
      const uint32_t kj = s_key[pj];
      const int ij = idx(pj);
      rank += (kj > kp || (kj == kp && ij < ip)) ? 1 : 0;
    }
    rank = min(rank, K - 1);
    ids[(size_t)r * K + rank] = ip;
    vals[(size_t)r * K + rank] = row[min(max(ip, 0), V - 1)];
  }
}

// ---------------------------------------------------------------------------------------------
hipError_t launch_vocab_topk(int R, int V, int K, const float* logits, uint32_t* cmax, int32_t* ids, float* vals,
                             hipStream_t stream) {
  const int C = vocab_chunk(K), nch = (V + C - 1) / C;
  static_assert(kVocabMaxK <= kTkMaxK && kVocabMaxK * 256 <= kTkMaxKeys && 1024 * 32 <= kTkMaxKeys,
                "K * C and the chunk count fit the LDS key buffer");
  const dim3 g1((nch + 3) / 4, R);
  const bool vec = (V % 4 == 0) && (reinterpret_cast<uintptr_t>(logits) % 16 == 0);
  if (vec)
    hipLaunchKernelGGL(k_chunk_max<true>, g1, dim3(256), 0, stream, V, C, nch, logits, cmax);
  else
    hipLaunchKernelGGL(k_chunk_max<false>, g1, dim3(256), 0, stream, V, C, nch, logits, cmax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_topk_rows, dim3(R), dim3(kTkThreads), 0, stream, V, K, C, nch, logits, cmax, ids, vals);
  return hipGetLastError();
}

}  // namespace moe
