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
//                 K chunks; their entries are read once more and reduced to sub-chunk maxima, a
//                 second select picks K sub-chunks, and a third picks the K entries among those
//                 sub-chunks' entries; a rank count orders them. Only K / (V / C) of the row is
//                 read a second time.
// Radix select: four passes over 8-bit digits from the top, each a histogram of the entries that
// still match the chosen prefix (per-wave LDS histograms that one wave then reads and sums in
// registers), which leaves the K-th
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

// Inclusive prefix sum over the wave's lanes: Hillis-Steele steps of 1, 2, 4, 8 lanes inside each
// row of 16 (DPP row shifts, zero from outside the row), then the earlier rows' totals.
template <int CTRL>
__device__ __forceinline__ int dpp_shr0(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ int wave_prefix_sum(int v) {
  v += dpp_shr0<0x111>(v);  // row_shr:1
  v += dpp_shr0<0x112>(v);  // row_shr:2
  v += dpp_shr0<0x114>(v);  // row_shr:4
  v += dpp_shr0<0x118>(v);  // row_shr:8
  const int t0 = __builtin_amdgcn_readlane(v, 15), t1 = __builtin_amdgcn_readlane(v, 31);
  const int t2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (int)(threadIdx.x & 63) >> 4;
  return v + (row == 0 ? 0 : row == 1 ? t0 : row == 2 ? t0 + t1 : t0 + t1 + t2);
}

template <class Part, class Val>
__device__ __forceinline__ Sel radix_select(int n, int K, Part part, Val val, uint32_t* s_hist /* kTkWaves x 256 */,
                                            int* s_ctl /* 4 ints */) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint32_t prefix = 0u, mask = 0u;
  int rem = K;  // how many are still to be taken at or below the current prefix
  int eq = 0;
  uint32_t* h = s_hist + wave * 256;
  for (int shift = 24; shift >= 0; shift -= 8) {
    // this wave's histogram: cleared and filled by the wave itself (a wave's LDS accesses
    // complete in order, so no barrier is needed between the two)
    *reinterpret_cast<uint4*>(h + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
    for (int i = tid; i < n; i += kTkThreads)
      if (part(i)) {
        const uint32_t v = val(i);
        if ((v & mask) == prefix) atomicAdd(&h[(v >> shift) & 255u], 1u);
      }
    __syncthreads();
    if (wave == 0) {
      // lane l sums digits 255 - 4l .. 252 - 4l (hb[0] the highest) over every wave's
      // histogram; a prefix sum over the lanes then counts from the top digit down, and the lane
      // holding the digit where that count reaches rem reports it
      const int hi = 252 - 4 * lane;
      uint32_t hb[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int w = 0; w < kTkWaves; ++w) {
        const uint4 t = *reinterpret_cast<const uint4*>(s_hist + w * 256 + hi);
        hb[0] += t.w;
        hb[1] += t.z;
        hb[2] += t.y;
        hb[3] += t.x;
      }
      const int mine = (int)(hb[0] + hb[1] + hb[2] + hb[3]);
      const int incl = wave_prefix_sum(mine);  // over lanes <= this one, i.e. digits >= hi
      const int excl = incl - mine;
      if (excl < rem && rem <= incl) {
        int cum = excl;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (cum + (int)hb[q] >= rem) {
            s_ctl[0] = hi + 3 - q;
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
  }
  __syncthreads();  // every thread has read s_ctl before anyone writes it again
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

// One block per row. A fast path (step 0 below) ranks the entries >= the K-th largest chunk
// maximum directly; when ties make those too many, three exact reductions in a row:
//   1. the K chunks with the largest maxima among the row's nch chunk maxima;
//   2. the chosen chunks' entries are read once (every wave issues all of its loads first) and
//      cut into sub-chunks of S = C / 64 consecutive entries, one per lane; the K sub-chunks with
//      the largest maxima are chosen among the K * 64 (the chunk argument again: the chosen
//      chunks hold the global top K, so the top K of their entries is the global top K);
//   3. the K entries among the K * S entries of the chosen sub-chunks, re-read from memory.
// Ties between equal maxima go to the lower range, ranges being ordered by their first entry.
// LDS: up to kTkMaxKeys keys, the chosen chunks, sub-chunks and entries, per-wave histograms.
constexpr int kTkMaxKeys = 8192;  // >= nch and >= K * 64
constexpr int kTkMaxK = 128;
constexpr int kTkMaxS = 16;       // C / 64 for C <= 1024
constexpr int kTkCap = 1024;      // candidates of the fast path (one per thread for the rank)

template <bool VEC>
__global__ __launch_bounds__(kTkThreads) void k_topk_rows(int V, int K, int C, int nch, const float* __restrict__ logits,
                                                          const uint32_t* __restrict__ cmax, int32_t* __restrict__ ids,
                                                          float* __restrict__ vals) {
  __shared__ uint32_t s_key[kTkMaxKeys];
  __shared__ uint32_t s_fin[kTkMaxK * kTkMaxS];  // keys of the chosen sub-chunks' entries
  __shared__ int s_chunk[kTkMaxK];
  __shared__ int s_sub[kTkMaxK];
  __shared__ int s_pos[kTkMaxK];
  __shared__ uint32_t s_hist[kTkWaves * 256];
  __shared__ int s_ctl[4];
  __shared__ uint32_t s_ck[kTkCap];  // fast path: candidate keys
  __shared__ int s_ci[kTkCap];       // ... and their indices
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = blockIdx.x;
  const float* row = logits + (size_t)r * V;
  const int S = C / 64;
  for (int i = tid; i < nch; i += kTkThreads) s_key[i] = cmax[(size_t)r * nch + i];
  __syncthreads();

  // 0. Fast path. tau1 = the K-th largest chunk maximum (0 when there are no more than K
  //    chunks). Those K maxima are K entries >= tau1, so every entry of the top K is >= tau1 and
  //    the entries >= tau1 (all in chunks whose maximum is >= tau1) hold the answer. When there
  //    are at most kTkMaxK such chunks and kTkCap such entries (the usual case; ties at the top
  //    of many chunks are not), they are gathered and ranked directly.
  {
    uint32_t tau1 = 0u;
    if (nch > K) {
      auto all = [](int) { return true; };
      auto ck = [&](int i) { return s_key[i]; };
      tau1 = radix_select(nch, K, all, ck, s_hist, s_ctl).tau;
    }
    if (tid == 0) s_ctl[3] = 0;
    __syncthreads();
    for (int i = tid; i < nch; i += kTkThreads)
      if (s_key[i] >= tau1) append(s_chunk, kTkMaxK, s_ctl, i);
    __syncthreads();
    const int nc = s_ctl[3];
    __syncthreads();
    if (nc <= kTkMaxK) {
      if (tid == 0) s_ctl[3] = 0;
      __syncthreads();
      for (int q0 = wave; q0 < nc; q0 += 4 * kTkWaves) {
        float v[4][kTkMaxS];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int q = q0 + u * kTkWaves;
          const int e0 = (q < nc ? min(max(s_chunk[q], 0), nch - 1) : 0) * C + lane * S;
#pragma unroll
          for (int j = 0; j < kTkMaxS; j += 4) {
            if (j >= S) break;
            if (VEC) {
              const float4 t =
                  e0 + j < V ? *reinterpret_cast<const float4*>(row + e0 + j) : make_float4(0.f, 0.f, 0.f, 0.f);
              v[u][j] = t.x;
              v[u][j + 1] = t.y;
              v[u][j + 2] = t.z;
              v[u][j + 3] = t.w;
            } else {
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) v[u][j + jj] = e0 + j + jj < V ? row[e0 + j + jj] : 0.f;
            }
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int q = q0 + u * kTkWaves;
          if (q >= nc) break;
          const int e0 = min(max(s_chunk[q], 0), nch - 1) * C + lane * S;
#pragma unroll
          for (int j = 0; j < kTkMaxS; ++j)
            if (j < S && e0 + j < V) {
              const uint32_t kk = logit_key(v[u][j]);
              if (kk >= tau1) {
                const int slot = atomicAdd(&s_ctl[3], 1);
                if (slot < kTkCap) {
                  s_ck[slot] = kk;
                  s_ci[slot] = e0 + j;
                }
              }
            }
        }
      }
      __syncthreads();
      const int M = s_ctl[3];
      if (M <= kTkCap) {
        // rank of each candidate by (key desc, index asc); the first K go out
        if (tid < M) {
          const uint32_t kp = s_ck[tid];
          const int ip = s_ci[tid];
          int rank = 0;
          for (int j = 0; j < M; ++j) {
            const uint32_t kj = s_ck[j];
            rank += (kj > kp || (kj == kp && s_ci[j] < ip)) ? 1 : 0;
          }
          if (rank < K) {
            ids[(size_t)r * K + rank] = ip;
            vals[(size_t)r * K + rank] = row[min(max(ip, 0), V - 1)];
          }
        }
        return;
      }
    }
    __syncthreads();  // the general path below starts from the chunk keys, still in s_key
  }

  // 1. chunks: all of them when there are no more than K
  const int nsel = min(K, nch);
  if (nch <= K) {
    for (int i = tid; i < nch; i += kTkThreads) s_chunk[i] = i;
    __syncthreads();
  } else {
    auto all = [](int) { return true; };
    auto ck = [&](int i) { return s_key[i]; };
    auto cid = [](int i) { return i; };
    select_k(nch, K, all, ck, cid, s_chunk, s_hist, s_ctl);
  }
  // 2. sub-chunk maxima of the chosen chunks: slot q's lane l covers entries
  //    chunk * C + l * S .. + S - 1; key 0 when the sub-chunk lies past V
  auto chunk_of = [&](int q) { return min(max(s_chunk[q], 0), nch - 1); };
  for (int q0 = wave; q0 < nsel; q0 += 4 * kTkWaves) {
    float v[4][kTkMaxS];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = q0 + u * kTkWaves;
      const int e0 = (q < nsel ? chunk_of(q) : 0) * C + lane * S;
#pragma unroll
      for (int j = 0; j < kTkMaxS; j += 4) {
        if (j >= S) break;
        if (VEC) {
          const float4 t = e0 + j < V ? *reinterpret_cast<const float4*>(row + e0 + j) : make_float4(0.f, 0.f, 0.f, 0.f);
          v[u][j] = t.x;
          v[u][j + 1] = t.y;
          v[u][j + 2] = t.z;
          v[u][j + 3] = t.w;
        } else {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) v[u][j + jj] = e0 + j + jj < V ? row[e0 + j + jj] : 0.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = q0 + u * kTkWaves;
      if (q >= nsel) break;
      const int e0 = chunk_of(q) * C + lane * S;
      uint32_t m = 0u;
#pragma unroll
      for (int j = 0; j < kTkMaxS; ++j)
        if (j < S && e0 + j < V) m = max(m, logit_key(v[u][j]));
      s_key[q * 64 + lane] = m;
    }
  }
  __syncthreads();
  const int nsub = nsel * 64;
  auto sub_first = [&](int i) { return chunk_of(i >> 6) * C + (i & 63) * S; };  // first entry of sub-chunk i
  // When every chunk was kept the live sub-chunks are 0 .. ceil(V / S) - 1, and there may be no
  // more than K of them: then all are kept. Otherwise K chosen chunks hold at least K live ones.
  const int nlive = nch <= K ? (V + S - 1) / S : nsub;
  const int nsubsel = min(K, nlive);
  if (nlive <= K) {
    for (int i = tid; i < nlive; i += kTkThreads) s_sub[i] = i;
    __syncthreads();
  } else {
    auto live = [&](int i) { return s_key[i] != 0u; };
    auto sk = [&](int i) { return s_key[i]; };
    select_k(nsub, K, live, sk, sub_first, s_sub, s_hist, s_ctl);
  }
  // 3. the chosen sub-chunks' entries (position p = slot * S + offset), and the K among them
  auto elem = [&](int p) {
    const int u = p / S;
    return sub_first(min(max(s_sub[u], 0), nsub - 1)) + (p - u * S);
  };
  const int nfin = nsubsel * S;
  for (int p = tid; p < nfin; p += kTkThreads) {
    const int i = elem(p);
    s_fin[p] = i < V ? logit_key(row[i]) : 0u;
  }
  __syncthreads();
  {
    auto live = [&](int p) { return s_fin[p] != 0u; };
    auto fk = [&](int p) { return s_fin[p]; };
    select_k(nfin, K, live, fk, elem, s_pos, s_hist, s_ctl);
  }
  // 4. order: rank of each chosen entry among the K by (key desc, index asc). Positions and
  //    indices are clamped to their ranges, so a selection gone wrong could give wrong answers
  //    but never an access outside the buffers.
  auto pos = [&](int j) { return min(max(s_pos[j], 0), nfin - 1); };
  if (tid < K) {
    const int p = pos(tid);
    const uint32_t kp = s_fin[p];
    const int ip = elem(p);
    int rank = 0;
    for (int j = 0; j < K; ++j) {
      const int pj = pos(j);
      const uint32_t kj = s_fin[pj];
      const int ij = elem(pj);
      rank += (kj > kp || (kj == kp && ij < ip)) ? 1 : 0;
    }
    rank = min(rank, K - 1);
    ids[(size_t)r * K + rank] = ip;
    vals[(size_t)r * K + rank] = row[min(max(ip, 0), V - 1)];
  }
}

// ---------------------------------------------------------------------------------------------
hipError_t launch_vocab_topk(int R, int V, int K, const float* logits, uint32_t* cmax, int32_t* ids, float* vals,
                             hipStream_t stream, int stage) {
  const int C = vocab_chunk(K), nch = (V + C - 1) / C;
  static_assert(kVocabMaxK <= kTkMaxK && kVocabMaxK * 64 <= kTkMaxKeys && kVocabMaxChunks <= kTkMaxKeys,
                "the chunk keys and the sub-chunk keys fit the LDS key buffer");
  const dim3 g1((nch + 3) / 4, R);
  const bool vec = (V % 4 == 0) && (reinterpret_cast<uintptr_t>(logits) % 16 == 0);
  if (stage != 1) {
    if (vec)
      hipLaunchKernelGGL(k_chunk_max<true>, g1, dim3(256), 0, stream, V, C, nch, logits, cmax);
    else
      hipLaunchKernelGGL(k_chunk_max<false>, g1, dim3(256), 0, stream, V, C, nch, logits, cmax);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || stage == 0) return e;
  }
  if (vec)
    hipLaunchKernelGGL(k_topk_rows<true>, dim3(R), dim3(kTkThreads), 0, stream, V, K, C, nch, logits, cmax, ids, vals);
  else
    hipLaunchKernelGGL(k_topk_rows<false>, dim3(R), dim3(kTkThreads), 0, stream, V, K, C, nch, logits, cmax, ids,
                       vals);
  return hipGetLastError();
}

}  // namespace moe
