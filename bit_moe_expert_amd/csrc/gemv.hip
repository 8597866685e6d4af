// Decode and other small calls (T <= kGemvMaxT tokens): bandwidth-bound GEMV over each token's
// k selected experts plus the shared expert, on the vector ALUs, with 128-bit loads of the
// 4-bit codes. A wave works for one token; an expert chosen by several tokens is read once per
// token (the repeats mostly hit L2), so no grouping step is needed.
//
// Decode has no weight reuse, so the aim is to move as few bytes per token as possible and to
// keep the arithmetic below the memory time ("Perplexity's Lily Beats MLX-LM on MacBook M5.
// Because It Only Runs One Model.", sections "Prefill and decode are different problems" and
// "What didn't work"). Two fusions follow the same page's "Decode: minimize bytes per token":
// the expert input projections with the gate activation (k_gemv_gateup), and the expert output
// projection with the routing scores and the shared expert (k_gemv_down_combine).
//
// Arithmetic: per 32-input segment with one scale s and bias b,
//   sum_i x_i (s q_i + b) = s * sum_i x_i (128 + q_i) + (b - 128 s) * sum_i x_i,
// where "128 + q" is built as a bf16 value straight from the code bits (one and-or per pair)
// and the inner sum runs on v_dot2_f32_bf16. No weight is rounded to bf16 on this path.
//
// Latency discipline: the kernels are a few microseconds long, so every index that is the same
// across a wave is made scalar (readfirstlane), kernel arguments are plain pointers selected by
// scalar conditions, and all loads of a wave are issued before its first arithmetic use.
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kGvWaves = 4;  // waves per block
constexpr int kGvRows = 4;   // h entries (each = one gate row + one up row) per wave

// Segment of 32 consecutive inputs as 16 re-paired bf16 dwords (seg_pairs order) + their sum.
struct Seg32 {
  uint32_t p[16];
  float sum;
};

template <int BITS>
__device__ __forceinline__ void make_seg(const uint32_t* v16, Seg32& s) {
  if (BITS == 4) {
#pragma unroll
    for (int m = 0; m < 4; ++m) repair8(v16 + 4 * m, s.p + 4 * m);
  } else {
    // pair 8h + i = inputs (16h + i, 16h + i + 8), as seg_pairs<3> and seg_pairs<2> lay out codes
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        s.p[8 * h + i] = __builtin_amdgcn_perm(v16[8 * h + 4 + i / 2], v16[8 * h + i / 2], i % 2 ? 0x07060302u : 0x05040100u);
  }
  float acc = 0.0f;
#pragma unroll
  for (int m = 0; m < 16; ++m) acc = dot2_bf16(v16[m], 0x3F803F80u, acc);  // (1.0, 1.0)
  s.sum = acc;
}

// sum over the segment of act * (128 + q), from the segment's raw code words.
template <int BITS>
__device__ __forceinline__ float seg_dot(const uint4& cw, const Seg32& a) {
  uint32_t q[16];
  seg_pairs<BITS>(cw, q);
  float acc = 0.0f;
#pragma unroll
  for (int n = 0; n < 16; ++n) acc = dot2_bf16(q[n], a.p[n], acc);
  return acc;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Stop the compiler from sinking the loads above below this point.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }
// ... and from hoisting any arithmetic above it either: every load above is issued before the
// first instruction below (the scheduler may otherwise interleave them to save registers).
__device__ __forceinline__ void issue_all() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

struct GemvPtrs {
  const uint8_t *gc, *uc, *dc;       // routed gate/up/down codes
  const uint16_t *gs, *gb, *us, *ub, *ds, *db;
  const uint8_t *sgc, *suc, *sdc;    // shared expert
  const uint16_t *sgs, *sgb, *sus, *sub, *sds, *sdb;
};

static GemvPtrs gemv_ptrs(const Ctx& c) {
  GemvPtrs p;
  p.gc = c.routed.gate.codes;
  p.gs = c.routed.gate.scales;
  p.gb = c.routed.gate.biases;
  p.uc = c.routed.up.codes;
  p.us = c.routed.up.scales;
  p.ub = c.routed.up.biases;
  p.dc = c.routed.down.codes;
  p.ds = c.routed.down.scales;
  p.db = c.routed.down.biases;
  p.sgc = c.shared.gate.codes;
  p.sgs = c.shared.gate.scales;
  p.sgb = c.shared.gate.biases;
  p.suc = c.shared.up.codes;
  p.sus = c.shared.up.scales;
  p.sub = c.shared.up.biases;
  p.sdc = c.shared.down.codes;
  p.sds = c.shared.down.scales;
  p.sdb = c.shared.down.biases;
  return p;
}

// ---------------------------------------------------------------------------------------------
// One wave computes h[i0 .. i0 + kGvRows) = bf16(silu(x . Wg[row]) * (x . Wu[row])) for the
// weight rows row0 .. row0 + kGvRows of one expert's gate and up matrices; lane l takes the
// 16-byte code pieces l, l+64, ... of each row.
template <int BITS>
__device__ __forceinline__ void gateup_wave(int d, size_t row0, const uint8_t* gc, const uint16_t* gs,
                                            const uint16_t* gb, const uint8_t* uc, const uint16_t* us,
                                            const uint16_t* ub, const uint16_t* __restrict__ x, uint16_t* hout) {
  const int lane = threadIdx.x & 63;
  const int nseg = d / 32;
  const size_t cstride = (size_t)d * BITS / 8, sstride = (size_t)d / kGroup;
  float acc[2 * kGvRows];
#pragma unroll
  for (int r = 0; r < 2 * kGvRows; ++r) acc[r] = 0.0f;
  for (int seg = lane; seg < nseg; seg += 64) {
    uint4 cw[2 * kGvRows];
    uint16_t sr[2 * kGvRows], br[2 * kGvRows];
#pragma unroll
    for (int r = 0; r < 2 * kGvRows; ++r) {
      const size_t row = row0 + (r % kGvRows);
      const uint8_t* cp = r < kGvRows ? gc : uc;
      cw[r] = load_code_words<BITS>(cp + row * cstride + (size_t)seg * 4 * BITS);
    }
#pragma unroll
    for (int r = 0; r < 2 * kGvRows; ++r) {
      const size_t row = row0 + (r % kGvRows);
      sr[r] = (r < kGvRows ? gs : us)[row * sstride + seg / 2];
      br[r] = (r < kGvRows ? gb : ub)[row * sstride + seg / 2];
    }
    uint32_t xv[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 t = reinterpret_cast<const uint4*>(x + (size_t)seg * 32)[q];
      xv[4 * q] = t.x;
      xv[4 * q + 1] = t.y;
      xv[4 * q + 2] = t.z;
      xv[4 * q + 3] = t.w;
    }
    issue_fence();
    Seg32 a;
    make_seg<BITS>(xv, a);
#pragma unroll
    for (int r = 0; r < 2 * kGvRows; ++r) {
      const float s = bf16_to_f32(sr[r]), b = bf16_to_f32(br[r]);
      const float pd = seg_dot<BITS>(cw[r], a);
      acc[r] = fmaf(s, pd, acc[r]);
      acc[r] = fmaf(fmaf(-128.0f, s, b), a.sum, acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < 2 * kGvRows; ++r) acc[r] = wave_sum(acc[r]);
  if (lane < kGvRows / 2) {
    // lane q writes h entries 2q, 2q + 1 (acc is the same in every lane after the sums)
    float hv[kGvRows];
#pragma unroll
    for (int r = 0; r < kGvRows; ++r) hv[r] = silu_mul(acc[r], acc[kGvRows + r]);
    float a0 = hv[0], a1 = hv[1];
#pragma unroll
    for (int q = 1; q < kGvRows / 2; ++q)
      if (lane == q) {
        a0 = hv[2 * q];
        a1 = hv[2 * q + 1];
      }
    reinterpret_cast<uint32_t*>(hout)[lane] = pack_bf16x2(a0, a1);
  }
}

// ---------------------------------------------------------------------------------------------
// Router of T <= kGemvMaxT tokens: chunk partials of the logits (see route.hip for the fixed
// order), stored [T][E][d/64]. A block holds one (chunk, 64 experts) item: wave w loads the
// chunk's router values once, then takes tokens (w, w + kGvWaves), (w + 2 kGvWaves, ...), ...
// in pairs: each pair's inputs are loaded before the first use and the two tokens' fma chains
// run interleaved (lane = expert).
__global__ __launch_bounds__(kGvWaves * 64) void k_router_decode(int d, int E, int T, const uint16_t* __restrict__ x,
                                                                 const float* __restrict__ wr,
                                                                 float* __restrict__ parts) {
  const int wave = uniform(threadIdx.x >> 6);
  const int nchunks = d / kGroup;
  const int item = blockIdx.x;
  const int c = item % nchunks;
  const int e = (item / nchunks) * 64 + (threadIdx.x & 63);
  if (wave >= T || e >= E) return;
  const float* wp = wr + (size_t)c * kGroup * E + e;
  float v[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup; ++i) v[i] = wp[(size_t)i * E];
  for (int ta = wave; ta < T; ta += 2 * kGvWaves) {
    const int tb = ta + kGvWaves;
    const int tb2 = tb < T ? tb : ta;  // without a second token the second chain repeats the first
    // the chunk's 64 inputs of both tokens (8 x 16 bytes each), all in flight with the weights;
    // a zero the compiler cannot see through keeps them vector loads (scalar loads return out
    // of order, so their uses would wait for all of them at once, in several rounds)
    int vz;
    asm volatile("v_mov_b32 %0, 0" : "=v"(vz));
    const uint4* xa = reinterpret_cast<const uint4*>(x + (size_t)ta * d + c * kGroup) + vz;
    const uint4* xb = reinterpret_cast<const uint4*>(x + (size_t)tb2 * d + c * kGroup) + vz;
    uint4 ua[kGroup / 8], ub[kGroup / 8];
#pragma unroll
    for (int q = 0; q < kGroup / 8; ++q) {
      ua[q] = xa[q];
      ub[q] = xb[q];
    }
    issue_all();
    // two independent chains, each over ascending inputs from +0
    float pa = 0.0f, pb = 0.0f;
#pragma unroll
    for (int q = 0; q < kGroup / 8; ++q) {
      const uint32_t wa[4] = {ua[q].x, ua[q].y, ua[q].z, ua[q].w};
      const uint32_t wb[4] = {ub[q].x, ub[q].y, ub[q].z, ub[q].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        pa = fmaf(bf16lo(wa[m]), v[8 * q + 2 * m], pa);
        pb = fmaf(bf16lo(wb[m]), v[8 * q + 2 * m], pb);
        pa = fmaf(bf16hi(wa[m]), v[8 * q + 2 * m + 1], pa);
        pb = fmaf(bf16hi(wb[m]), v[8 * q + 2 * m + 1], pb);
      }
    }
    parts[((size_t)ta * E + e) * nchunks + c] = pa;
    parts[((size_t)tb2 * E + e) * nchunks + c] = pb;  // same value as pa when tb2 == ta
  }
}

hipError_t launch_router_decode(const Ctx& c) {
  const int n_part = (c.d / kGroup) * ((c.E + 63) / 64);  // one (chunk, 64 experts) item per block
  hipLaunchKernelGGL(k_router_decode, dim3(n_part), dim3(kGvWaves * 64), 0, c.stream, c.d, c.E, c.T, c.x, c.w_router,
                     c.router_parts);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Pipelined variant of gateup_wave for d <= 2048 (one 32-input segment per lane, lanes past the
// segments idle): the caller holds the lane's x segment (re-paired once per token) and passes
// the loads of the next rows while these rows are computed.
struct GuLoads {
  uint4 cw[2 * kGvRows];      // gate rows, then up rows: the segment's code words each
  uint32_t sb[2 * kGvRows];   // scale | bias << 16 of the segment's group
};

struct GuRows {
  const uint8_t *gc, *uc;
  const uint16_t *gs, *gb, *us, *ub;
  size_t row0;
  uint16_t* hout;
};

template <int BITS>
__device__ __forceinline__ void gu_load(const GuRows& g, int d, int seg, GuLoads& L) {
  const size_t cstride = (size_t)d * BITS / 8, sstride = (size_t)d / kGroup;
#pragma unroll
  for (int r = 0; r < 2 * kGvRows; ++r) {
    const size_t row = g.row0 + (r % kGvRows);
    L.cw[r] = load_code_words<BITS>((r < kGvRows ? g.gc : g.uc) + row * cstride + (size_t)seg * 4 * BITS);
  }
#pragma unroll
  for (int r = 0; r < 2 * kGvRows; ++r) {
    const size_t row = g.row0 + (r % kGvRows);
    L.sb[r] = (uint32_t)(r < kGvRows ? g.gs : g.us)[row * sstride + seg / 2] |
              ((uint32_t)(r < kGvRows ? g.gb : g.ub)[row * sstride + seg / 2] << 16);
  }
}

template <int BITS>
__device__ __forceinline__ void gu_finish(const GuLoads& L, const Seg32& a, bool active, uint16_t* hout) {
  const int lane = threadIdx.x & 63;
  float acc[2 * kGvRows];
#pragma unroll
  for (int r = 0; r < 2 * kGvRows; ++r) {
    const float s = bf16lo(L.sb[r]), b = bf16hi(L.sb[r]);
    const float pd = seg_dot<BITS>(L.cw[r], a);
    // the same operations, in the same order, as one segment of gateup_wave
    const float v = fmaf(fmaf(-128.0f, s, b), a.sum, fmaf(s, pd, 0.0f));
    acc[r] = active ? v : 0.0f;
  }
#pragma unroll
  for (int r = 0; r < 2 * kGvRows; ++r) acc[r] = wave_sum(acc[r]);
  if (lane < kGvRows / 2) {
    float hv[kGvRows];
#pragma unroll
    for (int r = 0; r < kGvRows; ++r) hv[r] = silu_mul(acc[r], acc[kGvRows + r]);
    float a0 = hv[0], a1 = hv[1];
#pragma unroll
    for (int q = 1; q < kGvRows / 2; ++q)
      if (lane == q) {
        a0 = hv[2 * q];
        a1 = hv[2 * q + 1];
      }
    reinterpret_cast<uint32_t*>(hout)[lane] = pack_bf16x2(a0, a1);
  }
}

// h[t][j][i] for token t's k routed slots (e_j = topk_ids[t][j]) and, if include_shared, its
// shared slot. Blocks are laid out token by token.
// FUSED_TOPK: every block first sums its token's router chunk partials (in chunk order) and
// takes the top-k itself, so no kernel boundary or atomic sits between the router and the
// experts' reads; all blocks of a token reach bit-identical choices, and the token's first
// block publishes them for the down kernel. The launch starts with n_sh blocks of the shared
// expert's rows (n_sh / T per token), which need no routing and start loading at once, while
// the routed blocks take the top-k.
template <bool FUSED_TOPK, int BITS>
__global__ __launch_bounds__(kGvWaves * 64) void k_gemv_gateup(int d, int E, int k, int I, int Is, int include_shared,
                                                               int groups_per_token, int reps, int sh_bpt, int n_tok,
                                                               const uint16_t* __restrict__ x,
                                                               const float* __restrict__ parts,
                                                               const float* __restrict__ bias, int32_t* __restrict__ ids,
                                                               float* __restrict__ wts, GemvPtrs p,
                                                               uint16_t* __restrict__ h, uint16_t* __restrict__ hs) {
  __shared__ int s_ids[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  __shared__ float s_lg[FUSED_TOPK ? kMaxExperts : 1];
  const int wave = threadIdx.x >> 6;
  const int n_sh = FUSED_TOPK ? sh_bpt * n_tok : 0;
  if ((int)blockIdx.x < n_sh) {  // shared expert rows: kGvRows per wave
    const int t = uniform(blockIdx.x / sh_bpt), sb = uniform(blockIdx.x - t * sh_bpt);
    const int r0 = uniform((sb * kGvWaves + wave) * kGvRows);
    if (r0 >= Is) return;
    gateup_wave<BITS>(d, (size_t)r0, p.sgc, p.sgs, p.sgb, p.suc, p.sus, p.sub, x + (size_t)t * d, hs + (size_t)t * Is + r0);
    return;
  }
  const int bid = (int)blockIdx.x - (FUSED_TOPK ? n_sh : 0);
  const int bpt = (groups_per_token + reps - 1) / reps;  // blocks per token
  const int t = uniform(bid / bpt), tb0 = uniform(bid - t * bpt);
  if (FUSED_TOPK) {
    const int nchunks = d / kGroup;
    sum_chunk_partials(parts + (size_t)t * nchunks * E, bias, nchunks, E, s_lg);
    __syncthreads();
    if (threadIdx.x < 64) wave_topk_softmax(s_lg, E, k, s_ids, s_w);
    __syncthreads();
    if (tb0 == 0 && (int)threadIdx.x < k) {
      ids[(size_t)t * k + threadIdx.x] = s_ids[threadIdx.x];
      wts[(size_t)t * k + threadIdx.x] = s_w[threadIdx.x];
    }
  }
  const int total = k * I + (include_shared ? Is : 0);
  // rows of pass `rep` of this wave; false past the end
  auto rows_of = [&](int rep, GuRows& g) -> bool {
    const int tb = tb0 * reps + rep;  // this pass's group of kGvWaves * kGvRows rows
    const int r0 = uniform((tb * kGvWaves + wave) * kGvRows);
    if (rep >= reps || r0 >= total) return false;
    const bool routed = r0 < k * I;
    const int j = routed ? r0 / I : k;
    const int i0 = routed ? r0 - j * I : r0 - k * I;
    int mat = 0;
    if (routed) {
      mat = FUSED_TOPK ? s_ids[j] : ids[(size_t)t * k + j];
      if ((unsigned)mat >= (unsigned)E) mat = 0;  // a corrupt routing must not read out of bounds
    }
    g.gc = routed ? p.gc : p.sgc;
    g.uc = routed ? p.uc : p.suc;
    g.gs = routed ? p.gs : p.sgs;
    g.gb = routed ? p.gb : p.sgb;
    g.us = routed ? p.us : p.sus;
    g.ub = routed ? p.ub : p.sub;
    g.row0 = (size_t)mat * (routed ? I : Is) + i0;
    g.hout = routed ? h + ((size_t)t * k + j) * I + i0 : hs + (size_t)t * Is + i0;
    return true;
  };
  if (d > 64 * 32) {  // several segments per lane: one pass at a time
    for (int rep = 0; rep < reps; ++rep) {
      GuRows g;
      if (!rows_of(rep, g)) break;
      gateup_wave<BITS>(d, g.row0, g.gc, g.gs, g.gb, g.uc, g.us, g.ub, x + (size_t)t * d, g.hout);
    }
    return;
  }
  const int lane = threadIdx.x & 63;
  const bool active = lane < d / 32;
  const int seg = active ? lane : 0;
  GuRows g;
  if (!rows_of(0, g)) return;
  GuLoads cur;
  gu_load<BITS>(g, d, seg, cur);
  uint32_t xv[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = reinterpret_cast<const uint4*>(x + (size_t)t * d + (size_t)seg * 32)[q];
    xv[4 * q] = v.x;
    xv[4 * q + 1] = v.y;
    xv[4 * q + 2] = v.z;
    xv[4 * q + 3] = v.w;
  }
  issue_fence();
  Seg32 a;
  make_seg<BITS>(xv, a);
  for (int rep = 0;; ++rep) {
    GuRows gn;
    const bool more = rows_of(rep + 1, gn);
    GuLoads nxt;
    if (more) gu_load<BITS>(gn, d, seg, nxt);
    issue_fence();
    gu_finish<BITS>(cur, a, active, g.hout);
    if (!more) break;
    cur = nxt;
    g = gn;
  }
}

// Blocks take reps consecutive row groups of one token, so that a call keeps about 512 blocks
// whatever T, all resident at once: the top-k prologue is paid once per block rather than in
// several rounds of blocks, and a wave's next rows load while its current rows are computed.
hipError_t launch_gemv_gateup(const Ctx& c, bool fused_topk) {
  const int include_shared = fused_topk ? 0 : (c.Is > 0 ? 1 : 0);
  const int waves = (c.k * c.I + (include_shared ? c.Is : 0)) / kGvRows;
  const int groups = (waves + kGvWaves - 1) / kGvWaves;  // row groups per token
  const int reps = (groups * c.T + 511) / 512;
  // the fused launch also computes the shared expert's h (its own leading blocks)
  const bool with_shared = fused_topk && c.Is > 0 && c.shared.gate.codes != nullptr;
  const int sh_bpt = with_shared ? (c.Is / kGvRows + kGvWaves - 1) / kGvWaves : 0;
  const dim3 grid(((groups + reps - 1) / reps) * c.T + (fused_topk ? sh_bpt * c.T : 0));
  const auto go = [&](auto kernel, int shb) {
    hipLaunchKernelGGL(kernel, grid, dim3(kGvWaves * 64), 0, c.stream, c.d, c.E, c.k, c.I, c.Is, include_shared,
                       groups, reps, shb, c.T, c.x, c.router_parts, c.logit_bias, c.r.topk_ids, c.r.topk_w, gemv_ptrs(c),
                       c.h, c.hs);
  };
  if (fused_topk) {
    if (c.bits == 3)
      go(k_gemv_gateup<true, 3>, sh_bpt);
    else if (c.bits == 2)
      go(k_gemv_gateup<true, 2>, sh_bpt);
    else
      go(k_gemv_gateup<true, 4>, sh_bpt);
  } else {
    if (c.bits == 3)
      go(k_gemv_gateup<false, 3>, 0);
    else if (c.bits == 2)
      go(k_gemv_gateup<false, 2>, 0);
    else
      go(k_gemv_gateup<false, 4>, 0);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// y[t][o] = bf16( sum_j w_tj * (h_tj . Wd[e_tj][o]) + h_ts . Wd_s[o] ), token t = blockIdx.y.
// A block keeps every slot's h in LDS (re-paired) with per-segment sums. Slots v = 0 .. k-1 are
// the routed ones, v = k the shared expert. An output takes HALVES groups of 16 lanes (a wave
// owns 4 / HALVES outputs); with two, the halves take alternate slots (half 0: v = 0, 2, 4, ...;
// half 1: v = 1, 3, ...). At each of its slots a lane takes 16-byte pieces l16, l16 + 16, ... of
// row o of that slot's expert. A lane's slots are taken in batches of 9 / HALVES (rounded up)
// whose loads are all in flight together. Each 16-lane group is reduced with DPP, then the
// halves are added: no atomics. Two halves keep every SIMD busy for a single token; for more
// tokens one group per output does less redundant staging per output.
constexpr int kGdWaves = 4;  // waves per block

template <int PIECES, int HALVES, int BITS>  // PIECES: 16-lane rounds of 32-input pieces per row: I, Is <= 512 * PIECES
__global__ __launch_bounds__(kGdWaves * 64) void k_gemv_down_combine(int d, int E, int k, int I, int Is,
                                                                     const int32_t* __restrict__ ids,
                                                                     const float* __restrict__ wts, GemvPtrs p,
                                                                     const uint16_t* __restrict__ h,
                                                                     const uint16_t* __restrict__ hs,
                                                                     uint16_t* __restrict__ y) {
  extern __shared__ uint32_t s_h[];  // nseg * 16 dwords of re-paired h, then nseg sums
  const int tok = blockIdx.y;        // this block's token
  ids += (size_t)tok * k;
  wts += (size_t)tok * k;
  h += (size_t)tok * k * I;
  hs += (size_t)tok * Is;
  y += (size_t)tok * d;
  const int S = I / 32, Ss = Is / 32;
  const int nslot = k + (Is > 0 ? 1 : 0);
  const int nseg = k * S + Ss;
  float* s_sum = reinterpret_cast<float*>(s_h + (size_t)nseg * 16);
  constexpr int kGdBatch = (9 + HALVES - 1) / HALVES;  // slots per lane per batch
  constexpr int kOutW = 4 / HALVES;                     // outputs per wave
  const int lane = threadIdx.x & 63, l16 = lane & 15, half = HALVES == 2 ? (lane >> 4) & 1 : 0;
  const int o = (blockIdx.x * kGdWaves + (threadIdx.x >> 6)) * kOutW + (lane >> 4) / HALVES;
  const bool ovalid = o < d;
  const int orow = ovalid ? o : 0;
  // every routed slot's expert and weight with one load per wave; slots read them by lane
  const int lj = lane < k ? lane : 0;
  const int id_lane = ids[lj];
  const float w_lane = wts[lj];
  float acc = 0.0f;
  for (int i0 = 0; HALVES * i0 < nslot; i0 += kGdBatch) {
    // 1. this thread's h segments for the LDS staging (first batch only; clamped, never out of
    //    bounds); segments past 2 * blockDim.x are loaded in step 3
    const int g0 = threadIdx.x, g1 = g0 + (int)blockDim.x;
    const int gs0 = (i0 == 0) && g0 < nseg ? g0 : 0;
    const int gs1 = (i0 == 0) && g1 < nseg ? g1 : 0;
    const uint32_t* src0 = gs0 < k * S ? reinterpret_cast<const uint32_t*>(h) + (size_t)gs0 * 16
                                       : reinterpret_cast<const uint32_t*>(hs) + (size_t)(gs0 - k * S) * 16;
    const uint32_t* src1 = gs1 < k * S ? reinterpret_cast<const uint32_t*>(h) + (size_t)gs1 * 16
                                       : reinterpret_cast<const uint32_t*>(hs) + (size_t)(gs1 - k * S) * 16;
    uint32_t hv[16], hv1[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 t = reinterpret_cast<const uint4*>(src0)[q];
      hv[4 * q] = t.x;
      hv[4 * q + 1] = t.y;
      hv[4 * q + 2] = t.z;
      hv[4 * q + 3] = t.w;
      const uint4 t1 = reinterpret_cast<const uint4*>(src1)[q];
      hv1[4 * q] = t1.x;
      hv1[4 * q + 1] = t1.y;
      hv1[4 * q + 2] = t1.z;
      hv1[4 * q + 3] = t1.w;
    }
    // 2. the batch's code pieces, scales and biases: every load unconditional, addresses clamped
    uint4 cw[kGdBatch * PIECES];
    uint32_t sb[kGdBatch * PIECES];  // scale | bias << 16
    float wj[kGdBatch];
#pragma unroll
    for (int b = 0; b < kGdBatch; ++b) {
      const int v0 = HALVES * (i0 + b);  // half 0's slot; half 1 takes v0 + 1
      const int v = v0 + half;
      const bool valid = v < nslot;
      const bool sh = valid && v >= k;
      const int Ie = sh ? Is : I;
      const int m0 = __builtin_amdgcn_readlane(id_lane, v0 < k ? v0 : 0);
      const int m1 = __builtin_amdgcn_readlane(id_lane, v0 + 1 < k ? v0 + 1 : 0);
      const float w0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane), v0 < k ? v0 : 0));
      const float w1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane), v0 + 1 < k ? v0 + 1 : 0));
      int mat = half ? m1 : m0;
      if (!valid || sh || (unsigned)mat >= (unsigned)E) mat = 0;
      wj[b] = !valid ? 0.0f : (sh ? 1.0f : (half ? w1 : w0));
      const uint8_t* dc = sh ? p.sdc : p.dc;
      const uint16_t* ds = sh ? p.sds : p.ds;
      const uint16_t* db = sh ? p.sdb : p.db;
      const size_t row = (size_t)mat * d + orow;
#pragma unroll
      for (int q = 0; q < PIECES; ++q) {
        int seg = l16 + 16 * q;
        seg = seg < Ie / 32 ? seg : 0;
        cw[b * PIECES + q] = load_code_words<BITS>(dc + row * (size_t)(Ie * BITS / 8) + (size_t)seg * 4 * BITS);
        sb[b * PIECES + q] = (uint32_t)ds[row * (size_t)(Ie / kGroup) + seg / 2] |
                             ((uint32_t)db[row * (size_t)(Ie / kGroup) + seg / 2] << 16);
      }
    }
    issue_fence();
    // 3. stage h into LDS (first batch only)
    if (i0 == 0) {
      for (int g = g0, r = 0; g < nseg; g += blockDim.x, ++r) {
        if (r == 1) {
#pragma unroll
          for (int q = 0; q < 16; ++q) hv[q] = hv1[q];
        }
        if (r >= 2) {
          const uint32_t* src = g < k * S ? reinterpret_cast<const uint32_t*>(h) + (size_t)g * 16
                                          : reinterpret_cast<const uint32_t*>(hs) + (size_t)(g - k * S) * 16;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 t = reinterpret_cast<const uint4*>(src)[q];
            hv[4 * q] = t.x;
            hv[4 * q + 1] = t.y;
            hv[4 * q + 2] = t.z;
            hv[4 * q + 3] = t.w;
          }
        }
        Seg32 a;
        make_seg<BITS>(hv, a);
#pragma unroll
        for (int q = 0; q < 16; ++q) s_h[(size_t)g * 16 + q] = a.p[q];
        s_sum[g] = a.sum;
      }
      __syncthreads();
    }
    // 4. arithmetic
#pragma unroll
    for (int b = 0; b < kGdBatch; ++b) {
      const int v = HALVES * (i0 + b) + half;
      const bool valid = v < nslot;
      const bool sh = valid && v >= k;
      const int Sj = sh ? Ss : S;
      const int gbase = sh ? k * S : (valid ? v * S : 0);
#pragma unroll
      for (int q = 0; q < PIECES; ++q) {
        const int seg = l16 + 16 * q;
        const bool use = valid && seg < Sj;
        const int gi = use ? gbase + seg : 0;
        Seg32 a;
        const uint4* hp = reinterpret_cast<const uint4*>(s_h + (size_t)gi * 16);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint4 vv = hp[t];
          a.p[4 * t] = vv.x;
          a.p[4 * t + 1] = vv.y;
          a.p[4 * t + 2] = vv.z;
          a.p[4 * t + 3] = vv.w;
        }
        a.sum = s_sum[gi];
        const uint32_t w2 = sb[b * PIECES + q];
        const float s = bf16lo(w2), bb = bf16hi(w2);
        const float pd = seg_dot<BITS>(cw[b * PIECES + q], a);
        const float c = fmaf(s, pd, fmaf(-128.0f, s, bb) * a.sum);
        acc = fmaf(use ? wj[b] : 0.0f, c, acc);
      }
    }
  }
  // sum over each group's 16 lanes (a DPP row; every lane of the row ends with the row sum)
  acc += dpp_f32<0xB1>(acc);
  acc += dpp_f32<0x4E>(acc);
  acc += dpp_f32<0x124>(acc);
  acc += dpp_f32<0x128>(acc);
  if (HALVES == 1) {
    if (ovalid && l16 == 0) y[o] = f32_to_bf16(acc);
    return;
  }
  // the two halves of each output: outputs o0 = rows 0 + 1, o0 + 1 = rows 2 + 3 of the wave
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 48));
  const int o0 = o - (lane >> 5);  // the wave's first output (even)
  if (lane == 0) {
    if (o0 + 1 < d)
      reinterpret_cast<uint32_t*>(y)[o0 >> 1] = pack_bf16x2(r0 + r1, r2 + r3);
    else if (o0 < d)
      y[o0] = f32_to_bf16(r0 + r1);
  }
}

template <int BITS>
static void launch_down(const Ctx& c, size_t lds) {
  const bool small = c.I <= 512 && c.Is <= 512;
  const auto go = [&](auto kernel, int outs_per_block) {
    const dim3 grid((c.d + outs_per_block - 1) / outs_per_block, c.T);
    hipLaunchKernelGGL(kernel, grid, dim3(kGdWaves * 64), lds, c.stream, c.d, c.E, c.k, c.I, c.Is, c.r.topk_ids,
                       c.r.topk_w, gemv_ptrs(c), c.h, c.hs, c.y);
  };
  if (c.T == 1) {  // two 16-lane halves per output, 2 outputs per wave
    if (small)
      go(k_gemv_down_combine<1, 2, BITS>, 2 * kGdWaves);
    else
      go(k_gemv_down_combine<2, 2, BITS>, 2 * kGdWaves);
  } else {  // 16 lanes per output, 4 outputs per wave
    if (small)
      go(k_gemv_down_combine<1, 1, BITS>, 4 * kGdWaves);
    else
      go(k_gemv_down_combine<2, 1, BITS>, 4 * kGdWaves);
  }
}

hipError_t launch_gemv_down_combine(const Ctx& c) {
  const int nseg = c.k * (c.I / 32) + c.Is / 32;
  const size_t lds = (size_t)nseg * 16 * 4 + (size_t)nseg * 4;
  if (c.bits == 3)
    launch_down<3>(c, lds);
  else if (c.bits == 2)
    launch_down<2>(c, lds);
  else
    launch_down<4>(c, lds);
  return hipGetLastError();
}

}  // namespace moe
