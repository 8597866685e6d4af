// Batch-1 decode: bandwidth-bound grouped GEMV over the k selected experts plus the shared
// expert, on the vector ALUs, with 128-bit loads of the 4-bit codes.
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
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kGvWaves = 4;     // waves per block
constexpr int kGvRows = 2;      // h entries (each = one gate row + one up row) per wave

// Segment of 32 consecutive inputs as 16 re-paired bf16 dwords (magic_pair order) + their sum.
struct Seg32 {
  uint32_t p[16];
  float sum;
};

__device__ __forceinline__ void make_seg(const uint32_t* v16, Seg32& s) {
#pragma unroll
  for (int m = 0; m < 4; ++m) repair8(v16 + 4 * m, s.p + 4 * m);
  float acc = 0.0f;
#pragma unroll
  for (int m = 0; m < 16; ++m) acc = dot2_bf16(v16[m], 0x3F803F80u, acc);  // (1.0, 1.0)
  s.sum = acc;
}

// sum over the segment of act * (128 + q) for one 16-byte row piece of codes.
__device__ __forceinline__ float seg_dot(const uint4& cw, const Seg32& a) {
  const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
  float acc = 0.0f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc = dot2_bf16(magic_pair(w[m], n), a.p[4 * m + n], acc);
  return acc;
}

// ---------------------------------------------------------------------------------------------
// h[j][i] = bf16(silu(x . Wg[e_j][i]) * (x . Wu[e_j][i])) for the k routed slots (e_j =
// topk_ids[j]) and the shared slot. One wave owns kGvRows consecutive i of one slot; lane l
// takes the 16-byte code pieces l, l+64, ... of each of its rows.
__global__ __launch_bounds__(kGvWaves * 64) void k_gemv_gateup(int d, int E, int k, int I, int Is,
                                                               const uint16_t* __restrict__ x,
                                                               const int32_t* __restrict__ ids, moe_ffn_q4 routed,
                                                               moe_ffn_q4 shared, uint16_t* __restrict__ h,
                                                               uint16_t* __restrict__ hs) {
  extern __shared__ uint32_t s_x[];  // x as d/2 dwords
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < d / 2; i += blockDim.x) s_x[i] = reinterpret_cast<const uint32_t*>(x)[i];
  __syncthreads();
  const int wave_g = blockIdx.x * kGvWaves + (threadIdx.x >> 6);
  const int r0 = wave_g * kGvRows;
  const int total = k * I + Is;
  if (r0 >= total) return;
  int Ie, mat, i0;
  moe_q4 G, U;
  uint16_t* hout;
  if (r0 < k * I) {
    const int j = r0 / I;
    i0 = r0 - j * I;
    Ie = I;
    mat = ids[j];
    if ((unsigned)mat >= (unsigned)E) mat = 0;  // keeps a corrupt routing from reading out of bounds
    G = routed.gate;
    U = routed.up;
    hout = h + (size_t)j * I + i0;
  } else {
    i0 = r0 - k * I;
    Ie = Is;
    mat = 0;
    G = shared.gate;
    U = shared.up;
    hout = hs + i0;
  }
  const int nseg = d / 32;
  const size_t cstride = (size_t)d / 2, sstride = (size_t)d / kGroup;
  float acc[2 * kGvRows];
#pragma unroll
  for (int r = 0; r < 2 * kGvRows; ++r) acc[r] = 0.0f;
  for (int seg = lane; seg < nseg; seg += 64) {
    uint4 cw[2 * kGvRows];
    uint16_t sr[2 * kGvRows], br[2 * kGvRows];
#pragma unroll
    for (int r = 0; r < 2 * kGvRows; ++r) {
      const moe_q4& Q = r < kGvRows ? G : U;
      const size_t row = (size_t)mat * Ie + i0 + (r % kGvRows);
      cw[r] = *reinterpret_cast<const uint4*>(Q.codes + row * cstride + (size_t)seg * 16);
      sr[r] = Q.scales[row * sstride + seg / 2];
      br[r] = Q.biases[row * sstride + seg / 2];
    }
    Seg32 a;
    make_seg(s_x + seg * 16, a);
#pragma unroll
    for (int r = 0; r < 2 * kGvRows; ++r) {
      const float s = bf16_to_f32(sr[r]), b = bf16_to_f32(br[r]);
      const float p = seg_dot(cw[r], a);
      acc[r] = fmaf(s, p, acc[r]);
      acc[r] = fmaf(fmaf(-128.0f, s, b), a.sum, acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < 2 * kGvRows; ++r) acc[r] = wave_sum(acc[r]);
  if (lane == 0) {
    uint32_t packed = pack_bf16x2(silu_mul(acc[0], acc[kGvRows]), silu_mul(acc[1], acc[kGvRows + 1]));
    *reinterpret_cast<uint32_t*>(hout) = packed;
  }
}

hipError_t launch_gemv_gateup(const Ctx& c) {
  const int waves = (c.k * c.I + c.Is) / kGvRows;
  const int nblk = (waves + kGvWaves - 1) / kGvWaves;
  const size_t lds = (size_t)c.d * 2;
  hipLaunchKernelGGL(k_gemv_gateup, dim3(nblk), dim3(kGvWaves * 64), lds, c.stream, c.d, c.E, c.k, c.I, c.Is, c.x,
                     c.r.topk_ids, c.routed, c.shared, c.h, c.hs);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// y[o] = bf16( sum_j w_j * (h_j . Wd[e_j][o]) + h_s . Wd_s[o] ). A block keeps every slot's h
// in LDS (re-paired) with per-segment sums; a wave owns 4 outputs, 16 lanes per output, and
// those lanes walk the (slot, 32-input segment) pieces of that output's rows. Each output is
// reduced inside its 16 lanes, so there are no atomics.
constexpr int kGdOut = 16;  // outputs per block (4 waves x 4)

__global__ __launch_bounds__(256) void k_gemv_down_combine(int d, int E, int k, int I, int Is,
                                                           const int32_t* __restrict__ ids,
                                                           const float* __restrict__ wts, moe_ffn_q4 routed,
                                                           moe_ffn_q4 shared, const uint16_t* __restrict__ h,
                                                           const uint16_t* __restrict__ hs, uint16_t* __restrict__ y) {
  extern __shared__ uint32_t s_h[];  // nseg_total * 16 dwords of re-paired h, then nseg_total sums
  const int S = I / 32, Ss = Is / 32;
  const int nseg = k * S + Ss;
  float* s_sum = reinterpret_cast<float*>(s_h + (size_t)nseg * 16);
  for (int g = threadIdx.x; g < nseg; g += blockDim.x) {
    const uint32_t* src = g < k * S ? reinterpret_cast<const uint32_t*>(h) + (size_t)g * 16
                                    : reinterpret_cast<const uint32_t*>(hs) + (size_t)(g - k * S) * 16;
    uint32_t v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 t = reinterpret_cast<const uint4*>(src)[q];
      v[4 * q] = t.x;
      v[4 * q + 1] = t.y;
      v[4 * q + 2] = t.z;
      v[4 * q + 3] = t.w;
    }
    Seg32 a;
    make_seg(v, a);
#pragma unroll
    for (int q = 0; q < 16; ++q) s_h[(size_t)g * 16 + q] = a.p[q];
    s_sum[g] = a.sum;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, l16 = lane & 15;
  const int o = blockIdx.x * kGdOut + (threadIdx.x >> 6) * 4 + (lane >> 4);
  float acc = 0.0f;
  if (o < d) {
    for (int tau = l16; tau < nseg; tau += 16) {
      int mat, seg, Ie;
      moe_q4 D;
      float wj;
      if (tau < k * S) {
        const int j = tau / S;
        seg = tau - j * S;
        Ie = I;
        mat = ids[j];
        if ((unsigned)mat >= (unsigned)E) mat = 0;
        D = routed.down;
        wj = wts[j];
      } else {
        seg = tau - k * S;
        Ie = Is;
        mat = 0;
        D = shared.down;
        wj = 1.0f;
      }
      const size_t row = (size_t)mat * d + o;
      const uint4 cw = *reinterpret_cast<const uint4*>(D.codes + row * (size_t)(Ie / 2) + (size_t)seg * 16);
      const float s = bf16_to_f32(D.scales[row * (size_t)(Ie / kGroup) + seg / 2]);
      const float b = bf16_to_f32(D.biases[row * (size_t)(Ie / kGroup) + seg / 2]);
      Seg32 a;
#pragma unroll
      for (int q = 0; q < 16; ++q) a.p[q] = s_h[(size_t)tau * 16 + q];
      a.sum = s_sum[tau];
      const float p = seg_dot(cw, a);
      acc = fmaf(wj, fmaf(s, p, fmaf(-128.0f, s, b) * a.sum), acc);
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (o < d && l16 == 0) y[o] = f32_to_bf16(acc);
}

hipError_t launch_gemv_down_combine(const Ctx& c) {
  const int nseg = c.k * (c.I / 32) + c.Is / 32;
  const size_t lds = (size_t)nseg * 16 * 4 + (size_t)nseg * 4;
  const int nblk = (c.d + kGdOut - 1) / kGdOut;
  hipLaunchKernelGGL(k_gemv_down_combine, dim3(nblk), dim3(256), lds, c.stream, c.d, c.E, c.k, c.I, c.Is,
                     c.r.topk_ids, c.r.topk_w, c.routed, c.shared, c.h, c.hs, c.y);
  return hipGetLastError();
}

}  // namespace moe
