// Grouped GEMM launchers (4-bit codes here; 3- and 2-bit codes in gemm_b3.hip and gemm_b2.hip,
// the same templates from gemm_impl.h) and the weighted combine back to token order.
#include "gemm_impl.h"

namespace moe {

extern template hipError_t launch_gateup_gemm_bits<3>(const Ctx& c);
extern template hipError_t launch_gateup_gemm_bits<2>(const Ctx& c);
extern template hipError_t launch_down_gemm_bits<3>(const Ctx& c);
extern template hipError_t launch_down_gemm_bits<2>(const Ctx& c);

hipError_t launch_gateup_gemm(const Ctx& c) {
  return c.bits == 3 ? launch_gateup_gemm_bits<3>(c) : c.bits == 2 ? launch_gateup_gemm_bits<2>(c)
                                                                    : launch_gateup_gemm_bits<4>(c);
}

hipError_t launch_down_gemm(const Ctx& c) {
  return c.bits == 3 ? launch_down_gemm_bits<3>(c) : c.bits == 2 ? launch_down_gemm_bits<2>(c)
                                                                  : launch_down_gemm_bits<4>(c);
}

// ---------------------------------------------------------------------------------------------
// Weighted gather back to token order: y[t] = bf16(sum_j w[t][j] * row(inv_pos[t][j]) + row(P + t)),
// j ascending, in fp32, where row(i) is the down product's fp16 row i with each 32-column segment
// multiplied back by 2^e (exact). A block covers 1024 outputs of one token (one thread per 4
// outputs), so the token's k row indices and weights are block-uniform scalar loads.
constexpr int kCombineThreads = 256;
__global__ __launch_bounds__(kCombineThreads) void k_combine(int T, int d, int k, int P, int has_shared,
                                                             const int32_t* __restrict__ inv_pos,
                                                             const float* __restrict__ w,
                                                             const uint16_t* __restrict__ y_rows,
                                                             const uint8_t* __restrict__ y_exp,
                                                             uint16_t* __restrict__ y) {
  const int nb = (d + 4 * kCombineThreads - 1) / (4 * kCombineThreads);  // blocks per token
  const int t = blockIdx.x / nb;
  const int o = ((blockIdx.x % nb) * kCombineThreads + threadIdx.x) * 4;
  if (t >= T || o >= d) return;
  // every index, row and exponent load is issued before the first add
  int row[kMaxTopK];
  float wj[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    row[j] = j < k ? inv_pos[(size_t)t * k + j] : -1;
    wj[j] = j < k ? w[(size_t)t * k + j] : 0.0f;
  }
  const int seg = o / 32, nseg = d / 32;
  uint2 q[kMaxTopK], qs = make_uint2(0u, 0u);
  int ej[kMaxTopK], es = 0;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if ((unsigned)row[j] < (unsigned)P) {
      q[j] = *reinterpret_cast<const uint2*>(y_rows + (size_t)row[j] * d + o);
      ej[j] = y_exp[(size_t)row[j] * nseg + seg];
    }
  if (has_shared) {
    qs = *reinterpret_cast<const uint2*>(y_rows + (size_t)(P + t) * d + o);
    es = y_exp[(size_t)(P + t) * nseg + seg];
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if ((unsigned)row[j] < (unsigned)P) {
      acc.x = fmaf(wj[j], __builtin_ldexpf(f16lo(q[j].x), ej[j]), acc.x);
      acc.y = fmaf(wj[j], __builtin_ldexpf(f16hi(q[j].x), ej[j]), acc.y);
      acc.z = fmaf(wj[j], __builtin_ldexpf(f16lo(q[j].y), ej[j]), acc.z);
      acc.w = fmaf(wj[j], __builtin_ldexpf(f16hi(q[j].y), ej[j]), acc.w);
    }
  if (has_shared) {
    acc.x += __builtin_ldexpf(f16lo(qs.x), es);
    acc.y += __builtin_ldexpf(f16hi(qs.x), es);
    acc.z += __builtin_ldexpf(f16lo(qs.y), es);
    acc.w += __builtin_ldexpf(f16hi(qs.y), es);
  }
  uint2 out;
  out.x = pack_bf16x2(acc.x, acc.y);
  out.y = pack_bf16x2(acc.z, acc.w);
  *reinterpret_cast<uint2*>(y + (size_t)t * d + o) = out;
}

hipError_t launch_combine(const Ctx& c) {
  const int nb = (c.d + 4 * kCombineThreads - 1) / (4 * kCombineThreads);
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((size_t)c.T * nb)), dim3(kCombineThreads), 0, c.stream, c.T, c.d, c.k,
                     c.P, c.Is > 0 ? 1 : 0, c.r.inv_pos, c.r.topk_w, c.y_rows, c.y_exp, c.y);
  return hipGetLastError();
}

}  // namespace moe
