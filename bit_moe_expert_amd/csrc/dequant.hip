// Check export: dequantise whole matrices with the very routine the GEMV kernels use to unpack
// codes (seg_pairs, for 4-, 3- and 2-bit codes): the codes are read back out of its "128 + q"
// pairs and mapped through the groupwise affine map, so a bit-exact comparison of this output
// covers the unpack of every code width.
#include "device_common.h"
#include "kernels.h"

namespace moe {

// w = bf16(fp32(s * q + b)): s * q is exact in fp32, so fmaf gives the single fp32 rounding the
// definition asks for; the conversion to bf16 rounds to nearest even.
template <int BITS>
__global__ __launch_bounds__(256) void k_dequant(int64_t n_groups, int in_dim, const uint8_t* __restrict__ codes,
                                                 const uint16_t* __restrict__ scales,
                                                 const uint16_t* __restrict__ biases, uint16_t* __restrict__ out) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_groups) return;
  const int gpr = in_dim / kGroup;
  const int64_t row = g / gpr;
  const int gi = (int)(g % gpr);
  const uint8_t* cp = codes + row * ((int64_t)in_dim * BITS / 8) + gi * 8 * BITS;
  const float s = bf16_to_f32(scales[g]), b = bf16_to_f32(biases[g]);
  float v[kGroup];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    uint32_t p[16];
    seg_pairs<BITS>(load_code_words<BITS>(cp + half * 4 * BITS), p);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int i = 32 * half + pair_input<BITS>(k);
      v[i] = fmaf(s, (float)(p[k] & 0xffu), b);
      v[i + pair_gap<BITS>()] = fmaf(s, (float)((p[k] >> 16) & 0xffu), b);
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(out + row * in_dim + gi * kGroup);
#pragma unroll
  for (int q = 0; q < 8; ++q)
    dst[q] = make_uint4(pack_bf16x2(v[8 * q], v[8 * q + 1]), pack_bf16x2(v[8 * q + 2], v[8 * q + 3]),
                        pack_bf16x2(v[8 * q + 4], v[8 * q + 5]), pack_bf16x2(v[8 * q + 6], v[8 * q + 7]));
}

hipError_t launch_dequant(const moe_q4& w, int64_t rows, int in_dim, int bits, uint16_t* out, hipStream_t stream) {
  const int64_t n_groups = rows * (in_dim / kGroup);
  const int64_t nblk = (n_groups + 255) / 256;
  const auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)nblk), dim3(256), 0, stream, n_groups, in_dim, w.codes, w.scales,
                       w.biases, out);
  };
  if (bits == 3)
    go(k_dequant<3>);
  else if (bits == 2)
    go(k_dequant<2>);
  else
    go(k_dequant<4>);
  return hipGetLastError();
}

}  // namespace moe
