// Check export: dequantise whole matrices with the very routines the kernels use: the codes are
// read with load_codes32 (the GEMV kernels' unpack of 4-, 3- and 2-bit codes into nibbles) and
// expanded with dequant_group, so a bit-exact comparison of this output covers both.
#include "device_common.h"
#include "kernels.h"

namespace moe {

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
  const uint4 c0 = load_codes32<BITS>(cp);
  const uint4 c1 = load_codes32<BITS>(cp + 4 * BITS);
  uint32_t dq[32];
  dequant_group(c0, c1, bf16_to_f32(scales[g]), bf16_to_f32(biases[g]), dq);
  uint4* dst = reinterpret_cast<uint4*>(out + row * in_dim + gi * kGroup);
#pragma unroll
  for (int q = 0; q < 8; ++q) dst[q] = make_uint4(dq[4 * q], dq[4 * q + 1], dq[4 * q + 2], dq[4 * q + 3]);
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
