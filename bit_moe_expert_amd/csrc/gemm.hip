// Prefill: grouped GEMM over the expert groups of the block map, with the 4-bit weights
// dequantised tile by tile into LDS as bf16 and multiplied on the matrix cores with fp32
// accumulation; the expanded weights never reach HBM ("Perplexity's Lily Beats MLX-LM on MacBook
// M5. Because It Only Runs One Model.", section "Prefill: keep routing on the GPU, dequantize in
// flight"). Gate and up share a block so SwiGLU is applied in registers and h is written once,
// in bf16. The shared expert is one more group of T rows in the same launch.
//
// Tiling (gfx950, wave64, v_mfma_f32_16x16x32_bf16):
//   - a block is 4 waves; K advances 128 inputs (two quantisation groups) per step;
//   - each thread dequantises one 64-input group of one weight row per step (32 bytes of codes,
//     one scale, one bias) into LDS, while the next step's codes are already in flight;
//   - the A rows (tokens, gathered through sorted_token) are staged in LDS as they are in HBM;
//   - the M extent of a tile is 16, 32, 64 or 128 rows, the smallest that covers the tile's
//     rows, so small expert groups are not padded to a large tile;
//   - the grid is an upper bound (moe_max_tiles x column blocks); blocks past the device-side
//     tile count exit at once. Blocks are renumbered so that each XCD (blocks are dealt to the
//     8 XCDs round-robin) gets a contiguous range ordered (column block, tile): tiles of one
//     large expert that read the same weight rows then run on the same XCD and share its L2.
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kBK = 128;             // inputs per K step
constexpr int kLds = kBK + 8;        // LDS row stride in bf16 (16-byte pad)
constexpr int kGuCols = 64;          // h columns per gate/up block (64 gate + 64 up weight rows)
constexpr int kDnCols = 128;         // output columns per down block

struct GemmArgs {
  int d, E, k, I, Is, T, P, max_tiles, nb;
  const uint16_t* x;
  const int32_t* sorted_token;
  const int32_t* tiles;
  const int32_t* n_tiles;
  moe_ffn_q4 routed, shared;
  uint16_t* h;
  uint16_t* hs;
  float* y_rows;
};

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Decode the block's (column block, tile) and validate the tile. Returns false when the block
// has nothing to do.
__device__ __forceinline__ bool block_tile(const GemmArgs& a, int& nb, int& e, int& row0, int& rows) {
  const int per_xcd = gridDim.x / 8;
  const int L = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  nb = L / a.max_tiles;
  const int ti = L % a.max_tiles;
  if (nb >= a.nb) return false;
  const int nt = min(*a.n_tiles, a.max_tiles);
  if (ti >= nt) return false;
  e = a.tiles[3 * ti];
  row0 = a.tiles[3 * ti + 1];
  rows = a.tiles[3 * ti + 2];
  // a corrupt block map must not turn into out-of-bounds accesses
  if (e < 0 || e > a.E || (e == a.E && a.Is == 0) || rows < 1 || rows > kTileRows || row0 < 0 ||
      row0 + rows > a.P + (a.Is ? a.T : 0) || (e < a.E && row0 + rows > a.P) || (e == a.E && row0 < a.P))
    return false;
  return true;
}

// Load the next K step of one thread's weight group and A chunks.
struct StepRegs {
  uint4 c0, c1;
  uint16_t s, b;
  bool gv, av;  // group present / A chunk inside K (applied when the slot is consumed)
};

// K steps kept in flight per thread (codes, scale, bias and A chunks in registers), sized so the
// ring stays near 100 registers: HBM latency is several K steps long.
template <int MT>
constexpr int ring_depth() {
  return MT == 1 ? 4 : MT == 2 ? 4 : MT == 4 ? 2 : 1;
}

template <int MT>
__device__ __forceinline__ void store_step(uint16_t* Bs, uint16_t* As, int wr, int wh, const StepRegs& w,
                                          const uint4 (&areg)[MT], const bool (&amask)[MT]) {
  uint32_t dq[32];
  const float s = w.gv ? bf16_to_f32(w.s) : 0.0f, b = w.gv ? bf16_to_f32(w.b) : 0.0f;
  dequant_group(w.c0, w.c1, s, b, dq);
  uint4* dst = reinterpret_cast<uint4*>(Bs + wr * kLds + wh * 64);
#pragma unroll
  for (int q = 0; q < 8; ++q) dst[q] = make_uint4(dq[4 * q], dq[4 * q + 1], dq[4 * q + 2], dq[4 * q + 3]);
  const int tid = threadIdx.x;
#pragma unroll
  for (int mm = 0; mm < MT; ++mm) {
    const bool keep = w.av && amask[mm];
    const uint4 v = areg[mm];
    *reinterpret_cast<uint4*>(As + ((tid >> 4) + 16 * mm) * kLds + (tid & 15) * 8) =
        make_uint4(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
  }
}

// ---------------------------------------------------------------------------------------------
// gate/up: h[row][n0 + c] = bf16(silu(g) * u) for the 64 columns n0..n0+63 of one tile.
template <int MT>
__device__ __forceinline__ void gateup_body(const GemmArgs& a, int n0, int e, int row0, int rows, uint16_t* Bs,
                                            uint16_t* As) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool sh = (e == a.E);
  const int Ie = sh ? a.Is : a.I;
  const int mat = sh ? 0 : e;
  const moe_ffn_q4& F = sh ? a.shared : a.routed;
  const int d = a.d;
  // this thread's weight group: row wr of the 128 (64 gate rows, then 64 up rows), half wh
  const int wr = tid >> 1, wh = tid & 1;
  const moe_q4& Q = wr < kGuCols ? F.gate : F.up;
  const size_t wrow = (size_t)mat * Ie + n0 + (wr & (kGuCols - 1));
  const uint8_t* cp = Q.codes + wrow * (size_t)(d / 2) + wh * 32;
  const uint16_t* sp = Q.scales + wrow * (size_t)(d / kGroup) + wh;
  const uint16_t* bp = Q.biases + wrow * (size_t)(d / kGroup) + wh;
  // this thread's A chunks: row (tid >> 4) + 16 mm, inputs 8 (tid & 15) .. +7 of the step
  const uint16_t* ap[MT];
  bool amask[MT];
#pragma unroll
  for (int mm = 0; mm < MT; ++mm) {
    const int r = (tid >> 4) + 16 * mm;
    int tok = -1;
    if (r < rows) tok = sh ? (row0 - a.P + r) : a.sorted_token[row0 + r];
    amask[mm] = (unsigned)tok < (unsigned)a.T;
    ap[mm] = a.x + (size_t)(amask[mm] ? tok : 0) * d;
  }
  const int S = (d + kBK - 1) / kBK;
  constexpr int D = ring_depth<MT>();
  StepRegs w[D];
  uint4 areg[D][MT];
  // Every slot load is unconditional (step index clamped, A rows of absent tokens read row 0),
  // so the compiler can count outstanding loads exactly; padding steps and absent rows are
  // zeroed with selects instead of branches.
  const int kh_last = (d / 64) - 1;  // last 64-input group index
  auto load = [&](int s, StepRegs& wd, uint4 (&ad)[MT]) {
    const int g = min(2 * s + wh, kh_last);
    const bool gv = 2 * s + wh <= kh_last;
    wd.c0 = *reinterpret_cast<const uint4*>(cp - wh * 32 + g * 32);
    wd.c1 = *reinterpret_cast<const uint4*>(cp - wh * 32 + g * 32 + 16);
    wd.s = sp[g - wh];
    wd.b = bp[g - wh];
    wd.gv = gv;
    const int ka = min(s * kBK + (tid & 15) * 8, d - 8);
    wd.av = s * kBK + (tid & 15) * 8 < d;
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) ad[mm] = *reinterpret_cast<const uint4*>(ap[mm] + ka);
  };
  f32x4_t accg[MT], accu[MT];
#pragma unroll
  for (int mm = 0; mm < MT; ++mm) {
    accg[mm] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    accu[mm] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int u = 0; u < D; ++u) load(u, w[u], areg[u]);
  for (int s0 = 0; s0 < S; s0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      store_step<MT>(Bs, As, wr, wh, w[u], areg[u], amask);
      __syncthreads();
      load(s0 + u + D, w[u], areg[u]);
      const int kofs = (lane >> 4) * 8;
#pragma unroll
      for (int kk = 0; kk < kBK / 32; ++kk) {
        const uint4 bg = *reinterpret_cast<const uint4*>(Bs + (16 * wave + (lane & 15)) * kLds + kk * 32 + kofs);
        const uint4 bu =
            *reinterpret_cast<const uint4*>(Bs + (kGuCols + 16 * wave + (lane & 15)) * kLds + kk * 32 + kofs);
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) {
          const uint4 av = *reinterpret_cast<const uint4*>(As + (16 * mm + (lane & 15)) * kLds + kk * 32 + kofs);
          accg[mm] = mfma16x16x32(av, bg, accg[mm]);
          accu[mm] = mfma16x16x32(av, bu, accu[mm]);
        }
      }
      __syncthreads();
    }
  }
  uint16_t* hout = sh ? a.hs + (size_t)(row0 - a.P) * Ie : a.h + (size_t)row0 * Ie;
  const int col = n0 + 16 * wave + (lane & 15);
#pragma unroll
  for (int mm = 0; mm < MT; ++mm)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * mm + 4 * (lane >> 4) + r;
      if (row < rows) hout[(size_t)row * Ie + col] = f32_to_bf16(silu_mul(accg[mm][r], accu[mm][r]));
    }
}

__global__ __launch_bounds__(256) void k_gateup_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2 * kGuCols * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t As[kTileRows * kLds];
  int nb, e, row0, rows;
  if (!block_tile(a, nb, e, row0, rows)) return;
  const int n0 = nb * kGuCols;
  if (n0 >= (e == a.E ? a.Is : a.I)) return;
  if (rows <= 16)
    gateup_body<1>(a, n0, e, row0, rows, Bs, As);
  else if (rows <= 32)
    gateup_body<2>(a, n0, e, row0, rows, Bs, As);
  else if (rows <= 64)
    gateup_body<4>(a, n0, e, row0, rows, Bs, As);
  else
    gateup_body<8>(a, n0, e, row0, rows, Bs, As);
}

// ---------------------------------------------------------------------------------------------
// down: y_rows[row][n0 + c] = h[row] . Wd[e][n0 + c] for 128 output columns of one tile.
template <int MT>
__device__ __forceinline__ void down_body(const GemmArgs& a, int n0, int e, int row0, int rows, uint16_t* Bs,
                                          uint16_t* As) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool sh = (e == a.E);
  const int Ie = sh ? a.Is : a.I;
  const int mat = sh ? 0 : e;
  const moe_q4& Q = sh ? a.shared.down : a.routed.down;
  const int d = a.d;
  const int wr = tid >> 1, wh = tid & 1;
  const bool wvalid = n0 + wr < d;
  const size_t wrow = (size_t)mat * d + n0 + (wvalid ? wr : 0);
  const uint8_t* cp = Q.codes + wrow * (size_t)(Ie / 2) + wh * 32;
  const uint16_t* sp = Q.scales + wrow * (size_t)(Ie / kGroup) + wh;
  const uint16_t* bp = Q.biases + wrow * (size_t)(Ie / kGroup) + wh;
  const uint16_t* hbase = sh ? a.hs + (size_t)(row0 - a.P) * Ie : a.h + (size_t)row0 * Ie;
  const uint16_t* ap[MT];
  bool amask[MT];
#pragma unroll
  for (int mm = 0; mm < MT; ++mm) {
    const int r = (tid >> 4) + 16 * mm;
    amask[mm] = r < rows;
    ap[mm] = hbase + (size_t)(amask[mm] ? r : 0) * Ie;
  }
  const int S = (Ie + kBK - 1) / kBK;
  constexpr int D = ring_depth<MT>();
  StepRegs w[D];
  uint4 areg[D][MT];
  const int kh_last = (Ie / 64) - 1;
  auto load = [&](int s, StepRegs& wd, uint4 (&ad)[MT]) {
    const int g = min(2 * s + wh, kh_last);
    const bool gv = wvalid && 2 * s + wh <= kh_last;
    wd.c0 = *reinterpret_cast<const uint4*>(cp - wh * 32 + g * 32);
    wd.c1 = *reinterpret_cast<const uint4*>(cp - wh * 32 + g * 32 + 16);
    wd.s = sp[g - wh];
    wd.b = bp[g - wh];
    wd.gv = gv;
    const int ka = min(s * kBK + (tid & 15) * 8, Ie - 8);
    wd.av = s * kBK + (tid & 15) * 8 < Ie;
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) ad[mm] = *reinterpret_cast<const uint4*>(ap[mm] + ka);
  };
  f32x4_t acc[MT][2];
#pragma unroll
  for (int mm = 0; mm < MT; ++mm) acc[mm][0] = acc[mm][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < D; ++u) load(u, w[u], areg[u]);
  for (int s0 = 0; s0 < S; s0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      store_step<MT>(Bs, As, wr, wh, w[u], areg[u], amask);
      __syncthreads();
      load(s0 + u + D, w[u], areg[u]);
      const int kofs = (lane >> 4) * 8;
#pragma unroll
      for (int kk = 0; kk < kBK / 32; ++kk) {
        const uint4 b0 = *reinterpret_cast<const uint4*>(Bs + (32 * wave + (lane & 15)) * kLds + kk * 32 + kofs);
        const uint4 b1 =
            *reinterpret_cast<const uint4*>(Bs + (32 * wave + 16 + (lane & 15)) * kLds + kk * 32 + kofs);
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) {
          const uint4 av = *reinterpret_cast<const uint4*>(As + (16 * mm + (lane & 15)) * kLds + kk * 32 + kofs);
          acc[mm][0] = mfma16x16x32(av, b0, acc[mm][0]);
          acc[mm][1] = mfma16x16x32(av, b1, acc[mm][1]);
        }
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int mm = 0; mm < MT; ++mm)
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      const int col = n0 + 32 * wave + 16 * nn + (lane & 15);
      if (col >= d) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * mm + 4 * (lane >> 4) + r;
        if (row < rows) a.y_rows[(size_t)(row0 + row) * d + col] = acc[mm][nn][r];
      }
    }
}

__global__ __launch_bounds__(256) void k_down_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kDnCols * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t As[kTileRows * kLds];
  int nb, e, row0, rows;
  if (!block_tile(a, nb, e, row0, rows)) return;
  const int n0 = nb * kDnCols;
  if (rows <= 16)
    down_body<1>(a, n0, e, row0, rows, Bs, As);
  else if (rows <= 32)
    down_body<2>(a, n0, e, row0, rows, Bs, As);
  else if (rows <= 64)
    down_body<4>(a, n0, e, row0, rows, Bs, As);
  else
    down_body<8>(a, n0, e, row0, rows, Bs, As);
}

static GemmArgs gemm_args(const Ctx& c, int nb) {
  GemmArgs a;
  a.d = c.d;
  a.E = c.E;
  a.k = c.k;
  a.I = c.I;
  a.Is = c.Is;
  a.T = c.T;
  a.P = c.P;
  a.max_tiles = c.max_tiles;
  a.nb = nb;
  a.x = c.x;
  a.sorted_token = c.r.sorted_token;
  a.tiles = c.r.tiles;
  a.n_tiles = c.r.n_tiles;
  a.routed = c.routed;
  a.shared = c.shared;
  a.h = c.h;
  a.hs = c.hs;
  a.y_rows = c.y_rows;
  return a;
}

static int grid_blocks(int max_tiles, int nb) { return ((max_tiles * nb + 7) / 8) * 8; }

hipError_t launch_gateup_gemm(const Ctx& c) {
  const int nb = (max(c.I, c.Is) + kGuCols - 1) / kGuCols;
  hipLaunchKernelGGL(k_gateup_gemm, dim3(grid_blocks(c.max_tiles, nb)), dim3(256), 0, c.stream, gemm_args(c, nb));
  return hipGetLastError();
}

hipError_t launch_down_gemm(const Ctx& c) {
  const int nb = (c.d + kDnCols - 1) / kDnCols;
  hipLaunchKernelGGL(k_down_gemm, dim3(grid_blocks(c.max_tiles, nb)), dim3(256), 0, c.stream, gemm_args(c, nb));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Weighted gather back to token order: y[t] = bf16(sum_j w[t][j] * y_rows[inv_pos[t][j]] +
// y_rows[P + t]), j ascending, in fp32. One thread per 4 outputs.
__global__ __launch_bounds__(256) void k_combine(int T, int d, int k, int P, int has_shared,
                                                 const int32_t* __restrict__ inv_pos, const float* __restrict__ w,
                                                 const float* __restrict__ y_rows, uint16_t* __restrict__ y) {
  const int q = d / 4;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)T * q) return;
  const int t = (int)(idx / q), o = (int)(idx % q) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int row = inv_pos[(size_t)t * k + j];
    if ((unsigned)row >= (unsigned)P) continue;
    const float wj = w[(size_t)t * k + j];
    const float4 v = *reinterpret_cast<const float4*>(y_rows + (size_t)row * d + o);
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  if (has_shared) {
    const float4 v = *reinterpret_cast<const float4*>(y_rows + (size_t)(P + t) * d + o);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  uint2 out;
  out.x = pack_bf16x2(acc.x, acc.y);
  out.y = pack_bf16x2(acc.z, acc.w);
  *reinterpret_cast<uint2*>(y + (size_t)t * d + o) = out;
}

hipError_t launch_combine(const Ctx& c) {
  const size_t n = (size_t)c.T * (c.d / 4);
  const int nblk = (int)((n + 255) / 256);
  hipLaunchKernelGGL(k_combine, dim3(nblk), dim3(256), 0, c.stream, c.T, c.d, c.k, c.P, c.Is > 0 ? 1 : 0,
                     c.r.inv_pos, c.r.topk_w, c.y_rows, c.y);
  return hipGetLastError();
}

}  // namespace moe
