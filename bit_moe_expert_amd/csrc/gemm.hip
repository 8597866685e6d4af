// Prefill: grouped GEMM over the expert groups of the block map. The 4-bit weights of one K
// step are staged in LDS a tile at a time and multiplied on the matrix cores with fp32
// accumulation; no expanded weight ever reaches HBM ("Perplexity's Lily Beats MLX-LM on MacBook
// M5. Because It Only Runs One Model.", section "Prefill: keep routing on the GPU, dequantize in
// flight"). Gate and up share a block so SwiGLU is applied in registers and h is written once,
// in bf16. The shared expert is one more group of T rows in the same launch.
//
// Tiling (gfx950, wave64, v_mfma_f32_16x16x32_bf16):
//   - a tile is at most 32 rows of one expert group; its M extent is 16 or 32 rows, the
//     smallest that covers it (the same section's note that 32-row tiles beat 16-row ones);
//   - a block is 4 waves and covers 128 weight rows (gate/up: 64 gate + 64 up rows, giving 64 h
//     columns; down: 128 output columns); K advances 128 inputs (two quantisation groups) a step;
//   - the grid is an upper bound (moe_max_tiles x column blocks); blocks past the device-side
//     tile count exit at once. Blocks are renumbered so that each XCD (blocks are dealt to the
//     8 XCDs round-robin) gets a contiguous range ordered (column block, tile): tiles of one
//     expert that read the same weight rows then run on the same XCD and share its L2.
#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kBK = 128;             // inputs per K step
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
  return !(e < 0 || e > a.E || (e == a.E && a.Is == 0) || rows < 1 || rows > kTileRows || row0 < 0 ||
           row0 + rows > a.P + (a.Is ? a.T : 0) || (e < a.E && row0 + rows > a.P) || (e == a.E && row0 < a.P));
}

// ---------------------------------------------------------------------------------------------
// The matrix cores take the 4-bit codes themselves. Over one 64-input group with scale s and bias b,
//   sum_k x_k (s q_k + b) = s * sum_k x_k (128 + q_k) + (b - 128 s) * X_g,   X_g = sum_k x_k,
// and "128 + q" is an exact bf16 made from the code bits with one and-or per pair. So each group
// runs its two MFMA K-steps into a fresh accumulator, then two FMAs fold the group's scale and
// bias into the running sum; X_g comes from one more MFMA of the same A rows against ones. The
// weight enters as s * q + b evaluated in fp32 without rounding the weight itself to bf16 first
// (a difference of at most half a bf16 ulp per weight).
//
// Pipeline: every input of K step s (128 inputs) goes straight from memory to LDS with direct
// loads (no registers on the way), three steps ahead, into a ring of four stages:
//   - codes: 128 weight rows x 64 bytes; each row's four 16-byte quarters are XOR-swizzled by
//     row so the MFMA-side 8-byte reads spread over the banks;
//   - scales and biases: one 16-bit load per (weight row, group), each landing zero-extended in
//     its own dword; a group past K or a weight row past the matrix loads from a zero word, so
//     its codes and A values (read from clamped, in-bounds addresses) add exactly 0;
//   - A rows (up to 32 gathered x rows, or h rows) of 256 bytes; the 16-byte chunks of a row are
//     XOR-swizzled by row. A rows past the tile's rows repeat its last row and only reach
//     accumulator rows that are never written out.
// A is permuted to the code pair order as it is read for the MFMA. Loads complete in issue
// order, so before each barrier a wave waits until at most the two younger steps' loads are
// outstanding: its part of the next stage has then landed.
constexpr int kCodeStages = 4;               // LDS ring depth (3 steps in flight)
constexpr int kCodeStageBytes = 128 * 64;    // 128 weight rows x 128 inputs of codes
constexpr int kSbStageWords = 2 * 256;       // scale dwords [128 rows][2 groups], then biases
constexpr int kAStageBytes = 32 * 256;       // 32 A rows x 128 bf16

__device__ const uint16_t kZeroHalf[8] = {0, 0, 0, 0, 0, 0, 0, 0};

// The stages are separate LDS arrays so that the compiler can tell a direct load into one stage
// from reads of another and does not wait for loads that a read does not depend on.
struct GemmLds {
  uint8_t* c[kCodeStages];
  uint32_t* sb[kCodeStages];
  uint8_t* a[kCodeStages];
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

__device__ __forceinline__ int code_swz(int r) { return (r >> 1) & 3; }
__device__ __forceinline__ int a_swz(int r) { return r & 7; }

// Direct loads are written as inline assembly: the compiler's own wait insertion cannot follow
// them across the loop back-edge and would drain every outstanding load before the first LDS
// read of each unrolled round. Completion is handled explicitly (step_barrier, and a full wait
// before the block ends).
__device__ __forceinline__ uint32_t lds_addr(const void* l) {
  // wave-uniform by construction; readfirstlane puts it in a scalar register for m0
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)l);
}
__device__ __forceinline__ void dma16(const void* g, void* l) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_addr(l)) : "memory", "m0");
}
__device__ __forceinline__ void dma2(const void* g, void* l) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %0, off" ::"v"(g), "s"(lds_addr(l)) : "memory", "m0");
}

// Waits until at most N of this wave's vector memory loads are outstanding and its LDS reads
// have completed, then joins the workgroup barrier. No LDS release fence: a fence would also
// wait for every direct load.
template <int N>
__device__ __forceinline__ void step_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));  // vmcnt(N) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// GU: gate/up (A = gathered x rows, 64 gate + 64 up weight rows, SwiGLU epilogue to h);
// otherwise down (A = h rows, 128 weight rows of the down matrix, fp32 y_rows epilogue).
template <int MT, bool GU>
__device__ __forceinline__ void tile_body(const GemmArgs& a, int n0, int e, int row0, int rows, const GemmLds& L) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool sh = (e == a.E);
  const int Ie = sh ? a.Is : a.I;
  const int mat = sh ? 0 : e;
  const int d = a.d;
  const int K = GU ? d : Ie;        // reduction length
  const int ldc = K / 2;            // code bytes per weight row
  const int ldg = K / kGroup;       // groups per weight row
  const int nrows_w = GU ? Ie : d;  // weight rows of the matrix
  const int S = (K + kBK - 1) / kBK;

  // ---- codes: wave w fills block rows 32w .. 32w+31 (two 16-row loads per step). For GU, block
  // rows 0..63 are gate rows (waves 0, 1) and 64..127 up rows (waves 2, 3).
  const uint8_t *gate_c, *up_c;
  const uint16_t *gate_s, *up_s, *gate_b, *up_b;
  if (GU) {
    gate_c = sh ? a.shared.gate.codes : a.routed.gate.codes;
    up_c = sh ? a.shared.up.codes : a.routed.up.codes;
    gate_s = sh ? a.shared.gate.scales : a.routed.gate.scales;
    up_s = sh ? a.shared.up.scales : a.routed.up.scales;
    gate_b = sh ? a.shared.gate.biases : a.routed.gate.biases;
    up_b = sh ? a.shared.up.biases : a.routed.up.biases;
  } else {
    gate_c = up_c = sh ? a.shared.down.codes : a.routed.down.codes;
    gate_s = up_s = sh ? a.shared.down.scales : a.routed.down.scales;
    gate_b = up_b = sh ? a.shared.down.biases : a.routed.down.biases;
  }
  const size_t mrow0 = (size_t)mat * nrows_w + n0;  // first weight row of the block in its matrix
  const uint8_t* cbase = (GU && wave >= 2 ? up_c : gate_c) + mrow0 * (size_t)ldc;
  uint32_t coff[2];
  int cq16[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = 32 * wave + 16 * t + (lane >> 2);  // block row
    const int rl = GU ? (r & (kGuCols - 1)) : r;     // row within this matrix's block
    const int rc = min(rl, nrows_w - 1 - n0);        // rows past the matrix read its last row
    coff[t] = (uint32_t)rc * (uint32_t)ldc;
    cq16[t] = 16 * ((lane & 3) ^ code_swz(r));
  }
  // ---- scales / biases: wave w loads array (w >> 1) for block rows 64 (w & 1) .. +63
  const int sb_arr = wave >> 1;
  const uint16_t* sb_src[2];
  bool sb_rowvalid[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int p = 64 * (2 * (wave & 1) + t) + lane;  // index 2 * row + group within the array
    const int r = p >> 1;
    const int rl = GU ? (r & (kGuCols - 1)) : r;
    const bool up = GU && r >= kGuCols;
    sb_rowvalid[t] = n0 + rl < nrows_w;
    const uint16_t* arr = sb_arr ? (up ? up_b : gate_b) : (up ? up_s : gate_s);
    sb_src[t] = arr + (mrow0 + (sb_rowvalid[t] ? rl : 0)) * (size_t)ldg + (p & 1);
  }
  // ---- A rows: wave w loads rows 4 (w + 4 t) .. +3, lane j: row + (j >> 4), chunk slot j & 15
  const uint8_t* arow[MT];
  int achunk[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int r = 4 * (wave + 4 * t) + (lane >> 4);
    const int rr = min(r, rows - 1);
    const uint16_t* rp;
    if (GU) {
      int tok = sh ? (row0 - a.P + rr) : a.sorted_token[row0 + rr];
      tok = min(max(tok, 0), a.T - 1);
      rp = a.x + (size_t)tok * d;
    } else {
      rp = (sh ? a.hs + (size_t)(row0 - a.P) * Ie : a.h + (size_t)row0 * Ie) + (size_t)rr * Ie;
    }
    arow[t] = reinterpret_cast<const uint8_t*>(rp);
    achunk[t] = 16 * ((lane & 15) ^ a_swz(r));
  }
  const int amax = 2 * K - 16;  // last 16-byte chunk of a row

  auto issue = [&](int s, int st) __attribute__((always_inline)) {
    uint8_t* cdst = L.c[st] + wave * 2048;
#pragma unroll
    for (int t = 0; t < 2; ++t) dma16(cbase + coff[t] + min(64 * s + cq16[t], ldc - 16), cdst + 1024 * t);
    uint32_t* sdst = L.sb[st] + sb_arr * 256 + 128 * (wave & 1);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int g = 2 * s + (lane & 1);
      const bool ok = sb_rowvalid[t] && g < ldg;
      dma2(ok ? (const void*)(sb_src[t] + 2 * s) : (const void*)kZeroHalf, sdst + 64 * t);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) dma16(arow[t] + min(256 * s + achunk[t], amax), L.a[st] + 1024 * (wave + 4 * t));
  };

  const int n = lane & 15, kb = lane >> 4;
  // this lane's two weight rows in the block (subtiles 0 and 1)
  const int wrow0 = GU ? 16 * wave + n : 32 * wave + n;
  const int wrow1 = GU ? kGuCols + 16 * wave + n : 32 * wave + 16 + n;
  const int cread0 = wrow0 * 64 + 8 * (kb & 1), cread1 = wrow1 * 64 + 8 * (kb & 1);
  const int cswz0 = code_swz(wrow0), cswz1 = code_swz(wrow1);
  f32x4_t acc[2][MT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) acc[t][mm] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);

  auto compute = [&](int st) __attribute__((always_inline)) {
    const uint8_t* cs = L.c[st];
    const uint32_t* sb = L.sb[st];
    const uint8_t* as = L.a[st];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const int q = 2 * gg + (kb >> 1);
      const uint2 w0 = *reinterpret_cast<const uint2*>(cs + cread0 + 16 * (q ^ cswz0));
      const uint2 w1 = *reinterpret_cast<const uint2*>(cs + cread1 + 16 * (q ^ cswz1));
      f32x4_t tmp[2][MT], xs[MT];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint32_t c0 = kk ? w0.y : w0.x, c1 = kk ? w1.y : w1.x;
        const uint4 b0 = make_uint4(magic_pair(c0, 0), magic_pair(c0, 1), magic_pair(c0, 2), magic_pair(c0, 3));
        const uint4 b1 = make_uint4(magic_pair(c1, 0), magic_pair(c1, 1), magic_pair(c1, 2), magic_pair(c1, 3));
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) {
          const int r = 16 * mm + n, c = 8 * gg + 2 * kb + kk;
          const uint4 raw = *reinterpret_cast<const uint4*>(as + r * 256 + 16 * (c ^ a_swz(r)));
          const uint32_t v[4] = {raw.x, raw.y, raw.z, raw.w};
          uint32_t pr[4];
          repair8(v, pr);
          const uint4 av = make_uint4(pr[0], pr[1], pr[2], pr[3]);
          const f32x4_t z = f32x4_t{0.f, 0.f, 0.f, 0.f};
          tmp[0][mm] = mfma16x16x32(av, b0, kk == 0 ? z : tmp[0][mm]);
          tmp[1][mm] = mfma16x16x32(av, b1, kk == 0 ? z : tmp[1][mm]);
          xs[mm] = mfma16x16x32(raw, ones, kk == 0 ? z : xs[mm]);
        }
      }
      const float s0 = bf16lo(sb[2 * wrow0 + gg]), c0 = fmaf(-128.0f, s0, bf16lo(sb[256 + 2 * wrow0 + gg]));
      const float s1 = bf16lo(sb[2 * wrow1 + gg]), c1 = fmaf(-128.0f, s1, bf16lo(sb[256 + 2 * wrow1 + gg]));
#pragma unroll
      for (int mm = 0; mm < MT; ++mm)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[0][mm][r] = fmaf(c0, xs[mm][r], fmaf(s0, tmp[0][mm][r], acc[0][mm][r]));
          acc[1][mm][r] = fmaf(c1, xs[mm][r], fmaf(s1, tmp[1][mm][r], acc[1][mm][r]));
        }
    }
  };

  // Loads past the last step are issued anyway (clamped to it) so that every iteration issues
  // the same sequence; their data lands in stages that are not read again.
  constexpr int kOps = 2 + 2 + MT;  // loads one wave issues per step
  const int Sm = S - 1;
  issue(0, 0);
  issue(min(1, Sm), 1);
  issue(min(2, Sm), 2);
  auto iter = [&](int s, int j) __attribute__((always_inline)) {
    step_barrier<2 * kOps>();
    issue(min(s + 3, Sm), (j + 3) & 3);
    compute(j);
  };
  for (int s = 0; s < S; s += 4) {
    iter(s, 0);
    if (s + 1 < S) iter(s + 1, 1);
    if (s + 2 < S) iter(s + 2, 2);
    if (s + 3 < S) iter(s + 3, 3);
  }
  // the clamped loads past the end must land before the block (and its LDS) is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (GU) {
    uint16_t* hout = sh ? a.hs + (size_t)(row0 - a.P) * Ie : a.h + (size_t)row0 * Ie;
    const int col = n0 + 16 * wave + n;
#pragma unroll
    for (int mm = 0; mm < MT; ++mm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * mm + 4 * kb + r;
        if (row < rows) hout[(size_t)row * Ie + col] = f32_to_bf16(silu_mul(acc[0][mm][r], acc[1][mm][r]));
      }
  } else {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int col = n0 + 32 * wave + 16 * t + n;
      if (col >= d) continue;
#pragma unroll
      for (int mm = 0; mm < MT; ++mm)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mm + 4 * kb + r;
          if (row < rows) a.y_rows[(size_t)(row0 + row) * d + col] = acc[t][mm][r];
        }
    }
  }
}

template <bool GU>
__device__ __forceinline__ void gemm_block(const GemmArgs& a) {
  __shared__ __attribute__((aligned(16))) uint8_t c0[kCodeStageBytes], c1[kCodeStageBytes], c2[kCodeStageBytes],
      c3[kCodeStageBytes];
  __shared__ __attribute__((aligned(16))) uint32_t s0[kSbStageWords], s1[kSbStageWords], s2[kSbStageWords],
      s3[kSbStageWords];
  __shared__ __attribute__((aligned(16))) uint8_t a0[kAStageBytes], a1[kAStageBytes], a2[kAStageBytes],
      a3[kAStageBytes];
  const GemmLds L = {{c0, c1, c2, c3}, {s0, s1, s2, s3}, {a0, a1, a2, a3}};
  int nb, e, row0, rows;
  if (!block_tile(a, nb, e, row0, rows)) return;
  const int n0 = nb * (GU ? kGuCols : kDnCols);
  if (GU && n0 >= (e == a.E ? a.Is : a.I)) return;
  if (rows <= 16)
    tile_body<1, GU>(a, n0, e, row0, rows, L);
  else
    tile_body<2, GU>(a, n0, e, row0, rows, L);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gateup_gemm(GemmArgs a) {
  gemm_block<true>(a);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_down_gemm(GemmArgs a) {
  gemm_block<false>(a);
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
