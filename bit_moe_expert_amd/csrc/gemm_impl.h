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
//     tile count exit at once. Blocks are renumbered so that all column blocks of a tile run on
//     one XCD and read its A rows through that XCD's L2 (block_tile).
//
// Codes of 4, 3 or 2 bits (BITS): a weight row's codes are a little-endian bit stream; the
// kernels are templates on BITS, one translation unit per width, and differ only in how codes
// move to LDS and become "128 + q" pairs.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace moe {

constexpr int kBK = 128;             // inputs per K step
constexpr int kGuCols = 64;          // h columns per gate/up block (64 gate + 64 up weight rows)
constexpr int kDnCols = 128;         // output columns per down block
constexpr int kTileGroup = 2;        // tiles per XCD work unit

struct GemmArgs {
  int d, E, k, I, Is, T, P, max_tiles, nb;  // nb: runs of column blocks
  const uint16_t* xp;  // x, each 8-input chunk in pair order
  const int32_t* sorted_token;
  const int32_t* tiles;
  const int32_t* n_tiles;
  moe_ffn_q4 routed, shared;
  uint16_t* h;
  uint16_t* hs;
  uint16_t* y_rows;  // fp16 rows of the down product, each 32-column segment scaled by 2^-e ...
  uint8_t* y_exp;    // ... e per (row, segment)
  const float* xsum;  // [T][d/64] group sums of x (the bias term's factor on the gate/up side)
  float* hsum;        // [P][I/64] group sums of h (written by the gate/up epilogue, read by down)
  float* hsum_sh;     // [T][Is/64] the same for the shared expert's h
  float* dbg_g;  // check export of the gate/up kernel: fp32 g and u, [P][I] then [T][Is]
  float* dbg_u;
  float* dbg_y;  // check export of the down kernel: its fp32 rows, [P + T][d]
};

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Decode the block's (run of column blocks, tile) and validate the tile. Returns false when the
// block has nothing to do. Blocks are dealt to the 8 XCDs round-robin (block b runs on XCD
// b % 8); each XCD takes whole units of kTileGroup consecutive tiles with all their runs, so a
// tile's A rows are fetched into one L2 and served from there to every column block, and tiles of
// one expert within a unit share the weight rows. Units are dealt to the XCDs round-robin as well,
// which spreads the live tiles evenly whatever the grid's upper bound.
__device__ __forceinline__ bool block_tile(const GemmArgs& a, int& run, int& e, int& row0, int& rows) {
  const int xcd = blockIdx.x % 8, j = blockIdx.x / 8;
  const int unit_blocks = kTileGroup * a.nb;
  const int r = j % unit_blocks;
  const int ti = ((j / unit_blocks) * 8 + xcd) * kTileGroup + r / a.nb;
  run = r % a.nb;
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
// runs its two MFMA K-steps into a fresh accumulator and one FMA folds the group's scale into the
// running sum; the K loop needs the scales only. The bias terms of all groups form one small
// product per job, sum_g X[row][g] C[g][col] with C = b - 128 s, which the block runs on the matrix
// cores before its K loop: its operands (X from group sums computed once per row, for x by the pass
// that pairs it and for h by the gate/up epilogue; the scales and biases of the job's columns) are
// register loads issued ahead of the pipeline's first loads, so their latency hides under the
// pipeline's start. X and C are each split into a high and a low bf16 part (X_hi C_hi + X_hi C_lo +
// X_lo C_hi, 32 groups per v_mfma_f32_16x16x32_bf16): the dropped X_lo C_lo and the split leave a
// relative error near 2^-16 of the bias term, and none when X and C are bf16 values, as on
// exact-arithmetic inputs. The weight enters
// as s * q + b without rounding the weight itself to bf16 first (a difference of at most half a
// bf16 ulp per weight).
//
// Code words of the lane's 16 inputs (16 kb .. 16 kb + 15 of a group), as two words of 8 codes
// (inputs 16 kb .. + 7 and 16 kb + 8 .. + 15), code i of a word at bits [BITS i, BITS i + BITS):
//   4 bits: the two dwords at p;  2 bits: the halves of the dword at p;
//   3 bits: 6 bytes that start sh / 8 bytes after the 4-byte aligned p (sh = 0 or 16), taken from
//           the two dwords at p with funnel shifts.
template <int BITS>
__device__ __forceinline__ uint2 lane_codes(const uint8_t* p, uint32_t sh) {
  if constexpr (BITS == 4) return *reinterpret_cast<const uint2*>(p);
  const uint32_t* p32 = reinterpret_cast<const uint32_t*>(p);
  if constexpr (BITS == 2) {
    const uint32_t u = p32[0];
    return make_uint2(u, u >> 16);
  }
  const uint32_t d0 = p32[0], d1 = p32[1];
  const uint32_t lo = __builtin_amdgcn_alignbit(d1, d0, sh), hi = d1 >> sh;
  return make_uint2(lo, __builtin_amdgcn_alignbit(hi, lo, 24));
}

// The four "128 + q" pairs of a word of 8 codes: pair n holds inputs (n, n + 4), the pair order
// of the A operand. 4 bits: a shift and an and-or each. 2 bits: one byte permute first puts codes
// 0-3 in byte 0 and codes 4-7 in byte 2, so code n + 4 sits 16 bits above code n. 3 bits: codes
// n and n + 4 lie 12 bits apart; one shift and a bit-field insert move codes 4-7 up to bit 16.
template <int BITS>
__device__ __forceinline__ uint4 code_pairs8(uint32_t u) {
  if constexpr (BITS == 4)
    return make_uint4(magic_pair(u, 0), magic_pair(u, 1), magic_pair(u, 2), magic_pair(u, 3));
  constexpr uint32_t kMask = BITS == 2 ? 0x00030003u : 0x00070007u;
  const uint32_t t = BITS == 2 ? __builtin_amdgcn_perm(u, u, 0x0C010C00u) : ((u & 0xFFFu) | ((u << 4) & ~0xFFFu));
  const uint32_t m = opaque_v(kMask), g = opaque_v(0x43004300u);
  return make_uint4((t & m) | g, ((t >> BITS) & m) | g, ((t >> (2 * BITS)) & m) | g, ((t >> (3 * BITS)) & m) | g);
}

// Work item: one tile and a run of consecutive column blocks (gate/up: 64 h columns = 64 gate +
// 64 up weight rows; down: 128 output columns). The block streams the run's column blocks
// through one continuous pipeline, so the load latency at the start is paid once per run.
//
// Pipeline: every input goes straight from memory to LDS with direct loads (no registers on
// the way). A K step is 128 inputs (two quantisation groups).
//   - codes move per pair of K steps: 128 weight rows x 32 BITS bytes (for 4 bits a whole 128-byte
//     line of every row at once, which the memory system serves better than two 64-byte halves
//     a step apart). They go into a ring of two pair stages, issued at the first step of a pair
//     for the next pair. A row's codes move as 16-byte chunks (4 and 2 bits: 8 and 4 lanes per
//     row) or 12-byte chunks (3 bits, 8 lanes per row; the direct load places each lane's 12
//     bytes at a 16-byte stride in LDS); the chunks of a row are XOR-swizzled by row so the
//     MFMA-side reads spread over the banks. A job's steps are padded to an even count: the
//     padding step loads in-bounds stand-in data and multiplies nothing;
//   - scales: when K is whole steps, per pair of steps with the codes, into two pair stages:
//     two 4-byte loads per weight row (each a step's two groups), both lanes of a row in one
//     cache line and each wave loading its own 32 rows (a direct load's cost follows the cache
//     lines it touches, so one load per row and step, repeated by two waves, had cost a sixth
//     of the kernel). Otherwise per step, one 2-byte load per (row, group), each landing
//     zero-extended in its own dword;
//   - A rows (up to 32 gathered x rows, or h rows) of 256 bytes per step; the 16-byte chunks of
//     a row are XOR-swizzled by row. A rows past the tile's rows repeat its last row and only
//     reach accumulator rows that are never written out. Both x (paired once per call, before
//     the GEMMs) and h (written so by the gate/up epilogue) hold each chunk of 8 inputs in pair
//     order 0, 4, 1, 5, 2, 6, 3, 7, the order of the "128 + q" pairs, so A goes from LDS to the
//     matrix cores unchanged.
// A (and the per-step scales) run in a ring of AS stages, AS - 1 steps ahead.
// Addresses are a scalar base that advances per step plus a per-lane offset fixed for the run.
// When K is an odd number of groups, the last step's second group reads in-bounds stand-in data
// and is given scale 0 when it is multiplied. Weight rows past the down matrix repeat
// its last row; their outputs are not written. Loads complete in issue order, so before each
// barrier a wave waits until only the loads younger than the ones the step needs are
// outstanding: its part of the stages the step reads has then landed.
constexpr int kPairCodeStageBytes = 128 * 128;  // 128 weight rows x 256 inputs of codes (at most)
constexpr int kA16StageBytes = 16 * 256;        // 16 A rows x 128 bf16
constexpr int kRunGu = 1;                       // column blocks per gate/up work item
// column blocks per down work item: two when K is short (fewer than kRunMinSteps steps), so the
// pipeline start is paid over more steps; one otherwise, for more blocks and a lean loop
constexpr int kRunMinSteps = 6;
inline int down_run(int I) { return (I + kBK - 1) / kBK < kRunMinSteps ? 2 : 1; }

__device__ __forceinline__ int a_swz(int r) { return r & 7; }

// Direct loads are written as inline assembly: the compiler's own wait insertion cannot follow
// them across the loop back-edge and would drain every outstanding load before the first LDS
// read of each unrolled round. Completion is handled explicitly (step_barrier, and a full wait
// before the block ends). Address = 64-bit scalar base + 32-bit per-lane offset.
__device__ __forceinline__ uint32_t lds_addr(const void* l) {
  // wave-uniform by construction; readfirstlane puts it in a scalar register for m0
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)l);
}
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// The LDS destination is a wave-uniform 32-bit LDS address (the m0 value). The scalar operands come
// from v_readfirstlane, a vector instruction writing scalar registers, which a vector memory
// instruction may read only 5 wait states later; the compiler inserts such waits for its own
// loads but cannot see inside an asm statement, so the statement supplies them itself: the m0
// write and s_nop 3 (which also covers the one wait state a direct load needs after m0 is set).
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t l) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 3\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(uniform_ptr(base)),
               "s"(l)
               : "memory", "m0");
}
__device__ __forceinline__ void dma12(const void* base, uint32_t off, uint32_t l) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 3\n\tglobal_load_lds_dwordx3 %0, %1" ::"v"(off), "s"(uniform_ptr(base)),
               "s"(l)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t l) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 3\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(uniform_ptr(base)),
               "s"(l)
               : "memory", "m0");
}
__device__ __forceinline__ void dma2(const void* base, uint32_t off, uint32_t l) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 3\n\tglobal_load_lds_ushort %0, %1" ::"v"(off), "s"(uniform_ptr(base)),
               "s"(l)
               : "memory", "m0");
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
// PAIRED: K is a multiple of 128 (whole steps; scale/bias pairs load as one dword).
// MT: 16-row subtiles of A (1 for tiles of at most 16 rows, else 2); AS: depth of the A and
// scale ring, sized so that every layout fits the same LDS: 2 for MT = 2 (one step ahead),
// 3 for MT = 1 with an odd group count (two steps ahead), 4 for MT = 1 with whole steps (a pair
// of steps ahead, one barrier per pair).
template <int BITS, int MT, int AS, bool GU, bool PAIRED, int R, bool DBG, bool VEC8>
__device__ __forceinline__ void run_body(const GemmArgs& a, int run, int e, int row0, int rows, uint8_t* lds) {
  static_assert(AS == 2 || AS == 3 || (AS == 4 && MT == 1 && PAIRED), "A and scale ring depth");
  static_assert(!VEC8 || PAIRED, "a multiple of 8 groups is whole steps");
  constexpr int kSbBytes = 1024;            // without PAIRED: a scale stage per step
  constexpr int kSpBytes = 1024;            // with PAIRED: a scale stage per pair of steps
  constexpr int kAS = MT * kA16StageBytes;  // an A stage: 16 MT rows
  // codes of a pair of steps: 32 BITS bytes per weight row, kCB-byte chunks, kLPR lanes per row;
  // in LDS a chunk takes 16 bytes and a row kLRB bytes
  constexpr int kCB = BITS == 3 ? 12 : 16;
  constexpr int kLPR = BITS == 2 ? 4 : 8;
  constexpr int kLRB = 16 * kLPR;
  constexpr int kRPL = 64 / kLPR;        // rows per load instruction
  constexpr int kNL = 32 / kRPL;         // load instructions per wave and pair
  constexpr int kCPG = 8 * BITS / kCB;   // chunks per group
  static_assert(kCB * kLPR == 32 * BITS && kRPL * kLRB == 1024, "code chunking");
  // code pair stage st (0, 1), and stage st of the scales and of A, in the block's LDS
  const auto Lc = [lds](int st) { return lds + st * kPairCodeStageBytes; };
  const auto La = [lds](int st) { return lds + 2 * kPairCodeStageBytes + st * kAS; };
  const auto Lsb = [lds](int st) {
    return reinterpret_cast<uint32_t*>(lds + 2 * kPairCodeStageBytes + AS * kAS + st * (PAIRED ? kSpBytes : kSbBytes));
  };

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const bool sh = (e == a.E);
  const int Ie = sh ? a.Is : a.I;
  const int mat = sh ? 0 : e;
  const int d = a.d;
  const int K = GU ? d : Ie;        // reduction length
  const int ldc = K * BITS / 8;     // code bytes per weight row
  const int ldg = K / kGroup;       // groups per weight row
  const int nrows_w = GU ? Ie : d;  // weight rows of the matrix (per expert)
  const int S = (K + kBK - 1) / kBK;
  const int cols = GU ? kGuCols : kDnCols;
  const int ncb = (nrows_w + cols - 1) / cols;  // column blocks of this matrix
  const int nb0 = run * R;
  if (nb0 >= ncb) return;
  const int njobs = R == 1 ? 1 : min(R, ncb - nb0);

  // ---- weight matrices (for GU, waves 0, 1 load gate rows and waves 2, 3 up rows)
  const uint8_t* wc;
  const uint16_t* sb_arr;  // the scales this wave's direct loads read
  if (GU) {
    const bool upw = wave >= 2;
    wc = sh ? (upw ? a.shared.up.codes : a.shared.gate.codes) : (upw ? a.routed.up.codes : a.routed.gate.codes);
    // scale loads: with PAIRED wave w loads block rows 32 w .. 32 w + 31 (gate rows for w < 2, up
    // rows for w >= 2); otherwise block rows 64 (w & 1) .. +63, which are gate rows for w & 1 == 0
    // and up rows for w & 1 == 1 (waves 2, 3 repeat the loads of waves 0, 1 into the same slots)
    const bool ups = PAIRED ? wave >= 2 : (wave & 1) != 0;
    sb_arr = sh ? (ups ? a.shared.up.scales : a.shared.gate.scales) : (ups ? a.routed.up.scales : a.routed.gate.scales);
  } else {
    wc = sh ? a.shared.down.codes : a.routed.down.codes;
    sb_arr = sh ? a.shared.down.scales : a.routed.down.scales;
  }
  const size_t mrow = (size_t)mat * nrows_w;  // first row of this expert's matrix

  // ---- per-lane fixed offsets
  // codes: block row r = 32 wave + kRPL t + lane / kLPR, LDS slot lane % kLPR, which holds the
  // row's chunk (lane % kLPR) ^ (r % kLPR)
  int crow[kNL];
  uint32_t cq16[kNL];  // byte offset of that chunk in the row
#pragma unroll
  for (int t = 0; t < kNL; ++t) {
    const int r = 32 * wave + kRPL * t + lane / kLPR;
    crow[t] = GU ? (r & (kGuCols - 1)) : r;  // row within the column block's weight rows
    cq16[t] = kCB * ((lane % kLPR) ^ (r & (kLPR - 1)));
  }
  // scales: PAIRED: block row 32 wave + (lane >> 1), step lane & 1 of a pair; else (row, group) =
  // (p >> 1, p & 1) for p = 64 (2 (wave & 1) + t) + lane
  int srow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = PAIRED ? (32 * wave + (lane >> 1)) : ((64 * (2 * (wave & 1) + t) + lane) >> 1);
    srow[t] = GU ? (r & (kGuCols - 1)) : r;
  }
  // A: row 4 (wave + 4 t) + (lane >> 4), chunk slot lane & 15
  const uint16_t* abase;
  uint32_t aoff[MT], achk[MT];  // row offset, swizzled chunk offset within the step
  if (GU) {
    abase = a.xp;
  } else {
    abase = sh ? a.hs + (size_t)(row0 - a.P) * Ie : a.h + (size_t)row0 * Ie;
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int r = 4 * (wave + 4 * t) + (lane >> 4);
    const int rr = min(r, rows - 1);
    int arow;
    if (GU) {
      arow = sh ? (row0 - a.P + rr) : a.sorted_token[row0 + rr];
      arow = min(max(arow, 0), a.T - 1);
    } else {
      arow = rr;
    }
    aoff[t] = (uint32_t)arow * (uint32_t)(2 * K);
    achk[t] = 16u * (uint32_t)((lane & 15) ^ a_swz(r));
  }

  const int S2 = (S + 1) & ~1;
  const int SP = S2 / 2;  // code pairs per job

  // Load state of the job being issued, set once per job: uniform bases of its column block and
  // per-lane offsets (weight rows past the matrix repeat its last row). Destinations are 32-bit
  // LDS addresses: this wave's part of stage 0, plus the stage and load offsets.
  const uint32_t lbase = lds_addr(lds);
  const uint32_t lds_c = lbase + wave * (32 * kLRB);
  const uint32_t lds_a = lbase + 2 * kPairCodeStageBytes + wave * 1024;
  const uint32_t lds_s = lbase + 2 * kPairCodeStageBytes + AS * kAS + (PAIRED ? 256 * wave : 512 * (wave & 1));
  const uint8_t* cjb;
  uint32_t coq[kNL];  // codes: row offset + swizzled chunk
  const uint8_t* spb;  // PAIRED: the scale pairs move with the codes (base of the code job's rows)
  uint32_t spo;        // ... and this lane's offset: its row, plus 4 bytes for a pair's second step
  auto setup_codes = [&](int j) __attribute__((always_inline)) {
    const int n0 = (nb0 + j) * cols;
    const int lim = nrows_w - 1 - n0;
    cjb = wc + (mrow + n0) * (size_t)ldc;
#pragma unroll
    for (int t = 0; t < kNL; ++t) coq[t] = (uint32_t)min(crow[t], lim) * (uint32_t)ldc + cq16[t];
    if (PAIRED) {
      spb = reinterpret_cast<const uint8_t*>(sb_arr + (mrow + n0) * (size_t)ldg);
      spo = (uint32_t)min(srow[0], lim) * (uint32_t)(2 * ldg) + 4u * (uint32_t)(lane & 1);
    }
  };
  const uint16_t* sjb;
  uint32_t so[2];  // scale offsets in bytes
  auto setup_sb = [&](int j) __attribute__((always_inline)) {
    const int n0 = (nb0 + j) * cols;
    const int lim = nrows_w - 1 - n0;
    sjb = sb_arr + (mrow + n0) * (size_t)ldg;
    if (!PAIRED) {
#pragma unroll
      for (int t = 0; t < 2; ++t) so[t] = ((uint32_t)min(srow[t], lim) * (uint32_t)ldg + (uint32_t)(lane & 1)) * 2u;
    }
  };
  uint32_t aq[MT];  // A: row offset + swizzled chunk
#pragma unroll
  for (int t = 0; t < MT; ++t) aq[t] = aoff[t] + achk[t];
  const uint32_t vlast = (uint32_t)(ldc - 32 * BITS * (SP - 1));  // code bytes of a job's last pair (8 BITS .. 32 BITS)

  // issue the code loads of pair ss of the current code job into code stage st
  auto issue_codes = [&](int ss, int st) __attribute__((always_inline)) {
    const uint8_t* cb = cjb + 32 * BITS * ss;
    const uint32_t dst = lds_c + st * kPairCodeStageBytes;
    const auto dma = [&](uint32_t off, uint32_t l) __attribute__((always_inline)) {
      if constexpr (BITS == 3)
        dma12(cb, off, l);
      else
        dma16(cb, off, l);
    };
    if (ss == SP - 1 && vlast < (uint32_t)(32 * BITS)) {
#pragma unroll
      for (int t = 0; t < kNL; ++t) {
        uint32_t q = cq16[t];
        // chunks past K re-read a chunk of the pair's first group
        if (q + (uint32_t)kCB > vlast) q = (uint32_t)kCB * ((q / (uint32_t)kCB) % (uint32_t)kCPG);
        dma(coq[t] - cq16[t] + q, dst + 1024 * t);
      }
    } else {
#pragma unroll
      for (int t = 0; t < kNL; ++t) dma(coq[t], dst + 1024 * t);
    }
    if (PAIRED) {
      // the pair's scale dwords (a step's two groups each); a pair whose second step is past K
      // reads its first step's dword twice
      const uint32_t off = 2 * ss + 1 < S ? spo : spo - 4u * (uint32_t)(lane & 1);
      dma4(spb + 8 * ss, off, lds_s + st * kSpBytes);
    }
  };
  // issue the A and scale loads of step s of the current job into stage st; the padding step
  // (s == S) re-reads step S - 1
  auto issue = [&](int s, int st) __attribute__((always_inline)) {
    s = min(s, S - 1);
    const bool tail = !PAIRED && s == S - 1 && (ldg & 1);
    const uint32_t sdst = lds_s + st * kSbBytes;
    if (!PAIRED) {
#pragma unroll
      for (int t = 0; t < 2; ++t) dma2(sjb + 2 * s, tail ? so[t] - 2u * (uint32_t)(lane & 1) : so[t], sdst + 256 * t);
    }
    const uint16_t* ab = abase + 128 * s;
    const uint32_t adst = lds_a + st * kAS;
#pragma unroll
    for (int t = 0; t < MT; ++t)  // chunks past K re-read the first half
      dma16(ab, tail ? aoff[t] + (achk[t] & 127u) : aq[t], adst + 4096 * t);
  };

  const int n = lane & 15, kb = lane >> 4;
  // this lane's two weight rows in the block (subtiles 0 and 1)
  const int wrow0 = GU ? 16 * wave + n : 32 * wave + n;
  const int wrow1 = GU ? kGuCols + 16 * wave + n : 32 * wave + 16 + n;
  // code read offsets within a pair stage for group G = 2 h + gg of the pair (h: second step of the
  // pair): the lane's 16 codes start at stream byte 8 BITS G + 2 BITS kb of the row, in its chunk
  // c (LDS slot c ^ (row % kLPR)); 3 bits read the 4-byte aligned 8 bytes that hold those 6
  uint32_t crd[2][4];
#pragma unroll
  for (int G = 0; G < 4; ++G) {
    const int sbyte = 8 * BITS * G + 2 * BITS * kb;
    const int c = sbyte / kCB;
    const int o = BITS == 3 ? 4 * (kb & 1) : sbyte % kCB;
    crd[0][G] = wrow0 * kLRB + 16 * (c ^ (wrow0 & (kLPR - 1))) + o;
    crd[1][G] = wrow1 * kLRB + 16 * (c ^ (wrow1 & (kLPR - 1))) + o;
  }
  const uint32_t csh = 16u * (uint32_t)(kb & 1);  // 3 bits: where the 6 bytes start in the 8
  f32x4_t acc[2][MT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) acc[t][mm] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // step of A/scale stage st, codes from stage cst, second step of its pair when h
  auto compute = [&](int st, int cst, int h, bool half) __attribute__((always_inline)) {
    const uint8_t* cs = Lc(cst);
    const uint32_t* sb = Lsb(PAIRED ? cst : st);
    const uint8_t* as = La(st);
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const uint2 w0 = lane_codes<BITS>(cs + crd[0][2 * h + gg], csh);
      const uint2 w1 = lane_codes<BITS>(cs + crd[1][2 * h + gg], csh);
      f32x4_t tmp[2][MT];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint32_t c0 = kk ? w0.y : w0.x, c1 = kk ? w1.y : w1.x;
        const uint4 b0 = code_pairs8<BITS>(c0);
        const uint4 b1 = code_pairs8<BITS>(c1);
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) {
          const int r = 16 * mm + n, c = 8 * gg + 2 * kb + kk;
          const uint4 av = *reinterpret_cast<const uint4*>(as + r * 256 + 16 * (c ^ a_swz(r)));
          const f32x4_t z = f32x4_t{0.f, 0.f, 0.f, 0.f};
          tmp[0][mm] = mfma16x16x32(av, b0, kk == 0 ? z : tmp[0][mm]);
          tmp[1][mm] = mfma16x16x32(av, b1, kk == 0 ? z : tmp[1][mm]);
        }
      }
      float s0, s1;
      if (PAIRED) {
        const uint32_t sc0 = sb[2 * wrow0 + h], sc1 = sb[2 * wrow1 + h];
        s0 = gg ? bf16hi(sc0) : bf16lo(sc0);
        s1 = gg ? bf16hi(sc1) : bf16lo(sc1);
      } else {
        s0 = bf16lo(sb[2 * wrow0 + gg]);
        s1 = bf16lo(sb[2 * wrow1 + gg]);
        if (gg == 1 && half) s0 = s1 = 0.0f;  // the group past K adds nothing
      }
#pragma unroll
      for (int mm = 0; mm < MT; ++mm)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[0][mm][r] = fmaf(s0, tmp[0][mm][r], acc[0][mm][r]);
          acc[1][mm][r] = fmaf(s1, tmp[1][mm][r], acc[1][mm][r]);
        }
    }
  };

  // ---- bias terms: acc += X C for the job's columns, as split-bf16 products (see above). Lane
  // (n, kb) holds groups 8 kb .. 8 kb + 7 (of a chunk of 32) of tile row 16 mm + n (X, A operand)
  // and of the column n of each of its two subtiles (C, B operand).
  const float* xs_row[MT];  // group sums of the tile rows of the lane's A fragments
#pragma unroll
  for (int mm = 0; mm < MT; ++mm) {
    const int r = min(16 * mm + n, rows - 1);
    if (GU) {
      int tok = sh ? (row0 - a.P + r) : a.sorted_token[row0 + r];
      tok = min(max(tok, 0), a.T - 1);
      xs_row[mm] = a.xsum + (size_t)tok * (size_t)ldg;
    } else {
      xs_row[mm] = sh ? a.hsum_sh + (size_t)(row0 - a.P + r) * (size_t)ldg : a.hsum + (size_t)(row0 + r) * (size_t)ldg;
    }
  }
  // scales and biases of the two column subtiles (gate/up: the gate and the up matrix)
  const uint16_t* const bsc0 = GU ? (sh ? a.shared.gate.scales : a.routed.gate.scales)
                                  : (sh ? a.shared.down.scales : a.routed.down.scales);
  const uint16_t* const bbi0 = GU ? (sh ? a.shared.gate.biases : a.routed.gate.biases)
                                  : (sh ? a.shared.down.biases : a.routed.down.biases);
  const uint16_t* const bsc1 = GU ? (sh ? a.shared.up.scales : a.routed.up.scales) : bsc0;
  const uint16_t* const bbi1 = GU ? (sh ? a.shared.up.biases : a.routed.up.biases) : bbi0;
  // Groups gl .. gl + 7 (gl a multiple of 8) of a row of ldg values, those past the row 0, without
  // branches (a branch would make the compiler drain the loads at its join): every load reads an
  // in-bounds address, clamped to the row, and a select zeroes what lies past it. VEC8 (ldg a
  // multiple of 8): the 8 values are one aligned 16-byte load (two for fp32); whole K steps (ldg
  // even): 4-byte pairs; otherwise single values.
  const auto load8 = [&](const uint16_t* rowp, int gl) __attribute__((always_inline)) -> uint4 {
    if constexpr (VEC8) {
      const uint4 v = *reinterpret_cast<const uint4*>(rowp + min(gl, ldg - 8));
      const bool in = gl < ldg;
      return make_uint4(in ? v.x : 0u, in ? v.y : 0u, in ? v.z : 0u, in ? v.w : 0u);
    }
    uint32_t w[4];
    if constexpr (PAIRED) {
      const uint32_t* r32 = reinterpret_cast<const uint32_t*>(rowp);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g = gl + 2 * q;
        const uint32_t v = r32[min(g, ldg - 2) >> 1];
        w[q] = g < ldg ? v : 0u;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g = gl + 2 * q;
        const uint32_t lo = rowp[min(g, ldg - 1)], hi = rowp[min(g + 1, ldg - 1)];
        w[q] = (g < ldg ? lo : 0u) | ((g + 1 < ldg ? hi : 0u) << 16);
      }
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  };
  struct BiasOps {
    float x[MT][8];      // group sums of the lane's rows
    uint4 sc[2], bi[2];  // scales and biases of the lane's two columns (bf16)
  };
  const auto bias_load = [&](BiasOps& o, int j, int g0, bool want_x) __attribute__((always_inline)) {
    const int gl = g0 + 8 * kb;
    const int n0 = (nb0 + j) * cols;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int wr = t ? wrow1 : wrow0;
      const int rm = GU ? (wr & (kGuCols - 1)) : wr;  // row within the column block of its matrix
      const size_t row = mrow + (size_t)min(n0 + rm, nrows_w - 1);
      o.sc[t] = load8((t ? bsc1 : bsc0) + row * (size_t)ldg, gl);
      o.bi[t] = load8((t ? bbi1 : bbi0) + row * (size_t)ldg, gl);
    }
    if (want_x) {
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) {
        if constexpr (VEC8) {
          const float* xp8 = xs_row[mm] + min(gl, ldg - 8);
          const float4 v0 = reinterpret_cast<const float4*>(xp8)[0], v1 = reinterpret_cast<const float4*>(xp8)[1];
          const bool in = gl < ldg;
          const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) o.x[mm][i] = in ? v[i] : 0.0f;
        } else if constexpr (PAIRED) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int g = gl + 2 * q;
            const float2 v = *reinterpret_cast<const float2*>(xs_row[mm] + min(g, ldg - 2));
            o.x[mm][2 * q] = g < ldg ? v.x : 0.0f;
            o.x[mm][2 * q + 1] = g < ldg ? v.y : 0.0f;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float v = xs_row[mm][min(gl + i, ldg - 1)];
            o.x[mm][i] = gl + i < ldg ? v : 0.0f;
          }
        }
      }
    }
  };
  // X (this lane's rows) split once per chunk, then the products for the columns of `o` into dst
  const auto bias_mfma = [&](const BiasOps& o, const BiasOps& xo, f32x4_t (&dst)[2][MT]) __attribute__((always_inline)) {
    uint4 chi[2], clo[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t sv[4] = {o.sc[t].x, o.sc[t].y, o.sc[t].z, o.sc[t].w};
      const uint32_t bv[4] = {o.bi[t].x, o.bi[t].y, o.bi[t].z, o.bi[t].w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float c0 = fmaf(-128.0f, bf16lo(sv[q]), bf16lo(bv[q]));
        const float c1 = fmaf(-128.0f, bf16hi(sv[q]), bf16hi(bv[q]));
        hi[q] = pack_bf16x2(c0, c1);
        lo[q] = pack_bf16x2(c0 - bf16lo(hi[q]), c1 - bf16hi(hi[q]));
      }
      chi[t] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      clo[t] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      const float* v = xo.x[mm];
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        hi[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
        lo[q] = pack_bf16x2(v[2 * q] - bf16lo(hi[q]), v[2 * q + 1] - bf16hi(hi[q]));
      }
      const uint4 xhi = make_uint4(hi[0], hi[1], hi[2], hi[3]), xlo = make_uint4(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        dst[t][mm] = mfma16x16x32(xhi, chi[t], dst[t][mm]);
        dst[t][mm] = mfma16x16x32(xhi, clo[t], dst[t][mm]);
        dst[t][mm] = mfma16x16x32(xlo, chi[t], dst[t][mm]);
      }
    }
  };

  // gate/up: the sums of this wave's 16 h columns for each accumulator row of the lane (the same in
  // all 16 lanes of a DPP row), combined across the 4 waves after the loop into hsum
  float hpart[MT][4];
  // with two jobs (down), the bias terms of the second one, added when it starts
  f32x4_t bnext[2][MT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) bnext[t][mm] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto finish = [&](int j) __attribute__((always_inline)) {
    const int n0 = (nb0 + j) * cols;
    if (GU && DBG) {
      // the accumulators themselves (natural column order), before the activation
      const size_t base = sh ? (size_t)a.P * a.I + (size_t)(row0 - a.P) * Ie : (size_t)row0 * Ie;
      const int col = n0 + 16 * wave + n;
#pragma unroll
      for (int mm = 0; mm < MT; ++mm)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mm + 4 * kb + r;
          if (row < rows) {
            a.dbg_g[base + (size_t)row * Ie + col] = acc[0][mm][r];
            a.dbg_u[base + (size_t)row * Ie + col] = acc[1][mm][r];
          }
        }
    } else if (GU) {
      uint16_t* hout = sh ? a.hs + (size_t)(row0 - a.P) * Ie : a.h + (size_t)row0 * Ie;
      // h is stored in pair order, so that the down GEMM reads it as its A operand unchanged
      const int col = pair_pos(n0 + 16 * wave + n);
#pragma unroll
      for (int mm = 0; mm < MT; ++mm)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mm + 4 * kb + r;
          const uint16_t hb = f32_to_bf16(silu_mul(acc[0][mm][r], acc[1][mm][r]));
          if (row < rows) hout[(size_t)row * Ie + col] = hb;
          // the rounded value enters the down product, so it is what the group sum adds
          float v = bf16_to_f32(hb);
          v += dpp_f32<0xB1>(v);
          v += dpp_f32<0x4E>(v);
          v += dpp_f32<0x124>(v);
          v += dpp_f32<0x128>(v);
          hpart[mm][r] = v;
        }
    } else if (DBG) {
      // the check export: the fp32 rows themselves
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int col = n0 + 32 * wave + 16 * t + n;
        if (col >= d) continue;
#pragma unroll
        for (int mm = 0; mm < MT; ++mm)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * mm + 4 * kb + r;
            if (row < rows) a.dbg_y[(size_t)(row0 + row) * d + col] = acc[t][mm][r];
          }
      }
    } else if (n0 + 32 * wave < d) {  // d is a multiple of 64: the wave's 32 columns are whole
      // fp16 rows. The wave's 32 columns of a row form one segment with an exponent e >= 0 that
      // keeps the segment's largest magnitude below 2^15; the segment is stored as
      // fp16(v * 2^-e) (the scaling is exact), so any fp32 range survives with fp16's 11-bit
      // precision, and e goes to y_exp. First a 4 x 4 transpose within each quad of lanes turns the
      // MFMA layout (lane = column, register = row) into 4 consecutive columns of one row per lane
      // (row 4 kb + (n & 3), columns 4 (n >> 2) .. + 3 of each 16-column half), so each lane
      // stores 8 bytes per half. The lane shuffles run in every lane, outside any condition.
      const int cw = n0 + 32 * wave;
      const bool q0 = (n & 1) != 0, q1 = (n & 2) != 0;
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) {
        float tv[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const f32x4_t m = acc[t][mm];
          const float s0 = quad_swap<0xB1>(m[0]), s1 = quad_swap<0xB1>(m[1]);  // quad_perm 1,0,3,2
          const float s2 = quad_swap<0xB1>(m[2]), s3 = quad_swap<0xB1>(m[3]);
          const float b0 = q0 ? s1 : m[0], b1 = q0 ? m[1] : s0, b2 = q0 ? s3 : m[2], b3 = q0 ? m[3] : s2;
          const float u0 = quad_swap<0x4E>(b0), u1 = quad_swap<0x4E>(b1);  // quad_perm 2,3,0,1
          const float u2 = quad_swap<0x4E>(b2), u3 = quad_swap<0x4E>(b3);
          tv[t][0] = q1 ? u2 : b0;
          tv[t][1] = q1 ? u3 : b1;
          tv[t][2] = q1 ? b2 : u0;
          tv[t][3] = q1 ? b3 : u1;
        }
        // the exponent field of the row's largest magnitude (max ignores NaN): the lane's 8 values,
        // then lanes n + 4, n + 8 (mod 16), which hold the same row
        float mx = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(tv[t][r]));
        uint32_t be = __float_as_uint(mx) >> 23;
        be = max(be, dpp_u32<0x124>(be));  // row_ror 4
        be = max(be, dpp_u32<0x128>(be));  // row_ror 8
        // the largest magnitude is below 2^(be - 126), so e = be - 141 brings it below 2^15
        const int e = max(0, (int)be - 141);
        const int row = 16 * mm + 4 * kb + (n & 3);
        if (row < rows) {
          uint16_t* yr = a.y_rows + (size_t)(row0 + row) * d + cw + 4 * (n >> 2);
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = __builtin_ldexpf(tv[t][r], -e);
            *reinterpret_cast<uint2*>(yr + 16 * t) = make_uint2(pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]));
          }
          if ((n >> 2) == 0) a.y_exp[(size_t)(row0 + row) * (d / 32) + cw / 32] = (uint8_t)e;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int mm = 0; mm < MT; ++mm) {
        acc[t][mm] = R > 1 ? bnext[t][mm] : f32x4_t{0.f, 0.f, 0.f, 0.f};  // the next job starts from its bias terms
        if (R > 1) bnext[t][mm] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
  };

  // Positions run over (job, step) with each job's steps padded to an even count S2, so every
  // code pair is two positions. Positions past the end issue clamped re-loads of the last
  // position (same sequence every iteration); their data lands in a stage that is not read
  // again. Issue order per position p: A/scales of p + AS - 1, then, at the first step of a
  // pair, the codes of the next pair. With AS = 3 the loads younger than the ones a position
  // needs are one position's A/scales at an even position, and those plus one pair's codes at an
  // odd one; with AS = 2 they are nothing at an even position and one pair's codes at an odd one.
  // A stage is overwritten only after the barrier that follows its last read.
  constexpr int kOpsA = (PAIRED ? 0 : 2) + MT;  // A (and without PAIRED scale) loads one wave issues per position
  constexpr int kOpsC = kNL + (PAIRED ? 1 : 0);  // code (and with PAIRED scale) loads one wave issues per pair
  const int P2 = njobs * S2;
  int ij = 0, is = 0;    // position being issued (job, step); stays at the last position
  int icj = 0, ics = 0;  // code pair being issued (job, pair); stays at the last pair
  int cj = 0, cs = 0;    // position being computed
  // the first chunk of bias operands goes out before the pipeline's first loads; the products run
  // once those operands are in (the stage loads stay in flight meanwhile)
  BiasOps bo0, bo1;
  bias_load(bo0, 0, 0, true);
  if (R > 1 && njobs > 1) bias_load(bo1, 1, 0, false);
  setup_codes(0);
  setup_sb(0);
  issue_codes(0, 0);
  issue(0, 0);
  if (AS >= 3) {
    is = 1;  // S2 >= 2
    issue(1, 1);
  }
  // keep the products (and the wait for their operands) after the pipeline's first loads
  __builtin_amdgcn_sched_barrier(0);
  bias_mfma(bo0, bo0, acc);
  if (R > 1 && njobs > 1) bias_mfma(bo1, bo0, bnext);
  for (int g0 = 32; g0 < ldg; g0 += 32) {  // more than 32 groups: the further chunks in turn
    bias_load(bo0, 0, g0, true);
    bias_mfma(bo0, bo0, acc);
    if (R > 1 && njobs > 1) {
      bias_load(bo1, 1, g0, false);
      bias_mfma(bo1, bo0, bnext);
    }
  }
  if constexpr (AS == 4) {
    // Positions are pairs of steps, one barrier per pair: position i computes pair i from code
    // stage i & 1 and A/scale stages 2 (i & 1), 2 (i & 1) + 1, after issuing pair i + 1 into the
    // other halves of the rings. Every load a position needs was issued one position earlier,
    // and nothing younger is outstanding, so the barrier waits for all of this wave's loads.
    is = 0;  // first step of the pair being issued
    const int NP = njobs * SP;
    for (int p = 0; p < NP; p += 2) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (q == 0 || p + q < NP) {
          step_barrier<0>();
          if (is < S2 - 2) {
            is += 2;
          } else if (R > 1 && ij < njobs - 1) {
            is = 0;
            setup_sb(++ij);
          }
          issue(is, 2 * ((q + 1) & 1));
          issue(is + 1, 2 * ((q + 1) & 1) + 1);
          if (ics < SP - 1) {
            ++ics;
          } else if (R > 1 && icj < njobs - 1) {
            ics = 0;
            setup_codes(++icj);
          }
          issue_codes(ics, (q + 1) & 1);
          if (cs < S) compute(2 * q, q, 0, false);
          if (cs + 1 < S) compute(2 * q + 1, q, 1, false);
          if (cs == S2 - 2) {
            finish(cj);
            cs = 0;
            ++cj;
          } else {
            cs += 2;
          }
        }
      }
    }
  } else {
  constexpr int kWaitEven = AS == 3 ? kOpsA : 0, kWaitOdd = kWaitEven + kOpsC;
  // kUnroll positions per iteration, a multiple of 2 AS (A stage q % AS) and of 4 (code stage
  // (q >> 1) & 1: real pair i is issued as the i-th pair, into stage i & 1)
  constexpr int kUnroll = AS == 3 ? 12 : 4;
  for (int p = 0; p < P2; p += kUnroll) {
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
      if (q == 0 || p + q < P2) {
        if (q & 1)
          step_barrier<kWaitOdd>();
        else
          step_barrier<kWaitEven>();
        if (is < S2 - 1) {
          ++is;
        } else if (R > 1 && ij < njobs - 1) {
          is = 0;
          setup_sb(++ij);
        }
        issue(is, (q + AS - 1) % AS);
        if ((q & 1) == 0) {
          if (ics < SP - 1) {
            ++ics;
          } else if (R > 1 && icj < njobs - 1) {
            ics = 0;
            setup_codes(++icj);
          }
          issue_codes(ics, ((q >> 1) + 1) & 1);  // the (pos / 2 + 1)-th pair issued
        }
        if (cs < S) compute(q % AS, (q >> 1) & 1, q & 1, !PAIRED && cs == S - 1 && (ldg & 1));
        if (cs == S2 - 1) {
          finish(cj);
          cs = 0;
          ++cj;
        } else {
          ++cs;
        }
      }
    }
  }
  }
  // the clamped loads past the end must land before the block (and its LDS) is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (GU && !DBG) {
    // group sums of h: the block's 64 h columns are one group of the down product's reduction;
    // the 4 waves' partial sums meet in LDS (every load has landed and every read is done after
    // the barrier) and are added in wave order
    __syncthreads();
    float* s_part = reinterpret_cast<float*>(lds);  // [4 waves][16 MT rows]
    if (n == 0) {
#pragma unroll
      for (int mm = 0; mm < MT; ++mm)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_part[wave * 16 * MT + 16 * mm + 4 * kb + r] = hpart[mm][r];
    }
    __syncthreads();
    if (tid < 16 * MT && tid < rows) {
      const float v = ((s_part[tid] + s_part[16 * MT + tid]) + s_part[32 * MT + tid]) + s_part[48 * MT + tid];
      const int grp = nb0;  // column block = group of 64 h columns (one job per gate/up block)
      if (sh)
        a.hsum_sh[(size_t)(row0 - a.P + tid) * (size_t)(Ie / kGroup) + grp] = v;
      else
        a.hsum[(size_t)(row0 + tid) * (size_t)(Ie / kGroup) + grp] = v;
    }
  }
}

template <int BITS, bool GU, bool PAIRED, int R, bool DBG, bool VEC8>
__device__ __forceinline__ void gemm_block(const GemmArgs& a) {
  constexpr int kScB = PAIRED ? 0 : 1024;  // scale stage per step (without PAIRED)
  constexpr int kSpB = PAIRED ? 2048 : 0;  // two scale stages per pair of steps (PAIRED)
  // One LDS buffer, carved per tile height: two code pair stages, then four 16-row A stages
  // (tiles of at most 16 rows, whole steps), three 16-row A stages and three scale stages (at most
  // 16 rows, K an odd number of groups), or two 32-row A stages (and two scale stages without
  // PAIRED); with PAIRED the two scale pair stages last.
  constexpr int kLds1 = 2 * kPairCodeStageBytes + 3 * (kA16StageBytes + kScB) + kSpB;
  constexpr int kLds2 = 2 * kPairCodeStageBytes + 2 * (2 * kA16StageBytes + kScB) + kSpB;
  constexpr int kLds4 = PAIRED ? 2 * kPairCodeStageBytes + 4 * kA16StageBytes + kSpB : 0;
  constexpr int kLds12 = kLds1 > kLds2 ? kLds1 : kLds2;
  constexpr int kLds = kLds12 > kLds4 ? kLds12 : kLds4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  int run, e, row0, rows;
  if (!block_tile(a, run, e, row0, rows)) return;
  // the tile is the same for the whole block: keep it (and all that derives from it) scalar
  run = __builtin_amdgcn_readfirstlane(run);
  e = __builtin_amdgcn_readfirstlane(e);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  rows = __builtin_amdgcn_readfirstlane(rows);
  if (rows <= 16)
    run_body<BITS, 1, PAIRED ? 4 : 3, GU, PAIRED, R, DBG, VEC8>(a, run, e, row0, rows, lds);
  else
    run_body<BITS, 2, 2, GU, PAIRED, R, DBG, VEC8>(a, run, e, row0, rows, lds);
}

// DBG: the check export (fp32 pre-activations instead of h). VEC8: the reduction is a multiple of
// 8 groups (512 inputs), so the bias operands load as aligned 16-byte vectors.
template <int BITS, bool PAIRED, bool DBG, bool VEC8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_gateup_gemm(GemmArgs a) {
  gemm_block<BITS, true, PAIRED, kRunGu, DBG, VEC8>(a);
}

// DBG: the check export (the fp32 rows instead of fp16 rows and exponents).
template <int BITS, bool PAIRED, int R, bool DBG, bool VEC8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_down_gemm(GemmArgs a) {
  gemm_block<BITS, false, PAIRED, R, DBG, VEC8>(a);
}

inline GemmArgs gemm_args(const Ctx& c, int nruns) {
  GemmArgs a;
  a.d = c.d;
  a.E = c.E;
  a.k = c.k;
  a.I = c.I;
  a.Is = c.Is;
  a.T = c.T;
  a.P = c.P;
  a.max_tiles = c.max_tiles;
  a.nb = nruns;
  a.xp = c.xp;
  a.sorted_token = c.r.sorted_token;
  a.tiles = c.r.tiles;
  a.n_tiles = c.r.n_tiles;
  a.routed = c.routed;
  a.shared = c.shared;
  a.h = c.h;
  a.hs = c.hs;
  a.y_rows = c.y_rows;
  a.y_exp = c.y_exp;
  a.dbg_y = c.dbg_y;
  a.xsum = c.xsum;
  a.hsum = c.hsum;
  a.hsum_sh = c.hsum_sh;
  a.dbg_g = c.dbg_g;
  a.dbg_u = c.dbg_u;
  return a;
}

// Every (tile < max_tiles, run) pair has one block (see block_tile).
inline int grid_blocks(int max_tiles, int nruns) {
  const int units = (max_tiles + kTileGroup - 1) / kTileGroup;
  return ((units + 7) / 8) * 8 * kTileGroup * nruns;
}

template <int BITS>
hipError_t launch_gateup_gemm_bits(const Ctx& c) {
  const int ncb = (max(c.I, c.Is) + kGuCols - 1) / kGuCols;
  const int nruns = (ncb + kRunGu - 1) / kRunGu;
  const dim3 grid(grid_blocks(c.max_tiles, nruns));
  const bool dbg = c.dbg_g != nullptr;
  const bool vec8 = c.d % (8 * kGroup) == 0;
  const auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(256), 0, c.stream, gemm_args(c, nruns)); };
  if (vec8)
    dbg ? go(k_gateup_gemm<BITS, true, true, true>) : go(k_gateup_gemm<BITS, true, false, true>);
  else if (c.d % kBK == 0)
    dbg ? go(k_gateup_gemm<BITS, true, true, false>) : go(k_gateup_gemm<BITS, true, false, false>);
  else
    dbg ? go(k_gateup_gemm<BITS, false, true, false>) : go(k_gateup_gemm<BITS, false, false, false>);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_down_gemm_bits(const Ctx& c) {
  const int ncb = (c.d + kDnCols - 1) / kDnCols;
  const bool dbg = c.dbg_y != nullptr;
  const int R = down_run(c.I);
  const int nruns = (ncb + R - 1) / R;
  const dim3 grid(grid_blocks(c.max_tiles, nruns));
  // both the routed and the shared matrix must be whole steps for the paired form, and multiples
  // of 8 groups for the vector form
  const bool paired = c.I % kBK == 0 && (c.Is == 0 || c.Is % kBK == 0);
  const bool vec8 = c.I % (8 * kGroup) == 0 && (c.Is == 0 || c.Is % (8 * kGroup) == 0);
  const GemmArgs a = gemm_args(c, nruns);
  const auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(256), 0, c.stream, a); };
  // the check export runs the same block shapes with fp32 rows out
  const auto pick = [&](auto dbg_tag) {
    constexpr bool D = decltype(dbg_tag)::value;
    if (vec8)
      R == 1 ? go(k_down_gemm<BITS, true, 1, D, true>) : go(k_down_gemm<BITS, true, 2, D, true>);
    else if (paired)
      R == 1 ? go(k_down_gemm<BITS, true, 1, D, false>) : go(k_down_gemm<BITS, true, 2, D, false>);
    else
      R == 1 ? go(k_down_gemm<BITS, false, 1, D, false>) : go(k_down_gemm<BITS, false, 2, D, false>);
  };
  if (dbg)
    pick(std::true_type{});
  else
    pick(std::false_type{});
  return hipGetLastError();
}

}  // namespace moe
