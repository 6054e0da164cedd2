// GEMMs with a 384 x 256 tile: the projection and the backward recompute
// (both operands K-major, mainloop_w), dH (K-major G x MN-major W,
// mainloop_kmn) and dW computed transposed, dW^T = Xc^T G (K-major XcT x
// MN-major G, mainloop_kmn).  Each of the 4 waves owns 192 x 128 of the tile as 6 x 4
// blocks of v_mfma_f32_32x32x16_bf16.  Against the 256 x 256 tile, a k step
// issues 24 MFMAs per 10 fragments (16 per 8), and a stage moves 80 KB into
// LDS per 384 x 256 x 64 multiply-adds (64 KB per 256 x 256 x 64): about a
// sixth less LDS and L2 traffic per flop.  Measured against the 256-wide
// loops (same box, alternating runs): 6% faster on the llama3-8b head's
// projection, 5-6% on full rounds of the recompute shape, 10.8% on full
// rounds of the dH shape.
//
// 384 fp32 accumulators per lane do not fit the AGPR file (256).  Blocks 0-3
// of each wave's 6 rows of blocks accumulate in AGPRs and blocks 4-5 in
// VGPRs.  The compiler's MFMA builtin puts every accumulator in AGPRs and
// spills the rest, so these MFMAs are inline asm with AGPR ("a") or VGPR
// ("v") accumulator operands.  The compiler still places and waits for the
// LDS reads and DMAs (builtins) that feed them; the asm MFMAs have side
// effects, so memory operations keep their source order around them, which
// fixes the interleaving.  The wait states an MFMA needs after VALU writes
// of its accumulators, and VALU reads need after the last MFMA, are padded
// explicitly (acc_fence).
//
// Two LDS stages of 80 KB (A 48 KB, B 32 KB): the whole 160 KB of a CU.
// Every tile is full: the last 384-row tile (of the usable head rows, of a
// chunk, of the valid tokens, or of the hidden columns) is computed shifted
// down so that it ends at the last row, and the epilogue drops the rows that
// belong to the tile before it.  The 256-wide operand has whole tiles, or is
// clamped on load.
#pragma once

#include "gemm_tile.hpp"

namespace flce {
namespace gemm {

constexpr int WBM = 384;            // wide tile rows (head rows)
constexpr int WMB = WBM / 64;       // MFMA blocks per wave along M (6)
constexpr int WNBA = WBM / 32;      // 1 KB DMA blocks of A per wave per stage (12)
constexpr int WSTAGE_A = WBM * BK2;  // elements of one A stage
constexpr int WIDE_GROUP_M = 4;     // M tiles per group in the tile order

// Row of accumulator register r of block (mb, nb) in a tile whose waves own
// `wave_rows` rows each.
__device__ __forceinline__ int acc_row_w(int wave_rows, int wm, int mb, int r, int lane) {
  return wm * wave_rows + 32 * mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// K-major DMA sources of a tile whose rows all exist.  Block b of a wave is
// rows 8b..8b+7; a lane's byte offset within its block depends only on the
// block's parity (the chunk swizzle repeats every 16 rows), and the block's
// row offset is uniform, so it goes into the scalar offset with the stage's
// k offset: two VGPRs per operand instead of one per block.
template <int NBW>
struct FullLoader {
  __amdgpu_buffer_rsrc_t rsrc;
  unsigned off[2];
  unsigned rows8_bytes;
  unsigned wave_bytes;
  __device__ __forceinline__ FullLoader(const Operand& op, int mn0, int wave, int lane) {
    rsrc = make_rsrc(op.ptr + (int64_t)mn0 * op.ld);
    rows8_bytes = (unsigned)op.ld * 16u;
    wave_bytes = (unsigned)(wave * NBW) * rows8_bytes;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = q * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz64(r);
      off[q] = (unsigned)((lane >> 3) * (int)op.ld + c * 8) * 2u;
    }
  }
  // DMA of block q of this wave's share of the stage at k0.
  __device__ __forceinline__ void issue(bf16* tile, int k0, int wave, int q) const {
    const unsigned soff =
        __builtin_amdgcn_readfirstlane(wave_bytes + (unsigned)q * rows8_bytes + (unsigned)k0 * 2u);
    lds_dma16(rsrc, off[q & 1], soff, tile + (wave * NBW + q) * 512);
  }
};

__device__ __forceinline__ void mfma_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vgpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// 24 wait states with every accumulator as an operand, so that no write of
// an accumulator before it and no read after it can move across it.
__device__ __forceinline__ void acc_fence(f32x16 (&acc)[WMB][4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[1][0]),
                 "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]), "+a"(acc[2][0]), "+a"(acc[2][1]),
                 "+a"(acc[2][2]), "+a"(acc[2][3]), "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc[3][2]),
                 "+a"(acc[3][3]));
  asm volatile("s_nop 0"
               : "+v"(acc[4][0]), "+v"(acc[4][1]), "+v"(acc[4][2]), "+v"(acc[4][3]), "+v"(acc[5][0]),
                 "+v"(acc[5][1]), "+v"(acc[5][2]), "+v"(acc[5][3]));
}

// One k step: 24 MFMAs on (fa, fb).  With RD, the next k step's 10
// fragments (k step s_next of tiles sa / sb) are read after every other
// MFMA; NV DMAs go out evenly, dma(d) issuing the d-th.
template <bool RD, int NV, class DmaF>
__device__ __forceinline__ void kstep_w(f32x16 (&acc)[WMB][4], const bf16x8 (&fa)[WMB], const bf16x8 (&fb)[4],
                                        bf16x8 (&na)[WMB], bf16x8 (&nb)[4], const bf16* sa, const bf16* sb,
                                        int s_next, int wm, int wn, int lane, DmaF dma) {
#pragma unroll
  for (int m = 0; m < 4 * WMB; ++m) {
    const int i = m / 4, j = m % 4;
    if (i < 4) mfma_agpr(acc[i][j], fa[i], fb[j]);
    else mfma_vgpr(acc[i][j], fa[i], fb[j]);
    if (RD && (m % 2) == 0 && m / 2 < WMB + 4) {
      const int r = m / 2;
      if (r < WMB) na[r] = frag64(sa, wm * 32 * WMB + 32 * r + (lane & 31), s_next, lane);
      else nb[r - WMB] = frag64(sb, wn * 128 + 32 * (r - WMB) + (lane & 31), s_next, lane);
    }
    if constexpr (NV > 0) {
#pragma unroll
      for (int d = 0; d < NV; ++d)
        if (m == 1 + (4 * WMB * d) / NV) dma(d);
    }
  }
}

struct NoDma {
  __device__ __forceinline__ void operator()(int) const {}
};

// Stage D in (ca, cb), stage D+1 in (na, nb).  Stage D+1's DMAs: A blocks
// 0-7 in k step 3 of stage D-1, A blocks 8-11 and B blocks 0-3 in k step 0
// of D, B blocks 4-7 in k step 1.  The barrier at the start of k step 3
// (vmcnt(0), lgkmcnt(0)) makes D+1 visible and frees D's buffers, whose
// refill with D+2 starts right after it.
template <bool NEXT, bool NEXT2>
__device__ __forceinline__ void stage_w(bf16* ca, bf16* cb, bf16* na, bf16* nb, int D, const FullLoader<WNBA>& la,
                                        const FullLoader<8>& lb, int wave, int wm, int wn, int lane,
                                        bf16x8 (&fa)[2][WMB], bf16x8 (&fb)[2][4], f32x16 (&acc)[WMB][4]) {
  const int k1 = (D + 1) * BK2, k2 = (D + 2) * BK2;
  auto dma0 = [&](int d) {
    if (d < WNBA - 8) la.issue(na, k1, wave, 8 + d);
    else lb.issue(nb, k1, wave, d - (WNBA - 8));
  };
  auto dma1 = [&](int d) { lb.issue(nb, k1, wave, 4 + d); };
  auto dma3 = [&](int d) { la.issue(ca, k2, wave, d); };
  if constexpr (NEXT) kstep_w<true, WNBA - 4>(acc, fa[0], fb[0], fa[1], fb[1], ca, cb, 1, wm, wn, lane, dma0);
  else kstep_w<true, 0>(acc, fa[0], fb[0], fa[1], fb[1], ca, cb, 1, wm, wn, lane, NoDma{});
  if constexpr (NEXT) kstep_w<true, 4>(acc, fa[1], fb[1], fa[0], fb[0], ca, cb, 2, wm, wn, lane, dma1);
  else kstep_w<true, 0>(acc, fa[1], fb[1], fa[0], fb[0], ca, cb, 2, wm, wn, lane, NoDma{});
  kstep_w<true, 0>(acc, fa[0], fb[0], fa[1], fb[1], ca, cb, 3, wm, wn, lane, NoDma{});
  if constexpr (NEXT) {
    stage_barrier<0>();
    if constexpr (NEXT2) kstep_w<true, 8>(acc, fa[1], fb[1], fa[0], fb[0], na, nb, 0, wm, wn, lane, dma3);
    else kstep_w<true, 0>(acc, fa[1], fb[1], fa[0], fb[0], na, nb, 0, wm, wn, lane, NoDma{});
  } else {
    kstep_w<false, 0>(acc, fa[1], fb[1], fa[0], fb[0], na, nb, 0, wm, wn, lane, NoDma{});
  }
}

// nk counts 32-wide steps and is a multiple of NST: an even number (at least
// two) of 64-wide stages.  a0 / n0: first rows of the A / B tiles, both full.
__device__ __forceinline__ void mainloop_w(const Operand& A, const Operand& B, int a0, int n0, int nk, bf16* s0,
                                          bf16* s1, bf16* s2, bf16* s3, f32x16 (&acc)[WMB][4]) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < WMB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  acc_fence(acc);
  const int nd = nk / 2;
  const FullLoader<WNBA> la(A, a0, wave, lane);
  const FullLoader<8> lb(B, n0, wave, lane);
#pragma unroll
  for (int q = 0; q < WNBA; ++q) la.issue(s0, 0, wave, q);
#pragma unroll
  for (int q = 0; q < 8; ++q) lb.issue(s1, 0, wave, q);
#pragma unroll
  for (int q = 0; q < 8; ++q) la.issue(s2, BK2, wave, q);
  stage_barrier<8>();
  bf16x8 fa[2][WMB], fb[2][4];
#pragma unroll
  for (int r = 0; r < WMB; ++r) fa[0][r] = frag64(s0, wm * 32 * WMB + 32 * r + (lane & 31), 0, lane);
#pragma unroll
  for (int r = 0; r < 4; ++r) fb[0][r] = frag64(s1, wn * 128 + 32 * r + (lane & 31), 0, lane);
  int D = 0;
  for (; D + 2 < nd; D += 2) {
    stage_w<true, true>(s0, s1, s2, s3, D, la, lb, wave, wm, wn, lane, fa, fb, acc);
    stage_w<true, true>(s2, s3, s0, s1, D + 1, la, lb, wave, wm, wn, lane, fa, fb, acc);
  }
  // The two stages after the loop take the lane index through an opaque
  // move, so that their LDS addresses are computed here rather than before
  // the loop and kept in scratch across it.
  int lane_t = lane;
  asm volatile("" : "+v"(lane_t));
  stage_w<true, false>(s0, s1, s2, s3, D, la, lb, wave, wm, wn, lane_t, fa, fb, acc);
  stage_w<false, false>(s2, s3, s0, s1, D + 1, la, lb, wave, wm, wn, lane_t, fa, fb, acc);
  stage_barrier<0>();
  acc_fence(acc);
}

// ---- K-major A (384 rows) x MN-major B (256 columns): the dH contraction.
// B's fragments come from transposing reads (ds_read_b64_tr_b16), the slow
// ones, so each k step reads the next step's 4 B fragments first, after its
// first four MFMAs.  A's fragments use one register set: the next step's
// fragment i is read into fa[i] right after the step's last MFMA with it
// (the MFMAs run i-major), which leaves the registers that a second set
// would take to the 128 VGPR accumulators.

// MN-major operand: a stage is 64 k-rows x 256 columns (rows of 512 bytes);
// each wave DMAs 8 blocks of 2 k-rows.  Block b's k-row offset is uniform
// (scalar offset); a lane's offset within its block depends only on b's
// parity (the pair swizzle of k-row 2b + lane/32 repeats every 4 k-rows).
// k-rows past k_max read as zero.
struct MnLoaderW {
  const bf16* base;
  int64_t ld;
  int k_max;
  unsigned off[2];
  __device__ __forceinline__ MnLoaderW(const Operand& op, int mn0, int lane) {
    base = op.ptr;
    ld = op.ld;
    k_max = op.k_max;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int kk = q * 2 + (lane >> 5);
      const int c = (lane & 31) ^ swz_mn(kk);
      const int col = min(mn0 + c * 8, op.mn_max - 7);
      off[q] = (unsigned)((lane >> 5) * (int)op.ld + col) * 2u;
    }
  }
  __device__ __forceinline__ void issue(bf16* tile, int k0, int wave, int q) const {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (int64_t)k0 * ld);
    const int b = wave * 8 + q;
    const unsigned soff = __builtin_amdgcn_readfirstlane((unsigned)(b * 2) * (unsigned)ld * 2u);
    if (k0 + BK2 - 1 <= k_max) {
      lds_dma16(r, off[q & 1], soff, tile + b * 512);
    } else {
      const int kk = b * 2 + (int)((threadIdx.x >> 5) & 1);
      lds_dma16(r, kk <= k_max - k0 ? off[q & 1] : 0x80000000u, soff, tile + b * 512);
    }
  }
};

// frag_mnmajor with the second read's index laundered by a volatile asm
// (the alias-scope reason is given at frag_mnmajor): a non-volatile one is
// hoisted out of the main loop, and the 16 indices it then keeps live spill
// with this tile's register budget.
__device__ __forceinline__ bf16x8 frag_mn_w(const bf16* tile, int col0, int s, int lane) {
  const int g = lane >> 4;
  const int j = lane & 15;
  const int col = col0 + 16 * (g & 1) + 4 * (j & 3);
  const int k0 = 16 * s + 8 * (g >> 1) + (j >> 2);
  const int k1 = k0 + 4;
  const int i0 = k0 * 256 + (((col >> 3) ^ swz_mn(k0)) << 3) + (col & 7);
  int i1 = k1 * 256 + (((col >> 3) ^ swz_mn(k1)) << 3) + (col & 7);
  asm volatile("" : "+v"(i1));
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FLCE_LDS bf16x4*)(tile + i0));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FLCE_LDS bf16x4*)(tile + i1));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <bool RD, int NV, class DmaF>
__device__ __forceinline__ void kstep_kmn(f32x16 (&acc)[WMB][4], bf16x8 (&fa)[WMB], const bf16x8 (&fb)[4],
                                          bf16x8 (&nb)[4], const bf16* sa, const bf16* sb, int s_next, int wm,
                                          int wn, int lane, DmaF dma) {
#pragma unroll
  for (int m = 0; m < 4 * WMB; ++m) {
    const int i = m / 4, j = m % 4;
    if (i < 4) mfma_agpr(acc[i][j], fa[i], fb[j]);
    else mfma_vgpr(acc[i][j], fa[i], fb[j]);
    if (RD && m < 4) nb[m] = frag_mn_w(sb, wn * 128 + 32 * m, s_next, lane);
    if (RD && j == 3) fa[i] = frag64(sa, wm * 32 * WMB + 32 * i + (lane & 31), s_next, lane);
    if constexpr (NV > 0) {
#pragma unroll
      for (int d = 0; d < NV; ++d)
        if (m == 1 + (4 * WMB * d) / NV) dma(d);
    }
  }
}

// Same stage order, DMA split and barrier as stage_w.
template <bool NEXT, bool NEXT2>
__device__ __forceinline__ void stage_kmn(bf16* ca, bf16* cb, bf16* na, bf16* nb, int D, const FullLoader<WNBA>& la,
                                          const MnLoaderW& lb, int wave, int wm, int wn, int lane,
                                          bf16x8 (&fa)[WMB], bf16x8 (&fb)[2][4], f32x16 (&acc)[WMB][4]) {
  const int k1 = (D + 1) * BK2, k2 = (D + 2) * BK2;
  auto dma0 = [&](int d) {
    if (d < WNBA - 8) la.issue(na, k1, wave, 8 + d);
    else lb.issue(nb, k1, wave, d - (WNBA - 8));
  };
  auto dma1 = [&](int d) { lb.issue(nb, k1, wave, 4 + d); };
  auto dma3 = [&](int d) { la.issue(ca, k2, wave, d); };
  if constexpr (NEXT) kstep_kmn<true, WNBA - 4>(acc, fa, fb[0], fb[1], ca, cb, 1, wm, wn, lane, dma0);
  else kstep_kmn<true, 0>(acc, fa, fb[0], fb[1], ca, cb, 1, wm, wn, lane, NoDma{});
  if constexpr (NEXT) kstep_kmn<true, 4>(acc, fa, fb[1], fb[0], ca, cb, 2, wm, wn, lane, dma1);
  else kstep_kmn<true, 0>(acc, fa, fb[1], fb[0], ca, cb, 2, wm, wn, lane, NoDma{});
  kstep_kmn<true, 0>(acc, fa, fb[0], fb[1], ca, cb, 3, wm, wn, lane, NoDma{});
  if constexpr (NEXT) {
    stage_barrier<0>();
    if constexpr (NEXT2) kstep_kmn<true, 8>(acc, fa, fb[1], fb[0], na, nb, 0, wm, wn, lane, dma3);
    else kstep_kmn<true, 0>(acc, fa, fb[1], fb[0], na, nb, 0, wm, wn, lane, NoDma{});
  } else {
    kstep_kmn<false, 0>(acc, fa, fb[1], fb[0], na, nb, 0, wm, wn, lane, NoDma{});
  }
}

__device__ __forceinline__ void mainloop_kmn(const Operand& A, const Operand& B, int a0, int n0, int nk, bf16* s0,
                                            bf16* s1, bf16* s2, bf16* s3, f32x16 (&acc)[WMB][4]) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < WMB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  acc_fence(acc);
  const int nd = nk / 2;
  const FullLoader<WNBA> la(A, a0, wave, lane);
  const MnLoaderW lb(B, n0, lane);
#pragma unroll
  for (int q = 0; q < WNBA; ++q) la.issue(s0, 0, wave, q);
#pragma unroll
  for (int q = 0; q < 8; ++q) lb.issue(s1, 0, wave, q);
#pragma unroll
  for (int q = 0; q < 8; ++q) la.issue(s2, BK2, wave, q);
  stage_barrier<8>();
  bf16x8 fa[WMB], fb[2][4];
#pragma unroll
  for (int r = 0; r < WMB; ++r) fa[r] = frag64(s0, wm * 32 * WMB + 32 * r + (lane & 31), 0, lane);
#pragma unroll
  for (int r = 0; r < 4; ++r) fb[0][r] = frag_mn_w(s1, wn * 128 + 32 * r, 0, lane);
  int D = 0;
  for (; D + 2 < nd; D += 2) {
    stage_kmn<true, true>(s0, s1, s2, s3, D, la, lb, wave, wm, wn, lane, fa, fb, acc);
    stage_kmn<true, true>(s2, s3, s0, s1, D + 1, la, lb, wave, wm, wn, lane, fa, fb, acc);
  }
  int lane_t = lane;  // as in mainloop_w
  asm volatile("" : "+v"(lane_t));
  stage_kmn<true, false>(s0, s1, s2, s3, D, la, lb, wave, wm, wn, lane_t, fa, fb, acc);
  stage_kmn<false, false>(s2, s3, s0, s1, D + 1, la, lb, wave, wm, wn, lane_t, fa, fb, acc);
  stage_barrier<0>();
  acc_fence(acc);
}

// Tile order as tile_of, with groups of WIDE_GROUP_M M-tiles (the 32
// workgroups of an XCD then cover 4 x 8 tiles).
__device__ __forceinline__ void tile_of_wide(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int xcd = pid & 7;
  const int local = pid >> 3;
  const int l = xcd * (total >> 3) + min(xcd, total & 7) + local;
  const int per_group = WIDE_GROUP_M * tiles_n;
  const int gid = l / per_group;
  const int first_m = gid * WIDE_GROUP_M;
  const int gsz = min(tiles_m - first_m, WIDE_GROUP_M);
  const int r = l - gid * per_group;
  tm = first_m + r % gsz;
  tn = r / gsz;
}

// A: head rows (mn_max + 1 >= WBM rows, checked on the host); B: token rows,
// a whole number of 256-row tiles; tokens along N (sch.tok_dim == 2).
// Epi::apply(ep, acc, m0, a0, n0, smem): m0 is the tile's first row, a0 <= m0
// the row of accumulator row 0.
template <class Epi>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_wide_kernel(Operand A, Operand B, Schedule sch,
                                                                 typename Epi::Params ep) {
  __shared__ __attribute__((aligned(1024))) bf16 s0[WSTAGE_A];
  __shared__ __attribute__((aligned(1024))) bf16 s1[STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 s2[WSTAGE_A];
  __shared__ __attribute__((aligned(1024))) bf16 s3[STAGE_ELEMS];
  int tiles_m = sch.tiles_m, tiles_n = sch.tiles_n;
  if (sch.tok_dim == 2) {
    const int tv = *sch.tok_count;
    tiles_n = min(tiles_n, (tv + BN - 1) / BN);
  }
  const int pid = blockIdx.x;
  if (pid >= tiles_m * tiles_n) return;
  int tm, tn;
  tile_of_wide(pid, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * WBM;
  const int a0 = min(m0, A.mn_max + 1 - WBM);
  const int n0 = tn * BN;
  f32x16 acc[WMB][4];
  mainloop_w(A, B, a0, n0, sch.k_steps, s0, s1, s2, s3, acc);
  Epi::apply(ep, acc, m0, a0, n0, s0);
}

// One 384 x 256 tile of a K-major x MN-major product whose K is the valid
// tokens (sch.tok_dim == 3: ceil(Tv / 128) * 128 of them) or sch.k_steps:
// dW^T = Xc^T G of a chunk, A = XcT (hidden rows, all present; the last tile
// computed shifted down), B = G (the chunk's head rows as columns).  With no
// valid tokens the tile is all zeros.
template <class Epi>
__device__ __forceinline__ void run_wide_kmn(const Operand& A, const Operand& B, const Schedule& sch,
                                             const typename Epi::Params& ep, int pid, bf16* s0, bf16* s1,
                                             bf16* s2, bf16* s3) {
  if (pid >= sch.tiles_m * sch.tiles_n) return;
  int k_steps = sch.k_steps;
  if (sch.tok_dim == 3) {
    const int tv = *sch.tok_count;
    k_steps = (tv + NST * BK - 1) / (NST * BK) * NST;
  }
  int tm, tn;
  tile_of_wide(pid, sch.tiles_m, sch.tiles_n, tm, tn);
  const int m0 = tm * WBM;
  const int a0 = min(m0, A.mn_max + 1 - WBM);
  const int n0 = tn * BN;
  f32x16 acc[WMB][4];
  if (k_steps > 0) {
    mainloop_kmn(A, B, a0, n0, k_steps, s0, s1, s2, s3, acc);
  } else {
#pragma unroll
    for (int i = 0; i < WMB; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  }
  Epi::apply(ep, acc, m0, a0, n0, s0);
}

// dH of a chunk on 256-row token tiles (run_tile's K-major G x MN-major W)
// and its dW as 384-row tiles of dW^T (run_wide_kmn) in one launch;
// workgroups [0, n1) take dH's tiles, as in gemm_pair.
template <class Epi1, class Epi2>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_pair_nt(Operand A1, Operand B1, Schedule sch1,
                                                             typename Epi1::Params ep1, int n1, Operand A2,
                                                             Operand B2, Schedule sch2, typename Epi2::Params ep2) {
  __shared__ __attribute__((aligned(1024))) bf16 s0[WSTAGE_A];
  __shared__ __attribute__((aligned(1024))) bf16 s1[STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 s2[WSTAGE_A];
  __shared__ __attribute__((aligned(1024))) bf16 s3[STAGE_ELEMS];
  const int pid = blockIdx.x;
  if (pid < n1) {
    if (pid < sch1.tiles_m * sch1.tiles_n) run_tile<true, false, Epi1>(A1, B1, sch1, ep1, pid, s0, s1, s2, s3);
  } else {
    run_wide_kmn<Epi2>(A2, B2, sch2, ep2, pid - n1, s0, s1, s2, s3);
  }
}

// dH of one chunk (K-major G x MN-major W with 384-row token tiles) and dW
// of the chunk (run_tile's MN-major G x K-major XcT, 256-row tiles) in one
// launch.  Workgroups [0, n1) take dH's tiles (n1: its host-side tile count
// rounded up to a multiple of 8, so that dW's tiles keep the id-to-XCD
// mapping tile_of assumes), the rest dW's.  Only the ceil(Tv / 384) token
// tiles that hold valid tokens run; the last is computed shifted down to
// end at row Tvp - 1 (G's rows past Tv are zero).  With WIDE2, dW runs as
// 384-row tiles of dW^T (run_wide_kmn) instead.
template <class Epi1, class Epi2, bool WIDE2 = false>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_pair_wide(Operand A1, Operand B1, Schedule sch1,
                                                               typename Epi1::Params ep1, int n1, Operand A2,
                                                               Operand B2, Schedule sch2, typename Epi2::Params ep2) {
  __shared__ __attribute__((aligned(1024))) bf16 s0[WSTAGE_A];
  __shared__ __attribute__((aligned(1024))) bf16 s1[STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 s2[WSTAGE_A];
  __shared__ __attribute__((aligned(1024))) bf16 s3[STAGE_ELEMS];
  const int pid = blockIdx.x;
  if (pid < n1) {
    const int tv = *sch1.tok_count;
    const int tiles_m = min(sch1.tiles_m, (tv + WBM - 1) / WBM);
    const int tiles_n = sch1.tiles_n;
    if (pid >= tiles_m * tiles_n) return;
    int tm, tn;
    tile_of_wide(pid, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * WBM;
    const int a0 = min(m0, A1.mn_max + 1 - WBM);
    const int n0 = tn * BN;
    f32x16 acc[WMB][4];
    mainloop_kmn(A1, B1, a0, n0, sch1.k_steps, s0, s1, s2, s3, acc);
    Epi1::apply(ep1, acc, m0, a0, n0, s0);
  } else if constexpr (WIDE2) {
    run_wide_kmn<Epi2>(A2, B2, sch2, ep2, pid - n1, s0, s1, s2, s3);
  } else {
    run_tile<false, true, Epi2>(A2, B2, sch2, ep2, pid - n1, s0, s1, s2, s3);
  }
}

}  // namespace gemm
}  // namespace flce
