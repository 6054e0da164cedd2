// An fp32 head read straight by the projection and recompute GEMMs: each
// piece of a bf16 LDS tile of head rows is made from fp32 head elements,
// rounded to nearest even on the way ("nemo_automodel.components.models.
// inkling2.loss", class description: an fp32 head takes part through its
// bf16 value).  The LDS DMA (buffer_load ... lds) copies bytes as they are,
// so the head's tiles come in through registers (buffer_load_dwordx4,
// v_cvt_pk_bf16_f32, ds_write_b64; F32Loader) into the slots the DMA loader
// would have filled.  The LDS layout, the swizzles, the fragment reads and
// the MFMA order are those of gemm_tile.hpp, so the result is bit for bit
// that of the bf16 head rounded beforehand on the same tiles.
//
// The head operand's eight 1 KB pieces per wave and stage go out as two
// register sets of four, each loaded two k steps before it is written:
//   set 0 (pieces 0-3 of stage D+1): loaded in k step 3 of stage D-1, right
//     after the barrier, written in k step 1 of stage D;
//   set 1 (pieces 4-7 of stage D+1): loaded in k step 0 of stage D, written in
//     k step 2;
// both into the buffer stage D-1 used, which the barrier at k step 3 of
// stage D-1 freed, and both before the barrier at k step 3 of stage D that
// publishes stage D+1.  These kernels use the 256 x 256 tile: the 384-row
// tile has no registers left for the 64 staging VGPRs.
//
// In the backward recompute, the workgroups of the first token tile also
// write the rounded head rows of their tile to a bf16 copy of the chunk's
// rows, from the same registers: the dH contraction of the chunk then reads
// that copy as it reads a bf16 head.  No separate pass reads the fp32 head.
#pragma once

#include "gemm_tile.hpp"

namespace flce {
namespace gemm {

// An fp32 operand (the head).  ld in elements; mn_max / k_max as Operand.
struct OperandF32 {
  const float* ptr;
  int64_t ld;
  int mn_max;
  int k_max;
};

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Loads of the fp32 head for one K-major tile of 256 head rows x 64 k.  A
// 1 KB piece of the bf16 LDS tile (8 rows x 64 k) is 2 KB of fp32, which two
// buffer_load_dwordx4 bring in so that each instruction covers 4 whole rows
// of 64 k (whole 256-byte runs, so whole cache lines): lane l takes 4
// consecutive elements, rounds them to 4 bf16 and writes them with one
// ds_write_b64 into its half of the 16-byte slot the DMA loader would fill.
// (Two 16-byte loads per lane at a 32-byte stride touch twice the cache
// lines per instruction.)
//
// Registers: one lane byte offset, to which each load adds its piece's
// uniform row offset, and four LDS destinations (the slot swizzle of a row
// depends on the lane and on the row's place modulo 16 rows).  Rows past
// mn_max lie past the buffer resource's record count and read as zero.
struct F32Loader {
  int64_t ld;
  int mn_rows;          // rows of the tile that exist
  __amdgpu_buffer_rsrc_t rsrc;
  unsigned lane_off;    // byte offset of this lane's 4 elements within its piece row
  unsigned dst[4];      // LDS element offset of its bf16, by (piece parity, load)
  int lane;
  f32x4v set[2][4][2];

  __device__ __forceinline__ F32Loader(const OperandF32& op, int mn0, int wave, int lane_) {
    ld = op.ld;
    lane = lane_;
    mn_rows = min(op.mn_max - mn0 + 1, 256);
    const float* base = op.ptr + (int64_t)mn0 * op.ld;
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0,
                                             __builtin_amdgcn_readfirstlane(mn_rows * (int)op.ld * 4), 0x00020000);
    lane_off = (unsigned)((lane >> 4) * (int)op.ld + 4 * (lane & 15)) * 4u;
#pragma unroll
    for (int pi = 0; pi < 4; ++pi) {
      // row 8 p + 4 i + lane/16 of a piece p with p % 2 = pi / 2, load i = pi % 2
      const int r = 8 * (pi >> 1) + 4 * (pi & 1) + (lane >> 4);
      dst[pi] = (unsigned)(r * BK2 + ((((lane & 15) >> 1) ^ swz64(r)) << 3) + ((lane & 1) << 2));
    }
  }

  // Loads of pieces 4S .. 4S+3 of this wave's share of the stage at k0 into
  // register set S.
  template <int S>
  __device__ __forceinline__ void load(int k0, int wave) {
    unsigned lo = lane_off;
    asm volatile("" : "+v"(lo));  // keep the 8 sums below from being hoisted out of the main loop
    const int soff = k0 * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const unsigned row = (unsigned)((wave * 8 + 4 * S + j) * 8 + 4 * i);
        set[S][j][i] = __builtin_bit_cast(
            f32x4v, __builtin_amdgcn_raw_buffer_load_b128(rsrc, lo + row * (unsigned)ld * 4u, soff, 0));
      }
  }

  // Round register set S to bf16 and write it to its places in `tile`; with
  // `copy` (row stride ld_copy, at the tile's first row) also to the copy's
  // rows that exist, elements k0 ...
  template <int S>
  __device__ __forceinline__ void store(bf16* tile, int wave, bf16* copy = nullptr, int64_t ld_copy = 0,
                                        int k0 = 0) const {
    bf16* t = tile + wave * 8 * 512;  // this wave's 8 pieces
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int q = 4 * S + j;
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)set[S][j][i][e];
        // piece q starts at q * 512 elements; rows repeat their swizzle every
        // 2 pieces
        const int pi = ((q & 1) << 1) | i;
        *(FLCE_LDS bf16x4*)(t + (q >> 1) * 1024 + dst[pi]) = v;
        if (copy) {
          const int r = (wave * 8 + q) * 8 + 4 * i + (lane >> 4);
          if (r < mn_rows) *reinterpret_cast<bf16x4*>(copy + (int64_t)r * ld_copy + k0 + 4 * (lane & 15)) = v;
        }
      }
  }
};

// ---- fp32 head as operand A, both operands K-major (projection, recompute).
// Stage order and B's DMAs as stage_kk; A as described at the top.
template <bool NEXT, bool NEXT2>
__device__ __forceinline__ void stage_kk_f32a(bf16* ca, bf16* cb, bf16* na, bf16* nb, int D, F32Loader& la,
                                             const Loader<true>& lb, int wave, int wm, int wn, int lane,
                                             bf16x8 (&fa)[2][4], bf16x8 (&fb)[2][4], f32x16 (&acc)[4][4],
                                             bf16* copy, int64_t ld_copy) {
  read_frags<true, true>(ca, cb, 1, wm, wn, lane, fa[1], fb[1]);
  if constexpr (NEXT) {
    la.load<1>((D + 1) * BK2, wave);
    lb.issue<0, 3>(nb, (D + 1) * BK2, wave);
  }
  mfma_step(fa[0], fb[0], acc);
  interleave_step<8, NEXT ? 11 : 0>();
  __builtin_amdgcn_sched_barrier(0);

  read_frags<true, true>(ca, cb, 2, wm, wn, lane, fa[0], fb[0]);
  if constexpr (NEXT) {
    la.store<0>(na, wave, copy, ld_copy, (D + 1) * BK2);
    lb.issue<3, 8>(nb, (D + 1) * BK2, wave);
  }
  mfma_step(fa[1], fb[1], acc);
  interleave_step<8, NEXT ? 5 : 0>();
  __builtin_amdgcn_sched_barrier(0);

  read_frags<true, true>(ca, cb, 3, wm, wn, lane, fa[1], fb[1]);
  if constexpr (NEXT) la.store<1>(na, wave, copy, ld_copy, (D + 1) * BK2);
  mfma_step(fa[0], fb[0], acc);
  interleave_step<8, 0>();
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (NEXT) {
    stage_barrier<0>();
    read_frags<true, true>(na, nb, 0, wm, wn, lane, fa[0], fb[0]);
    if constexpr (NEXT2) la.load<0>((D + 2) * BK2, wave);
  }
  mfma_step(fa[1], fb[1], acc);
  interleave_step<NEXT ? 8 : 0, NEXT2 ? 8 : 0>();
  __builtin_amdgcn_sched_barrier(0);
}

// copy: the bf16 copy's row m0 (nullptr: none), row stride ld_copy.
__device__ __forceinline__ void mainloop_kk_f32a(const OperandF32& A, const Operand& B, int m0, int n0, int nk,
                                                bf16* s0, bf16* s1, bf16* s2, bf16* s3, f32x16 (&acc)[4][4],
                                                bf16* copy, int64_t ld_copy) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave >> 1;
  const int wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  if (nk <= 0) return;
  const int nd = nk / 2;
  F32Loader la(A, m0, wave, lane);
  const Loader<true> lb(B, n0, wave, lane);
  // Prologue: stage 0 whole (A through registers), then A's first register
  // set of stage 1, which k step 1 of stage 0 writes.
  la.load<0>(0, wave);
  la.load<1>(0, wave);
  lb.issue<0, 8>(s1, 0, wave);
  la.store<0>(s0, wave, copy, ld_copy, 0);
  la.store<1>(s0, wave, copy, ld_copy, 0);
  la.load<0>(BK2, wave);
  stage_barrier<8>();
  bf16x8 fa[2][4], fb[2][4];
  read_frags<true, true>(s0, s1, 0, wm, wn, lane, fa[0], fb[0]);
  int D = 0;
  for (; D + 2 < nd; D += 2) {
    stage_kk_f32a<true, true>(s0, s1, s2, s3, D, la, lb, wave, wm, wn, lane, fa, fb, acc, copy, ld_copy);
    stage_kk_f32a<true, true>(s2, s3, s0, s1, D + 1, la, lb, wave, wm, wn, lane, fa, fb, acc, copy, ld_copy);
  }
  stage_kk_f32a<true, false>(s0, s1, s2, s3, D, la, lb, wave, wm, wn, lane, fa, fb, acc, copy, ld_copy);
  stage_kk_f32a<false, false>(s2, s3, s0, s1, D + 1, la, lb, wave, wm, wn, lane, fa, fb, acc, copy, ld_copy);
  stage_barrier<0>();
}

// ---- Kernels ---------------------------------------------------------------

// Projection / recompute with the fp32 head as operand A (256 x 256 tiles).
// copy (nullptr: none): the bf16 copy of A's rows (row stride A.ld), written
// by the workgroups of the first token tile.
template <class Epi>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_kernel_f32a(OperandF32 A, Operand B, Schedule sch,
                                                                 typename Epi::Params ep, bf16* copy) {
  __shared__ __attribute__((aligned(1024))) bf16 s0[STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 s1[STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 s2[STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 s3[STAGE_ELEMS];
  int m0, n0, k_steps;
  if (!map_tile(sch, blockIdx.x, m0, n0, k_steps)) return;
  f32x16 acc[4][4];
  bf16* cp = (copy && n0 == 0) ? copy + (int64_t)m0 * A.ld : nullptr;
  mainloop_kk_f32a(A, B, m0, n0, k_steps, s0, s1, s2, s3, acc, cp, A.ld);
  Epi::apply(ep, acc, m0, n0, s0);
}

}  // namespace gemm
}  // namespace flce
