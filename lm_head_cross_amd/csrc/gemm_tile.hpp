// MFMA bf16 -> fp32 tile GEMM for gfx950, shared by every contraction of the
// fused linear cross-entropy path.
//
// One workgroup of 256 threads (4 wave64s arranged 2 x 2) owns a 256 x 256
// output tile; each wave owns 128 x 128 of it as 4 x 4 blocks of the
// v_mfma_f32_32x32x16_bf16 instruction, whose fp32 accumulators live in the
// AGPR half of the register file (one wave per SIMD).
//
// K advances 64 at a time through two LDS stages of 64 KB: A in the arrays
// s0 / s2, B in s1 / s3, each array its own __shared__ object so that the
// compiler can see that a DMA in flight into one stage never aliases the
// stage being read (it then does not make the LDS reads wait for it).
// Stages are filled by buffer_load_dwordx4 ... lds, which writes each lane's
// 16 bytes straight into LDS (no VGPR staging, no LDS write instructions),
// spread between the MFMAs.  A stage runs as four k steps of 16, 16 MFMAs
// per wave each; one workgroup barrier per stage hands the next stage over.
//
// Either operand may be K-major (element (mn, k) at ptr[mn*ld + k]) or
// MN-major (element (mn, k) at ptr[k*ld + mn]); the LDS tile keeps the
// global layout, so global loads stay fully coalesced either way:
//  - K-major tile: 256 rows x 64 k, rows of 128 bytes, so every DMA moves
//    whole cache lines.  A fragment (one row, 8 consecutive k) is one
//    ds_read_b128.  The 16-byte chunk c of row r sits at slot c ^ swz64(r).
//  - MN-major tile: 64 k-rows x 256 mn (512-byte rows).  A fragment is two
//    ds_read_b64_tr_b16: within each 16-lane group the hardware transposes a
//    4 (k) x 16 (mn) block so that lane i receives column i, four
//    consecutive k.  Pairs of 16-byte chunks are XOR-swizzled per k-row,
//    which leaves these reads free of bank conflicts.
// With both operands K-major (the projection and the recompute) fragments
// are read one k step ahead (mainloop_kk); with an MN-major operand (dH, dW)
// two k steps ahead, since the transposing reads take a few hundred cycles
// under load (mainloop_mn).
//
// The accumulator layout of the 32x32 MFMA: lane l, register r holds element
// (row 8*(r/4) + 4*(l/32) + r%4, column l%32) of its block.
#pragma once

#include "device_common.hpp"

namespace flce {
namespace gemm {

constexpr int BM = 256;
constexpr int BN = 256;
static_assert(BM == BN, "token tiles are BM wide along M and N alike");
constexpr int BK = 32;                        // K is counted in steps of 32 (Schedule::k_steps) ...
constexpr int NST = 4;                        // ... and padded to a multiple of NST steps (128)
constexpr int BK2 = 64;                       // k per LDS stage
constexpr int NTHREADS = 256;
constexpr int STAGE_ELEMS = 256 * BK2;        // one operand's tile of one stage (32 KB)

// One GEMM operand.
struct Operand {
  const bf16* ptr;
  int64_t ld;     // elements between consecutive rows of the stored layout
  int mn_max;     // largest mn index that may be read (rows or columns beyond are clamped)
  int k_max;      // largest k index that may be read (MN-major only)
};

// Tile bookkeeping shared by every GEMM launch.
struct Schedule {
  int tiles_m, tiles_n;
  int k_steps;              // K / BK (a multiple of NST) when K is known on the host
  const int* tok_count;     // device count of valid tokens (may be null)
  int tok_dim;              // 0: none, 1: M is tokens, 2: N is tokens, 3: K is tokens
};

// Chunk slot of a K-major row: chunk c of row r sits at c ^ swz64(r), which
// keeps the 8- and 16-lane phases of a fragment read (consecutive rows, one
// chunk) on distinct banks.
__device__ __forceinline__ int swz64(int r) { return (r >> 1) & 7; }

// Chunk XOR for MN-major rows: pairs of 16-byte chunks are XOR-ed with
// t(k % 4) in {0, 3, 5, 6}; t and t ^ 1 cover all eight pair slots of 256 B.
// Chosen by measuring SQ_LDS_BANK_CONFLICT for this read pattern: 0.
__device__ __forceinline__ int swz_mn(int k) { return ((0x6530 >> ((k & 3) * 4)) & 0xF) << 1; }

// Global -> LDS copy of 16 bytes per lane through a buffer resource: the
// base address is uniform (SGPRs) and each lane supplies a 32-bit byte
// offset, which costs the address unit half of what 64-bit per-lane
// addresses do.  The LDS destination is wave-uniform; lane i's 16 bytes land
// at lds_dst + 16 * i.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFF0, 0x00020000);
}
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, unsigned voff, unsigned soff, bf16* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (FLCE_LDS void*)lds_dst, 16, voff, soff, 0, 0);
}

// s_waitcnt with vmcnt <= n (n < 64) and lgkmcnt = 0 (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier after this wave's DMA instructions older than the newest
// `n_out` have landed and its LDS reads are done.  A fence-based barrier
// would also wait for the DMAs still in flight into the other stage.
template <int N_OUT>
__device__ __forceinline__ void stage_barrier() {
  wait_vm_lgkm0<N_OUT>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-thread DMA sources of one operand for 64-wide stages, fixed along K:
// the byte offset of each of this thread's 16-byte pieces (8 blocks of 1 KB
// per wave) relative to the tile's origin.
//  - K-major: a block is 8 rows x 128 B; the resource is based at the tile's
//    first row, and stage k0 adds 2*k0 bytes through the scalar offset.
//  - MN-major: a block is 2 k-rows x 512 B; the resource is rebased at k-row
//    k0 for every stage (scalar work), and rows past k_max read as zero (the
//    partner operand is zero there too).
template <bool KMAJOR>
struct Loader {
  const bf16* base;
  int64_t ld;
  int k_max;
  __amdgpu_buffer_rsrc_t rsrc;
  unsigned off[8];
  int kk[8];
  __device__ __forceinline__ Loader(const Operand& op, int mn0, int wave, int lane) {
    ld = op.ld;
    k_max = op.k_max;
    if constexpr (KMAJOR) {
      base = op.ptr + (int64_t)mn0 * op.ld;
      rsrc = make_rsrc(base);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int b = wave * 8 + q;
        const int r = b * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz64(r);
        const int gr = min(mn0 + r, op.mn_max) - mn0;
        off[q] = (unsigned)(gr * (int)op.ld + c * 8) * 2u;
        kk[q] = 0;
      }
    } else {
      base = op.ptr;
      rsrc = make_rsrc(base);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int b = wave * 8 + q;            // 1 KB block: 2 k-rows of 512 B
        kk[q] = b * 2 + (lane >> 5);
        const int c = (lane & 31) ^ swz_mn(kk[q]);
        const int col = min(mn0 + c * 8, op.mn_max - 7);
        off[q] = (unsigned)(kk[q] * (int)op.ld + col) * 2u;
      }
    }
  }
  template <int Q0, int Q1>
  __device__ __forceinline__ void issue(bf16* tile, int k0, int wave) const {
    if constexpr (KMAJOR) {
      const unsigned soff = (unsigned)k0 * 2u;
#pragma unroll
      for (int q = Q0; q < Q1; ++q) lds_dma16(rsrc, off[q], soff, tile + (wave * 8 + q) * 512);
    } else {
      const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (int64_t)k0 * ld);
      if (k0 + BK2 - 1 <= k_max) {
#pragma unroll
        for (int q = Q0; q < Q1; ++q) lds_dma16(r, off[q], 0, tile + (wave * 8 + q) * 512);
      } else {
        const int krem = k_max - k0;
#pragma unroll
        for (int q = Q0; q < Q1; ++q) {
          const unsigned o = kk[q] <= krem ? off[q] : 0x80000000u;
          lds_dma16(r, o, 0, tile + (wave * 8 + q) * 512);
        }
      }
    }
  }
};


// Fragment of a 64-wide K-major tile: row `row`, k = 16*s + 8*(lane/32) + 0..7.
__device__ __forceinline__ bf16x8 frag64(const bf16* tile, int row, int s, int lane) {
  const int c = (2 * s + (lane >> 5)) ^ swz64(row);
  return *(const FLCE_LDS bf16x8*)(tile + row * BK2 + c * 8);
}

// Fragment of an MN-major tile for the 32 columns starting at col0:
// lane l gets column col0 + l%32, k = 16*s + 8*(l/32) + 0..7.
__device__ __forceinline__ bf16x8 frag_mnmajor(const bf16* tile, int col0, int s, int lane) {
  const int g = lane >> 4;
  const int j = lane & 15;
  const int col = col0 + 16 * (g & 1) + 4 * (j & 3);
  const int k0 = 16 * s + 8 * (g >> 1) + (j >> 2);
  const int k1 = k0 + 4;
  const int i0 = k0 * 256 + (((col >> 3) ^ swz_mn(k0)) << 3) + (col & 7);
  int i1 = k1 * 256 + (((col >> 3) ^ swz_mn(k1)) << 3) + (col & 7);
  // i1 is i0 + 1024; left visible, the optimizer splits that constant into a
  // GEP of its own, one level too deep for the LDS lowering to attach the
  // per-array alias scope, and the waitcnt pass then makes this read wait
  // for every DMA in flight (vmcnt(0) each stage).  The empty asm keeps both
  // addresses one GEP away from the tile.
  asm("" : "+v"(i1));
  const bf16* p0 = tile + i0;
  const bf16* p1 = tile + i1;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FLCE_LDS bf16x4*)p0);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FLCE_LDS bf16x4*)p1);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// This wave's fragments of k step s: rows wm*128 + 32*i (A), wn*128 + 32*i (B).
template <bool A_KMAJOR, bool B_KMAJOR>
__device__ __forceinline__ void read_frags(const bf16* sa, const bf16* sb, int s, int wm, int wn, int lane,
                                            bf16x8 (&fa)[4], bf16x8 (&fb)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (A_KMAJOR) fa[i] = frag64(sa, wm * 128 + 32 * i + (lane & 31), s, lane);
    else fa[i] = frag_mnmajor(sa, wm * 128 + 32 * i, s, lane);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (B_KMAJOR) fb[i] = frag64(sb, wn * 128 + 32 * i + (lane & 31), s, lane);
    else fb[i] = frag_mnmajor(sb, wn * 128 + 32 * i, s, lane);
  }
}

__device__ __forceinline__ void mfma_step(const bf16x8 (&fa)[4], const bf16x8 (&fb)[4], f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
}

// Map a workgroup id to a tile.  The hardware deals workgroup ids to the 8
// XCDs round-robin, so ids equal mod 8 share an XCD (and its L2): each XCD
// gets a contiguous run of tiles, and within the run tiles go in groups of
// 8 M-tiles per N-tile column, so the 32 workgroups an XCD runs at once
// cover about 8 x 4 tiles and share both operands' k-slabs in L2.
constexpr int GROUP_M = 8;
__device__ __forceinline__ void tile_of(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int xcd = pid & 7;
  const int local = pid >> 3;
  const int l = xcd * (total >> 3) + min(xcd, total & 7) + local;
  const int per_group = GROUP_M * tiles_n;
  const int gid = l / per_group;
  const int first_m = gid * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int r = l - gid * per_group;
  tm = first_m + r % gsz;
  tn = r / gsz;
}

// LDS read instructions one read_frags issues.
template <bool A_KMAJOR, bool B_KMAJOR>
constexpr int frag_reads() { return (A_KMAJOR ? 4 : 8) + (B_KMAJOR ? 4 : 8); }

// Scheduling masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;

// Instruction order is pinned per k step: NR LDS reads and NV DMAs spread
// evenly between the 16 MFMAs.  A DMA issue can stall the wave while the
// address unit is busy, and a stalled wave issues no MFMA, so no two DMAs sit
// next to each other.
template <int NR, int NV>
__device__ __forceinline__ void interleave_step() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if (i < NR) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    if (NV > 0 && (i % (16 / (NV > 0 ? NV : 1))) == 0 && i / (16 / (NV > 0 ? NV : 1)) < NV)
      __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
  }
}

// ---- Both operands K-major: fragments one k step ahead (two register sets).
// Stage D+1's DMAs go out over the last k step of stage D-1 and the first two
// of stage D.  At the start of stage D's last k step one barrier (after
// vmcnt(0), lgkmcnt(0)) makes D+1 visible everywhere and frees D's buffer,
// whose refill with stage D+2 starts right there.
//
// Why 64-wide stages: with 32-wide ones every row of a K-major tile is a
// 64-byte piece, so each 1 KB DMA covers 16 half cache lines; the address
// unit then spent about 33 cycles per DMA (TA_BUSY over the DMA count) and 32
// of them per 1024 MFMA cycles kept it saturated.  Measured on the
// projection, recompute and a square shape: 7.5-10.6% faster than the
// earlier four-buffer 32-wide loop.
//
// Stage D in buffers (ca, cb), stage D+1 in (na, nb).  NEXT: there is a stage
// D+1 (whose remaining DMAs go out in k steps 0 and 1).  NEXT2: there is a
// stage D+2 (its first DMAs go out in k step 3, into (ca, cb)).
template <bool NEXT, bool NEXT2>
__device__ __forceinline__ void stage_kk(bf16* ca, bf16* cb, bf16* na, bf16* nb, int D, const Loader<true>& la,
                                        const Loader<true>& lb, int wave, int wm, int wn, int lane,
                                        bf16x8 (&fa)[2][4], bf16x8 (&fb)[2][4], f32x16 (&acc)[4][4]) {
  read_frags<true, true>(ca, cb, 1, wm, wn, lane, fa[1], fb[1]);
  if constexpr (NEXT) {
    la.issue<6, 8>(na, (D + 1) * BK2, wave);
    lb.issue<0, 3>(nb, (D + 1) * BK2, wave);
  }
  mfma_step(fa[0], fb[0], acc);
  interleave_step<8, NEXT ? 5 : 0>();
  __builtin_amdgcn_sched_barrier(0);

  read_frags<true, true>(ca, cb, 2, wm, wn, lane, fa[0], fb[0]);
  if constexpr (NEXT) lb.issue<3, 8>(nb, (D + 1) * BK2, wave);
  mfma_step(fa[1], fb[1], acc);
  interleave_step<8, NEXT ? 5 : 0>();
  __builtin_amdgcn_sched_barrier(0);

  read_frags<true, true>(ca, cb, 3, wm, wn, lane, fa[1], fb[1]);
  mfma_step(fa[0], fb[0], acc);
  interleave_step<8, 0>();
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (NEXT) {
    stage_barrier<0>();
    read_frags<true, true>(na, nb, 0, wm, wn, lane, fa[0], fb[0]);
    if constexpr (NEXT2) la.issue<0, 6>(ca, (D + 2) * BK2, wave);
  }
  mfma_step(fa[1], fb[1], acc);
  interleave_step<NEXT ? 8 : 0, NEXT2 ? 6 : 0>();
  __builtin_amdgcn_sched_barrier(0);
}

// nk counts 32-wide steps and is a multiple of NST, so there is an even
// number (at least two) of 64-wide stages.
__device__ __forceinline__ void mainloop_kk(const Operand& A, const Operand& B, int m0, int n0, int nk, bf16* s0,
                                           bf16* s1, bf16* s2, bf16* s3, f32x16 (&acc)[4][4]) {
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
  const Loader<true> la(A, m0, wave, lane);
  const Loader<true> lb(B, n0, wave, lane);
  // Prologue: stage 0 whole, the first part of stage 1 (the rest goes out in
  // stage 0's first two k steps, as in the steady state).
  la.issue<0, 8>(s0, 0, wave);
  lb.issue<0, 8>(s1, 0, wave);
  la.issue<0, 6>(s2, BK2, wave);
  stage_barrier<6>();
  bf16x8 fa[2][4], fb[2][4];
  read_frags<true, true>(s0, s1, 0, wm, wn, lane, fa[0], fb[0]);
  int D = 0;
  for (; D + 2 < nd; D += 2) {
    stage_kk<true, true>(s0, s1, s2, s3, D, la, lb, wave, wm, wn, lane, fa, fb, acc);
    stage_kk<true, true>(s2, s3, s0, s1, D + 1, la, lb, wave, wm, wn, lane, fa, fb, acc);
  }
  // The two stages after the loop take the lane index through an opaque
  // move, so that their LDS addresses are computed here rather than before
  // the loop and kept in scratch across it.
  int lane_t = lane;
  asm volatile("" : "+v"(lane_t));
  stage_kk<true, false>(s0, s1, s2, s3, D, la, lb, wave, wm, wn, lane_t, fa, fb, acc);
  stage_kk<false, false>(s2, s3, s0, s1, D + 1, la, lb, wave, wm, wn, lane_t, fa, fb, acc);
  stage_barrier<0>();
}

// ---- An MN-major operand (dH, dW): fragments two k steps ahead, into four
// register sets, one per k step of a stage.  The barrier sits at the start of
// k step 2, where stage D+1's first fragments are read; stage D+1's DMAs go
// out in k steps 2 and 3 of stage D-1 and k step 0 of stage D.  Against the
// earlier 32-wide four-buffer loop: dH 1.2% and dW 1.7% faster.
template <bool A_KMAJOR, bool B_KMAJOR, bool NEXT, bool NEXT2>
__device__ __forceinline__ void stage_mn(bf16* ca, bf16* cb, bf16* na, bf16* nb, int D, const Loader<A_KMAJOR>& la,
                                       const Loader<B_KMAJOR>& lb, int wave, int wm, int wn, int lane,
                                       bf16x8 (&fa)[4][4], bf16x8 (&fb)[4][4], f32x16 (&acc)[4][4]) {
  constexpr int NR = frag_reads<A_KMAJOR, B_KMAJOR>();
  // s0: part 3 of D+1
  read_frags<A_KMAJOR, B_KMAJOR>(ca, cb, 2, wm, wn, lane, fa[2], fb[2]);
  if constexpr (NEXT) lb.template issue<3, 8>(nb, (D + 1) * BK2, wave);
  mfma_step(fa[0], fb[0], acc);
  interleave_step<NR, NEXT ? 5 : 0>();
  __builtin_amdgcn_sched_barrier(0);
  // s1
  read_frags<A_KMAJOR, B_KMAJOR>(ca, cb, 3, wm, wn, lane, fa[3], fb[3]);
  mfma_step(fa[1], fb[1], acc);
  interleave_step<NR, 0>();
  __builtin_amdgcn_sched_barrier(0);
  // s2: barrier, D+1's first fragments, part 1 of D+2
  if constexpr (NEXT) {
    stage_barrier<0>();
    read_frags<A_KMAJOR, B_KMAJOR>(na, nb, 0, wm, wn, lane, fa[0], fb[0]);
    if constexpr (NEXT2) la.template issue<0, 6>(ca, (D + 2) * BK2, wave);
  }
  mfma_step(fa[2], fb[2], acc);
  interleave_step<NEXT ? NR : 0, NEXT2 ? 6 : 0>();
  __builtin_amdgcn_sched_barrier(0);
  // s3: part 2 of D+2
  if constexpr (NEXT) read_frags<A_KMAJOR, B_KMAJOR>(na, nb, 1, wm, wn, lane, fa[1], fb[1]);
  if constexpr (NEXT2) {
    la.template issue<6, 8>(ca, (D + 2) * BK2, wave);
    lb.template issue<0, 3>(cb, (D + 2) * BK2, wave);
  }
  mfma_step(fa[3], fb[3], acc);
  interleave_step<NEXT ? NR : 0, NEXT2 ? 5 : 0>();
  __builtin_amdgcn_sched_barrier(0);
}

template <bool A_KMAJOR, bool B_KMAJOR>
__device__ __forceinline__ void mainloop_mn(const Operand& A, const Operand& B, int m0, int n0, int nk, bf16* s0,
                                          bf16* s1, bf16* s2, bf16* s3, f32x16 (&acc)[4][4]) {
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
  const Loader<A_KMAJOR> la(A, m0, wave, lane);
  const Loader<B_KMAJOR> lb(B, n0, wave, lane);
  la.template issue<0, 8>(s0, 0, wave);
  lb.template issue<0, 8>(s1, 0, wave);
  la.template issue<0, 8>(s2, BK2, wave);
  lb.template issue<0, 3>(s3, BK2, wave);
  stage_barrier<11>();
  bf16x8 fa[4][4], fb[4][4];
  read_frags<A_KMAJOR, B_KMAJOR>(s0, s1, 0, wm, wn, lane, fa[0], fb[0]);
  read_frags<A_KMAJOR, B_KMAJOR>(s0, s1, 1, wm, wn, lane, fa[1], fb[1]);
  int D = 0;
  for (; D + 2 < nd; D += 2) {
    stage_mn<A_KMAJOR, B_KMAJOR, true, true>(s0, s1, s2, s3, D, la, lb, wave, wm, wn, lane, fa, fb, acc);
    stage_mn<A_KMAJOR, B_KMAJOR, true, true>(s2, s3, s0, s1, D + 1, la, lb, wave, wm, wn, lane, fa, fb, acc);
  }
  int lane_t = lane;  // as in mainloop_kk
  asm volatile("" : "+v"(lane_t));
  stage_mn<A_KMAJOR, B_KMAJOR, true, false>(s0, s1, s2, s3, D, la, lb, wave, wm, wn, lane_t, fa, fb, acc);
  stage_mn<A_KMAJOR, B_KMAJOR, false, false>(s2, s3, s0, s1, D + 1, la, lb, wave, wm, wn, lane_t, fa, fb, acc);
  stage_barrier<0>();
}

// Row / column of accumulator register r of block (mb, nb) within the tile.
__device__ __forceinline__ int acc_row(int wm, int mb, int r, int lane) {
  return wm * 128 + 32 * mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int nb, int lane) { return wn * 128 + 32 * nb + (lane & 31); }

// Workgroup pid's tile: its first rows (m0, n0) and K steps; false for a
// workgroup with no tile.  With tokens along M or N, the grid covers every
// token tile the host allows for, but only ceil(Tv / 256) of them hold valid
// tokens (Tv is read on the device).  The workgroup ids are mapped onto those
// tiles alone and the rest exit: mapped over the full grid, the tiles past Tv
// took whole XCDs' shares (tile_of gives each XCD a contiguous run), and at
// half the tokens ignored half the XCDs sat idle in dH.
__device__ __forceinline__ bool map_tile(const Schedule& sch, int pid, int& m0, int& n0, int& k_steps) {
  int tiles_m = sch.tiles_m, tiles_n = sch.tiles_n;
  k_steps = sch.k_steps;
  if (sch.tok_dim != 0) {
    const int tv = *sch.tok_count;
    const int tok_tiles = (tv + BM - 1) / BM;
    if (sch.tok_dim == 1) tiles_m = min(tiles_m, tok_tiles);
    if (sch.tok_dim == 2) tiles_n = min(tiles_n, tok_tiles);
    if (sch.tok_dim == 3) k_steps = (tv + NST * BK - 1) / (NST * BK) * NST;
    if (pid >= tiles_m * tiles_n) return false;
  }
  int tm, tn;
  tile_of(pid, tiles_m, tiles_n, tm, tn);
  m0 = tm * BM;
  n0 = tn * BN;
  return true;
}

// One tile: schedule, early exit for tiles past the valid tokens, main loop,
// then the epilogue (which may reuse the first stage's LDS).
template <bool A_KMAJOR, bool B_KMAJOR, class Epi>
__device__ __forceinline__ void run_tile(const Operand& A, const Operand& B, const Schedule& sch,
                                         const typename Epi::Params& ep, int pid, bf16* s0, bf16* s1, bf16* s2,
                                         bf16* s3) {
  int m0, n0, k_steps;
  if (!map_tile(sch, pid, m0, n0, k_steps)) return;
  f32x16 acc[4][4];
  if constexpr (A_KMAJOR && B_KMAJOR) mainloop_kk(A, B, m0, n0, k_steps, s0, s1, s2, s3, acc);
  else mainloop_mn<A_KMAJOR, B_KMAJOR>(A, B, m0, n0, k_steps, s0, s1, s2, s3, acc);
  Epi::apply(ep, acc, m0, n0, s0);
}

template <bool A_KMAJOR, bool B_KMAJOR, class Epi>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_kernel(Operand A, Operand B, Schedule sch,
                                                            typename Epi::Params ep) {
  __shared__ __attribute__((aligned(1024))) bf16 s0[STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 s1[STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 s2[STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 s3[STAGE_ELEMS];
  run_tile<A_KMAJOR, B_KMAJOR, Epi>(A, B, sch, ep, blockIdx.x, s0, s1, s2, s3);
}

// Two independent GEMMs in one launch: workgroups [0, n1) take the first
// problem's tiles (n1 is its tile count rounded up to a multiple of 8, so
// that the second problem's tiles keep the id-to-XCD mapping tile_of
// assumes), the rest the second's.  The hardware hands out workgroups in id
// order, so compute units that finish the first problem's last, partly
// filled round of tiles go on to the second problem at once.
template <bool A1_KMAJOR, bool B1_KMAJOR, class Epi1, bool A2_KMAJOR, bool B2_KMAJOR, class Epi2>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_pair(Operand A1, Operand B1, Schedule sch1,
                                                          typename Epi1::Params ep1, int n1, Operand A2, Operand B2,
                                                          Schedule sch2, typename Epi2::Params ep2) {
  __shared__ __attribute__((aligned(1024))) bf16 s0[STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 s1[STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 s2[STAGE_ELEMS];
  __shared__ __attribute__((aligned(1024))) bf16 s3[STAGE_ELEMS];
  const int pid = blockIdx.x;
  if (pid < n1) {
    if (pid < sch1.tiles_m * sch1.tiles_n)
      run_tile<A1_KMAJOR, B1_KMAJOR, Epi1>(A1, B1, sch1, ep1, pid, s0, s1, s2, s3);
  } else {
    run_tile<A2_KMAJOR, B2_KMAJOR, Epi2>(A2, B2, sch2, ep2, pid - n1, s0, s1, s2, s3);
  }
}

}  // namespace gemm
}  // namespace flce
