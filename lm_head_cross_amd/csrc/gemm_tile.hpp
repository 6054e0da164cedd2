// MFMA bf16 -> fp32 tile GEMM for gfx950, shared by every contraction of the
// fused linear cross-entropy path.
//
// One workgroup of 256 threads (4 wave64s arranged 2 x 2) owns a 256 x 256
// output tile; each wave owns 128 x 128 of it as 4 x 4 blocks of the
// v_mfma_f32_32x32x16_bf16 instruction, whose fp32 accumulators live in the
// AGPR half of the register file (one wave per SIMD).
//
// With both operands K-major (the projection and the recompute), K advances
// 64 at a time through two 64 KB LDS stages (mainloop64, described there).
// Otherwise K advances 32 at a time through four LDS stages of 32 KB (A and B
// tiles of 16 KB each), each its own __shared__ array.  Stages are filled by
// buffer_load_dwordx4 ... lds, which writes each lane's 16 bytes straight
// into LDS (no VGPR staging, no LDS write instructions), three stages ahead
// of the stage being multiplied and spread across a stage's MFMAs.  Separate
// arrays let the compiler see that a DMA in flight never aliases the stage
// being read, so it does not stall LDS reads on it; the wait before each
// workgroup barrier names how many DMA instructions may still be
// outstanding.
//
// The MFMA fragments of the next stage (both 16-wide k steps) are read while
// the current stage's 32 MFMAs issue, into four register sets that rotate
// every two stages.  One barrier per stage, at its start, hands the next
// stage over.
//
// Either operand may be K-major (element (mn, k) at ptr[mn*ld + k]) or
// MN-major (element (mn, k) at ptr[k*ld + mn]); the LDS tile keeps the
// global layout, so global loads stay fully coalesced either way:
//  - K-major tile: 256 rows x 32 k (64-byte rows).  A fragment (one row,
//    8 consecutive k) is one ds_read_b128.  The 16-byte chunk c of row r sits
//    at chunk c ^ swz_k(r), which leaves these reads free of bank conflicts.
//  - MN-major tile: 32 k-rows x 256 mn (512-byte rows).  A fragment is two
//    ds_read_b64_tr_b16: within each 16-lane group the hardware transposes a
//    4 (k) x 16 (mn) block so that lane i receives column i, four
//    consecutive k.  Pairs of 16-byte chunks are XOR-swizzled per k-row,
//    which leaves these reads free of bank conflicts.
//
// The accumulator layout of the 32x32 MFMA: lane l, register r holds element
// (row 8*(r/4) + 4*(l/32) + r%4, column l%32) of its block.
#pragma once

#include "device_common.hpp"

namespace flce {
namespace gemm {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 32;
constexpr int NST = 4;                        // LDS stages
constexpr int SUB = BK / 16;                  // MFMA k steps per stage
constexpr int NTHREADS = 256;
constexpr int TILE_ELEMS = 256 * BK;          // one operand, one stage (16 KB)
constexpr int STAGE_ELEMS = 2 * TILE_ELEMS;   // A + B (32 KB)
constexpr int LOADS_PER_STAGE = STAGE_ELEMS * 2 / 16 / NTHREADS;  // DMA instructions per thread (8)
constexpr int LOADS_PER_TILE = LOADS_PER_STAGE / 2;               // per operand (4)

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

// Chosen by measurement (SQ_LDS_BANK_CONFLICT on gfx950 for this exact
// read pattern): XOR-ing chunks with bits 2..3 of the row leaves the
// ds_read_b128 of both k steps conflict-free.
__device__ __forceinline__ int swz_k(int r) { return (r >> 2) & 3; }

// Chunk XOR for MN-major rows: pairs of 16-byte chunks are XOR-ed with
// t(k % 4) in {0, 3, 5, 6}; t and t ^ 1 cover all eight pair slots of 256 B.
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
// would also wait for the DMAs still in flight into the other stages.
template <int N_OUT>
__device__ __forceinline__ void stage_barrier() {
  wait_vm_lgkm0<N_OUT>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-thread DMA sources for one operand, fixed along K: the byte offset of
// each of this thread's 16-byte pieces relative to the tile's origin.
//  - K-major: resource based at the tile's first row; stage k0 adds 2*k0
//    bytes through the scalar offset.
//  - MN-major: resource rebased at k-row k0 for every stage (scalar work);
//    rows past k_max read as zero (the partner operand is zero there too).
template <bool KMAJOR>
struct Loader {
  const bf16* base;
  int64_t ld;
  int k_max;
  __amdgpu_buffer_rsrc_t rsrc;      // K-major only
  unsigned off[LOADS_PER_TILE];     // bytes
  int kk[LOADS_PER_TILE];           // MN-major: k row within the stage
  int col[LOADS_PER_TILE];          // MN-major: column (elements)

  __device__ __forceinline__ Loader(const Operand& op, int mn0, int wave, int lane) {
    ld = op.ld;
    k_max = op.k_max;
    if constexpr (KMAJOR) {
      base = op.ptr + (int64_t)mn0 * op.ld;
      rsrc = make_rsrc(base);
#pragma unroll
      for (int q = 0; q < LOADS_PER_TILE; ++q) {
        const int b = wave * LOADS_PER_TILE + q;   // 1 KB block: 16 rows of 64 B
        const int r = b * 16 + (lane >> 2);
        const int c = (lane & 3) ^ swz_k(r);
        const int gr = min(mn0 + r, op.mn_max) - mn0;
        off[q] = (unsigned)(gr * (int)op.ld + c * 8) * 2u;
        kk[q] = 0;
        col[q] = 0;
      }
    } else {
      base = op.ptr;
      rsrc = make_rsrc(base);
#pragma unroll
      for (int q = 0; q < LOADS_PER_TILE; ++q) {
        const int b = wave * LOADS_PER_TILE + q;   // 1 KB block: 2 k-rows of 512 B
        kk[q] = b * 2 + (lane >> 5);
        const int c = (lane & 31) ^ swz_mn(kk[q]);
        col[q] = min(mn0 + c * 8, op.mn_max - 7);
        off[q] = (unsigned)(kk[q] * (int)op.ld + col[q]) * 2u;
      }
    }
  }

  // Issue this thread's share of the stage starting at k0 into `tile`.
  __device__ __forceinline__ void issue(bf16* tile, int k0, int wave) const {
    if constexpr (KMAJOR) {
      const unsigned soff = (unsigned)k0 * 2u;
#pragma unroll
      for (int q = 0; q < LOADS_PER_TILE; ++q)
        lds_dma16(rsrc, off[q], soff, tile + (wave * LOADS_PER_TILE + q) * 512);
    } else {
      const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (int64_t)k0 * ld);
      if (k0 + BK - 1 <= k_max) {
#pragma unroll
        for (int q = 0; q < LOADS_PER_TILE; ++q)
          lds_dma16(r, off[q], 0, tile + (wave * LOADS_PER_TILE + q) * 512);
      } else {
        // Rows past k_max read as zero: their offsets are made out of range,
        // which the buffer unit answers with zeros and no memory access.
        const int krem = k_max - k0;
#pragma unroll
        for (int q = 0; q < LOADS_PER_TILE; ++q) {
          const unsigned o = kk[q] <= krem ? off[q] : 0x80000000u;
          lds_dma16(r, o, 0, tile + (wave * LOADS_PER_TILE + q) * 512);
        }
      }
    }
  }
};

// Fragment of a K-major tile: row `row` (0..255), k = 16*s + 8*(lane/32) + 0..7.
__device__ __forceinline__ bf16x8 frag_kmajor(const bf16* tile, int row, int s, int lane) {
  const int c = (2 * s + (lane >> 5)) ^ swz_k(row);
  return *(const FLCE_LDS bf16x8*)(tile + row * BK + c * 8);
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

template <bool A_KMAJOR, bool B_KMAJOR>
__device__ __forceinline__ void read_frags(const bf16* stage, int s, int wm, int wn, int lane, bf16x8 (&fa)[4],
                                           bf16x8 (&fb)[4]) {
  const bf16* sa = stage;
  const bf16* sb = stage + TILE_ELEMS;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (A_KMAJOR) fa[i] = frag_kmajor(sa, wm * 128 + 32 * i + (lane & 31), s, lane);
    else fa[i] = frag_mnmajor(sa, wm * 128 + 32 * i, s, lane);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (B_KMAJOR) fb[i] = frag_kmajor(sb, wn * 128 + 32 * i + (lane & 31), s, lane);
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

// s_waitcnt vmcnt <= VM, lgkmcnt <= LG, then the workgroup barrier.
template <int VM, int LG>
__device__ __forceinline__ void stage_barrier_lg() {
  static_assert(VM >= 0 && VM < 64 && LG >= 0 && LG < 16, "waitcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LG << 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One stage of the main loop.  Stage j's fragments (both k steps) were read
// during stage j-1 into register sets U0, U1; this stage reads stage j+1's
// into R0, R1 while its 32 MFMAs issue, and refills the buffer of stage j-1
// with stage `refill_step` (A half during the first k step, B half during
// the second).
//  - The barrier at the start makes stage j+1 visible (WAIT_OUT: this
//    thread's DMA instructions that may still be in flight, those issued
//    after stage j+1's) and frees stage j-1's buffer: every wave finished
//    its reads of stage j-1 before the LDS reads of stage j it issued last,
//    and LDS reads complete in order, so the wait may leave this stage's own
//    2*NR reads outstanding (capped by the 4-bit lgkmcnt field).
//  - HAS_NEXT: there is a stage j+1.  REFILL: there is a stage to issue.
// Instruction order is pinned per k step: LDS reads and DMAs spread evenly
// between the 16 MFMAs.  A DMA issue can stall the wave while the address
// unit is busy, and a stalled wave issues no MFMA, so no two DMAs sit next
// to each other.
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

template <bool A_KMAJOR, bool B_KMAJOR, int WAIT_OUT, bool HAS_NEXT, bool REFILL, int U0, int U1, int R0, int R1,
          class LA, class LB>
__device__ __forceinline__ void stage_compute(bf16* nxt, bf16* refill, int refill_step, const LA& la, const LB& lb,
                                              int wave, int wm, int wn, int lane, bf16x8 (&fa)[4][4],
                                              bf16x8 (&fb)[4][4], f32x16 (&acc)[4][4]) {
  constexpr int NR = frag_reads<A_KMAJOR, B_KMAJOR>();
  constexpr int LG = 2 * NR < 15 ? 2 * NR : 15;
  constexpr int NRD = HAS_NEXT ? NR : 0;
  constexpr int NV = REFILL ? LOADS_PER_TILE : 0;
  if constexpr (HAS_NEXT) {
    stage_barrier_lg<WAIT_OUT, LG>();
    read_frags<A_KMAJOR, B_KMAJOR>(nxt, 0, wm, wn, lane, fa[R0], fb[R0]);
  }
  if constexpr (REFILL) la.issue(refill, refill_step * BK, wave);
  mfma_step(fa[U0], fb[U0], acc);
  interleave_step<NRD, NV>();
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (HAS_NEXT) read_frags<A_KMAJOR, B_KMAJOR>(nxt, 1, wm, wn, lane, fa[R1], fb[R1]);
  if constexpr (REFILL) lb.issue(refill + TILE_ELEMS, refill_step * BK, wave);
  mfma_step(fa[U1], fb[U1], acc);
  interleave_step<NRD, NV>();
  __builtin_amdgcn_sched_barrier(0);
}

// The main loop over nk stages of BK; nk must be a multiple of NST (callers
// pad K to NST * BK with operands that are zero there).  acc[mb][nb] is the
// 32x32 block at rows wm*128 + 32*mb, columns wn*128 + 32*nb of the tile.
//
// Stage j lives in buffer j % 4.  Stages 0..2 are issued up front; stage
// j+3 is issued during stage j into the buffer of stage j-1, so a DMA has
// about two stages of MFMA time to land.  Fragments are read a whole stage
// (two k steps) ahead: the transposing LDS reads of MN-major operands take
// a few hundred cycles under load, more than one k step of MFMAs covers.
// Stage j's k steps use register sets (2j) % 4 and (2j+1) % 4, so the
// pattern repeats every two stages and the loop unrolls over the four
// buffers.
template <bool A_KMAJOR, bool B_KMAJOR>
__device__ __forceinline__ void mainloop(const Operand& A, const Operand& B, int m0, int n0, int nk, bf16* s0,
                                         bf16* s1, bf16* s2, bf16* s3, f32x16 (&acc)[4][4]) {
  const int tid = threadIdx.x;
  // Wave-uniform in an SGPR, so LDS destinations of the DMAs are scalar.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave >> 1;
  const int wn = wave & 1;

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  if (nk <= 0) return;

  const Loader<A_KMAJOR> la(A, m0, wave, lane);
  const Loader<B_KMAJOR> lb(B, n0, wave, lane);
  auto dma = [&](bf16* stage, int step) {
    la.issue(stage, step * BK, wave);
    lb.issue(stage + TILE_ELEMS, step * BK, wave);
  };
  constexpr int L = LOADS_PER_STAGE;

  // Prologue: stages 0..2 in flight; stage 0's fragments read.
  dma(s0, 0);
  dma(s1, 1);
  dma(s2, 2);
  stage_barrier<2 * L>();
  bf16x8 fa[4][4], fb[4][4];
  read_frags<A_KMAJOR, B_KMAJOR>(s0, 0, wm, wn, lane, fa[0], fb[0]);
  read_frags<A_KMAJOR, B_KMAJOR>(s0, 1, wm, wn, lane, fa[1], fb[1]);

  // At the barrier of stage it+J, stage it+J+1 must have landed; stage
  // it+J+2 may still be in flight.
#define FLCE_STAGE(J, REFILL, HAS_NEXT, WAIT)                                                                   \
  stage_compute<A_KMAJOR, B_KMAJOR, WAIT, HAS_NEXT, REFILL, (2 * (J)) % 4, (2 * (J) + 1) % 4, (2 * (J) + 2) % 4, \
                (2 * (J) + 3) % 4>((J) == 0 ? s1 : (J) == 1 ? s2 : (J) == 2 ? s3 : s0,                           \
                                   (J) == 0 ? s3 : (J) == 1 ? s0 : (J) == 2 ? s1 : s2, it + (J) + 3, la, lb, wave, \
                                   wm, wn, lane, fa, fb, acc)
  int it = 0;
  for (; it + NST < nk; it += NST) {
    FLCE_STAGE(0, true, true, L);
    FLCE_STAGE(1, true, true, L);
    FLCE_STAGE(2, true, true, L);
    FLCE_STAGE(3, true, true, L);
  }
  // Last four stages: one refill left, then the in-flight count drains.
  FLCE_STAGE(0, true, true, L);
  FLCE_STAGE(1, false, true, L);
  FLCE_STAGE(2, false, true, 0);
  FLCE_STAGE(3, false, false, 0);
#undef FLCE_STAGE
  stage_barrier<0>();
}


// ---- The K x K main loop: 64-wide k stages, two LDS buffers. ----
//
// With both operands K-major, a 32-wide k stage gives every row a 64-byte
// piece, so each 1 KB DMA instruction covers 16 half cache lines; the address
// path then spends about 33 cycles per instruction (TA_BUSY against the DMA
// count), and 32 of them per 1024 MFMA cycles leave it saturated.  With
// 64-wide stages each DMA covers 8 whole 128-byte lines.  Measured on the
// projection, recompute and a square shape: 7.5-10.6% faster than the
// four-buffer 32-wide loop below.
//
// A stage of 64 k is 64 KB (A and B, 256 rows x 128 B each), so LDS holds two:
// A in s0 / s2, B in s1 / s3, each its own array (own alias scope).  A stage
// runs as four k steps of 16 (16 MFMAs per wave each); fragments are read one
// k step ahead from LDS with ds_read_b128.  Stage D+1's DMAs go out over the
// last k step of stage D-1 and the first two of stage D; at the start of
// stage D's last k step one barrier (after vmcnt(0), lgkmcnt(0)) makes D+1
// visible everywhere and frees D's buffer, whose refill with stage D+2 starts
// right there.  Rows of 128 B hold 8 chunks of 16 B; chunk c of row r sits at
// slot c ^ ((r >> 1) & 7), which keeps the 8- and 16-lane phases of a
// fragment read (consecutive rows, one chunk) on distinct banks.
constexpr int BK2 = 64;
__device__ __forceinline__ int swz64(int r) { return (r >> 1) & 7; }

// Per-thread DMA sources of one K-major operand for 64-wide stages: 8 blocks
// of 1 KB (8 rows x 128 B) per wave; stage k0 adds 2*k0 bytes through the
// scalar offset.
struct Loader64 {
  __amdgpu_buffer_rsrc_t rsrc;
  unsigned off[8];
  __device__ __forceinline__ Loader64(const Operand& op, int mn0, int wave, int lane) {
    rsrc = make_rsrc(op.ptr + (int64_t)mn0 * op.ld);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int b = wave * 8 + q;
      const int r = b * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz64(r);
      const int gr = min(mn0 + r, op.mn_max) - mn0;
      off[q] = (unsigned)(gr * (int)op.ld + c * 8) * 2u;
    }
  }
  // Blocks [Q0, Q1) of this wave's share of the stage starting at k0.
  template <int Q0, int Q1>
  __device__ __forceinline__ void issue(bf16* tile, int k0, int wave) const {
    const unsigned soff = (unsigned)k0 * 2u;
#pragma unroll
    for (int q = Q0; q < Q1; ++q) lds_dma16(rsrc, off[q], soff, tile + (wave * 8 + q) * 512);
  }
};

// Fragment of a 64-wide K-major tile: row `row`, k = 16*s + 8*(lane/32) + 0..7.
__device__ __forceinline__ bf16x8 frag64(const bf16* tile, int row, int s, int lane) {
  const int c = (2 * s + (lane >> 5)) ^ swz64(row);
  return *(const FLCE_LDS bf16x8*)(tile + row * BK2 + c * 8);
}

__device__ __forceinline__ void read_frags64(const bf16* sa, const bf16* sb, int s, int wm, int wn, int lane,
                                             bf16x8 (&fa)[4], bf16x8 (&fb)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[i] = frag64(sa, wm * 128 + 32 * i + (lane & 31), s, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) fb[i] = frag64(sb, wn * 128 + 32 * i + (lane & 31), s, lane);
}

// Stage D in buffers (ca, cb), stage D+1 in (na, nb).  NEXT: there is a stage
// D+1 (whose remaining DMAs go out in k steps 0 and 1).  NEXT2: there is a
// stage D+2 (its first DMAs go out in k step 3, into (ca, cb)).
template <bool NEXT, bool NEXT2>
__device__ __forceinline__ void stage64(bf16* ca, bf16* cb, bf16* na, bf16* nb, int D, const Loader64& la,
                                        const Loader64& lb, int wave, int wm, int wn, int lane,
                                        bf16x8 (&fa)[2][4], bf16x8 (&fb)[2][4], f32x16 (&acc)[4][4]) {
  read_frags64(ca, cb, 1, wm, wn, lane, fa[1], fb[1]);
  if constexpr (NEXT) {
    la.issue<6, 8>(na, (D + 1) * BK2, wave);
    lb.issue<0, 3>(nb, (D + 1) * BK2, wave);
  }
  mfma_step(fa[0], fb[0], acc);
  interleave_step<8, NEXT ? 5 : 0>();
  __builtin_amdgcn_sched_barrier(0);

  read_frags64(ca, cb, 2, wm, wn, lane, fa[0], fb[0]);
  if constexpr (NEXT) lb.issue<3, 8>(nb, (D + 1) * BK2, wave);
  mfma_step(fa[1], fb[1], acc);
  interleave_step<8, NEXT ? 5 : 0>();
  __builtin_amdgcn_sched_barrier(0);

  read_frags64(ca, cb, 3, wm, wn, lane, fa[1], fb[1]);
  mfma_step(fa[0], fb[0], acc);
  interleave_step<8, 0>();
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (NEXT) {
    stage_barrier<0>();
    read_frags64(na, nb, 0, wm, wn, lane, fa[0], fb[0]);
    if constexpr (NEXT2) la.issue<0, 6>(ca, (D + 2) * BK2, wave);
  }
  mfma_step(fa[1], fb[1], acc);
  interleave_step<NEXT ? 8 : 0, NEXT2 ? 6 : 0>();
  __builtin_amdgcn_sched_barrier(0);
}

// nk counts 32-wide steps and is a multiple of NST, so there is an even
// number (at least two) of 64-wide stages.
__device__ __forceinline__ void mainloop64(const Operand& A, const Operand& B, int m0, int n0, int nk, bf16* s0,
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
  const Loader64 la(A, m0, wave, lane);
  const Loader64 lb(B, n0, wave, lane);
  // Prologue: stage 0 whole, the first part of stage 1 (the rest goes out in
  // stage 0's first two k steps, as in the steady state).
  la.issue<0, 8>(s0, 0, wave);
  lb.issue<0, 8>(s1, 0, wave);
  la.issue<0, 6>(s2, BK2, wave);
  stage_barrier<6>();
  bf16x8 fa[2][4], fb[2][4];
  read_frags64(s0, s1, 0, wm, wn, lane, fa[0], fb[0]);
  int D = 0;
  for (; D + 2 < nd; D += 2) {
    stage64<true, true>(s0, s1, s2, s3, D, la, lb, wave, wm, wn, lane, fa, fb, acc);
    stage64<true, true>(s2, s3, s0, s1, D + 1, la, lb, wave, wm, wn, lane, fa, fb, acc);
  }
  stage64<true, false>(s0, s1, s2, s3, D, la, lb, wave, wm, wn, lane, fa, fb, acc);
  stage64<false, false>(s2, s3, s0, s1, D + 1, la, lb, wave, wm, wn, lane, fa, fb, acc);
  stage_barrier<0>();
}

// Row / column of accumulator register r of block (mb, nb) within the tile.
__device__ __forceinline__ int acc_row(int wm, int mb, int r, int lane) {
  return wm * 128 + 32 * mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int nb, int lane) { return wn * 128 + 32 * nb + (lane & 31); }

// One tile: schedule, early exit for tiles past the valid tokens, main loop,
// then the epilogue (which may reuse the first stage's LDS).
template <bool A_KMAJOR, bool B_KMAJOR, class Epi>
__device__ __forceinline__ void run_tile(const Operand& A, const Operand& B, const Schedule& sch,
                                         const typename Epi::Params& ep, int pid, bf16* s0, bf16* s1, bf16* s2,
                                         bf16* s3) {
  int tm, tn;
  tile_of(pid, sch.tiles_m, sch.tiles_n, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  int k_steps = sch.k_steps;
  if (sch.tok_dim != 0) {
    const int tv = *sch.tok_count;
    if (sch.tok_dim == 1 && m0 >= tv) return;
    if (sch.tok_dim == 2 && n0 >= tv) return;
    if (sch.tok_dim == 3) k_steps = (tv + NST * BK - 1) / (NST * BK) * NST;
  }
  f32x16 acc[4][4];
  if constexpr (A_KMAJOR && B_KMAJOR) mainloop64(A, B, m0, n0, k_steps, s0, s1, s2, s3, acc);
  else mainloop<A_KMAJOR, B_KMAJOR>(A, B, m0, n0, k_steps, s0, s1, s2, s3, acc);
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
