// MFMA bf16 -> fp32 tile GEMM for gfx950, shared by every contraction of the
// fused linear cross-entropy path.
//
// One workgroup of 256 threads (4 wave64s arranged 2 x 2) owns a 256 x 256
// output tile; each wave owns 128 x 128 of it as 4 x 4 blocks of the
// v_mfma_f32_32x32x16_bf16 instruction, whose fp32 accumulators live in the
// AGPR half of the register file.  The K dimension advances 64 at a time
// through two LDS stages (2 operands x 32 KB each per stage, 128 KB total),
// filled by global_load_lds_dwordx4: the load unit writes each lane's 16 bytes
// straight into LDS, so staging uses no VGPRs and no LDS write instructions.
//
// Either operand may be K-major (element (mn, k) at ptr[mn*ld + k]) or
// MN-major (element (mn, k) at ptr[k*ld + mn]); the LDS tile keeps the
// global layout, so loads stay fully coalesced either way:
//  - K-major tile: 256 rows x 64 k (128-byte rows).  An MFMA fragment (one
//    row, 8 consecutive k) is one ds_read_b128.  The 16-byte chunk c of row r
//    sits at chunk c ^ swz_k(r), which spreads the 16 (or 8) lanes that the
//    LDS services together over distinct banks.
//  - MN-major tile: 64 k-rows x 256 mn (512-byte rows).  A fragment is built
//    from two ds_read_b64_tr_b16: within each 16-lane group the hardware
//    transposes a 4 (k) x 16 (mn) block so that lane i receives column i,
//    four consecutive k.  Chunk pairs are XOR-swizzled per k-row so the four
//    rows one group reads, and the two groups of a half-wave, hit distinct
//    banks.
//
// The accumulator layout of the 32x32 MFMA: lane l, register r holds element
// (row 8*(r/4) + 4*(l/32) + r%4, column l%32) of its block.
#pragma once

#include "device_common.hpp"

namespace flce {
namespace gemm {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int NTHREADS = 256;
constexpr int TILE_ELEMS = 256 * BK;          // one operand, one stage
constexpr int STAGE_ELEMS = 2 * TILE_ELEMS;   // A + B
constexpr int SMEM_ELEMS = 2 * STAGE_ELEMS;   // two stages: 128 KB

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
  int k_steps;              // K / BK when the K extent is known on the host
  const int* tok_count;     // device count of valid tokens (may be null)
  int tok_dim;              // 0: none, 1: M is tokens, 2: N is tokens, 3: K is tokens
};

__device__ __forceinline__ int swz_k(int r) { return (r ^ (r >> 3)) & 7; }

// Chunk XOR for MN-major rows: pairs of 16-byte chunks are XOR-ed with
// t(k % 4) in {0, 3, 5, 6}; t and t ^ 1 cover all eight pair slots of 256 B.
__device__ __forceinline__ int swz_mn(int k) { return ((0x6530 >> ((k & 3) * 4)) & 0xF) << 1; }

__device__ __forceinline__ void lds_dma16(const bf16* src, bf16* lds_dst) {
  __builtin_amdgcn_global_load_lds((const void*)src, (FLCE_LDS void*)lds_dst, 16, 0, 0);
}

// Stage one 256 (mn) x 64 (k) K-major tile: 32 KB = 32 wave-instructions of
// 1 KB (8 rows), 8 per wave.
__device__ __forceinline__ void load_tile_kmajor(const Operand& op, int mn0, int k0, bf16* dst,
                                                 int wave, int lane) {
  const bf16* base = op.ptr + (int64_t)k0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int b = wave * 8 + q;
    const int r = b * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz_k(r);
    const int gr = min(mn0 + r, op.mn_max);
    lds_dma16(base + (int64_t)gr * op.ld + c * 8, dst + b * 512);
  }
}

// Stage one 64 (k) x 256 (mn) MN-major tile: 32 wave-instructions of 1 KB
// (2 k-rows of 512 B), 8 per wave.
__device__ __forceinline__ void load_tile_mnmajor(const Operand& op, int mn0, int k0, bf16* dst,
                                                  int wave, int lane) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int b = wave * 8 + q;
    const int kk = b * 2 + (lane >> 5);
    const int c = (lane & 31) ^ swz_mn(kk);
    const int gk = min(k0 + kk, op.k_max);
    const int col = min(mn0 + c * 8, op.mn_max - 7);
    lds_dma16(op.ptr + (int64_t)gk * op.ld + col, dst + b * 512);
  }
}

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
  const int kb = 16 * s + 8 * (g >> 1) + (j >> 2);
  const int k0 = kb;
  const int k1 = kb + 4;
  const bf16* p0 = tile + k0 * 256 + (((col >> 3) ^ swz_mn(k0)) << 3) + (col & 7);
  const bf16* p1 = tile + k1 * 256 + (((col >> 3) ^ swz_mn(k1)) << 3) + (col & 7);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FLCE_LDS bf16x4*)p0);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FLCE_LDS bf16x4*)p1);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Map a workgroup id to a tile so that the workgroups one XCD runs (ids that
// are equal mod 8) get a contiguous run of tiles, with N varying fastest.
__device__ __forceinline__ void tile_of(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int xcd = pid & 7;
  const int local = pid >> 3;
  const int base = xcd * (total >> 3) + min(xcd, total & 7);
  const int logical = base + local;
  tm = logical / tiles_n;
  tn = logical - tm * tiles_n;
}

// The main loop.  acc[mb][nb] is the 32x32 block at rows wm*128 + 32*mb,
// columns wn*128 + 32*nb of the tile.
template <bool A_KMAJOR, bool B_KMAJOR>
__device__ __forceinline__ void mainloop(const Operand& A, const Operand& B, int m0, int n0,
                                         int k_steps, bf16* smem, f32x16 (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wm = wave >> 1;
  const int wn = wave & 1;

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  auto stage_load = [&](int stage, int k0) {
    bf16* sa = smem + stage * STAGE_ELEMS;
    bf16* sb = sa + TILE_ELEMS;
    if constexpr (A_KMAJOR) load_tile_kmajor(A, m0, k0, sa, wave, lane);
    else load_tile_mnmajor(A, m0, k0, sa, wave, lane);
    if constexpr (B_KMAJOR) load_tile_kmajor(B, n0, k0, sb, wave, lane);
    else load_tile_mnmajor(B, n0, k0, sb, wave, lane);
  };

  if (k_steps > 0) stage_load(0, 0);
  for (int it = 0; it < k_steps; ++it) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 1 < k_steps) stage_load((it + 1) & 1, (it + 1) * BK);
    const bf16* sa = smem + (it & 1) * STAGE_ELEMS;
    const bf16* sb = sa + TILE_ELEMS;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (A_KMAJOR) fa[i] = frag_kmajor(sa, wm * 128 + 32 * i + (lane & 31), s, lane);
        else fa[i] = frag_mnmajor(sa, wm * 128 + 32 * i, s, lane);
        if constexpr (B_KMAJOR) fb[i] = frag_kmajor(sb, wn * 128 + 32 * i + (lane & 31), s, lane);
        else fb[i] = frag_mnmajor(sb, wn * 128 + 32 * i, s, lane);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }
  __syncthreads();
}

// Row / column of accumulator register r of block (mb, nb) within the tile.
__device__ __forceinline__ int acc_row(int wm, int mb, int r, int lane) {
  return wm * 128 + 32 * mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int nb, int lane) { return wn * 128 + 32 * nb + (lane & 31); }

// The kernel: schedule, early exit for tiles past the valid tokens, main loop,
// then the epilogue.
template <bool A_KMAJOR, bool B_KMAJOR, class Epi>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_kernel(Operand A, Operand B, Schedule sch,
                                                            typename Epi::Params ep) {
  __shared__ __attribute__((aligned(1024))) bf16 smem[SMEM_ELEMS];
  int tm, tn;
  tile_of(blockIdx.x, sch.tiles_m, sch.tiles_n, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  int k_steps = sch.k_steps;
  if (sch.tok_dim != 0) {
    const int tv = *sch.tok_count;
    if (sch.tok_dim == 1 && m0 >= tv) return;
    if (sch.tok_dim == 2 && n0 >= tv) return;
    if (sch.tok_dim == 3) k_steps = (tv + BK - 1) / BK;
  }
  f32x16 acc[4][4];
  mainloop<A_KMAJOR, B_KMAJOR>(A, B, m0, n0, k_steps, smem, acc);
  Epi::apply(ep, acc, m0, n0, smem);
}

}  // namespace gemm
}  // namespace flce
