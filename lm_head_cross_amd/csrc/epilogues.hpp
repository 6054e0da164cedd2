// Epilogues of the tile GEMM: what happens to a 256 x 256 fp32 accumulator
// tile once its K loop is done.
#pragma once

#include "gemm_tile.hpp"

namespace flce {
namespace epi {

using gemm::acc_col;
using gemm::acc_row;

// Forward: logits tile z^T (rows = head rows v, columns = compacted tokens t).
// Applies the softcap, drops rows v >= Vu, and reduces each token column to a
// (max, sum exp(z' - max)) pair for this vocab tile; the tile that holds a
// token's label also records z'[t, y_t].  ("nemo_automodel.components.
// models.inkling2.loss", class description: the softcap and the loss are fp32
// arithmetic, and only head rows below unpadded_vocab_size take part in the
// softmax.)
//
// MB: MFMA blocks per wave along the head rows (4 for the 256-row tile, 6
// for the 384-row one); the waves' two rows of 32*MB head rows are merged
// through LDS at the end.
template <bool CAP, int MB = 4>
struct Lse {
  struct Params {
    float2* partials;       // [tiles_v][ldp]
    int ldp;
    float* label_logit;     // [Tvp]
    const int32_t* yc;      // compacted labels [Tvp]
    const int* tok_count;   // Tv
    int vocab_limit;        // Vu
    float softcap, inv_softcap;
  };
  static constexpr int kWaveRows = 32 * MB;
  static constexpr int kTileRows = 2 * kWaveRows;

  static __device__ __forceinline__ void apply(const Params& p, f32x16 (&acc)[MB][4], int m0, int n0,
                                               bf16* smem) {
    apply(p, acc, m0, m0, n0, smem);
  }

  // m0: the tile's first head row (its partials slot is m0 / kTileRows);
  // a0 <= m0: the head row of accumulator row 0.  Rows outside [m0, Vu) are
  // dropped: past Vu they are not in the softmax, below m0 (a last tile
  // computed shifted down) they belong to the tile before.
  //
  // Per lane and token column, the 16 values of one MFMA block at a time:
  // the running (max, sum) pair takes each block with one rescale, which
  // keeps a block's 16 values the only temporaries.
  static __device__ __forceinline__ void apply(const Params& p, f32x16 (&acc)[MB][4], int m0, int a0, int n0,
                                               bf16* smem) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tv = *p.tok_count;
    float* xchg = reinterpret_cast<float*>(smem);  // [2][256][4]
    const bool ragged = a0 < m0 || a0 + kTileRows > p.vocab_limit;
    const int row0 = a0 + wm * kWaveRows;   // head row of this wave's first accumulator row
    const float k2 = 2.0f * kLog2e * p.inv_softcap;
    const float c = p.softcap;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int tc = acc_col(wn, nb, lane);
      const int t = n0 + tc;
      const int y_in = p.yc[t];  // t < Tvp: always inside the buffer
      const int y = t < tv ? y_in : -1;
      // The label's logit is looked for only when some lane's label falls in
      // this wave's rows (about 5% of the time at V = 128256).
      const bool scan = __builtin_amdgcn_ballot_w64((unsigned)(y - row0) < (unsigned)kWaveRows) != 0;
      float m = kNegInf, s = 0.0f, lab = 0.0f, found = 0.0f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float z[16];
        float bm = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = acc[mb][nb][r];
          if constexpr (CAP) v = __builtin_fmaf(softcap_recip(v, k2), -2.0f * c, c);  // c tanh(z / c)
          z[r] = v;
        }
        if (ragged) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = row0 + 32 * mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            z[r] = (row >= m0 && row < p.vocab_limit) ? z[r] : kNegInf;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) bm = __builtin_fmaxf(bm, z[r]);
        if (scan) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = row0 + 32 * mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const bool hit = row == y && row >= m0;
            lab = hit ? z[r] : lab;
            found = hit ? 1.0f : found;
          }
        }
        const float mn = __builtin_fmaxf(m, bm);
        if (mn != kNegInf) {
          // exp(z - mn) as one fma and the hardware base-2 exponential; the
          // running sum is rescaled from the old max (exp2(-inf) = 0 first).
          const float mn2 = mn * kLog2e;
          float bs = 0.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) bs += __builtin_amdgcn_exp2f(__builtin_fmaf(z[r], kLog2e, -mn2));
          s = s * __builtin_amdgcn_exp2f(__builtin_fmaf(m, kLog2e, -mn2)) + bs;
          m = mn;
        }
      }
      // The two lane halves hold the same token column.
      lse_merge(m, s, lane_xor32(m), lane_xor32(s));
      const float lab2 = lane_xor32(lab);
      const float found2 = lane_xor32(found);
      if (found2 != 0.0f) { lab = lab2; found = 1.0f; }
      if (lane < 32) {
        float* e = xchg + ((wm * 256 + tc) << 2);
        e[0] = m; e[1] = s; e[2] = lab; e[3] = found;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    // Waves of the top row merge the bottom row's pairs and write out.
    if (wm == 0 && lane < 32) {
      const int tile_v = m0 / kTileRows;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int tc = acc_col(wn, nb, lane);
        const int t = n0 + tc;
        if (t >= tv) continue;
        const float* e0 = xchg + (tc << 2);
        const float* e1 = xchg + ((256 + tc) << 2);
        float m = e0[0], s = e0[1];
        lse_merge(m, s, e1[0], e1[1]);
        p.partials[(int64_t)tile_v * p.ldp + t] = make_float2(m, s);
        if (e0[3] != 0.0f) p.label_logit[t] = e0[2];
        else if (e1[3] != 0.0f) p.label_logit[t] = e1[2];
      }
    }
  }
};

// Backward recompute: logits tile z^T of one vocabulary chunk (rows = chunk
// rows, columns = compacted tokens) turned into the logit gradient
//   G[t, v] = (g/D) (exp(z'[t,v] - lse_t) - [v == y_t]) (1 - (z'/c)^2),
// rounded to bf16 and stored token-major, G[t][v - chunk start].  Positions
// past the valid tokens or the chunk get 0.  (chunked_ce page,
// _ChunkedCrossEntropySum.backward: the fp32 softmax is recomputed.)
//
// The epilogue runs while no MFMA issues, so its per-logit work is kept to
// the minimum: exp(z' - lse) is one fma into the base-2 exponential; g/D
// and the token mask are one per-column factor (0 past the valid tokens);
// with the softcap, t = tanh(z/c) is one exponential, one reciprocal and one
// fma, z' - lse = c t - lse one fma, and the slope 1 - t^2 another.  The
// one-hot term is subtracted only in the columns whose label falls into the
// wave's rows (a wave-uniform branch, about 5% of columns at V = 128256).
template <bool CAP, int MB = 4>
struct Grad {
  struct Params {
    bf16* G;
    int64_t ldg;
    int v0;                  // global row of chunk row 0
    int vw;                  // valid rows in this chunk
    const float* lse;        // [T], original token order
    const int32_t* valid_idx;
    const int32_t* yc;
    const int* tok_count;
    const float* scale;      // g / D
    float softcap, inv_softcap;
  };
  static constexpr int kWaveRows = 32 * MB;

  static __device__ __forceinline__ void apply(const Params& p, f32x16 (&acc)[MB][4], int m0, int n0,
                                               bf16* smem) {
    apply(p, acc, m0, m0, n0, smem);
  }

  // One token column of the wave's accumulators (column block nb): its
  // 16 * MB values, stored from chunk row m0 on.  LABEL: the column's label
  // may fall into these rows (y_rel: label row relative to row0).
  template <bool LABEL, int nb>
  static __device__ __forceinline__ void column(const Params& p, const f32x16 (&acc)[MB][4], int hi,
                                                int row0, int m0, bool shifted, int y_rel, float nl2, float st,
                                                float k2, float cl2, bf16* grow) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 out;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rel = 32 * mb + 8 * q + 4 * hi + i;   // row within the wave's rows
          const float z = acc[mb][nb][4 * q + i];
          float g;
          if constexpr (CAP) {
            const float t = __builtin_fmaf(-2.0f, softcap_recip(z, k2), 1.0f);  // tanh(z / c)
            float d = __builtin_amdgcn_exp2f(__builtin_fmaf(t, cl2, nl2));       // exp(z' - lse)
            if constexpr (LABEL) d -= rel == y_rel ? 1.0f : 0.0f;
            g = d * (__builtin_fmaf(-t, t, 1.0f) * st);
          } else {
            float d = __builtin_amdgcn_exp2f(__builtin_fmaf(z, kLog2e, nl2));
            if constexpr (LABEL) d -= rel == y_rel ? 1.0f : 0.0f;
            g = d * st;
          }
          // A 256-row tile can reach past the chunk's last row (a 384-row
          // tile is shifted to end there).
          if constexpr (MB == 4) g = row0 + rel < p.vw ? g : 0.0f;
          out[i] = (bf16)g;
        }
        const int mq = row0 + 32 * mb + 8 * q + 4 * hi;
        if (!shifted) {
          *reinterpret_cast<bf16x4*>(grow + mq) = out;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (mq + i >= m0) grow[mq + i] = out[i];
        }
      }
  }

  // m0: the tile's first chunk row; a0 <= m0: the chunk row of accumulator
  // row 0.  A tile computed shifted down (a0 < m0) ends at the chunk's last
  // row and stores only its rows from m0 on, one value at a time; the rows
  // below belong to the tile before.  Otherwise rows past the chunk get 0.
  static __device__ __forceinline__ void apply(const Params& p, f32x16 (&acc)[MB][4], int m0, int a0, int n0,
                                               bf16*) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int hi = lane >> 5;
    const int tv = *p.tok_count;  // > 0: tiles past the valid tokens never get here
    const float scale = *p.scale;
    const bool shifted = a0 < m0;
    const int row0 = a0 + wm * kWaveRows;
    const float k2 = 2.0f * kLog2e * p.inv_softcap;
    const float cl2 = p.softcap * kLog2e;
    columns<0>(p, acc, wn, lane, hi, n0, tv, scale, row0, m0, shifted, k2, cl2);
  }

  // Token column blocks nb, nb+1, .. 3 (a compile-time index, so that the
  // accumulators stay in registers).
  template <int nb>
  static __device__ __forceinline__ void columns(const Params& p, const f32x16 (&acc)[MB][4], int wn, int lane,
                                                 int hi, int n0, int tv, float scale, int row0, int m0, bool shifted,
                                                 float k2, float cl2) {
    const int t = n0 + acc_col(wn, nb, lane);
    const bool tok_ok = t < tv;
    const int ts = tok_ok ? t : 0;
    const float nl2 = -p.lse[p.valid_idx[ts]] * kLog2e;
    const float st = tok_ok ? scale : 0.0f;
    const int y_rel = tok_ok ? p.yc[ts] - p.v0 - row0 : -1;
    // The lane holding the label's row: rows 8k + 4 hi + 0..3 of the wave's.
    const bool own = (unsigned)y_rel < (unsigned)kWaveRows && ((y_rel >> 2) & 1) == hi;
    bf16* grow = p.G + (int64_t)t * p.ldg;
    if (__builtin_amdgcn_ballot_w64(own) != 0)
      column<true, nb>(p, acc, hi, row0, m0, shifted, y_rel, nl2, st, k2, cl2, grow);
    else
      column<false, nb>(p, acc, hi, row0, m0, shifted, y_rel, nl2, st, k2, cl2, grow);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (nb < 3) columns<nb + 1>(p, acc, wn, lane, hi, n0, tv, scale, row0, m0, shifted, k2, cl2);
  }
};

// dW rows of one chunk: fp32 store of the rows / columns in range.  The
// rows are final and nothing in the step reads them again, so they go out
// with streaming (nontemporal) stores, which measured about 3% faster on
// this kernel than plain ones.
struct StoreF32 {
  struct Params {
    float* out;
    int64_t ldo;
    int rows, cols;
  };
  static __device__ __forceinline__ void apply(const Params& p, f32x16 (&acc)[4][4], int m0, int n0,
                                               bf16*) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = n0 + acc_col(wn, nb, lane);
      if (n >= p.cols) continue;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + acc_row(wm, mb, r, lane);
          if (m < p.rows) __builtin_nontemporal_store(acc[mb][nb][r], p.out + (int64_t)m * p.ldo + n);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// A transposed fp32 tile: accumulator rows are hidden columns h, accumulator
// columns are rows v of the output, stored at out[v * ldo + h] (dW computed
// as Xc^T G).  A lane's registers 4q..4q+3 of a block are 4 consecutive h of
// one v: one 16-byte store each.  H is a multiple of 8 and a0 / m0 are too,
// so each such group lies wholly inside or outside [m0, hcols).  Rows below
// m0 (a last tile computed shifted down) belong to the tile before.  Plain
// stores: the 32-byte pieces of 4 consecutive stores fill whole 128-byte
// lines, which the L2 merges before they go out (streaming stores of the
// same pieces made the dH + dW launch 6% slower at T=8192, H=3072).
template <int MB>
struct StoreF32T {
  struct Params {
    float* out;
    int64_t ldo;
    int vrows;   // columns v >= vrows are not stored
    int hcols;   // accumulator rows h >= hcols are not stored
  };
  static constexpr int kWaveRows = 32 * MB;

  static __device__ __forceinline__ void apply(const Params& p, f32x16 (&acc)[MB][4], int m0, int a0, int n0,
                                               bf16*) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int v = n0 + acc_col(wn, nb, lane);
      if (v >= p.vrows) continue;
      float* row = p.out + (int64_t)v * p.ldo;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int h = a0 + wm * kWaveRows + 32 * mb + 8 * q + 4 * (lane >> 5);
          if (h < m0 || h >= p.hcols) continue;
          const float4 x = make_float4(acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1], acc[mb][nb][4 * q + 2],
                                       acc[mb][nb][4 * q + 3]);
          *reinterpret_cast<float4*>(row + h) = x;
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// dHidden: fp32 accumulation over the vocabulary chunks in a fixed order; the
// last chunk rounds to bf16 and writes each compacted token's row back to its
// original position.
enum { kAccFirst = 1, kAccLast = 2 };
template <int MB = 4>
struct AccumH {
  struct Params {
    float* acc_buf;           // [Tvp][ld] fp32
    int64_t ld;
    bf16* dh;                 // [T][ld] bf16
    const int32_t* valid_idx;
    const int* tok_count;
    int cols;
    int mode;
  };
  static constexpr int kWaveRows = 32 * MB;

  static __device__ __forceinline__ void apply(const Params& p, f32x16 (&acc)[MB][4], int m0, int n0,
                                               bf16* smem) {
    apply(p, acc, m0, m0, n0, smem);
  }

  // m0: the tile's first token row; a0 <= m0: the row of accumulator row 0
  // (a last tile computed shifted down); rows below m0 belong to the tile
  // before and are left alone.  The running sum is read back one 64-row
  // block (per wave: 16 rows x 4 column blocks) at a time, all 64 loads in
  // flight together: the pass is bound by memory latency, since every tile
  // of the launch (one round of tiles) reaches it at once.  It is written
  // back with streaming stores.
  static __device__ __forceinline__ void apply(const Params& p, f32x16 (&acc)[MB][4], int m0, int a0, int n0,
                                               bf16*) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tv = *p.tok_count;
    const bool first = (p.mode & kAccFirst) != 0;
    const bool last = (p.mode & kAccLast) != 0;
    int hc[4];
    bool hok[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int h = n0 + acc_col(wn, nb, lane);
      hok[nb] = h < p.cols;
      hc[nb] = hok[nb] ? h : 0;   // loads stay inside the row
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      // Rows t < Tvp always exist in the running sum (rows at or past the
      // valid-token count are loaded but never used).  The first chunk reads
      // nothing: with a single chunk there is no running sum at all.
      float prev[16][4] = {};
      if (!first) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row =
              (int64_t)(a0 + wm * kWaveRows + 32 * mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * p.ld;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) prev[r][nb] = p.acc_buf[row + hc[nb]];
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = a0 + wm * kWaveRows + 32 * mb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (t >= tv || t < m0) continue;
        const int64_t orig = last ? (int64_t)p.valid_idx[t] : 0;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          if (!hok[nb]) continue;
          const float v = acc[mb][nb][r] + prev[r][nb];
          const int h = hc[nb];
          if (last) p.dh[orig * p.ld + h] = (bf16)v;
          else __builtin_nontemporal_store(v, p.acc_buf + (int64_t)t * p.ld + h);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

}  // namespace epi
}  // namespace flce
