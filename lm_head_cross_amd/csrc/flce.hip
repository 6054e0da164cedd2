// Fused linear cross-entropy for AMD MI355X (gfx950): the small kernels, the
// GEMM instantiations and the C ABI declared in include/flce.h.
//
// Forward (one stream, no host synchronisation):
//   compact   labels -> compacted token list (valid_idx, yc) and Tv
//   gather    Xc[t] = X[valid_idx[t]], zero rows up to the 256-row padding
//   proj+lse  MFMA tiles of W Xc^T with the softcap / log-sum-exp epilogue
//   combine   per token: merge the vocab-tile partials in order -> lse, loss
//   finalize  fixed-order fp64 sum of per-block sums, divided by D
// Backward:
//   compact, gather, scale = g / D, zero dH and the padding rows of dW, then
//   per vocabulary chunk: recompute z^T tiles -> G chunk (bf16), dW rows of
//   the chunk = G^T Xc, dH_acc += G W[chunk] (the last chunk writes bf16 dH).
#include <math.h>
#include <algorithm>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/flce.h"
#include "epilogues.hpp"
#include "gemm_f32w.hpp"
#include "gemm_wide.hpp"
#include "host_common.hpp"

namespace flce {

// ---------------------------------------------------------------------------
// Small kernels
// ---------------------------------------------------------------------------

constexpr int kCompactThreads = 1024;

// Stable compaction of the valid positions (label != ignore_index and inside
// [0, Vu)); an out-of-range label is treated as ignored and flagged.  Also
// clears the per-token outputs so that ignored positions read 0.
__global__ __launch_bounds__(kCompactThreads) void k_compact(const int64_t* __restrict__ labels, int T,
                                                             int Vu, int64_t ignore_index, Meta* meta,
                                                             int32_t* __restrict__ valid_idx,
                                                             int32_t* __restrict__ yc, int32_t* status,
                                                             float* lse_out, float* tl_out) {
  __shared__ int scan[kCompactThreads];
  const int tid = threadIdx.x;
  const int per = (T + kCompactThreads - 1) / kCompactThreads;
  const int lo = min(tid * per, T);
  const int hi = min(lo + per, T);
  int count = 0;
  int bad = 0;
  for (int t = lo; t < hi; ++t) {
    const int64_t y = labels[t];
    if (lse_out) lse_out[t] = 0.0f;
    if (tl_out) tl_out[t] = 0.0f;
    if (y == ignore_index) continue;
    if (y < 0 || y >= Vu) { bad = 1; continue; }
    ++count;
  }
  if (bad && status) atomicOr(status, FLCE_DEVICE_BAD_LABEL);
  scan[tid] = count;
  __syncthreads();
  for (int off = 1; off < kCompactThreads; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  int pos = scan[tid] - count;
  if (tid == kCompactThreads - 1) meta->n_valid = scan[tid];
  for (int t = lo; t < hi; ++t) {
    const int64_t y = labels[t];
    if (y == ignore_index || y < 0 || y >= Vu) continue;
    valid_idx[pos] = t;
    yc[pos] = (int32_t)y;
    ++pos;
  }
}

// Xc[t, :H] = X[valid_idx[t], :] for t < Tv; every other element of the
// Tvp x Hp buffer (rows Tv..Tvp, columns H..Hp) is 0.  Rows are moved in
// 16-byte pieces: in_vec = H/8 of them per input row, out_vec = Hp/8 per
// output row.
__global__ __launch_bounds__(256) void k_gather(const uint4* __restrict__ X, int64_t in_vec, int64_t out_vec,
                                                 const int32_t* __restrict__ valid_idx, const Meta* meta,
                                                 uint4* __restrict__ Xc, int64_t Tvp) {
  const int tv = meta->n_valid;
  const int64_t total = Tvp * out_vec;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / out_vec;
    const int64_t c = i - t * out_vec;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t < tv && c < in_vec) v = X[(int64_t)valid_idx[t] * in_vec + c];
    Xc[i] = v;
  }
}

// XcT[h][t] = Xc[t][h] through a 64 x 64 LDS tile: 16-byte reads along h,
// 16-byte writes along t.  dW reads the gathered hidden states K-major
// (along the tokens it sums over) from this copy.
__global__ __launch_bounds__(256) void k_transpose_xc(const bf16* __restrict__ Xc, int64_t H, int64_t Tvp,
                                                       bf16* __restrict__ XcT) {
  __shared__ bf16 tile[64][64 + 2];
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int64_t h0 = (int64_t)blockIdx.y * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int r = pass * 32 + (tid >> 3);
    const int c = (tid & 7) * 8;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(Xc + (t0 + r) * H + h0 + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[r][c + e] = v[e];
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int h = pass * 32 + (tid >> 3);
    const int c = (tid & 7) * 8;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[c + e][h];
    *reinterpret_cast<bf16x8*>(XcT + (h0 + h) * Tvp + t0 + c) = v;
  }
}

// Per compacted token: merge the vocab-tile partials into the log-sum-exp,
// form the token loss, and reduce the block's losses in fp64.  A block takes
// kCombineTokens consecutive tokens; its kCombineSlices thread rows each merge
// every kCombineSlices-th tile (reads stay coalesced across the tokens), then
// the slices are merged in slice order.  The order is fixed, so the result is
// deterministic.
constexpr int kCombineTokens = 64;
constexpr int kCombineSlices = 16;
__global__ __launch_bounds__(kCombineTokens * kCombineSlices) void k_combine(
    const float2* __restrict__ partials, int tiles_v, int ldp, const float* __restrict__ label_logit,
    const int32_t* __restrict__ valid_idx, const Meta* meta, float* lse_out, float* tl_out, double* block_sums) {
  __shared__ float2 red[kCombineSlices][kCombineTokens];
  __shared__ double lred[kCombineTokens];
  const int tv = meta->n_valid;
  const int tok = threadIdx.x % kCombineTokens;
  const int slice = threadIdx.x / kCombineTokens;
  const int t = blockIdx.x * kCombineTokens + tok;
  float m = kNegInf, s = 0.0f;
  if (t < tv) {
    for (int j = slice; j < tiles_v; j += kCombineSlices) {
      const float2 pr = partials[(int64_t)j * ldp + t];
      lse_merge(m, s, pr.x, pr.y);
    }
  }
  red[slice][tok] = make_float2(m, s);
  __syncthreads();
  if (slice == 0) {
    for (int k = 1; k < kCombineSlices; ++k) lse_merge(m, s, red[k][tok].x, red[k][tok].y);
    double loss = 0.0;
    if (t < tv) {
      const float lse = m + log_e(s);
      const float l = lse - label_logit[t];
      const int orig = valid_idx[t];
      lse_out[orig] = lse;
      if (tl_out) tl_out[orig] = l;
      loss = (double)l;
    }
    lred[tok] = loss;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double acc = 0.0;
    for (int k = 0; k < kCombineTokens; ++k) acc += lred[k];
    block_sums[blockIdx.x] = acc;
  }
}

// Normaliser D: num_label_tokens when given, else Tv for MEAN, else 1.
__device__ __forceinline__ double divisor(const Meta* meta, int reduction, int64_t num_label_tokens) {
  if (num_label_tokens > 0) return (double)num_label_tokens;
  if (reduction == FLCE_REDUCTION_MEAN) return (double)meta->n_valid;
  return 1.0;
}

// loss = (fixed-order fp64 sum of the block sums) / D.
__global__ __launch_bounds__(256) void k_finalize(const double* __restrict__ block_sums, int nblocks,
                                                   const Meta* meta, int reduction, int64_t num_label_tokens,
                                                   float* loss) {
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < nblocks; i += 256) s += block_sums[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = (float)(red[0] / divisor(meta, reduction, num_label_tokens));
}

// The loss for T == 0: 0 for SUM (or a given count), NaN for MEAN.
__global__ void k_empty_loss(int reduction, int64_t num_label_tokens, float* loss) {
  *loss = (num_label_tokens <= 0 && reduction == FLCE_REDUCTION_MEAN) ? __builtin_nanf("") : 0.0f;
}

__global__ void k_scale(const float* grad_out, const Meta* meta, int reduction, int64_t num_label_tokens,
                        float* scale) {
  *scale = (float)((double)*grad_out / divisor(meta, reduction, num_label_tokens));
}

__global__ __launch_bounds__(256) void k_zero(uint4* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

// G[t, c0:c1] = 0 for t < rows (row stride ld): the K padding of the dH
// contraction past a chunk's last row, which a shifted last tile of the
// recompute does not write.
__global__ __launch_bounds__(256) void k_zero_cols(bf16* __restrict__ G, int64_t ld, int64_t rows, int c0, int c1) {
  const int w = c1 - c0;
  const int64_t n = rows * w;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / w;
    G[t * ld + c0 + (int)(i - t * w)] = (bf16)0.0f;
  }
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__global__ __launch_bounds__(256) void k_round_bf16(const float* __restrict__ src, bf16* __restrict__ dst,
                                                     int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = (bf16)src[i];
}

// Rows < `rows` of a head [*, H] into a bf16 copy [rows, Hp] whose columns
// H..Hp are 0: an fp32 head is rounded to nearest even, a bf16 head copied.
// H is a multiple of 8, so each 16-byte output piece lies wholly inside or
// wholly past the end of its source row.
template <class Src>
__global__ __launch_bounds__(256) void k_stage_head(const Src* __restrict__ src, int64_t H, int64_t Hp,
                                                     int64_t rows, uint4* __restrict__ dst) {
  const int64_t vec = Hp / 8;
  const int64_t n = rows * vec;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t r = i / vec;
    const int64_t c = (i - r * vec) * 8;
    uint4 o = make_uint4(0, 0, 0, 0);
    if (c < H) {
      if constexpr (sizeof(Src) == 4) {
        const float4 a = *reinterpret_cast<const float4*>(src + r * H + c);
        const float4 b = *reinterpret_cast<const float4*>(src + r * H + c + 4);
        bf16x8 v;
        v[0] = (bf16)a.x; v[1] = (bf16)a.y; v[2] = (bf16)a.z; v[3] = (bf16)a.w;
        v[4] = (bf16)b.x; v[5] = (bf16)b.y; v[6] = (bf16)b.z; v[7] = (bf16)b.w;
        o = *reinterpret_cast<const uint4*>(&v);
      } else {
        o = *reinterpret_cast<const uint4*>(src + r * H + c);
      }
    }
    dst[i] = o;
  }
}

__global__ __launch_bounds__(256) void k_round_bf16_vec(const float4* __restrict__ src, bf16x4* __restrict__ dst,
                                                         int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 v = src[i];
    bf16x4 o;
    o[0] = (bf16)v.x; o[1] = (bf16)v.y; o[2] = (bf16)v.z; o[3] = (bf16)v.w;
    dst[i] = o;
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// The launch tracer shared by every entry point of the library.
namespace host {
Tracer g_trace;
}  // namespace host

namespace {

using namespace host;

constexpr size_t kAlign = 256;


// Sizes derived from a validated problem.
struct Plan {
  int64_t T, H, V, Vu;
  int64_t Hp;           // H rounded up to 128: the row length of Xc, XcT's row count and a staged head's rows
  bool stage_head;      // the kernels read a bf16 copy of the head's rows < Vu (fp32 head, or H != Hp)
  bool f32_head;        // the GEMMs read an fp32 head directly, rounding each piece on its way into LDS
                        // (FLCE_FLAG_ROUND_HEAD_ON_LOAD)
  int64_t Tvp;          // T rounded up to 256 (the token tile)
  int64_t tiles_t;      // Tvp / 256
  int64_t tiles_v;      // ceil(Vu / 256): forward vocab tiles
  int64_t tiles_h;      // ceil(H / 256)
  int64_t vc;           // backward vocabulary chunk width (multiple of 256)
  int64_t nchunks;
  bool dw_wide;         // dW of a chunk as 384-row tiles of Xc^T G (stored transposed)
  int n_cu;             // compute units the chunk width was chosen for
  // workspace byte offsets
  size_t off_meta, off_valid, off_yc, off_label, off_scale, off_bsum, off_xc;
  size_t off_wst;       // the staged head [Vu, Hp] bf16 (0 bytes when the caller's head is read directly)
  size_t off_part;      // forward region
  size_t off_g, off_hacc, off_xct;  // backward region
  size_t off_wcopy;     // backward, fp32 head read directly: bf16 copy of one chunk's head rows [vc, Hp]
  size_t fwd_total;     // bytes the forward pass touches (a prefix of the workspace)
  size_t total;
};

int validate(const flce_problem_t* p) {
  if (!p) return FLCE_ERR_INVALID_ARG;
  if (p->num_tokens < 0 || p->hidden <= 0 || p->vocab <= 0) return FLCE_ERR_INVALID_ARG;
  if (p->unpadded_vocab <= 0 || p->unpadded_vocab > p->vocab) return FLCE_ERR_INVALID_ARG;
  if (!(p->softcap >= 0.0f) || isinf(p->softcap)) return FLCE_ERR_INVALID_ARG;
  if (p->reduction != FLCE_REDUCTION_SUM && p->reduction != FLCE_REDUCTION_MEAN) return FLCE_ERR_INVALID_ARG;
  if (p->num_label_tokens == 0) return FLCE_ERR_INVALID_ARG;
  if (p->weight_dtype != FLCE_DTYPE_BF16 && p->weight_dtype != FLCE_DTYPE_FP32) return FLCE_ERR_UNSUPPORTED;
  if ((p->flags & ~(FLCE_FLAG_ROUND_HEAD_ON_LOAD | FLCE_FLAG_DW_TILE_256 | FLCE_FLAG_DW_TILE_384 |
                    FLCE_FLAG_HEAD_STAGED)) != 0)
    return FLCE_ERR_INVALID_ARG;
  if ((p->flags & FLCE_FLAG_DW_TILE_256) && (p->flags & FLCE_FLAG_DW_TILE_384)) return FLCE_ERR_INVALID_ARG;
  if ((p->flags & FLCE_FLAG_DW_TILE_384) && p->hidden < 384) return FLCE_ERR_INVALID_ARG;
  if ((p->flags & FLCE_FLAG_ROUND_HEAD_ON_LOAD) && p->weight_dtype != FLCE_DTYPE_FP32) return FLCE_ERR_INVALID_ARG;
  if (p->hidden % 8 != 0) return FLCE_ERR_UNSUPPORTED;
  // The GEMM loaders address a 256-row tile with 32-bit byte offsets from a
  // buffer resource of under 2 GB: 256 rows of ld bf16 elements must stay
  // below 2^31 bytes for every row length the kernels use (Hp, the padded
  // token count, and the chunk width, at most V/4).  These bounds keep each
  // at or below 2^30 bytes, and every tile count within an int.
  if (p->num_tokens > (int64_t(1) << 21) || p->vocab > (int64_t(1) << 23) || p->hidden > (int64_t(1) << 20))
    return FLCE_ERR_UNSUPPORTED;
  return FLCE_OK;
}

// Width, in 256-row vocabulary tiles, of the backward pass's chunks, and the
// tile of their dW.  A chunk of ct tiles launches tiles_t * ceil(256 ct / 384)
// recompute tiles (depth H; 256-row tiles for chunks under 384 rows) and
// either ct * tiles_h dW tiles (depth Tvp) or, with dW computed as Xc^T G on
// 384-row tiles, ct * ceil(H / 384) of them; a launch of n tiles runs in
// about ceil(n / CUs) rounds, one tile per CU per round.  The dH
// contraction's cost does not depend on the split, apart from its fp32
// accumulator pass, which is counted with the launch overhead as a fixed cost
// per chunk.  For each dW tile this picks, among widths up to ct_max, the one
// with the least estimated time (ties: the wider); the 384-row dW tiles are
// taken when they save at least 1%, or when the caller fixes the tile
// (dw_tile 256 or 384; 0 leaves it to the estimate).  A round of 384-row
// recompute tiles costs kWideRound 256-row rounds of the same depth: 1.5
// times the work at the 5-6% better rate measured on full rounds of the
// recompute shape.  A round of 384-row dW^T tiles costs kWideRoundDw,
// calibrated on four head shapes (each measured with both dW tiles at the
// width this estimate picks for each, same box, alternating runs): per step,
// T=8192, H=3072 39.6 -> 37.7 ms with the 384-row tiles, T=16384 (8192
// valid), H=5120 40.6 -> 39.7, T=65536, H=8192 424.4 -> 419.8, and T=4096,
// H=4096 13.02 against 13.04 (a tie, which the 1% margin leaves on 256-row
// tiles).
constexpr int64_t kChunkOverheadDepth = 1536;  // per chunk, in units of one round's depth
constexpr double kWideRound = 1.42;
constexpr double kWideRoundDw = 1.38;
constexpr double kWideDwMargin = 0.99;
struct ChunkChoice {
  int64_t ct;
  bool dw_wide;
};
ChunkChoice pick_chunks(int64_t Vu, int64_t tiles_t, int64_t tiles_h, int64_t H, int64_t Hp, int64_t Tvp,
                        int64_t ct_max, int n_cu, int dw_tile) {
  const int64_t tiles_v = ceil_div(Vu, 256);
  const int64_t tiles_wh = ceil_div(H, gemm::WBM);
  auto cost = [&](int64_t ct, bool wide) {
    const int64_t full = tiles_v / ct;
    const int64_t rem = tiles_v - full * ct;
    auto chunk = [&](int64_t c, int64_t rows) {
      const double rec = rows >= gemm::WBM
                             ? (double)ceil_div(ceil_div(rows, gemm::WBM) * tiles_t, n_cu) * Hp * kWideRound
                             : (double)ceil_div(tiles_t * c, n_cu) * Hp;
      const double dw = wide ? (double)ceil_div(c * tiles_wh, n_cu) * Tvp * kWideRoundDw
                             : (double)(ceil_div(c * tiles_h, n_cu) * Tvp);
      return rec + dw + (double)kChunkOverheadDepth;
    };
    return full * chunk(ct, ct * 256) + (rem ? chunk(rem, Vu - full * ct * 256) : 0.0);
  };
  auto best_width = [&](bool wide, double& best_cost) {
    int64_t best = ct_max;
    best_cost = cost(ct_max, wide);
    for (int64_t ct = ct_max - 1; ct >= 1; --ct) {
      const double c = cost(ct, wide);
      if (c < best_cost) {
        best = ct;
        best_cost = c;
      }
    }
    return best;
  };
  double narrow_cost = 0.0, wide_cost = 0.0;
  if (dw_tile == 384) return {best_width(true, wide_cost), true};
  const int64_t ct_narrow = best_width(false, narrow_cost);
  if (dw_tile == 0 && H >= gemm::WBM) {
    const int64_t ct_wide = best_width(true, wide_cost);
    if (wide_cost < kWideDwMargin * narrow_cost) return {ct_wide, true};
  }
  return {ct_narrow, false};
}

// Whether a chunk's dH runs on 384-row token tiles (it needs at least 384
// token rows).  The wide tile is about 9% faster per flop, but the launch
// hands out dH's deep tiles before dW's, and the tile counts decide how the
// two pack onto the compute units.  Measured back to back, all chunks wide
// against all narrow: workloads 3, 4 and 5 (384, 640 and 8032 narrow dH
// tiles per chunk on the device) gained 2.1%, 2.9% and 5.1% per step;
// workload 2, whose 256 narrow dH tiles fill exactly one round of the 256
// compute units, lost 1.3%.  So the narrow tiles are kept when they make
// exactly one full round.  (The host sees T, not the valid count.)
bool dh_wide(int64_t tiles_t, int64_t tiles_h, int64_t Tvp, int n_cu) {
  if (Tvp < gemm::WBM) return false;
  return tiles_t * tiles_h != n_cu;
}

// Compute units of the current device (256 on MI355X when the query fails).
int device_cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

Plan make_plan(const flce_problem_t* p, int n_cu = 256) {
  Plan pl{};
  pl.T = p->num_tokens;
  pl.H = p->hidden;
  pl.V = p->vocab;
  pl.Vu = p->unpadded_vocab;
  pl.Hp = align_up((size_t)pl.H, 128);
  pl.f32_head = p->weight_dtype == FLCE_DTYPE_FP32 && pl.Hp == pl.H && (p->flags & FLCE_FLAG_ROUND_HEAD_ON_LOAD);
  pl.stage_head = (p->weight_dtype == FLCE_DTYPE_FP32 && !pl.f32_head) || pl.Hp != pl.H;
  pl.Tvp = align_up((size_t)pl.T, 256);
  pl.tiles_t = pl.Tvp / 256;
  pl.tiles_v = ceil_div(pl.Vu, 256);
  pl.tiles_h = ceil_div(pl.H, 256);
  // Chunk width: at most a quarter of the usable vocabulary (whole tiles), at
  // least one tile; chunks of equal width up to the last.  The G buffer is
  // sized for the widest chunk, so the workspace does not depend on the
  // device.
  const int64_t ct_max = std::max<int64_t>(1, pl.Vu / 1024);
  const int dw_tile = (p->flags & FLCE_FLAG_DW_TILE_384) ? 384 : (p->flags & FLCE_FLAG_DW_TILE_256) ? 256 : 0;
  const ChunkChoice cc = pick_chunks(pl.Vu, pl.tiles_t, pl.tiles_h, pl.H, pl.Hp, pl.Tvp, ct_max, n_cu, dw_tile);
  const int64_t ct = cc.ct;
  pl.vc = ct * 256;
  pl.dw_wide = cc.dw_wide;
  pl.n_cu = n_cu;
  pl.nchunks = ceil_div(pl.tiles_v, ct);

  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, kAlign); return at; };
  pl.off_meta = take(sizeof(Meta));
  pl.off_valid = take(pl.Tvp * 4);
  pl.off_yc = take(pl.Tvp * 4);
  pl.off_label = take(pl.Tvp * 4);
  pl.off_scale = take(16);
  pl.off_bsum = take(pl.Tvp / kCombineTokens * 8);
  pl.off_xc = take(pl.Tvp * pl.Hp * 2);
  // An fp32 head (unless rounded on load), or rows not a multiple of 128
  // long: the bf16 copy of the head's usable rows, zero-padded to Hp and
  // staged here by each call.
  pl.off_wst = take(pl.stage_head ? pl.Vu * pl.Hp * 2 : 0);
  const size_t common = o;
  pl.off_part = take(pl.tiles_v * pl.Tvp * 8);
  const size_t fwd_end = o;
  o = common;
  pl.off_g = take(pl.Tvp * ct_max * 256 * 2);
  // Every chunk width below tiles_v gives more than one chunk.
  pl.off_hacc = take(pl.tiles_v > 1 ? pl.Tvp * pl.H * 4 : 0);
  pl.off_xct = take(pl.Tvp * pl.Hp * 2);
  // An fp32 head read directly: the recompute writes the rounded rows of the
  // chunk here for the chunk's dH contraction.
  pl.off_wcopy = take(pl.f32_head ? ct_max * 256 * pl.Hp * 2 : 0);
  const size_t bwd_end = o;
  pl.fwd_total = fwd_end;
  pl.total = std::max(fwd_end, bwd_end);
  return pl;
}

template <class T>
T* ws_at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

int check_workspace(const Plan& pl, void* ws, size_t bytes) {
  if (pl.total == 0) return FLCE_OK;
  if (!ws || !aligned(ws, kAlign) || bytes < pl.total) return FLCE_ERR_WORKSPACE;
  return FLCE_OK;
}

// K steps of BK for a K extent, padded to whole groups of NST stages (the
// operands are zero, or multiplied by zero, in the padding).
int k_steps_for(int64_t K) {
  const int64_t group = (int64_t)gemm::NST * gemm::BK;
  return (int)(ceil_div(K, group) * gemm::NST);
}

void zero_fill(void* p, int64_t bytes, hipStream_t s) {
  if (bytes <= 0) return;
  TraceScope tr(FLCE_KERNEL_AUX, 0.0, s);
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(k_zero, dim3(grid_for(n16, 256, 8192)), dim3(256), 0, s, (uint4*)p, n16);
}

// The bf16 head the kernels read, rows of Hp elements: the caller's for a
// bf16 head with H a multiple of 128; otherwise its rows < Vu copied into
// the workspace with zero columns H..Hp, an fp32 head rounded to nearest
// even ("nemo_automodel.components.models.inkling2.loss", class description:
// an fp32 head is used at its bf16 value).  An fp32 head rounded on load
// (FLCE_FLAG_ROUND_HEAD_ON_LOAD) is not staged: the projection and recompute
// GEMMs read it directly (gemm_f32w.hpp), and this returns nullptr.  Rows
// >= Vu are never read.
const bf16* staged_head(const Plan& pl, const flce_problem_t& p, const void* weight, void* workspace,
                        hipStream_t stream) {
  if (pl.f32_head) return nullptr;
  if (!pl.stage_head) return static_cast<const bf16*>(weight);
  bf16* wst = ws_at<bf16>(workspace, pl.off_wst);
  TraceScope tr(FLCE_KERNEL_AUX, 0.0, stream);
  if (p.weight_dtype == FLCE_DTYPE_FP32 && pl.Hp == pl.H) {
    const int64_t n4 = pl.Vu * pl.H / 4;
    hipLaunchKernelGGL(k_round_bf16_vec, dim3(grid_for(n4, 256, 16384)), dim3(256), 0, stream,
                       static_cast<const float4*>(weight), reinterpret_cast<bf16x4*>(wst), n4);
  } else if (p.weight_dtype == FLCE_DTYPE_FP32) {
    hipLaunchKernelGGL(k_stage_head<float>, dim3(grid_for(pl.Vu * pl.Hp / 8, 256, 16384)), dim3(256), 0,
                       stream, static_cast<const float*>(weight), pl.H, pl.Hp, pl.Vu, reinterpret_cast<uint4*>(wst));
  } else {
    hipLaunchKernelGGL(k_stage_head<bf16>, dim3(grid_for(pl.Vu * pl.Hp / 8, 256, 16384)), dim3(256), 0,
                       stream, static_cast<const bf16*>(weight), pl.H, pl.Hp, pl.Vu, reinterpret_cast<uint4*>(wst));
  }
  return wst;
}

void launch_compact_gather(const Plan& pl, const flce_problem_t& p, const int64_t* labels, const void* hidden,
                           Meta* meta, int32_t* valid_idx, int32_t* yc, int32_t* device_status, float* lse,
                           float* token_loss, bf16* xc, hipStream_t stream) {
  {
    TraceScope tr(FLCE_KERNEL_COMPACT, 0.0, stream);
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(kCompactThreads), 0, stream, labels, (int)pl.T, (int)pl.Vu,
                       p.ignore_index, meta, valid_idx, yc, device_status, lse, token_loss);
  }
  const int64_t in_vec = pl.H / 8, out_vec = pl.Hp / 8;
  TraceScope tr(FLCE_KERNEL_GATHER, 0.0, stream);
  hipLaunchKernelGGL(k_gather, dim3(grid_for(pl.Tvp * out_vec, 256, 16384)), dim3(256), 0, stream,
                     (const uint4*)hidden, in_vec, out_vec, (const int32_t*)valid_idx, (const Meta*)meta,
                     (uint4*)xc, pl.Tvp);
}

// The no-allocation forward's scratch (flce_forward_noalloc): device memory
// of fixed size that the code object brings, one copy per device, held until
// the process ends.  Its name is a host-side stand-in: host code uses only
// the per-device address hipGetSymbolAddress returns.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;

}  // namespace
}  // namespace flce

static __device__ __align__(256) unsigned char scratch[flce::kStaticScratchBytes];

namespace flce {
namespace {

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
void* static_scratch_ptr() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

}  // namespace
}  // namespace flce

using namespace flce;

extern "C" {

const char* flce_status_string(int status) {
  switch (status) {
    case FLCE_OK: return "ok";
    case FLCE_ERR_INVALID_ARG: return "invalid argument";
    case FLCE_ERR_UNSUPPORTED: return "unsupported problem";
    case FLCE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case FLCE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int flce_version(void) { return 100; }

int flce_round_to_bf16(const float* src, void* dst, int64_t count, hipStream_t stream) {
  if (count < 0) return FLCE_ERR_INVALID_ARG;
  if (count == 0) return FLCE_OK;
  if (!src || !dst) return FLCE_ERR_INVALID_ARG;
  if (!aligned(src, 4) || !aligned(dst, 2)) return FLCE_ERR_UNSUPPORTED;
  TraceScope tr(FLCE_KERNEL_AUX, 0.0, stream);
  if (aligned(src, 16) && aligned(dst, 8) && count % 4 == 0) {
    hipLaunchKernelGGL(k_round_bf16_vec, dim3(grid_for(count / 4, 256, 16384)), dim3(256), 0, stream,
                       (const float4*)src, (bf16x4*)dst, count / 4);
  } else {
    hipLaunchKernelGGL(k_round_bf16, dim3(grid_for(count, 256, 16384)), dim3(256), 0, stream, src, (bf16*)dst,
                       count);
  }
  return launch_status();
}

int flce_workspace_size(const flce_problem_t* problem, size_t* bytes) {
  const int st = validate(problem);
  if (st != FLCE_OK) return st;
  if (!bytes) return FLCE_ERR_INVALID_ARG;
  *bytes = problem->num_tokens == 0 ? 0 : make_plan(problem).total;
  return FLCE_OK;
}

int flce_backward_plan(const flce_problem_t* problem, int cu_count, int64_t* chunk_rows, int64_t* chunks,
                       int* dw_tile_rows) {
  const int st = validate(problem);
  if (st != FLCE_OK) return st;
  if (!chunk_rows || !chunks || !dw_tile_rows) return FLCE_ERR_INVALID_ARG;
  const Plan pl = make_plan(problem, cu_count > 0 ? cu_count : device_cu_count());
  *chunk_rows = pl.vc;
  *chunks = problem->num_tokens == 0 ? 0 : pl.nchunks;
  *dw_tile_rows = pl.dw_wide ? gemm::WBM : 256;
  return FLCE_OK;
}

}  // extern "C"

namespace flce {
namespace {

// Which scratch the forward pass runs in.
enum class ScratchSource { kCallerWorkspace, kStaticScratch };

void* static_scratch_ptr();

// The forward pass on a caller's workspace (which must hold both passes'
// bytes) or on the library's static scratch (which must hold the forward's).
int forward_impl(const flce_problem_t* problem, const void* hidden, const void* weight, const int64_t* labels,
                 float* loss, float* lse, float* token_loss, int32_t* device_status, void* workspace,
                 size_t workspace_bytes, hipStream_t stream, ScratchSource src) {
  int st = validate(problem);
  if (st != FLCE_OK) return st;
  const flce_problem_t& p = *problem;
  if (!loss || !weight) return FLCE_ERR_INVALID_ARG;
  if (p.num_tokens > 0 && (!hidden || !labels || !lse)) return FLCE_ERR_INVALID_ARG;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(loss, 4) || !aligned(lse, 4) ||
      !aligned(token_loss, 4) || !aligned(labels, 8) || !aligned(device_status, 4))
    return FLCE_ERR_UNSUPPORTED;
  if (p.num_tokens == 0) {
    TraceScope tr(FLCE_KERNEL_FINALIZE, 0.0, stream);
    hipLaunchKernelGGL(k_empty_loss, dim3(1), dim3(1), 0, stream, (int)p.reduction, p.num_label_tokens, loss);
    return launch_status();
  }
  const Plan pl = make_plan(&p);
  if (src == ScratchSource::kStaticScratch) {
    if (pl.fwd_total > kStaticScratchBytes) return FLCE_ERR_WORKSPACE;
    workspace = static_scratch_ptr();
    if (!workspace) return FLCE_ERR_HIP;
  } else if ((st = check_workspace(pl, workspace, workspace_bytes)) != FLCE_OK) {
    return st;
  }

  Meta* meta = ws_at<Meta>(workspace, pl.off_meta);
  int32_t* valid_idx = ws_at<int32_t>(workspace, pl.off_valid);
  int32_t* yc = ws_at<int32_t>(workspace, pl.off_yc);
  float* label_logit = ws_at<float>(workspace, pl.off_label);
  double* bsum = ws_at<double>(workspace, pl.off_bsum);
  bf16* xc = ws_at<bf16>(workspace, pl.off_xc);
  float2* part = ws_at<float2>(workspace, pl.off_part);
  const int* tv = &meta->n_valid;

  const bf16* Wb = staged_head(pl, p, weight, workspace, stream);
  launch_compact_gather(pl, p, labels, hidden, meta, valid_idx, yc, device_status, lse, token_loss, xc, stream);
  // The projection runs with 384-row head tiles (gemm_wide.hpp) when the
  // usable head has at least that many rows, else with 256-row tiles; an
  // fp32 head read directly takes the 256-row tiles (gemm_f32w.hpp).
  const bool wide = pl.Vu >= gemm::WBM && !pl.f32_head;
  const int64_t tiles_v = wide ? ceil_div(pl.Vu, gemm::WBM) : pl.tiles_v;
  {
    gemm::Operand A{Wb, pl.Hp, (int)pl.Vu - 1, 0};
    gemm::OperandF32 Af{static_cast<const float*>(weight), pl.H, (int)pl.Vu - 1, 0};
    gemm::Operand B{xc, pl.Hp, (int)pl.Tvp - 1, 0};
    gemm::Schedule sch{(int)tiles_v, (int)pl.tiles_t, k_steps_for(pl.Hp), tv, 2};
    const dim3 grid(tiles_v * pl.tiles_t);
    const float c = p.softcap, inv_c = c > 0.0f ? 1.0f / c : 0.0f;
    TraceScope tr(FLCE_KERNEL_PROJ_LSE, 2.0 * pl.T * pl.Vu * pl.H, stream);
    if (pl.f32_head && c > 0.0f) {
      using E = epi::Lse<true>;
      E::Params ep{part, (int)pl.Tvp, label_logit, yc, tv, (int)pl.Vu, c, inv_c};
      hipLaunchKernelGGL((gemm::gemm_kernel_f32a<E>), grid, dim3(gemm::NTHREADS), 0, stream, Af, B, sch, ep,
                         (bf16*)nullptr);
    } else if (pl.f32_head) {
      using E = epi::Lse<false>;
      E::Params ep{part, (int)pl.Tvp, label_logit, yc, tv, (int)pl.Vu, c, inv_c};
      hipLaunchKernelGGL((gemm::gemm_kernel_f32a<E>), grid, dim3(gemm::NTHREADS), 0, stream, Af, B, sch, ep,
                         (bf16*)nullptr);
    } else if (wide && c > 0.0f) {
      using E = epi::Lse<true, gemm::WMB>;
      E::Params ep{part, (int)pl.Tvp, label_logit, yc, tv, (int)pl.Vu, c, inv_c};
      hipLaunchKernelGGL((gemm::gemm_wide_kernel<E>), grid, dim3(gemm::NTHREADS), 0, stream, A, B, sch, ep);
    } else if (wide) {
      using E = epi::Lse<false, gemm::WMB>;
      E::Params ep{part, (int)pl.Tvp, label_logit, yc, tv, (int)pl.Vu, c, inv_c};
      hipLaunchKernelGGL((gemm::gemm_wide_kernel<E>), grid, dim3(gemm::NTHREADS), 0, stream, A, B, sch, ep);
    } else if (c > 0.0f) {
      using E = epi::Lse<true>;
      E::Params ep{part, (int)pl.Tvp, label_logit, yc, tv, (int)pl.Vu, c, inv_c};
      hipLaunchKernelGGL((gemm::gemm_kernel<true, true, E>), grid, dim3(gemm::NTHREADS), 0, stream, A, B, sch, ep);
    } else {
      using E = epi::Lse<false>;
      E::Params ep{part, (int)pl.Tvp, label_logit, yc, tv, (int)pl.Vu, c, inv_c};
      hipLaunchKernelGGL((gemm::gemm_kernel<true, true, E>), grid, dim3(gemm::NTHREADS), 0, stream, A, B, sch, ep);
    }
  }
  {
    TraceScope tr(FLCE_KERNEL_COMBINE, 0.0, stream);
    hipLaunchKernelGGL(k_combine, dim3(pl.Tvp / kCombineTokens), dim3(kCombineTokens * kCombineSlices), 0, stream,
                       (const float2*)part, (int)tiles_v,
                       (int)pl.Tvp, (const float*)label_logit, (const int32_t*)valid_idx, (const Meta*)meta, lse,
                       token_loss, bsum);
  }
  {
    TraceScope tr(FLCE_KERNEL_FINALIZE, 0.0, stream);
    hipLaunchKernelGGL(k_finalize, dim3(1), dim3(256), 0, stream, (const double*)bsum,
                       (int)(pl.Tvp / kCombineTokens),
                       (const Meta*)meta, (int)p.reduction, p.num_label_tokens, loss);
  }
  return launch_status();
}

}  // namespace
}  // namespace flce

extern "C" {

int flce_forward(const flce_problem_t* problem, const void* hidden, const void* weight, const int64_t* labels,
                 float* loss, float* lse, float* token_loss, int32_t* device_status, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  return forward_impl(problem, hidden, weight, labels, loss, lse, token_loss, device_status, workspace,
                      workspace_bytes, stream, ScratchSource::kCallerWorkspace);
}

int flce_forward_noalloc(const flce_problem_t* problem, const void* hidden, const void* weight,
                         const int64_t* labels, float* loss, float* lse, float* token_loss,
                         int32_t* device_status, hipStream_t stream) {
  return forward_impl(problem, hidden, weight, labels, loss, lse, token_loss, device_status, nullptr, 0, stream,
                      ScratchSource::kStaticScratch);
}

int flce_backward(const flce_problem_t* problem, const void* hidden, const void* weight, const int64_t* labels,
                  const float* lse, const float* grad_out, void* d_hidden, float* d_weight,
                  int32_t* device_status, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = validate(problem);
  if (st != FLCE_OK) return st;
  const flce_problem_t& p = *problem;
  if (!weight || !grad_out || !d_weight) return FLCE_ERR_INVALID_ARG;
  if (p.num_tokens > 0 && (!hidden || !labels || !lse || !d_hidden)) return FLCE_ERR_INVALID_ARG;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(d_hidden, 16) || !aligned(d_weight, 16) ||
      !aligned(lse, 4) || !aligned(grad_out, 4) || !aligned(labels, 8) || !aligned(device_status, 4))
    return FLCE_ERR_UNSUPPORTED;
  if (p.num_tokens == 0) {
    zero_fill(d_weight, p.vocab * p.hidden * 4, stream);
    return launch_status();
  }
  const Plan pl = make_plan(&p, device_cu_count());
  if ((st = check_workspace(pl, workspace, workspace_bytes)) != FLCE_OK) return st;

  Meta* meta = ws_at<Meta>(workspace, pl.off_meta);
  int32_t* valid_idx = ws_at<int32_t>(workspace, pl.off_valid);
  int32_t* yc = ws_at<int32_t>(workspace, pl.off_yc);
  float* scale = ws_at<float>(workspace, pl.off_scale);
  bf16* xc = ws_at<bf16>(workspace, pl.off_xc);
  bf16* G = ws_at<bf16>(workspace, pl.off_g);
  float* hacc = ws_at<float>(workspace, pl.off_hacc);
  const int* tv = &meta->n_valid;
  // The head copy the matching forward staged (the caller vouches for it),
  // or this call's own.
  const bf16* W = (p.flags & FLCE_FLAG_HEAD_STAGED) && pl.stage_head ? ws_at<const bf16>(workspace, pl.off_wst)
                                                                      : staged_head(pl, p, weight, workspace, stream);

  launch_compact_gather(pl, p, labels, hidden, meta, valid_idx, yc, device_status, nullptr, nullptr, xc, stream);
  bf16* xct = ws_at<bf16>(workspace, pl.off_xct);
  {
    TraceScope tr(FLCE_KERNEL_GATHER, 0.0, stream);
    hipLaunchKernelGGL(k_transpose_xc, dim3((unsigned)(pl.Tvp / 64), (unsigned)(pl.Hp / 64)), dim3(256), 0,
                       stream, (const bf16*)xc, pl.Hp, pl.Tvp, xct);
  }
  {
    TraceScope tr(FLCE_KERNEL_AUX, 0.0, stream);
    hipLaunchKernelGGL(k_scale, dim3(1), dim3(1), 0, stream, grad_out, (const Meta*)meta, (int)p.reduction,
                       p.num_label_tokens, scale);
  }
  zero_fill(d_hidden, pl.T * pl.H * 2, stream);
  zero_fill(d_weight + pl.Vu * pl.H, (pl.V - pl.Vu) * pl.H * 4, stream);

  const float inv_c = p.softcap > 0.0f ? 1.0f / p.softcap : 0.0f;
  const bool wide_h = dh_wide(pl.tiles_t, pl.tiles_h, pl.Tvp, pl.n_cu);
  bf16* wcopy = ws_at<bf16>(workspace, pl.off_wcopy);
  for (int64_t c = 0; c < pl.nchunks; ++c) {
    const int64_t v0 = c * pl.vc;
    const int64_t vw = std::min(pl.vc, pl.Vu - v0);
    const int64_t tiles_c = ceil_div(vw, 256);
    // The chunk's bf16 head rows: the caller's or staged head, or (an fp32
    // head read directly) the copy the chunk's recompute writes.
    const bf16* Wc = pl.f32_head ? wcopy : W + v0 * pl.Hp;
    const float* Wcf = static_cast<const float*>(weight) + v0 * pl.H;
    const double chunk_flops = 2.0 * pl.T * vw * pl.H;

    // 1. logits of the chunk -> G (bf16, token-major); 384-row tiles when
    //    the chunk has at least 384 rows (256-row tiles for an fp32 head
    //    read directly).
    if (pl.f32_head) {
      gemm::OperandF32 A{Wcf, pl.H, (int)vw - 1, 0};
      gemm::Operand B{xc, pl.Hp, (int)pl.Tvp - 1, 0};
      gemm::Schedule sch{(int)tiles_c, (int)pl.tiles_t, k_steps_for(pl.Hp), tv, 2};
      const dim3 grid(tiles_c * pl.tiles_t);
      TraceScope tr(FLCE_KERNEL_RECOMPUTE_G, chunk_flops, stream);
      if (p.softcap > 0.0f) {
        using E = epi::Grad<true>;
        E::Params ep{G, pl.vc, (int)v0, (int)vw, lse, valid_idx, yc, tv, scale, p.softcap, inv_c};
        hipLaunchKernelGGL((gemm::gemm_kernel_f32a<E>), grid, dim3(gemm::NTHREADS), 0, stream, A, B, sch, ep, wcopy);
      } else {
        using E = epi::Grad<false>;
        E::Params ep{G, pl.vc, (int)v0, (int)vw, lse, valid_idx, yc, tv, scale, 0.0f, 0.0f};
        hipLaunchKernelGGL((gemm::gemm_kernel_f32a<E>), grid, dim3(gemm::NTHREADS), 0, stream, A, B, sch, ep, wcopy);
      }
    } else {
      const bool wide = vw >= gemm::WBM;
      const int64_t tiles_r = wide ? ceil_div(vw, gemm::WBM) : tiles_c;
      gemm::Operand A{Wc, pl.Hp, (int)vw - 1, 0};
      gemm::Operand B{xc, pl.Hp, (int)pl.Tvp - 1, 0};
      gemm::Schedule sch{(int)tiles_r, (int)pl.tiles_t, k_steps_for(pl.Hp), tv, 2};
      const dim3 grid(tiles_r * pl.tiles_t);
      const float c = p.softcap;
      if (wide && vw % 128 != 0) {
        // The dH contraction reads G's columns up to the next multiple of
        // 128 (against zero rows of W): the shifted last tile leaves them.
        const int c1 = (int)std::min<int64_t>(align_up((size_t)vw, 128), pl.vc);
        TraceScope tz(FLCE_KERNEL_AUX, 0.0, stream);
        hipLaunchKernelGGL(k_zero_cols, dim3(grid_for(pl.Tvp * (c1 - vw), 256, 1024)), dim3(256), 0, stream, G,
                           pl.vc, pl.Tvp, (int)vw, c1);
      }
      TraceScope tr(FLCE_KERNEL_RECOMPUTE_G, chunk_flops, stream);
      if (wide && c > 0.0f) {
        using E = epi::Grad<true, gemm::WMB>;
        E::Params ep{G, pl.vc, (int)v0, (int)vw, lse, valid_idx, yc, tv, scale, c, inv_c};
        hipLaunchKernelGGL((gemm::gemm_wide_kernel<E>), grid, dim3(gemm::NTHREADS), 0, stream, A, B, sch, ep);
      } else if (wide) {
        using E = epi::Grad<false, gemm::WMB>;
        E::Params ep{G, pl.vc, (int)v0, (int)vw, lse, valid_idx, yc, tv, scale, 0.0f, 0.0f};
        hipLaunchKernelGGL((gemm::gemm_wide_kernel<E>), grid, dim3(gemm::NTHREADS), 0, stream, A, B, sch, ep);
      } else if (c > 0.0f) {
        using E = epi::Grad<true>;
        E::Params ep{G, pl.vc, (int)v0, (int)vw, lse, valid_idx, yc, tv, scale, c, inv_c};
        hipLaunchKernelGGL((gemm::gemm_kernel<true, true, E>), grid, dim3(gemm::NTHREADS), 0, stream, A, B, sch, ep);
      } else {
        using E = epi::Grad<false>;
        E::Params ep{G, pl.vc, (int)v0, (int)vw, lse, valid_idx, yc, tv, scale, 0.0f, 0.0f};
        hipLaunchKernelGGL((gemm::gemm_kernel<true, true, E>), grid, dim3(gemm::NTHREADS), 0, stream, A, B, sch, ep);
      }
    }
    // 2. dH_acc (+)= G W[v0 : v0 + vw]   (M = tokens, N = H, K = chunk rows) and
    //    dW[v0 : v0 + vw] = G^T Xc          (M = chunk rows, N = H, K = tokens)
    //    in one launch, dH's tiles first.  dH's K-major G and MN-major W, on
    //    384-row token tiles when there are at least 384 token rows.  dW reads
    //    G MN-major (transposing LDS reads) and Xc K-major from XcT; with
    //    dw_wide it runs as dW^T = Xc^T G on 384-row tiles over the hidden
    //    columns (XcT K-major, G's chunk rows as columns), stored transposed.
    {
      const int64_t tiles_hm = wide_h ? ceil_div(pl.Tvp, gemm::WBM) : pl.tiles_t;
      gemm::Operand Ah{G, pl.vc, (int)pl.Tvp - 1, 0};
      gemm::Operand Bh{Wc, pl.Hp, (int)pl.H - 1, (int)vw - 1};
      gemm::Schedule sh{(int)tiles_hm, (int)pl.tiles_h, k_steps_for(vw), tv, 1};
      int mode = 0;
      if (c == 0) mode |= epi::kAccFirst;
      if (c == pl.nchunks - 1) mode |= epi::kAccLast;
      const int64_t n_h = align_up((size_t)(tiles_hm * pl.tiles_h), 8);
      TraceScope tr(FLCE_KERNEL_DGRAD, 2.0 * chunk_flops, stream);
      if (pl.dw_wide) {
        using EW = epi::StoreF32T<gemm::WMB>;
        const int64_t tiles_wh = ceil_div(pl.H, gemm::WBM);
        gemm::Operand Aw{xct, pl.Tvp, (int)pl.H - 1, 0};
        gemm::Operand Bw{G, pl.vc, (int)pl.vc - 1, (int)pl.Tvp - 1};
        gemm::Schedule sw{(int)tiles_wh, (int)tiles_c, 0, tv, 3};
        EW::Params ew{d_weight + v0 * pl.H, pl.H, (int)vw, (int)pl.H};
        const dim3 grid(n_h + tiles_wh * tiles_c);
        if (wide_h) {
          using EH = epi::AccumH<gemm::WMB>;
          EH::Params eh{hacc, pl.H, (bf16*)d_hidden, valid_idx, tv, (int)pl.H, mode};
          hipLaunchKernelGGL((gemm::gemm_pair_wide<EH, EW, true>), grid, dim3(gemm::NTHREADS), 0, stream, Ah, Bh,
                             sh, eh, (int)n_h, Aw, Bw, sw, ew);
        } else {
          using EH = epi::AccumH<>;
          EH::Params eh{hacc, pl.H, (bf16*)d_hidden, valid_idx, tv, (int)pl.H, mode};
          hipLaunchKernelGGL((gemm::gemm_pair_nt<EH, EW>), grid, dim3(gemm::NTHREADS), 0, stream, Ah, Bh, sh, eh,
                             (int)n_h, Aw, Bw, sw, ew);
        }
      } else {
        gemm::Operand Aw{G, pl.vc, (int)pl.vc - 1, (int)pl.Tvp - 1};
        gemm::Operand Bw{xct, pl.Tvp, (int)pl.H - 1, 0};
        gemm::Schedule sw{(int)tiles_c, (int)pl.tiles_h, 0, tv, 3};
        epi::StoreF32::Params ew{d_weight + v0 * pl.H, pl.H, (int)vw, (int)pl.H};
        const dim3 grid(n_h + tiles_c * pl.tiles_h);
        if (wide_h) {
          using EH = epi::AccumH<gemm::WMB>;
          EH::Params eh{hacc, pl.H, (bf16*)d_hidden, valid_idx, tv, (int)pl.H, mode};
          hipLaunchKernelGGL((gemm::gemm_pair_wide<EH, epi::StoreF32>), grid, dim3(gemm::NTHREADS), 0, stream, Ah,
                             Bh, sh, eh, (int)n_h, Aw, Bw, sw, ew);
        } else {
          using EH = epi::AccumH<>;
          EH::Params eh{hacc, pl.H, (bf16*)d_hidden, valid_idx, tv, (int)pl.H, mode};
          hipLaunchKernelGGL((gemm::gemm_pair<true, false, EH, false, true, epi::StoreF32>), grid,
                             dim3(gemm::NTHREADS), 0, stream, Ah, Bh, sh, eh, (int)n_h, Aw, Bw, sw, ew);
        }
      }
    }
  }
  return launch_status();
}

int flce_trace_start(int capacity) {
  if (capacity <= 0) return FLCE_ERR_INVALID_ARG;
  g_trace.release();
  g_trace.ev.resize(2 * (size_t)capacity, nullptr);
  for (auto& e : g_trace.ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      g_trace.release();
      return FLCE_ERR_HIP;
    }
  }
  g_trace.kind.assign(capacity, 0);
  g_trace.flops.assign(capacity, 0.0);
  g_trace.cap = capacity;
  g_trace.n = 0;
  g_trace.on = true;
  return FLCE_OK;
}

int flce_trace_select(uint32_t kind_mask) {
  g_trace.mask = kind_mask;
  return FLCE_OK;
}

int flce_trace_stop(void) {
  g_trace.on = false;
  return FLCE_OK;
}

int flce_trace_count(void) { return g_trace.n; }

int flce_trace_get(int i, int* kind, float* ms, double* flops) {
  if (i < 0 || i >= g_trace.n) return FLCE_ERR_INVALID_ARG;
  if (kind) *kind = g_trace.kind[i];
  if (flops) *flops = g_trace.flops[i];
  if (ms) {
    if (hipEventSynchronize(g_trace.ev[2 * i + 1]) != hipSuccess) return FLCE_ERR_HIP;
    if (hipEventElapsedTime(ms, g_trace.ev[2 * i], g_trace.ev[2 * i + 1]) != hipSuccess) return FLCE_ERR_HIP;
  }
  return FLCE_OK;
}

}  // extern "C"
