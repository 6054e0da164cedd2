/*
 * flce.h -- C ABI of the fused linear cross-entropy library for AMD MI355X
 * (gfx950).
 *
 * One call computes, for bf16 hidden states X[T,H] and a bf16 head W[V,H]:
 *
 *   z[t,v]  = sum_h X[t,h] W[v,h]            fp32 accumulation, v < Vu only
 *   z'      = c * tanh(z / c)                 if c > 0 (softcap), else z
 *   lse[t]  = log sum_{v<Vu} exp z'[t,v]
 *   l[t]    = lse[t] - z'[t, y_t]             0 where y_t == ignore_index
 *   loss    = (sum_t l[t]) / D
 *
 * and the backward pass gives dX = G W[:Vu] and dW[:Vu] = G^T X with
 * G[t,v] = (g/D) (softmax(z')[t,v] - [v == y_t]) (1 - (z'/c)^2), where g is the
 * upstream scalar gradient.  The [T,V] logits are never stored: the forward
 * keeps per-token log-sum-exp partials and the backward recomputes logit tiles
 * over bounded vocabulary chunks.
 *
 * Sources (NVIDIA NeMo AutoModel API pages):
 *  - "nemo_automodel.components.models.inkling2.loss",
 *    Inkling2FusedLinearCrossEntropy (constructor and class description):
 *    a bf16 x bf16 projection accumulated in fp32, then the softcap and the
 *    loss in fp32 arithmetic; only head rows below unpadded_vocab_size take
 *    part in the softmax; an fp32 head takes part through its bf16 rounding.
 *  - "nemo_automodel.components.loss.linear_ce", FusedLinearCrossEntropy
 *    (constructor: ignore_index, logit_softcapping, reduction; forward:
 *    hidden_states, labels, lm_weight, num_label_tokens; scalar result).
 *  - "nemo_automodel.components.loss.chunked_ce", _ChunkedCrossEntropySum
 *    (forward: ignored positions give zero loss and gradient, fp32 scalar
 *    result, inputs not mutated; backward: fp32 softmax chunks recomputed,
 *    scalar upstream gradient).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers on the current HIP device,
 *    row-major and contiguous.  The caller owns every buffer; the library
 *    allocates no device memory, and no compute call carries state to the
 *    next one.  The one process-wide state is the launch trace
 *    (flce_trace_*, for measurement): while it runs, every launch also
 *    records a pair of HIP events into it.  Inputs are read only.
 *  - Work is enqueued on `stream` and the call returns without waiting for
 *    it (no host synchronisation).
 *  - The return value is an flce_status_t.  Argument errors are detected on
 *    the host before any device work is enqueued, so a non-zero return means
 *    nothing was launched (except FLCE_ERR_HIP, which reports a failed launch).
 *  - A label that is neither ignore_index nor in [0, unpadded_vocab) can only
 *    be seen on the device: that position is treated as ignored and
 *    FLCE_DEVICE_BAD_LABEL is OR-ed into *device_status (if not NULL).
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum flce_status {
  FLCE_OK = 0,
  FLCE_ERR_INVALID_ARG = 1, /* a size, knob or pointer is out of its domain   */
  FLCE_ERR_UNSUPPORTED = 2, /* valid, but outside what the kernels handle     */
  FLCE_ERR_WORKSPACE = 3,   /* workspace NULL, misaligned or too small         */
  FLCE_ERR_HIP = 4          /* a HIP launch failed                             */
} flce_status_t;

/* Bits OR-ed into the optional device status word. */
#define FLCE_DEVICE_BAD_LABEL 1

typedef enum flce_reduction {
  FLCE_REDUCTION_SUM = 0,  /* loss = sum of per-token losses                 */
  FLCE_REDUCTION_MEAN = 1  /* loss = sum / (number of non-ignored positions) */
} flce_reduction_t;

typedef enum flce_dtype {
  FLCE_DTYPE_BF16 = 0,
  FLCE_DTYPE_FP32 = 1
} flce_dtype_t;

/*
 * Problem description, shared by every entry point.
 *
 * num_tokens        T >= 0: flattened [batch, sequence] positions.
 *                   Sizes beyond T = 2^21, V = 2^23 or H = 2^20 return
 *                   FLCE_ERR_UNSUPPORTED (the kernels address a 256-row
 *                   tile of any operand with 32-bit byte offsets).
 * hidden            H > 0, a multiple of 8 (rows of 16-byte pieces).  The
 *                   kernels step through H in groups of 128: when H is not a
 *                   multiple of 128, each call copies the head's rows < Vu
 *                   into the workspace with zero-padded rows of Hp =
 *                   ceil(H/128)*128 elements (Vu*Hp*2 more bytes), and the
 *                   gathered hidden rows are padded the same way.
 * vocab             V: rows of the head, padding included.
 * unpadded_vocab    Vu, 0 < Vu <= V: rows that take part in the softmax
 *                   (Inkling2 page, constructor argument unpadded_vocab_size).
 * softcap           c >= 0 and finite; 0 turns the softcap off (linear_ce page,
 *                   constructor argument logit_softcapping).
 * ignore_index      label value of positions that do not count (default -100).
 * reduction         FLCE_REDUCTION_SUM or FLCE_REDUCTION_MEAN.
 * num_label_tokens  > 0: divide the summed loss by this count whatever the
 *                   reduction (linear_ce page, forward argument
 *                   num_label_tokens); < 0: not given.  0 is invalid.
 * weight_dtype      FLCE_DTYPE_BF16, or FLCE_DTYPE_FP32 for an fp32 head that
 *                   each call rounds to bf16 itself (Inkling2 page, class
 *                   description: an fp32 head is used at its bf16 value,
 *                   rounded to nearest even like torch's cast).  By default
 *                   each call stages the rounded copy of rows < Vu in the
 *                   workspace (Vu*Hp*2 more bytes, one pass over the head per
 *                   call); rows >= Vu are never read.
 * flags             0, or FLCE_FLAG_ROUND_HEAD_ON_LOAD with an fp32 head whose
 *                   H is a multiple of 128: no staged copy; the projection and
 *                   recompute GEMMs read the fp32 head and round each piece on
 *                   its way into their bf16 LDS tiles, and the recompute keeps
 *                   one chunk's rounded rows for the dH contraction (vc*Hp*2
 *                   workspace bytes instead of Vu*Hp*2).  Results equal the
 *                   staged path's within rounding order (bit for bit where both
 *                   use 256-row tiles).  It reads twice the head bytes per
 *                   tile and runs slower (about 1.3x the staged step at
 *                   T=8192, H=3072, Vu=256000): a choice of memory over time.
 *                   Ignored for H not a multiple of 128 (the head is staged).
 *                   FLCE_FLAG_DW_TILE_256 or FLCE_FLAG_DW_TILE_384 (at most
 *                   one; 384 needs H >= 384) fix the tile of the backward's
 *                   dW contraction, which the library otherwise picks with
 *                   the vocabulary chunk width from an estimate of rounds of
 *                   tiles on the device's compute units: 256-row tiles of
 *                   G^T Xc, or 384-row tiles of Xc^T G stored transposed.
 *                   Either gives the same result up to the order of fp32
 *                   rounding.  FLCE_FLAG_HEAD_STAGED, read by flce_backward
 *                   only (flce_forward accepts and ignores it, so one problem
 *                   can serve both calls): the caller asserts that the
 *                   workspace still holds the head copy that the matching
 *                   flce_forward staged in it (an fp32 head, or H not a
 *                   multiple of 128), with the same problem and head and
 *                   nothing written to the workspace since; the backward
 *                   then skips its own staging pass (one read of the head's
 *                   usable rows).  Without a staged copy the bit changes
 *                   nothing.  Not for a workspace other than the forward's
 *                   (flce_forward_noalloc stages into its own scratch): the
 *                   backward would read whatever the region holds.  Other
 *                   bits are invalid.
 */
typedef struct flce_problem {
  int64_t num_tokens;
  int64_t hidden;
  int64_t vocab;
  int64_t unpadded_vocab;
  float softcap;
  int32_t reduction;
  int64_t ignore_index;
  int64_t num_label_tokens;
  int32_t weight_dtype;
  int32_t flags;
} flce_problem_t;

/* flce_problem_t.flags bits. */
#define FLCE_FLAG_ROUND_HEAD_ON_LOAD 1
#define FLCE_FLAG_DW_TILE_256 2
#define FLCE_FLAG_DW_TILE_384 4
#define FLCE_FLAG_HEAD_STAGED 8

/* Human-readable name of a status code (static string, never NULL). */
const char* flce_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int flce_version(void);

/*
 * Bytes of device workspace the forward and backward calls need for this
 * problem (one size serves both).  Writes it to *bytes.  The bound keeps every
 * logit-shaped scratch buffer at most a quarter of a bf16 [T, Vu] array.
 * Errors: FLCE_ERR_INVALID_ARG / FLCE_ERR_UNSUPPORTED as for flce_forward.
 */
int flce_workspace_size(const flce_problem_t* problem, size_t* bytes);

/*
 * The backward pass's launch plan for this problem on a device with cu_count
 * compute units (<= 0: the current device's count, 256 when it cannot be
 * read): the vocabulary chunk width in head rows (*chunk_rows, a multiple of
 * 256, at most max(256, a quarter of Vu)), the number of chunks (*chunks; 0
 * for a problem with no tokens, where the backward launches no chunk) and the
 * rows of the dW contraction's tiles (*dw_tile_rows: 256 for tiles of G^T Xc,
 * 384 for tiles of Xc^T G stored transposed).  It follows the problem's
 * FLCE_FLAG_DW_TILE_* bits.  Host only: launches nothing, and with
 * cu_count > 0 makes no HIP call.  The workspace size does not depend on it.
 * Errors: as flce_workspace_size; FLCE_ERR_INVALID_ARG for a NULL output.
 */
int flce_backward_plan(const flce_problem_t* problem, int cu_count, int64_t* chunk_rows, int64_t* chunks,
                       int* dw_tile_rows);

/*
 * Forward pass.
 *
 * hidden       bf16 [T, H], 16-byte aligned.
 * weight       [V, H] in weight_dtype (bf16 or fp32), 16-byte aligned; rows
 *              >= Vu are never read.
 * labels       int64 [T].
 * loss         fp32 scalar (device): the reduced loss; NaN for MEAN with no
 *              valid position and no num_label_tokens (0/0, as PyTorch).
 * lse          fp32 [T] (required): per-token log-sum-exp over the usable
 *              rows, 0 at ignored positions.  The backward pass reads it.
 * token_loss   fp32 [T] or NULL: per-token loss, 0 at ignored positions.
 * device_status int32 scalar or NULL; see FLCE_DEVICE_BAD_LABEL.  It is only
 *              OR-ed into, never cleared.
 * workspace    device buffer of at least flce_workspace_size() bytes,
 *              256-byte aligned; its contents need not be initialised and
 *              are scratch only after the call.
 */
int flce_forward(const flce_problem_t* problem, const void* hidden, const void* weight,
                 const int64_t* labels, float* loss, float* lse, float* token_loss,
                 int32_t* device_status, void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/*
 * Forward pass without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving or
 * scoring loops, harnesses that forbid allocation).  Same arguments and
 * results as flce_forward, bit for bit, but the scratch is the library's own
 * fixed array of 64 MiB per device (device memory that the library's code
 * object brings, held until the process ends); the call allocates nothing.
 *
 * Limit: the forward's scratch must fit the 64 MiB, about
 *   Tp*Hp*2 + ceil(Vu/256)*Tp*8 + 13*Tp + 1 KiB   bytes
 * with Tp = T rounded up to 256 and Hp = H rounded up to 128, plus Vu*Hp*2
 * when the head is staged (an fp32 head, or H not a multiple of 128).  The
 * llama3-8b head at T = 4096 (H = 4096, V = 128256) needs 48 MiB.  A larger
 * problem returns FLCE_ERR_WORKSPACE before anything is launched.
 * FLCE_ERR_HIP if the scratch's device address cannot be looked up.
 *
 * Every call on one device shares that device's scratch: calls that overlap
 * in time on one device (several streams or host threads) race and give
 * wrong results.  Nothing in the scratch needs to start at zero.
 */
int flce_forward_noalloc(const flce_problem_t* problem, const void* hidden, const void* weight,
                         const int64_t* labels, float* loss, float* lse, float* token_loss,
                         int32_t* device_status, hipStream_t stream);

/*
 * Backward pass: gradients of grad_out * loss.
 *
 * hidden, weight, labels   as passed to flce_forward.
 * lse          fp32 [T] written by flce_forward for the same inputs.
 * grad_out     fp32 scalar (device): upstream gradient of the loss.
 * d_hidden     bf16 [T, H] (output, overwritten): rows of ignored positions 0.
 * d_weight     fp32 [V, H] (output, overwritten): rows >= Vu are 0.
 * device_status, workspace  as for flce_forward.
 *
 * Results are deterministic: no atomics take part in any sum.
 */
int flce_backward(const flce_problem_t* problem, const void* hidden, const void* weight,
                  const int64_t* labels, const float* lse, const float* grad_out,
                  void* d_hidden, float* d_weight, int32_t* device_status, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);

/*
 * Round an fp32 head to the bf16 compute copy the kernels read: nearest
 * value, ties to even, NaN stays NaN ("nemo_automodel.components.models.
 * inkling2.loss", class description: an fp32 head is used at its bf16
 * value, the rounding sharded training applies to the model's own head).
 *
 * src    fp32 [count], 4-byte aligned (device).
 * dst    bf16 [count], 2-byte aligned (device); may not overlap src.
 * count  >= 0 elements.
 * Errors: FLCE_ERR_INVALID_ARG for a negative count or a NULL pointer with
 * count > 0; FLCE_ERR_UNSUPPORTED for misaligned pointers.
 */
int flce_round_to_bf16(const float* src, void* dst, int64_t count, hipStream_t stream);

/*
 * Launch tracing, for measurement.  While a trace is running, every kernel
 * launch the library makes is bracketed by a pair of HIP events recorded on
 * the launch's stream, tagged with the kernel's kind below; a caller can then
 * read each launch's duration.  The trace is process-wide state: start, run
 * the calls to measure, stop, then read.  Not for concurrent use from several
 * host threads.
 */
typedef enum flce_kernel_kind {
  FLCE_KERNEL_COMPACT = 0,      /* label compaction                           */
  FLCE_KERNEL_GATHER = 1,       /* gather of the valid hidden rows            */
  FLCE_KERNEL_PROJ_LSE = 2,     /* forward projection + softcap + lse partials */
  FLCE_KERNEL_COMBINE = 3,      /* per-token lse / loss                       */
  FLCE_KERNEL_FINALIZE = 4,     /* loss reduction                             */
  FLCE_KERNEL_RECOMPUTE_G = 5,  /* backward logit recompute -> G chunk         */
  FLCE_KERNEL_DWEIGHT = 6,      /* dW rows of a chunk = G^T X (not launched on
                                   its own: part of FLCE_KERNEL_DGRAD)        */
  FLCE_KERNEL_DHIDDEN = 7,      /* dH += G W[chunk] (likewise)                 */
  FLCE_KERNEL_AUX = 8,          /* zero fills, scale, rounding                 */
  FLCE_KERNEL_CE_FORWARD = 9,   /* chunked CE: per-row lse and loss            */
  FLCE_KERNEL_CE_BACKWARD = 10, /* chunked CE: per-row logits gradient         */
  FLCE_KERNEL_DGRAD = 11        /* dH += G W[chunk] and dW rows = G^T X of one
                                   chunk, in one launch; its flops are both   */
} flce_kernel_kind_t;

/*
 * Start recording up to `capacity` launches (events are created here, so this
 * call is not for a timed region).  Restarting discards the previous trace.
 * Errors: FLCE_ERR_INVALID_ARG for capacity <= 0, FLCE_ERR_HIP if events
 * cannot be created.
 */
int flce_trace_start(int capacity);

/*
 * Record only launches of the kinds whose bit (1 << kind) is set in
 * kind_mask; the default, and 0xFFFFFFFF, is every kind.  Applies to launches
 * made after the call, and stays in force across flce_trace_start.  With
 * fewer kinds recorded, fewer events sit between the launches being timed.
 */
int flce_trace_select(uint32_t kind_mask);

/* Stop recording; the recorded launches stay readable. */
int flce_trace_stop(void);

/* Number of launches recorded (at most the capacity). */
int flce_trace_count(void);

/*
 * Kind and duration in milliseconds of recorded launch i.
 * Waits for that launch's end event.  `flops` receives the launch's
 * algorithmic multiply-add work (2 per multiply-add) for the contraction
 * kinds, else 0; any output pointer may be NULL.
 * Errors: FLCE_ERR_INVALID_ARG for i out of range, FLCE_ERR_HIP.
 */
int flce_trace_get(int i, int* kind, float* ms, double* flops);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H */
