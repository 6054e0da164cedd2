/*
 * chunked_ce.h -- C ABI of the cross-entropy over given logits ("chunked CE")
 * in the same library as flce.h, for AMD MI355X (gfx950).
 *
 * For logits L[T,V] (bf16 or fp32, any leading token dimensions flattened to
 * T) and labels y[T]:
 *
 *   y'[t]   = ignore_index where mask[t] == 0, else y[t]   (mask optional)
 *   lse[t]  = log sum_v exp L[t,v]                      in fp32
 *   l[t]    = lse[t] - L[t, y'[t]]                      0 where y'[t] == ignore_index
 *   loss    = (sum_t l[t]) / D
 *
 * and the backward pass gives dL[t,v] = (g/D) (softmax(L[t])[v] - [v == y'[t]])
 * for counted positions, 0 for ignored ones, in the logits' dtype.  D is
 * num_label_tokens when given, else the number of counted positions for
 * MEAN, else 1.  The logits stay in their dtype; nothing of logits size is
 * written by the forward.
 *
 * Source (NVIDIA NeMo AutoModel API pages): "nemo_automodel.components.loss.
 * chunked_ce" -- ChunkedCrossEntropy (constructor: chunk_len, compile,
 * ignore_index, reduction; forward: logits [..., vocab], labels, mask,
 * num_label_tokens; scalar result; with a mask, ignored positions are
 * replaced with ignore_index in the labels tensor), _ChunkedCrossEntropySum
 * (forward: sum-reduced cross-entropy in fp32 chunks, logits kept in their
 * dtype and not mutated, ignored positions give zero loss and gradient;
 * backward: softmax recomputed, scalar upstream gradient, logits gradient
 * returned), _validate_chunk_len (chunk_len must be positive) and
 * compute_cross_entropy (sum of per-position cross-entropies).
 *
 * Conventions are those of flce.h: device pointers on the current HIP
 * device, row-major and contiguous; caller-owned buffers (no allocation, no
 * state between calls); work enqueued on `stream` without host waits; the
 * return value is an flce_status_t and argument errors are reported before
 * any device work.  A label that is neither ignore_index nor in [0, V), at a
 * position the mask keeps, is treated as ignored and FLCE_DEVICE_BAD_LABEL
 * is OR-ed into *device_status (if not NULL).
 */
#ifndef CHUNKED_CE_H
#define CHUNKED_CE_H

#include "flce.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Problem description, shared by every chunked_ce entry point.
 *
 * num_tokens        T >= 0 positions (the logits' leading dimensions, flattened).
 * vocab             V > 0 columns of the logits.
 * ignore_index      label value of positions that do not count (default -100).
 * reduction         FLCE_REDUCTION_SUM or FLCE_REDUCTION_MEAN.
 * num_label_tokens  > 0: divide the summed loss by this count whatever the
 *                   reduction; < 0: not given; 0 is invalid.
 * logits_dtype      FLCE_DTYPE_BF16 or FLCE_DTYPE_FP32; the gradient has the
 *                   same dtype.
 * chunk_len         > 0.  The page's bound on how many rows are upcast to fp32
 *                   at once; these kernels never hold an fp32 copy of the
 *                   logits, so it does not change the result or the memory
 *                   used.  Checked for the page's validation only.
 */
typedef struct chunked_ce_problem {
  int64_t num_tokens;
  int64_t vocab;
  int64_t ignore_index;
  int32_t reduction;
  int64_t num_label_tokens;
  int32_t logits_dtype;
  int64_t chunk_len;
} chunked_ce_problem_t;

/*
 * Workspace bytes chunked_ce_forward / chunked_ce_backward need (one size
 * serves both): O(T), never logits-sized.  Writes it to *bytes.
 * Errors: FLCE_ERR_INVALID_ARG for an invalid problem.
 */
int chunked_ce_workspace_size(const chunked_ce_problem_t* problem, size_t* bytes);

/*
 * Forward pass.
 *
 * logits          [T, V] in logits_dtype, 16-byte aligned.  A row is read only
 *                 if its position counts.
 * labels          int64 [T], 8-byte aligned.
 * mask            NULL, or [T] elements of mask_elem_bytes bytes (1, 2, 4 or
 *                 8: bool/uint8, int16, int32/fp32 bit patterns, int64): a
 *                 position counts only where its element is not all-zero
 *                 bits.  (A -0.0 float mask entry counts; pass integer or
 *                 bool masks.)
 * mask_elem_bytes 1, 2, 4 or 8 when mask is given; ignored otherwise.
 * loss            fp32 scalar (device): the reduced loss; NaN for MEAN with no
 *                 counted position and no num_label_tokens.
 * lse             fp32 [T] (required): per-position log-sum-exp, 0 at ignored
 *                 positions.  The backward pass reads it.
 * token_loss      fp32 [T] or NULL: per-position loss, 0 at ignored positions.
 * device_status   int32 scalar or NULL (only OR-ed into).
 * workspace       at least chunked_ce_workspace_size() bytes, 256-byte aligned.
 */
int chunked_ce_forward(const chunked_ce_problem_t* problem, const void* logits, const int64_t* labels,
                       const void* mask, int32_t mask_elem_bytes, float* loss, float* lse, float* token_loss,
                       int32_t* device_status, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward pass: gradient of grad_out * loss with respect to the logits.
 *
 * logits, labels, mask, mask_elem_bytes   as passed to chunked_ce_forward.
 * lse             fp32 [T] written by chunked_ce_forward for the same inputs.
 * grad_out        fp32 scalar (device).
 * d_logits        [T, V] in logits_dtype, 16-byte aligned (output, overwritten;
 *                 rows of ignored positions are 0).  May not overlap logits.
 * device_status, workspace   as for chunked_ce_forward.
 */
int chunked_ce_backward(const chunked_ce_problem_t* problem, const void* logits, const int64_t* labels,
                        const void* mask, int32_t mask_elem_bytes, const float* lse, const float* grad_out,
                        void* d_logits, int32_t* device_status, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * In-place label rewrite the page describes for ChunkedCrossEntropy.forward
 * with a mask: labels[t] = ignore_index wherever mask[t] is all-zero bits.
 *
 * labels  int64 [count], 8-byte aligned (device, modified).
 * mask    [count] elements of mask_elem_bytes bytes (1, 2, 4 or 8).
 * Errors: FLCE_ERR_INVALID_ARG for count < 0, NULL pointers with count > 0 or
 * another element size; FLCE_ERR_UNSUPPORTED for misaligned pointers.
 */
int chunked_ce_mask_labels(int64_t* labels, const void* mask, int32_t mask_elem_bytes, int64_t count,
                           int64_t ignore_index, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CHUNKED_CE_H */
