/*
 * bdattn_lce — token-chunked linear cross-entropy on one MI355X (gfx950).
 *
 * The output layer's loss of language-model training as "Block Parallelism
 * for Efficient Distributed Long-Context Diffusion Language Model Training"
 * (§5.1, Experimental setup) computes it: the vocabulary projection is done
 * chunk of tokens by chunk of tokens with library matrix products, and fused
 * softmax/cross-entropy kernels turn each chunk's logits into the loss and
 * the logit gradient, so that full-sequence logits never exist. For token i
 * with hidden state h_i, vocabulary entry j with projection row w_j and
 * target t_i:
 *   z_ij = <h_i, w_j>,  LSE_i = ln sum_j exp(z_ij),  loss_i = LSE_i - z_{i,t_i}
 * (loss_i = 0 when t_i == ignore_index), and for an upstream gradient g_i of
 * each token's loss:
 *   G_ij = g_i (exp(z_ij - LSE_i) - [j == t_i])  (0 on ignored tokens),
 *   dH_i = sum_j G_ij w_j,  dW_j = sum_i G_ij h_i.
 *
 * Per chunk of `chunk` tokens: logits [chunk, V] in float32 by rocBLAS
 * (bf16 operands, fp32 accumulation) into the workspace; a fused kernel
 * computes LSE and the loss, and/or G rounded to bf16; rocBLAS then gives
 * dH of the chunk (bf16) and adds the chunk's part of dW (float32).
 *
 * Layouts (row-major, contiguous): h [N, D] bf16, w [V, D] bf16, targets [N]
 * int32, loss/lse/dloss [N] float32, dh [N, D] bf16, dw [V, D] float32. Every
 * pointer is a DEVICE pointer owned by the caller, 16-byte aligned (targets,
 * loss, lse, dloss: 4-byte). Calls enqueue on `hip_stream` and return without
 * waiting; the workspace (bdattn_lce_workspace_size bytes, 256-byte aligned)
 * must not be used by anything else until the work is done. dw is
 * overwritten (the chunks' parts are summed into it in float32, in chunk
 * order). Errors are returned as bdattn_status codes (include/bdattn.h);
 * nothing aborts. bdattn_last_error() explains the last failure.
 */
#ifndef BDATTN_LCE_H
#define BDATTN_LCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int64_t n_tokens;     /* N >= 0 */
  int32_t hidden;       /* D >= 8, a multiple of 8 */
  int32_t vocab;        /* V >= 8, a multiple of 8 (pad the vocabulary) */
  int32_t chunk;        /* tokens per chunk, >= 1; chunk * V < 2^31 */
  int32_t ignore_index; /* a target equal to it contributes no loss and no gradient */
} bdattn_lce_problem;

/* Bytes of workspace for bdattn_lce_fwd (pass 0) or bdattn_lce_bwd and
 * bdattn_lce_fwd_bwd (pass 1): float32 logits of one chunk, plus (pass 1) its
 * bf16 logit gradient. Host-only. BDATTN_ERR_SHAPE for an invalid problem. */
int bdattn_lce_workspace_size(const bdattn_lce_problem* p, int pass, size_t* bytes);

/* Forward: loss [N] and LSE [N] (float32). A target outside [0, V) other than
 * ignore_index gets a NaN loss (and, in the backward, no one-hot term). */
int bdattn_lce_fwd(const bdattn_lce_problem* p, const void* h, const void* w,
                   const int32_t* targets, float* loss, float* lse,
                   void* workspace, size_t ws_bytes, void* hip_stream);

/* Backward from the forward's LSE and the upstream gradient dloss [N]
 * (e.g. 1/n_valid for a mean): dh [N, D] bf16 and dw [V, D] float32. The
 * logits are recomputed chunk by chunk. */
int bdattn_lce_bwd(const bdattn_lce_problem* p, const void* h, const void* w,
                   const int32_t* targets, const float* lse, const float* dloss,
                   void* dh, float* dw, void* workspace, size_t ws_bytes, void* hip_stream);

/* Forward and backward in one pass over the chunks (one logits product per
 * chunk instead of two), for an upstream gradient dloss known in advance, as
 * when the loss ends the graph: loss, LSE, dh and dw. */
int bdattn_lce_fwd_bwd(const bdattn_lce_problem* p, const void* h, const void* w,
                       const int32_t* targets, const float* dloss, float* loss, float* lse,
                       void* dh, float* dw, void* workspace, size_t ws_bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* BDATTN_LCE_H */
