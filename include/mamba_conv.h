/*
 * C ABI of the causal depthwise convolution front-end of the SSM branch
 * (gfx950), in the same library as mamba_scan.h (libmamba_scan.so).
 *
 * Operation ("Mamba and selective state spaces, from first principles",
 * section "The Mamba block": the SSM branch is a causal depthwise convolution
 * of width 4, then SiLU, then the selective SSM; "Mamba" reading notes,
 * section "Mamba": the short depthwise convolution mixes nearby sequence
 * positions within each channel):
 *
 *   v[b,t,d]   = bias[d] + sum_{j=0}^{width-1} weight[d,j] * xin[b, t-(width-1)+j, d]
 *   out[b,t,d] = silu(v[b,t,d]) = v / (1 + exp(-v))
 *
 * weight[d, width-1] multiplies the current input (the tap order of a causal
 * Conv1d padded by width-1 steps on the left). Inputs before t = 0 are taken
 * from a state that holds the last width-1 inputs of an earlier piece of the
 * sequence, oldest first (zeros without one). For decode, that state is the
 * per-channel part of the recurrent state next to the SSM's D x N numbers.
 *
 * All pointers are device pointers owned by the caller; row-major,
 * contiguous. io tensors (xin, out, states) are float32 or bfloat16
 * (mamba_dtype); weight and bias are float32. Calls are asynchronous on
 * `stream` (a hipStream_t, NULL = default stream); validation happens before
 * any HIP call and reports through mamba_status / mamba_last_error().
 */
#ifndef MAMBA_CONV_H
#define MAMBA_CONV_H

#include <stddef.h>
#include <stdint.h>

#include "mamba_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Sizes. width must be 1, 2, 3 or 4 (the pages' blocks use 4); flags 0. */
typedef struct mamba_conv_desc {
  int64_t batch;    /* >= 0                                          */
  int64_t seqlen;   /* L >= 0 (must be 1 for mamba_conv1d_update)    */
  int64_t dim;      /* channels >= 0                                  */
  int64_t width;    /* taps per channel                               */
  int32_t io_dtype; /* mamba_dtype of xin, out and the states         */
  uint32_t flags;   /* 0                                              */
} mamba_conv_desc;

/*
 * Convolution + SiLU over full sequences.
 *   xin       : (batch, seqlen, dim) io dtype.
 *   weight    : (dim, width) float32.
 *   bias      : (dim) float32 or NULL (zero).
 *   state_in  : (batch, dim, width-1) io dtype or NULL (zeros): the inputs
 *               before t = 0, oldest first.
 *   out       : (batch, seqlen, dim) io dtype, written (the scan's x).
 *   state_out : (batch, dim, width-1) io dtype or NULL: receives the last
 *               width-1 inputs (from state_in where the sequence is shorter),
 *               for a later piece or for mamba_conv1d_update.
 * out and state_out must not overlap any input or each other (so state_in
 * and state_out cannot be the same buffer). Alignment: io tensors to their
 * element size, weight and bias to 4 bytes.
 */
mamba_status mamba_conv1d_fwd(const mamba_conv_desc *desc, const void *xin,
                              const float *weight, const float *bias,
                              const void *state_in, void *out, void *state_out,
                              void *stream);

/*
 * One decode token (desc->seqlen must be 1):
 *   out[b,d] = silu(bias[d] + sum_{j<width-1} weight[d,j] * state[b,d,j]
 *                   + weight[d,width-1] * xin[b,d]),
 * then state[b,d,:] shifts by one (oldest value out) and takes xin[b,d].
 *   state : (batch, dim, width-1) io dtype, read and written in place
 *           (ignored, may be NULL, when width == 1).
 *   xin, out : (batch, dim) io dtype; weight, bias as mamba_conv1d_fwd.
 * out must not overlap any input or the state.
 */
mamba_status mamba_conv1d_update(const mamba_conv_desc *desc, void *state,
                                 const void *xin, const float *weight,
                                 const float *bias, void *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_CONV_H */
