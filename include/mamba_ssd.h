/*
 * C ABI of the Mamba-2 state space duality (SSD) layer (gfx950), in the same
 * library as mamba_scan.h (libmamba_scan.so).
 *
 * Operation ("Mamba and selective state spaces, from first principles",
 * section "Mamba-2: state space duality": A_t is a scalar times the identity,
 * a_t = exp(Delta_t A_h) with one A_h per head; the channels form heads of P
 * channels that share a_t, B_t and C_t; each head's state is an N x P matrix),
 * per batch row b and head h, with the first-order input weight and the
 * softplus step of the S6 layer (mamba_scan.h):
 *
 *   Delta_t = softplus(dt[b,t,h] + dt_bias[h])
 *   S_t     = exp(Delta_t A[h]) S_{t-1} + Delta_t B_t x_t^T      (N x P)
 *   y_t     = S_t^T C_t + D[h] x_t                               (P)
 *
 * with S_{-1} = h0 (zeros without one). The call computes it by the chunked
 * algorithm of the same section (chunks of 256 steps: the masked matrix form
 * inside a chunk on the matrix cores, the scalar recurrence across chunks).
 *
 * Conventions as in mamba_scan.h. This build supports io_dtype MAMBA_BF16,
 * headdim P = 64 and dstate N = 128 (the Mamba-2 2.7B layer's head shape);
 * other values give MAMBA_ERR_UNSUPPORTED. The products take bf16 operands
 * (the state entering each chunk and the masked scores are rounded to bf16)
 * and accumulate in fp32.
 */
#ifndef MAMBA_SSD_H
#define MAMBA_SSD_H

#include <stddef.h>
#include <stdint.h>

#include "mamba_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mamba_ssd_desc {
  int64_t batch;    /* >= 0                                             */
  int64_t seqlen;   /* L >= 0                                           */
  int64_t nheads;   /* H >= 0                                           */
  int64_t headdim;  /* P: must be 64                                    */
  int64_t dstate;   /* N: must be 128                                   */
  int64_t ngroups;  /* G >= 1 dividing H: head h reads B, C group h/(H/G) */
  int32_t io_dtype; /* MAMBA_BF16                                       */
  uint32_t flags;   /* 0                                                */
} mamba_ssd_desc;

/* Bytes of device workspace mamba_ssd_fwd needs (0 for an invalid desc):
 * per (batch, head, chunk) one fp32 and one bf16 N x P state. */
size_t mamba_ssd_workspace_size(const mamba_ssd_desc *desc);

/*
 *   x          : (batch, seqlen, H, P) bf16, 16-byte aligned.
 *   dt         : (batch, seqlen, H) bf16, Delta before the bias and softplus.
 *   A          : (H) float32 (negative for a decaying state).
 *   B, C       : (batch, seqlen, G, N) bf16, 16-byte aligned.
 *   D, dt_bias : (H) float32 or NULL (zero).
 *   h0         : (batch, H, N, P) float32 or NULL (zeros).
 *   out        : (batch, seqlen, H, P) bf16, written.
 *   last_state : (batch, H, N, P) float32 or NULL; receives S_{L-1} (h0 or
 *                zeros when seqlen == 0).
 *   workspace  : mamba_ssd_workspace_size(desc) bytes, 256-byte aligned.
 * Outputs must not overlap any input, the workspace or each other.
 */
mamba_status mamba_ssd_fwd(const mamba_ssd_desc *desc, const void *x, const void *dt,
                           const float *A, const void *B, const void *C, const float *D,
                           const float *dt_bias, const float *h0, void *out,
                           float *last_state, void *workspace, size_t workspace_bytes,
                           void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SSD_H */
