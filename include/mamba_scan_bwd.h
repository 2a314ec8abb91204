/*
 * C ABI of the backward pass of the full-sequence selective scan (gfx950), in
 * the same library as mamba_scan.h (libmamba_scan.so).
 *
 * Given the inputs of a mamba_scan_fwd / mamba_scan_fwd_init call, the
 * gradient dout = dLoss/dout and optionally dlast = dLoss/d(last_state), it
 * returns the gradient of the loss with respect to every input of the scan.
 * The intermediate states are not taken from the forward pass: the call
 * recomputes them from the inputs (erikxu.me notes "Mamba: Linear-Time
 * Sequence Modeling with Selective State Spaces", section "GPU Memory
 * Hierarchy": states are recomputed in the backward pass instead of being
 * stored; "Mamba and selective state spaces, from first principles", section
 * "The hardware-aware scan").
 *
 * With the forward operation of mamba_scan.h (first-order Bbar, y_t =
 * (C_t . h_t + D x_t) silu(z_t)), per batch row b, channel d and state n:
 *   ds_t       = dout_t silu(z_t)                   (dout_t without z)
 *   lam_t      = C_t ds_t + abar_{t+1} lam_{t+1},   lam_{L-1} = C_{L-1} ds_{L-1} + dlast
 *   dx_t       = D ds_t + Delta_t sum_n lam_t,n B_t,n
 *   ddelta_t   = sigmoid(delta_t + delta_bias) sum_n lam_t,n (A_n abar_t,n h_{t-1},n + B_t,n x_t)
 *   dz_t       = dout_t (C_t . h_t + D x_t) silu'(z_t)
 *   dA[d,n]    = sum_{b,t} Delta_t lam_t,n abar_t,n h_{t-1},n
 *   dB[b,t,g,n] = sum_{d in group g} lam_t,n Delta_t x_t
 *   dC[b,t,g,n] = sum_{d in group g} ds_t h_t,n
 *   dD[d]      = sum_{b,t} ds_t x_t
 *   ddelta_bias[d] = sum_{b,t} ddelta_t
 *   dh0        = abar_0 lam_0       (the gradient of the initial state)
 * where abar_t = exp(Delta_t A), Delta_t = softplus(delta_t + delta_bias) and
 * h_{-1} = h0 (zeros without one).
 *
 * Conventions as in mamba_scan.h (device pointers owned by the caller,
 * asynchronous on `stream`, synchronous validation, mamba_last_error()).
 * dx, ddelta and dz are in the io dtype; all other gradients are float32
 * (dB and dC too, whatever the io dtype: they are sums over channels).
 * Results are deterministic: every sum is taken in a fixed order.
 */
#ifndef MAMBA_SCAN_BWD_H
#define MAMBA_SCAN_BWD_H

#include <stddef.h>
#include <stdint.h>

#include "mamba_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Bytes of device workspace mamba_scan_bwd needs (0 when none). Bits 0-15 of
 * desc->flags force the number of time segments (0 = the library's choice,
 * which depends on the compute-unit count of the current device); other bits
 * must be 0 (the backward of the MAMBA_SCAN_ZOH mode is not provided:
 * mamba_scan_bwd returns MAMBA_ERR_UNSUPPORTED for it). The workspace holds,
 * among others, one fp32 copy of the state per 8 time steps (about
 * batch * seqlen * dim * dstate / 2 bytes); one such copy, batch * dim *
 * dstate * 4 bytes, must stay below 2^31 (else mamba_scan_bwd returns
 * MAMBA_ERR_UNSUPPORTED and this function 0). Returns 0 for an invalid
 * descriptor as well.
 */
size_t mamba_scan_bwd_workspace_size(const mamba_scan_desc *desc);

/*
 * Gradients of the full-sequence scan.
 *   Inputs as mamba_scan_fwd_init: x, delta, z, B, C (io dtype), A, D,
 *   delta_bias, h0 (float32); z, D, delta_bias, h0 may be NULL.
 *   dout        : (batch, seqlen, dim) io dtype, dLoss/dout.
 *   dlast       : (batch, dim, dstate) float32 or NULL (zero): dLoss/d(last_state).
 *   dx, ddelta  : (batch, seqlen, dim) io dtype, written (ddelta is the
 *                 gradient of delta, before the bias and the softplus).
 *   dz          : (batch, seqlen, dim) io dtype, written, or NULL to skip;
 *                 not touched when z is NULL.
 *   dA          : (dim, dstate) float32, written.
 *   dB, dC      : (batch, seqlen, G, dstate) float32 (the shape of B),
 *                 written; each is summed over its group's channels.
 *   dD, ddelta_bias : (dim) float32 or NULL (skip), written.
 *   dh0         : (batch, dim, dstate) float32 or NULL (skip), written.
 *   workspace   : at least mamba_scan_bwd_workspace_size(desc) bytes, 256-byte
 *                 aligned; contents on entry ignored; not shared by calls that
 *                 run concurrently.
 * Outputs must not overlap any input, the workspace or each other. Alignment
 * as mamba_scan_fwd; fp32 tensors to 4 bytes.
 * With seqlen == 0 (or batch == 0) dA, dD and ddelta_bias are zero and dh0 =
 * dlast (zero without it).
 */
mamba_status mamba_scan_bwd(const mamba_scan_desc *desc, const void *x,
                            const void *delta, const float *A, const void *B,
                            const void *C, const float *D, const void *z,
                            const float *delta_bias, const float *h0,
                            const void *dout, const float *dlast, void *dx,
                            void *ddelta, float *dA, float *dB, float *dC,
                            float *dD, void *dz, float *ddelta_bias, float *dh0,
                            void *workspace, size_t workspace_bytes,
                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SCAN_BWD_H */
