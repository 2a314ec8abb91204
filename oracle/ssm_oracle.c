/*
 * fp64 CPU oracle for the selective state-space scan (S6) and its one-token
 * state update.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file: only the test suite, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header or constant with the HIP
 * library; it is a plain, slow, literal restatement of what the pages define.
 *
 * What it computes, for every batch row b and channel d independently (one SSM
 * per channel: erikxu.me "Mamba" notes, section "State Space Models", the
 * paragraph on multidimensional inputs; ai.thesatyajit.com "Mamba and
 * selective state spaces", section "A state space model": the state of a
 * layer is D x N numbers):
 *
 *   h_{-1} = 0 (or a given initial state)          erikxu.me, "State Space
 *                                                   Models", discrete system
 *   for t = 0 .. L-1:
 *     Delta_t = softplus(delta[b,t,d] + bias[d])    ai.thesatyajit.com,
 *                                                   "Selection: B, C and Delta
 *                                                   from the token"
 *     abar_n  = exp(Delta_t * A[d,n])               same page, "Discretisation:
 *                                                   zero-order hold" and
 *                                                   "Selection" (A acts only
 *                                                   through exp(Delta A))
 *     bbar_n  = Delta_t * B[b,t,n]                  "Discretisation": the
 *                                                   first-order B-bar that the
 *                                                   reference code computes
 *             (or (abar_n - 1) / A[d,n] * B[b,t,n]  exact zero-order hold, a
 *                                                   test-only mode)
 *     h_n     = abar_n * h_n + bbar_n * x[b,t,d]    recurrence h_t = A-bar
 *                                                   h_{t-1} + B-bar x_t
 *     y       = sum_n C[b,t,n] * h_n + D[d] * x     y_t = C h_t + D x_t
 *                                                   (datarekha.com "State space
 *                                                   models and Mamba", "One
 *                                                   system, two views")
 *     y      *= silu(z[b,t,d]) if z is given        ai.thesatyajit.com, "The
 *                                                   Mamba block": the SSM
 *                                                   branch is multiplied by a
 *                                                   SiLU gate
 *   last_state[b,d,:] = h
 *
 * Layouts (row-major, contiguous): x, delta, z, out: (batch, seqlen, dim);
 * B, C: (batch, seqlen, ngroups, dstate): the channels form ngroups equal
 * consecutive groups, channel d reading group d / (dim / ngroups) (one group
 * shared by every channel is the S6 layer of ai.thesatyajit.com, "Selection";
 * groups of channels sharing B and C are the grouping of the same page's
 * "Mamba-2" section); A: (dim, dstate); D, bias: (dim); h0, last_state,
 * state: (batch, dim, dstate).
 * Optional arguments are NULL when absent (no D skip, no gate, zero bias, zero
 * initial state, no final state).
 *
 * Every value is double precision; libm exp/log1p; no fast-math.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(u) = log(1 + exp(u)), written so that neither branch overflows. */
static double softplus(double u) {
  if (u > 0.0) return u + log1p(exp(-u));
  return log1p(exp(u));
}

/* silu(v) = v * sigmoid(v) = v / (1 + exp(-v)). */
static double silu(double v) { return v / (1.0 + exp(-v)); }

/* One token of one (b, d) row: updates h[0..N-1] in place, returns y. */
static double row_step(int64_t N, double *h, double x, double delta_raw,
                       double bias, const double *A_d, const double *B_t,
                       const double *C_t, const double *D_d, const double *z,
                       int zoh) {
  double Delta = softplus(delta_raw + bias);
  double y = 0.0;
  for (int64_t n = 0; n < N; ++n) {
    double abar = exp(Delta * A_d[n]);
    double bbar;
    if (zoh)
      bbar = (abar - 1.0) / A_d[n] * B_t[n];
    else
      bbar = Delta * B_t[n];
    h[n] = abar * h[n] + bbar * x;
    y += C_t[n] * h[n];
  }
  if (D_d) y += (*D_d) * x;
  if (z) y *= silu(*z);
  return y;
}

/*
 * Full-sequence scan. Returns 0 on success, -1 on bad sizes or a missing
 * required pointer, -2 when zoh is requested with a zero entry of A.
 */
int oracle_scan_f64(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                    int64_t ngroups, const double *x, const double *delta, const double *A,
                    const double *B, const double *C, const double *D,
                    const double *z, const double *delta_bias,
                    const double *h0, int zoh, double *out, double *last_state,
                    int nthreads) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1) return -1;
  if (ngroups < 1 || dim % ngroups != 0) return -1;
  if (!x || !delta || !A || !B || !C || !out) return -1;
  if (zoh)
    for (int64_t i = 0; i < dim * dstate; ++i)
      if (A[i] == 0.0) return -2;
  if (nthreads < 1) nthreads = 1;
  const int64_t per_group = dim / ngroups;

#pragma omp parallel for collapse(2) schedule(static) num_threads(nthreads)
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t d = 0; d < dim; ++d) {
      const int64_t g = d / per_group;
      double *h = (double *)malloc(sizeof(double) * (size_t)dstate);
      for (int64_t n = 0; n < dstate; ++n)
        h[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;
      double bias = delta_bias ? delta_bias[d] : 0.0;
      for (int64_t t = 0; t < seqlen; ++t) {
        int64_t i = (b * seqlen + t) * dim + d;   /* (b, t, d) */
        int64_t j = ((b * seqlen + t) * ngroups + g) * dstate; /* (b, t, g, 0) */
        out[i] = row_step(dstate, h, x[i], delta[i], bias, A + d * dstate,
                          B + j, C + j, D ? D + d : NULL, z ? z + i : NULL, zoh);
      }
      if (last_state)
        for (int64_t n = 0; n < dstate; ++n)
          last_state[(b * dim + d) * dstate + n] = h[n];
      free(h);
    }
  }
  return 0;
}

/*
 * One decode token for every (b, d) row: the same step as one iteration of
 * the scan, against a resident state that is read and written in place.
 * x, delta, z, out: (batch, dim); B, C: (batch, ngroups, dstate).
 */
int oracle_state_update_f64(int64_t batch, int64_t dim, int64_t dstate, int64_t ngroups,
                            double *state, const double *x,
                            const double *delta, const double *A,
                            const double *B, const double *C, const double *D,
                            const double *z, const double *delta_bias, int zoh,
                            double *out, int nthreads) {
  if (batch < 0 || dim < 0 || dstate < 1) return -1;
  if (ngroups < 1 || dim % ngroups != 0) return -1;
  if (!state || !x || !delta || !A || !B || !C || !out) return -1;
  if (zoh)
    for (int64_t i = 0; i < dim * dstate; ++i)
      if (A[i] == 0.0) return -2;
  if (nthreads < 1) nthreads = 1;
  const int64_t per_group = dim / ngroups;

#pragma omp parallel for collapse(2) schedule(static) num_threads(nthreads)
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t d = 0; d < dim; ++d) {
      int64_t i = b * dim + d;
      int64_t j = (b * ngroups + d / per_group) * dstate; /* (b, g, 0) */
      out[i] = row_step(dstate, state + i * dstate, x[i], delta[i],
                        delta_bias ? delta_bias[d] : 0.0, A + d * dstate,
                        B + j, C + j, D ? D + d : NULL,
                        z ? z + i : NULL, zoh);
    }
  }
  return 0;
}

/*
 * Causal depthwise convolution followed by SiLU: the front-end of the SSM
 * branch (ai.thesatyajit.com, "The Mamba block": a causal depthwise
 * convolution of width 4, then SiLU, then the selective SSM; erikxu.me notes,
 * "Mamba": the short depthwise convolution mixes nearby sequence positions
 * within each channel, then SiLU, then the SSM).
 *
 * For every batch row b and channel d independently, with the inputs before
 * t = 0 taken from state_in (the last width - 1 inputs of an earlier piece of
 * the sequence, oldest first; zeros without it):
 *   v_t = bias[d] + sum_{j=0}^{width-1} weight[d, j] * xin[b, t - (width-1) + j, d]
 *   out[b, t, d] = silu(v_t)
 * so weight[d, width - 1] multiplies the current input (the tap order of a
 * causal Conv1d padded by width - 1 steps on the left).
 * state_out[b, d, j] = xin[b, seqlen - (width-1) + j, d] for j < width - 1
 * (taken from state_in where that time index is negative): what a later
 * piece, or the one-token update, needs.
 * Layouts: xin, out: (batch, seqlen, dim); weight: (dim, width); bias: (dim);
 * state_in, state_out: (batch, dim, width - 1).
 */
static double conv_input(const double *xin, const double *state_in, int64_t seqlen,
                         int64_t dim, int64_t width, int64_t b, int64_t d, int64_t t) {
  if (t >= 0) return xin[(b * seqlen + t) * dim + d];
  if (!state_in) return 0.0;
  return state_in[(b * dim + d) * (width - 1) + (width - 1) + t];
}

int oracle_conv1d_silu_f64(int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                           const double *xin, const double *weight, const double *bias,
                           const double *state_in, double *out, double *state_out,
                           int nthreads) {
  if (batch < 0 || seqlen < 0 || dim < 0 || width < 1) return -1;
  if ((batch * seqlen * dim > 0) && (!xin || !out || !weight)) return -1;
  if (nthreads < 1) nthreads = 1;

#pragma omp parallel for collapse(2) schedule(static) num_threads(nthreads)
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t d = 0; d < dim; ++d) {
      for (int64_t t = 0; t < seqlen; ++t) {
        double v = bias ? bias[d] : 0.0;
        for (int64_t j = 0; j < width; ++j)
          v += weight[d * width + j] *
               conv_input(xin, state_in, seqlen, dim, width, b, d, t - (width - 1) + j);
        out[(b * seqlen + t) * dim + d] = silu(v);
      }
      if (state_out)
        for (int64_t j = 0; j < width - 1; ++j)
          state_out[(b * dim + d) * (width - 1) + j] =
              conv_input(xin, state_in, seqlen, dim, width, b, d, seqlen - (width - 1) + j);
    }
  }
  return 0;
}

/*
 * One token of the convolution against its state (the decode step): the
 * state holds the last width - 1 inputs, oldest first; the output uses them
 * and the new input, then the state shifts by one and takes the new input.
 * state: (batch, dim, width - 1), read and written in place; xin, out:
 * (batch, dim).
 */
int oracle_conv1d_update_f64(int64_t batch, int64_t dim, int64_t width, double *state,
                             const double *xin, const double *weight, const double *bias,
                             double *out, int nthreads) {
  if (batch < 0 || dim < 0 || width < 1) return -1;
  if ((batch * dim > 0) && (!xin || !out || !weight || (width > 1 && !state))) return -1;
  if (nthreads < 1) nthreads = 1;

#pragma omp parallel for collapse(2) schedule(static) num_threads(nthreads)
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t d = 0; d < dim; ++d) {
      double *s = state ? state + (b * dim + d) * (width - 1) : NULL;
      const double *w = weight + d * width;
      double v = bias ? bias[d] : 0.0;
      for (int64_t j = 0; j < width - 1; ++j) v += w[j] * s[j];
      v += w[width - 1] * xin[b * dim + d];
      out[b * dim + d] = silu(v);
      for (int64_t j = 0; j + 1 < width - 1; ++j) s[j] = s[j + 1];
      if (width > 1) s[width - 2] = xin[b * dim + d];
    }
  }
  return 0;
}

/*
 * Gradients of the scan (first-order B-bar) by the plain reverse pass: the
 * backward pass of the method ("Mamba and selective state spaces, from first
 * principles", section "The hardware-aware scan": the backward pass recomputes
 * the intermediate states instead of storing them; here, on the CPU, every
 * state of a row is simply kept).
 *
 * Given dout = dLoss/dout (batch, seqlen, dim) and optionally
 * dlast = dLoss/dlast_state (batch, dim, dstate), with
 *   s_t = sum_n C[t,n] h[t,n] + D x_t,  y_t = s_t * silu(z_t)  (s_t without z),
 * the adjoint of the state, lambda_t = dLoss/dh_t, obeys
 *   lambda_{L-1} = ds_{L-1} C_{L-1} + dlast,
 *   lambda_t     = ds_t C_t + abar_{t+1} lambda_{t+1},     ds_t = dout_t silu(z_t),
 * and, from h_t = abar_t h_{t-1} + Delta_t x_t B_t with abar_t = exp(Delta_t A):
 *   dDelta_t = sum_n lambda_t,n (A_n abar_t,n h_{t-1,n} + x_t B_t,n)
 *   dx_t     = D ds_t + sum_n lambda_t,n Delta_t B_t,n
 *   dB_t,n  += lambda_t,n Delta_t x_t          (summed over the group's channels)
 *   dC_t,n  += ds_t h_t,n                       (summed over the group's channels)
 *   dA_n    += lambda_t,n Delta_t abar_t,n h_{t-1,n}  (summed over batch, time)
 *   dz_t     = dout_t s_t silu'(z_t)
 *   ddelta_t = dDelta_t sigmoid(delta_t + bias)  (softplus' = sigmoid)
 *   dbias   += ddelta_t; dD += ds_t x_t;  dh0 = abar_0 lambda_0.
 * Outputs: dx, ddelta, dz (batch, seqlen, dim); dA (dim, dstate); dB, dC
 * (batch, seqlen, ngroups, dstate); dD, dbias (dim); dh0 (batch, dim, dstate). dz, dD,
 * dbias, dh0 may be NULL (not wanted); all outputs are overwritten.
 * Parallel over channels; dB and dC are accumulated per thread, then summed.
 */
static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

int oracle_scan_bwd_f64(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                        int64_t ngroups, const double *x, const double *delta, const double *A,
                        const double *B, const double *C, const double *D,
                        const double *z, const double *delta_bias, const double *h0,
                        const double *dout, const double *dlast, double *dx,
                        double *ddelta, double *dA, double *dB, double *dC, double *dD,
                        double *dz, double *dbias, double *dh0, int nthreads) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1 || dstate > 64) return -1;
  if (ngroups < 1 || dim % ngroups != 0) return -1;
  if (!x || !delta || !A || !B || !C || !dout || !dx || !ddelta || !dA || !dB || !dC)
    return -1;
  if (nthreads < 1) nthreads = 1;
  const int64_t N = dstate, L = seqlen, G = ngroups, per_group = dim / ngroups;
  const int64_t bcn = batch * L * G * N;
  double *part = (double *)calloc((size_t)(nthreads * 2 * bcn + 1), sizeof(double));
  double *hist = (double *)malloc((size_t)(nthreads * (L + 1) * N + 1) * sizeof(double));
  if (!part || !hist) {
    free(part);
    free(hist);
    return -3;
  }

#pragma omp parallel for schedule(static) num_threads(nthreads)
  for (int64_t d = 0; d < dim; ++d) {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    double *pB = part + (int64_t)tid * 2 * bcn, *pC = pB + bcn;
    double *hs = hist + (int64_t)tid * (L + 1) * N; /* hs[(t+1)*N + n] = h_t, hs[n] = h_{-1} */
    const double *A_d = A + d * N;
    const double bias = delta_bias ? delta_bias[d] : 0.0;
    double dA_acc[64] = {0}, dD_acc = 0.0, dbias_acc = 0.0;
    for (int64_t b = 0; b < batch; ++b) {
      for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * dim + d) * N + n] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        const int64_t i = (b * L + t) * dim + d, j = ((b * L + t) * G + d / per_group) * N;
        const double Dl = softplus(delta[i] + bias);
        for (int64_t n = 0; n < N; ++n)
          hs[(t + 1) * N + n] = exp(Dl * A_d[n]) * hs[t * N + n] + Dl * B[j + n] * x[i];
      }
      double lam[64];
      for (int64_t n = 0; n < N; ++n) lam[n] = dlast ? dlast[(b * dim + d) * N + n] : 0.0;
      for (int64_t t = L - 1; t >= 0; --t) {
        const int64_t i = (b * L + t) * dim + d, j = ((b * L + t) * G + d / per_group) * N;
        const double u = delta[i] + bias, Dl = softplus(u), xt = x[i];
        double s = D ? D[d] * xt : 0.0;
        for (int64_t n = 0; n < N; ++n) s += C[j + n] * hs[(t + 1) * N + n];
        const double g = z ? silu(z[i]) : 1.0;
        const double ds = dout[i] * g;
        if (dz) {
          if (z) {
            const double sg = sigmoid(z[i]);
            dz[i] = dout[i] * s * sg * (1.0 + z[i] * (1.0 - sg));
          } else {
            dz[i] = 0.0; /* no gate: y does not depend on z */
          }
        }
        double dDl = 0.0, dxt = D ? D[d] * ds : 0.0;
        for (int64_t n = 0; n < N; ++n) {
          lam[n] += ds * C[j + n];
          const double abar = exp(Dl * A_d[n]), hprev = hs[t * N + n];
          pC[j + n] += ds * hs[(t + 1) * N + n];
          pB[j + n] += lam[n] * Dl * xt;
          dDl += lam[n] * (A_d[n] * abar * hprev + xt * B[j + n]);
          dxt += lam[n] * Dl * B[j + n];
          dA_acc[n] += lam[n] * Dl * abar * hprev;
          lam[n] *= abar;
        }
        dx[i] = dxt;
        ddelta[i] = dDl * sigmoid(u);
        dbias_acc += ddelta[i];
        dD_acc += ds * xt;
      }
      if (dh0)
        for (int64_t n = 0; n < N; ++n) dh0[(b * dim + d) * N + n] = lam[n];
    }
    for (int64_t n = 0; n < N; ++n) dA[d * N + n] = dA_acc[n];
    if (dD) dD[d] = dD_acc;
    if (dbias) dbias[d] = dbias_acc;
  }
  for (int64_t k = 0; k < bcn; ++k) {
    double sb = 0.0, sc = 0.0;
    for (int th = 0; th < nthreads; ++th) {
      sb += part[(int64_t)th * 2 * bcn + k];
      sc += part[(int64_t)th * 2 * bcn + bcn + k];
    }
    dB[k] = sb;
    dC[k] = sc;
  }
  free(part);
  free(hist);
  return 0;
}

/*
 * Mamba-2 state space duality (SSD) layer, by its linear recurrence
 * (ai.thesatyajit.com, "Mamba and selective state spaces, from first
 * principles", section "Mamba-2: state space duality"): A_t is a scalar times
 * the identity, a_t = exp(Delta_t A_h) with one A_h per head; the channels form
 * heads of P channels that share a_t, B_t and C_t, and each head's state is an
 * N x P matrix. Written, like the S6 layer above, with the first-order input
 * weight and the softplus(Delta_raw + bias) step:
 *
 *   Delta_t = softplus(dt[b,t,h] + dt_bias[h])
 *   S_t     = exp(Delta_t A[h]) S_{t-1} + Delta_t B_t x_t^T     (N x P)
 *   y_t     = S_t^T C_t + D[h] x_t                              (P)
 *
 * with S_{-1} = h0 (or 0). Heads form ngroups equal consecutive groups; head h
 * reads the B and C of group h / (nheads / ngroups).
 * Layouts (row-major, contiguous): x, out: (batch, seqlen, nheads, headdim);
 * dt: (batch, seqlen, nheads); A, D, dt_bias: (nheads); B, C: (batch, seqlen,
 * ngroups, dstate); h0, last_state: (batch, nheads, dstate, headdim). D,
 * dt_bias, h0, last_state may be NULL.
 */
int oracle_ssd_f64(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                   int64_t dstate, int64_t ngroups, const double *x, const double *dt,
                   const double *A, const double *B, const double *C, const double *D,
                   const double *dt_bias, const double *h0, double *out, double *last_state,
                   int nthreads) {
  if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 1 || dstate < 1) return -1;
  if (ngroups < 1 || nheads % ngroups != 0) return -1;
  if (!x || !dt || !A || !B || !C || !out) return -1;
  if (nthreads < 1) nthreads = 1;
  const int64_t H = nheads, P = headdim, N = dstate, G = ngroups, per_group = nheads / ngroups;

#pragma omp parallel for collapse(2) schedule(static) num_threads(nthreads)
  for (int64_t b = 0; b < batch; ++b) {
    for (int64_t h = 0; h < H; ++h) {
      double *S = (double *)malloc(sizeof(double) * (size_t)(N * P));
      for (int64_t k = 0; k < N * P; ++k) S[k] = h0 ? h0[(b * H + h) * N * P + k] : 0.0;
      const int64_t g = h / per_group;
      for (int64_t t = 0; t < seqlen; ++t) {
        const double Delta = softplus(dt[(b * seqlen + t) * H + h] + (dt_bias ? dt_bias[h] : 0.0));
        const double a = exp(Delta * A[h]);
        const double *Bt = B + ((b * seqlen + t) * G + g) * N;
        const double *Ct = C + ((b * seqlen + t) * G + g) * N;
        const double *xt = x + ((b * seqlen + t) * H + h) * P;
        double *yt = out + ((b * seqlen + t) * H + h) * P;
        for (int64_t n = 0; n < N; ++n)
          for (int64_t p = 0; p < P; ++p) S[n * P + p] = a * S[n * P + p] + Delta * Bt[n] * xt[p];
        for (int64_t p = 0; p < P; ++p) {
          double y = D ? D[h] * xt[p] : 0.0;
          for (int64_t n = 0; n < N; ++n) y += Ct[n] * S[n * P + p];
          yt[p] = y;
        }
      }
      if (last_state)
        for (int64_t k = 0; k < N * P; ++k) last_state[(b * H + h) * N * P + k] = S[k];
      free(S);
    }
  }
  return 0;
}
