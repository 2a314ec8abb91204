/*
 * mamba_scan.h — C ABI of the gfx950 selective state-space scan (S6).
 *
 * The operation (per batch row b, channel d, state n; one independent SSM per
 * channel with a D x N state per layer — "Mamba and selective state spaces,
 * from first principles", section "A state space model"):
 *
 *   Delta_t  = softplus(delta[b,t,d] + delta_bias[d])
 *              (section "Selection: B, C and Delta from the token")
 *   Abar     = exp(Delta_t * A[d,n])
 *              (sections "Discretisation: zero-order hold" and "Selection")
 *   Bbar x   = Delta_t * B[b,t,n] * x[b,t,d]
 *              (first-order Bbar, the form the page says the reference code
 *               computes, section "Discretisation: zero-order hold")
 *   h_t[n]   = Abar * h_{t-1}[n] + Bbar x,   h_{-1} = 0
 *              (erikxu.me notes "Mamba: Linear-Time Sequence Modeling with
 *               Selective State Spaces", section "State Space Models")
 *   y_t      = (sum_n C[b,t,n] h_t[n] + D[d] x[b,t,d]) * silu(z[b,t,d])
 *              (D term: "State space models and Mamba", section "One system,
 *               two views"; gate: "Mamba and selective state spaces", section
 *               "The Mamba block")
 *
 * The full-sequence call loads the inputs once, keeps every state on chip and
 * writes back only y of shape (batch, L, D) and the final state ("Mamba and
 * selective state spaces", section "The hardware-aware scan"). The decode call
 * advances a resident fp32 state by one token (erikxu.me notes, "State Space
 * Models": constant work per generated token).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers on the current HIP device, owned
 *    by the caller, dense and row-major in the shapes given below. The library
 *    never allocates, frees or retains them.
 *  - io tensors (x, delta, z, B, C, out) are float32 (MAMBA_F32) or bfloat16
 *    bit patterns (MAMBA_BF16, 2 bytes each); A, D, delta_bias, state and
 *    last_state are always float32. All arithmetic is float32.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *    is enqueued asynchronously on it; nothing synchronises the host.
 *  - Argument validation is synchronous and happens before any HIP call: a
 *    non-OK status means nothing was enqueued. MAMBA_ERR_HIP reports a launch
 *    failure; faults during execution surface at the caller's next
 *    synchronisation. A thread-local message for the last non-OK status is
 *    returned by mamba_last_error(). No C++ exception crosses the ABI.
 *  - Calls on different streams may run concurrently as long as their output
 *    buffers (and workspaces) do not overlap.
 *  - Non-finite inputs are not checked; they propagate.
 */
#ifndef MAMBA_SCAN_H
#define MAMBA_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mamba_status {
  MAMBA_OK = 0,
  MAMBA_ERR_INVALID_ARG = 1, /* null required pointer, bad size, overlap, ... */
  MAMBA_ERR_UNSUPPORTED = 2, /* valid request this build does not implement   */
  MAMBA_ERR_HIP = 3          /* a HIP runtime call or kernel launch failed     */
} mamba_status;

typedef enum mamba_dtype {
  MAMBA_F32 = 0,
  MAMBA_BF16 = 1
} mamba_dtype;

/*
 * Input weight of the discretisation. By default Bbar x = Delta B x, the
 * first-order form ("Mamba and selective state spaces, from first principles",
 * section "Discretisation: zero-order hold": the form the reference code
 * computes). With MAMBA_SCAN_ZOH in desc->flags the exact zero-order hold is
 * used instead: Bbar_n = (exp(Delta A[d,n]) - 1) / A[d,n] B_n (its limit Delta B_n
 * where Delta A[d,n] is 0); Abar is exp(Delta A) either way. The ZOH mode runs
 * the general decay path (an exponential per state and step), so it is slower.
 */
#define MAMBA_SCAN_ZOH (1u << 16)

/*
 * Kernel choice of mamba_scan_fwd (results agree to rounding either way).
 * By default the segmented scan runs: one lane per (batch, channel) row with
 * all N states in its registers; when there are too few rows to fill the GPU
 * the sequence is cut into time segments (bits 0-15 of flags can force their
 * number), which costs a second pass over the inputs and a workspace.
 * MAMBA_SCAN_SPLIT_STATES selects the state-split scan instead: the 16 states
 * of a row on four lanes, the whole sequence in one pass, no workspace
 * (mamba_scan_workspace_size reports 0). It takes dstate 16 and the
 * first-order input weight only, and rows (strides) of fewer than
 * 2^31 / 9 bytes: otherwise MAMBA_ERR_UNSUPPORTED; with nonzero bits 0-15
 * too, MAMBA_ERR_INVALID_ARG. It is not the default because it measured
 * slower on the layers tried (0.42 against 0.35 ms per call on 8 x 2048 x 5120
 * bf16 on an MI355X, and no faster from 2 to 16 sequences).
 */
#define MAMBA_SCAN_SPLIT_STATES (1u << 17)

/*
 * Problem sizes. dstate (N) must be 1, 2, 4, 8 or 16.
 * flags: for mamba_scan_fwd, bits 0-15 force the number of time segments the
 * sequence is cut into (0 = the library's choice; results agree to rounding
 * for any value, and the workspace size depends on it); MAMBA_SCAN_ZOH selects
 * the exact zero-order-hold input weight for mamba_scan_fwd, mamba_scan_fwd_init
 * and mamba_state_update; MAMBA_SCAN_SPLIT_STATES (full-sequence entry points
 * only) forces the state-split kernel; all other bits, and bits 0-15 for
 * mamba_state_update, must be 0.
 */
typedef struct mamba_scan_desc {
  int64_t batch;   /* >= 0                                         */
  int64_t seqlen;  /* L >= 0 (must be 1 for mamba_state_update)    */
  int64_t dim;     /* D_inner channels >= 0                        */
  int64_t dstate;  /* N                                            */
  int32_t io_dtype;/* mamba_dtype of x, delta, z, B, C and out     */
  uint32_t flags;  /* see above                                    */
  int64_t ngroups; /* G: groups of channels with their own B and C
                      (0 or 1: one group shared by every channel)  */
} mamba_scan_desc;

/*
 * Groups. With G = ngroups > 1 the channels form G equal consecutive groups
 * and channel d reads the B and C of group d / (dim / G): B and C have the
 * shape (batch, seqlen, G, dstate) (decode: (batch, G, dstate)). One group is
 * the S6 layer ("Mamba and selective state spaces, from first principles",
 * section "Selection": N numbers of B and C per token, shared by every
 * channel); channels grouped to share B and C are the grouping the same page
 * describes in its section "Mamba-2". dim must be a multiple of G; for the
 * full-sequence entry points each group must also be a whole number of
 * 256-channel tiles (dim / G a multiple of 256), else MAMBA_ERR_UNSUPPORTED.
 */

/*
 * Bytes of device workspace mamba_scan_fwd needs for this problem (0 when
 * none). The amount depends on the sizes in `desc` and, unless bits 0-15 of
 * flags fix the number of time segments, on the compute-unit count of the
 * current HIP device (call it with the device current that the scan will run
 * on). Returns 0 for an invalid descriptor as well; mamba_scan_fwd reports
 * the error.
 */
size_t mamba_scan_workspace_size(const mamba_scan_desc *desc);

/*
 * Full-sequence selective scan.
 *   x, delta, z : (batch, seqlen, dim) io dtype. delta is Delta_raw, before the
 *                 bias and the softplus. z may be NULL (no gate).
 *   A           : (dim, dstate) float32.
 *   B, C        : (batch, seqlen, G, dstate) io dtype (G = max(1, ngroups)):
 *                 group g is shared by channels g * dim / G .. (g + 1) * dim / G - 1.
 *   D           : (dim) float32 or NULL (no direct term).
 *   delta_bias  : (dim) float32 or NULL (zero bias).
 *   out         : (batch, seqlen, dim) io dtype, written.
 *   last_state  : (batch, dim, dstate) float32 or NULL; receives h_{L-1}
 *                 (zeros when seqlen == 0).
 *   workspace   : device scratch of at least mamba_scan_workspace_size(desc)
 *                 bytes, 256-byte aligned (may be NULL when that size is 0).
 *                 Its contents on entry are ignored; calls running
 *                 concurrently must not share it.
 * out and last_state must not overlap any input or each other. Alignment:
 * io tensors to their element size, B and C to 4 bytes (2 for bf16 with
 * dstate 1), fp32 tensors to 4 bytes.
 */
mamba_status mamba_scan_fwd(const mamba_scan_desc *desc, const void *x,
                            const void *delta, const float *A, const void *B,
                            const void *C, const float *D, const void *z,
                            const float *delta_bias, void *out,
                            float *last_state, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * mamba_scan_fwd from a given initial state instead of zeros: the state
 * before the first step is h0 ("State space models and Mamba", "A worked
 * example" and the convolution view: the state carries everything earlier
 * input contributed, so a sequence scanned in pieces, each piece starting from
 * the previous piece's final state, gives the result of one scan over the
 * whole sequence).
 *   h0 : (batch, dim, dstate) float32, 4-byte aligned, or NULL (zeros, the
 *        same as mamba_scan_fwd). Read only; it must not overlap out,
 *        last_state or the workspace (so one call's last_state cannot be its
 *        own h0: pass a copy). With seqlen == 0, last_state receives h0.
 * All other arguments, sizes, workspace and errors as mamba_scan_fwd.
 */
mamba_status mamba_scan_fwd_init(const mamba_scan_desc *desc, const void *x,
                                 const void *delta, const float *A, const void *B,
                                 const void *C, const float *D, const void *z,
                                 const float *delta_bias, const float *h0,
                                 void *out, float *last_state, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * One decode token for every sequence, against a resident state
 * (desc->seqlen must be 1).
 *   state       : (batch, dim, dstate) float32, read and overwritten in place
 *                 with the state after this token.
 *   x, delta, z : (batch, dim) io dtype (z may be NULL).
 *   B, C        : (batch, G, dstate) io dtype.
 *   A, D, delta_bias : as in mamba_scan_fwd.
 *   out         : (batch, dim) io dtype, written; must not overlap any input.
 */
mamba_status mamba_state_update(const mamba_scan_desc *desc, float *state,
                                const void *x, const void *delta,
                                const float *A, const void *B, const void *C,
                                const float *D, const void *z,
                                const float *delta_bias, void *out,
                                void *stream);

/*
 * Strided token tensors. A caller whose x, delta, z, out, B or C are column
 * slices of wider row-major tensors (x and z as the two halves of an input
 * projection's output rows, B and C as slices of another projection's rows:
 * "Mamba and selective state spaces, from first principles", section "The
 * Mamba block", and section "Selection" for B_t, C_t computed per token from
 * x_t) passes the row strides instead of copying. A row is one time step of
 * one batch row for mamba_scan_fwd_strided (batch row b's first row is row
 * b * seqlen, so that batch row b starts b * seqlen * stride elements in) and
 * one batch row for mamba_state_update_strided. Strides count elements of
 * the io dtype; 0 means contiguous rows (dim for x, delta, z, out;
 * G * dstate for B and C). Elements within a row stay contiguous; B and C
 * share one stride. A stride below its row length returns
 * MAMBA_ERR_INVALID_ARG, one above 2^26 MAMBA_ERR_UNSUPPORTED. Overlap checks
 * use each tensor's span (first to last element): out may not interleave
 * with an input's rows. Inputs may share memory (x and z interleaved in one
 * buffer are fine). The direct global-to-LDS copy path is used when every
 * row of x, delta, z and out starts 16- (or 4-) byte aligned; otherwise the
 * register-staged path is taken, with the same results.
 */
typedef struct mamba_scan_strides {
  int64_t x, delta, z, out; /* elements between consecutive rows, or 0 */
  int64_t bc;               /* B and C, or 0                          */
} mamba_scan_strides;

/* Workspace of mamba_scan_fwd_strided (the segment plan keeps every in-segment
 * byte offset within 31 bits, so the widest stride can change it). strides
 * may be NULL (then it equals mamba_scan_workspace_size). 0 for an invalid
 * descriptor or stride. */
size_t mamba_scan_workspace_size_strided(const mamba_scan_desc *desc,
                                         const mamba_scan_strides *strides);

/* mamba_scan_fwd_init with strided token tensors (strides may be NULL: all
 * contiguous). Same semantics, conventions and results as mamba_scan_fwd_init;
 * workspace sized by mamba_scan_workspace_size_strided. */
mamba_status mamba_scan_fwd_strided(const mamba_scan_desc *desc,
                                    const mamba_scan_strides *strides,
                                    const void *x, const void *delta,
                                    const float *A, const void *B, const void *C,
                                    const float *D, const void *z,
                                    const float *delta_bias, const float *h0,
                                    void *out, float *last_state,
                                    void *workspace, size_t workspace_bytes,
                                    void *stream);

/* mamba_state_update with strided token tensors (strides may be NULL): row b
 * of x, delta, z, out starts b * stride elements in; B and C likewise with
 * stride bc. The state stays contiguous (batch, dim, dstate). */
mamba_status mamba_state_update_strided(const mamba_scan_desc *desc,
                                        const mamba_scan_strides *strides,
                                        float *state, const void *x,
                                        const void *delta, const float *A,
                                        const void *B, const void *C,
                                        const float *D, const void *z,
                                        const float *delta_bias, void *out,
                                        void *stream);

/*
 * mamba_scan_fwd_init for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It takes no workspace argument and allocates nothing (no
 * hipMalloc, hipFree or allocating library call): the time segments' end
 * states, Delta sums and tile flags go to a fixed array of
 * MAMBA_SCAN_NOALLOC_SCRATCH_BYTES inside the library, one per GPU the library
 * runs on, held until the process ends. Its device address is looked up on
 * the first call on each device (that call may load the library's code
 * object onto the device; the caller may make one small call during
 * set-up).
 *  - Every call on a GPU shares that GPU's array: calls that overlap in time
 *    on one GPU (different streams, without ordering between them) race and
 *    give wrong results; order them on one stream or with events. Calls on
 *    different GPUs are independent.
 *  - Nothing needs clearing: every word a call reads from the array is
 *    written earlier in the same call, in stream order.
 *  - The library's own segment plan needs at most about 36 MB on a 256-CU
 *    device; a plan that needs more than the array holds (a large forced
 *    segment count in flags bits 0-15, or very long sequences whose byte
 *    offsets force extra segments) returns MAMBA_ERR_UNSUPPORTED before any
 *    HIP call, with the sizes in mamba_last_error(). MAMBA_ERR_HIP if the
 *    array's address cannot be obtained.
 * All other arguments, semantics, validation and results are those of
 * mamba_scan_fwd_init (h0 may be NULL: zeros).
 */
#define MAMBA_SCAN_NOALLOC_SCRATCH_BYTES (48u << 20)
mamba_status mamba_scan_fwd_noalloc(const mamba_scan_desc *desc, const void *x,
                                    const void *delta, const float *A,
                                    const void *B, const void *C, const float *D,
                                    const void *z, const float *delta_bias,
                                    const float *h0, void *out,
                                    float *last_state, void *stream);

/* Static name of a status code ("MAMBA_OK", ...). */
const char *mamba_status_string(int status);

/* Detail for the last non-OK status returned on this thread ("" if none). */
const char *mamba_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SCAN_H */
