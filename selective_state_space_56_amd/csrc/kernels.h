// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace mscan {

enum Io : int { kIoF32 = 0, kIoBf16 = 1 };

struct ScanProblem {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;      // nullable
  const void* z;       // nullable
  const float* bias;   // nullable
  const float* h0;     // nullable (zeros): state before the first step
  void* out;
  float* last_state;   // nullable
  int64_t batch, seqlen, dim;
  int dstate;
  int io;
  bool zoh;            // exact zero-order-hold input weight instead of Delta
  int64_t ngroups;     // G >= 1: B, C are (batch, seqlen, G, dstate); dim / G a multiple of 256
  // elements between consecutive steps (rows), per tensor: x, Delta_raw, z,
  // out (at least dim) and B, C (at least G * dstate); batch row b starts at
  // b * seqlen * stride
  int64_t sx, sd, sz, so, sbc;
};

// Time segmentation of a full-sequence scan: the sequence is cut into
// `segments` pieces of `seg_len` steps (the last takes the rest: shorter, or
// longer in plans that lengthen it) that are scanned in parallel and stitched
// by the affine-pair combine.
struct ScanPlan {
  int64_t seg_len;
  int segments;
  size_t workspace_bytes;
};

// forced_segments > 0 overrides the library's choice of time segments.
// row_elems: the widest step stride (elements) of the scan's tensors (dim when contiguous)
ScanPlan plan_scan(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int forced_segments,
                   int64_t row_elems);

hipError_t launch_scan_fwd(const ScanProblem& p, const ScanPlan& plan, void* workspace,
                           hipStream_t stream);

// Bytes of the fixed device scratch array of the allocation-free entry point,
// and its device address on the current device (looked up once per device).
constexpr size_t kScanScratchBytes = size_t(48) << 20;
hipError_t scan_scratch(void** ptr);

// The combine launch of launch_scan_fwd on its own: folds segment
// aggregates ws_h[k][rows][dstate] (end state from zero) and ws_s[k][rows]
// (sum of Delta), k < segments - 1, from h0 (or zero) in time order, leaving
// the state that enters segment k + 1 in slot k.
hipError_t launch_scan_combine(const float* A, float* ws_h, const float* ws_s, const float* h0,
                               int64_t rows, int64_t dim, int dstate, int segments,
                               hipStream_t stream);

// Compute units of the current HIP device (256 when it cannot be queried).
int device_cu_count();

// Backward of the full-sequence scan: gradients for dLoss/dy = dout and
// optionally dLoss/d(final state) = dlast. dx, ddelta, dz in the io dtype;
// every other gradient fp32. Nullable: z (no gate), dz, D, bias, h0, dlast,
// dD, dbias, dh0.
struct ScanBwdProblem {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  const float* h0;
  const void* dout;
  const float* dlast;
  void* dx;
  void* ddelta;
  float* dA;
  float* dB;
  float* dC;
  float* dD;
  void* dz;
  float* dbias;
  float* dh0;
  int64_t batch, seqlen, dim;
  int dstate;
  int io;
  int64_t ngroups;     // G >= 1: B, C, dB, dC are (batch, seqlen, G, dstate)
};

// Time segmentation and byte offsets of the backward's workspace regions
// (the forward carries come first).
struct ScanBwdPlan {
  ScanPlan seg;
  size_t adj_off, ck_off, cks_off, pa_off, pdb_off, pbc_off, flags_off;
  size_t workspace_bytes;
};

ScanBwdPlan plan_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int dstate,
                          int forced_segments);

hipError_t launch_scan_bwd(const ScanBwdProblem& p, const ScanBwdPlan& plan, void* workspace,
                           hipStream_t stream);

struct DecodeProblem {
  float* state;
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;      // nullable
  const void* z;       // nullable
  const float* bias;   // nullable
  void* out;
  int64_t batch, dim;
  int dstate;
  int io;
  bool zoh;            // exact zero-order-hold input weight instead of Delta
  int64_t ngroups;     // G >= 1 dividing dim: B, C are (batch, G, dstate)
  // elements between consecutive batch rows, per tensor: x, Delta_raw, z, out
  // (at least dim) and B, C (at least G * dstate)
  int64_t sx, sd, sz, so, sbc;
};

hipError_t launch_state_update(const DecodeProblem& p, hipStream_t stream);

// Mamba-2 SSD layer (bf16 io; headdim 64, dstate 128; chunks of 256 steps).
struct SsdProblem {
  const void* x;        // (batch, seqlen, nheads, 64)
  const void* dt;       // (batch, seqlen, nheads), before bias and softplus
  const float* A;       // (nheads)
  const void* B;        // (batch, seqlen, ngroups, 128)
  const void* C;
  const float* D;       // (nheads), nullable
  const float* dt_bias; // (nheads), nullable
  const float* h0;      // (batch, nheads, 128, 64), nullable
  void* out;            // (batch, seqlen, nheads, 64)
  float* last_state;    // (batch, nheads, 128, 64), nullable
  int64_t batch, seqlen, nheads, ngroups;
};

size_t ssd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t ngroups);
hipError_t launch_ssd_fwd(const SsdProblem& p, void* workspace, hipStream_t stream);

}  // namespace mscan
