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
};

// Time segmentation of a full-sequence scan: the sequence is cut into
// `segments` pieces of `seg_len` steps (the last may be shorter) that are
// scanned in parallel and stitched by the affine-pair combine.
struct ScanPlan {
  int64_t seg_len;
  int segments;
  size_t workspace_bytes;
};

// forced_segments > 0 overrides the library's choice of time segments.
ScanPlan plan_scan(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int forced_segments);

hipError_t launch_scan_fwd(const ScanProblem& p, const ScanPlan& plan, void* workspace,
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
};

hipError_t launch_state_update(const DecodeProblem& p, hipStream_t stream);

}  // namespace mscan
