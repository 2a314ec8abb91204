// Internal launch interface for the causal convolution front-end (api.cpp ->
// conv1d.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "kernels.h"

namespace mscan {

struct ConvProblem {
  const void* xin;        // (batch, seqlen, dim) io, or (batch, dim) for the update
  const float* weight;    // (dim, width)
  const float* bias;      // (dim) or null
  const void* state_in;   // (batch, dim, width - 1) io or null (zeros)
  void* out;              // like xin
  void* state_out;        // (batch, dim, width - 1) io or null
  void* state;            // the update's in-place state (batch, dim, width - 1) io
  int64_t batch, seqlen, dim;
  int width;              // 1 .. 4
  int io;
};

hipError_t launch_conv1d(const ConvProblem& p, hipStream_t stream);
hipError_t launch_conv1d_update(const ConvProblem& p, hipStream_t stream);

}  // namespace mscan
