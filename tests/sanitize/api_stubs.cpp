// Host-only stand-ins for the library's internal launch and planning
// functions (kernels.h, conv.h, scan_split.h), so that the C ABI layer
// (api.cpp) can be built with AddressSanitizer / UndefinedBehaviorSanitizer
// and driven without a GPU: every validation path runs for real, and a call
// that passes validation lands here, which counts it and touches nothing.
// Test infrastructure only.
#include <hip/hip_runtime_api.h>

#include "conv.h"
#include "kernels.h"
#include "scan_split.h"

int g_stub_launches = 0;

extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

namespace mscan {

// The library's real plan cuts time into segments by the device's size; here
// one segment unless a count is forced (the workspace formula of the real
// plan for that count), which is all the validation code looks at.
ScanPlan plan_scan(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int forced_segments,
                   int64_t) {
  ScanPlan p{seqlen, 1, 0};
  if (batch * dim <= 0 || seqlen <= 0) return p;
  int64_t segs = forced_segments > 0 ? forced_segments : 1;
  if (segs > seqlen) segs = seqlen;
  p.segments = static_cast<int>(segs);
  p.seg_len = (seqlen + segs - 1) / segs;
  if (segs > 1)
    p.workspace_bytes = (static_cast<size_t>(segs - 1) * static_cast<size_t>(batch * dim) *
                             static_cast<size_t>(dstate + 1) * 4 + 255) / 256 * 256;
  return p;
}

ScanBwdPlan plan_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int forced) {
  ScanBwdPlan p{};
  p.seg = plan_scan(batch, seqlen, dim, dstate, forced, dim);
  p.workspace_bytes = batch * dim * seqlen > 0 ? 4096 : 0;
  return p;
}

size_t ssd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t ngroups) {
  return static_cast<size_t>(batch * nheads * ((seqlen + 255) / 256) + ngroups) * 256;
}

bool scan_split_fits(int64_t dstate, int64_t row_elems, int io) {
  return dstate == 16 && row_elems * (io == kIoBf16 ? 2 : 4) * 9 < (int64_t(1) << 31);
}

hipError_t scan_scratch(void** ptr) {
  *ptr = reinterpret_cast<void*>(uintptr_t(0x7E0000000000));
  return hipSuccess;
}

int device_cu_count() { return 256; }

hipError_t launch_scan_fwd(const ScanProblem&, const ScanPlan&, void*, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
hipError_t launch_scan_split(const ScanProblem&, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
hipError_t launch_scan_bwd(const ScanBwdProblem&, const ScanBwdPlan&, void*, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
hipError_t launch_state_update(const DecodeProblem&, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
hipError_t launch_ssd_fwd(const SsdProblem&, void*, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
hipError_t launch_conv1d(const ConvProblem&, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
hipError_t launch_conv1d_update(const ConvProblem&, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}

}  // namespace mscan
