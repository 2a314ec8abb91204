// The state-split full-sequence scan (scan_split.hip): each (batch, channel)
// row's 16 states on four lanes, the whole sequence in one pass, no
// workspace. Chosen only on request (MAMBA_SCAN_SPLIT_STATES).
#pragma once

#include "kernels.h"

namespace mscan {

// Whether the state-split scan takes this problem: dstate 16, and every byte
// offset within 9 steps of the widest row (row_elems elements of the io type)
// fits in 31 bits. (The first-order input weight only: the caller rules out
// the exact zero-order hold.)
bool scan_split_fits(int64_t dstate, int64_t row_elems, int io);

// Launch it for p (seqlen > 0, dstate 16, !p.zoh) on `stream`.
hipError_t launch_scan_split(const ScanProblem& p, hipStream_t stream);

}  // namespace mscan
