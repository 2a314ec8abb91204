// Full-sequence selective scan (S6) on gfx950.
//
// One lane owns one (batch, channel) row and keeps its N fp32 states in
// registers for the whole time range it covers; every step is fused: softplus
// front-end, N decays exp(Delta A_n), first-order Bbar x = Delta B x, state
// update, C read-out, D skip and silu(z) gate, one store of y
// ("Mamba and selective state spaces, from first principles", section
// "The hardware-aware scan": only the (batch, L, D) output leaves the chip).
//
// Rows are independent (one SSM per channel), so lanes need no communication.
// When there are too few rows to fill the GPU, the sequence is cut into time
// segments that run in parallel and are stitched with the associative
// affine-pair combine (a1, b1) then (a2, b2) = (a2 a1, a2 b1 + b2) (same page,
// same section), in three launches:
//   1. aggregate: each segment but the last scans from h = 0 and records its
//      end state and the sum of its Delta (the segment's decay for state n is
//      exp(A_n * sum Delta), a product of per-step decays);
//   2. combine: a sequential fold over segments per (row, n) turns the
//      aggregates into each segment's carry-in state;
//   3. output: every segment re-scans from its carry-in and writes y (and the
//      last one the final state).
#include "device_math.h"
#include "kernels.h"

namespace mscan {

namespace {

constexpr int kBlock = 256;   // 4 wave64s, one lane per row
constexpr int kChunk = 8;     // time steps whose inputs are loaded together

struct ScanKernelArgs {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  void* out;
  float* last_state;
  float* ws_h;   // (segments - 1, batch, dim, N)
  float* ws_s;   // (segments - 1, batch, dim)
  int64_t seqlen;
  int64_t dim;
  int64_t rows;  // batch * dim
  int64_t seg_len;
  int segments;
  unsigned tiles;  // channel tiles of kBlock per batch row
};

// Grid: x = batch * channel tiles, y = time segment.
// MODE kOutput: scan segment blockIdx.y from its carry-in, write y (and the
//               final state after the last segment).
// MODE kAggregate: scan segment blockIdx.y from zero, write its end state and
//               its sum of Delta to the workspace.
enum Mode { kOutput = 0, kAggregate = 1 };

template <int N, class IO, int MODE>
__global__ __launch_bounds__(kBlock) void scan_segment_kernel(ScanKernelArgs a) {
  using raw = typename IO::raw;
  const int64_t b = blockIdx.x / a.tiles;
  const int64_t d = static_cast<int64_t>(blockIdx.x % a.tiles) * kBlock + threadIdx.x;
  const int s = blockIdx.y;
  if (d >= a.dim) return;
  const int64_t t_begin = static_cast<int64_t>(s) * a.seg_len;
  const int64_t t_end = t_begin + a.seg_len < a.seqlen ? t_begin + a.seg_len : a.seqlen;
  const int64_t row = b * a.dim + d;
  const int64_t dim = a.dim;

  float A2[N];
#pragma unroll
  for (int n = 0; n < N; ++n) A2[n] = a.A[d * N + n] * kLog2e;
  const float Dd = (MODE == kOutput && a.D) ? a.D[d] : 0.0f;
  const float bias = a.bias ? a.bias[d] : 0.0f;

  float h[N];
  if (MODE == kOutput && s > 0) {
    const float* hin = a.ws_h + (static_cast<int64_t>(s - 1) * a.rows + row) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = hin[n];
  } else {
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = 0.0f;
  }

  const int64_t base = b * a.seqlen * dim + d;
  const raw* xp = static_cast<const raw*>(a.x) + base;
  const raw* dp = static_cast<const raw*>(a.delta) + base;
  const raw* zp = a.z ? static_cast<const raw*>(a.z) + base : nullptr;
  raw* op = static_cast<raw*>(a.out) + base;
  const raw* Bp = static_cast<const raw*>(a.B) + b * a.seqlen * N;
  const raw* Cp = static_cast<const raw*>(a.C) + b * a.seqlen * N;

  float S = 0.0f, S_c = 0.0f;  // Kahan-compensated sum of Delta (aggregate mode)

  for (int64_t t0 = t_begin; t0 < t_end; t0 += kChunk) {
    raw xv[kChunk], dv[kChunk], zv[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const int64_t t = t0 + j;
      if (t < t_end) {
        xv[j] = xp[t * dim];
        dv[j] = dp[t * dim];
        if (MODE == kOutput && zp) zv[j] = zp[t * dim];
      }
    }
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const int64_t t = t0 + j;
      if (t < t_end) {
        const float xf = IO::to_f32(xv[j]);
        const float Delta = softplus_f(IO::to_f32(dv[j]) + bias);
        const float dx = Delta * xf;
        const raw* Bt = Bp + t * N;
        const raw* Ct = Cp + t * N;
        float y = 0.0f;
#pragma unroll
        for (int n = 0; n < N; ++n) {
          const float abar = hw_exp2(Delta * A2[n]);
          h[n] = fmaf(abar, h[n], dx * IO::to_f32(Bt[n]));
          if (MODE == kOutput) y = fmaf(IO::to_f32(Ct[n]), h[n], y);
        }
        if (MODE == kOutput) {
          y = fmaf(Dd, xf, y);
          if (zp) y *= silu_f(IO::to_f32(zv[j]));
          op[t * dim] = IO::from_f32(y);
        } else {
          const float v = Delta - S_c;
          const float tsum = S + v;
          S_c = (tsum - S) - v;
          S = tsum;
        }
      }
    }
  }

  if (MODE == kOutput) {
    if (s == a.segments - 1 && a.last_state) {
      float* ls = a.last_state + row * N;
#pragma unroll
      for (int n = 0; n < N; ++n) ls[n] = h[n];
    }
  } else {
    float* agg = a.ws_h + (static_cast<int64_t>(s) * a.rows + row) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) agg[n] = h[n];
    a.ws_s[static_cast<int64_t>(s) * a.rows + row] = S;
  }
}

// Fold the segment aggregates of one (row, n) in time order. Slot k of the
// workspace holds segment k's (end state from zero, sum of Delta) on entry and
// the carry-in state of segment k + 1 on exit.
template <int N>
__global__ __launch_bounds__(kBlock) void scan_combine_kernel(const float* A, float* ws_h,
                                                              const float* ws_s, int64_t rows,
                                                              int64_t dim, int segments) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= rows * N) return;
  const int64_t row = i / N;
  const int n = static_cast<int>(i % N);
  const int64_t d = row % dim;
  const float a2 = A[d * N + n] * kLog2e;
  float h = 0.0f;
  for (int k = 0; k < segments - 1; ++k) {
    float* slot = ws_h + static_cast<int64_t>(k) * rows * N + i;
    const float decay = hw_exp2(a2 * ws_s[static_cast<int64_t>(k) * rows + row]);
    h = fmaf(decay, h, *slot);
    *slot = h;
  }
}

__global__ __launch_bounds__(kBlock) void fill_zero_kernel(float* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

template <int N, class IO>
hipError_t launch_typed(const ScanProblem& p, const ScanPlan& plan, void* workspace,
                        hipStream_t stream) {
  ScanKernelArgs a;
  a.x = p.x;
  a.delta = p.delta;
  a.A = p.A;
  a.B = p.B;
  a.C = p.C;
  a.D = p.D;
  a.z = p.z;
  a.bias = p.bias;
  a.out = p.out;
  a.last_state = p.last_state;
  a.seqlen = p.seqlen;
  a.dim = p.dim;
  a.rows = p.batch * p.dim;
  a.seg_len = plan.seg_len;
  a.segments = plan.segments;
  a.ws_h = static_cast<float*>(workspace);
  a.tiles = static_cast<unsigned>((p.dim + kBlock - 1) / kBlock);
  a.ws_s = a.ws_h ? a.ws_h + static_cast<int64_t>(plan.segments - 1) * a.rows * N : nullptr;

  const dim3 block(kBlock);
  const unsigned blocks = a.tiles * static_cast<unsigned>(p.batch);
  if (plan.segments > 1) {
    const dim3 grid_agg(blocks, plan.segments - 1);
    hipLaunchKernelGGL((scan_segment_kernel<N, IO, kAggregate>), grid_agg, block, 0, stream, a);
    const int64_t work = a.rows * N;
    const dim3 grid_c(static_cast<unsigned>((work + kBlock - 1) / kBlock));
    hipLaunchKernelGGL((scan_combine_kernel<N>), grid_c, block, 0, stream, p.A, a.ws_h, a.ws_s,
                       a.rows, p.dim, plan.segments);
  }
  const dim3 grid(blocks, plan.segments);
  hipLaunchKernelGGL((scan_segment_kernel<N, IO, kOutput>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <class IO>
hipError_t dispatch_n(const ScanProblem& p, const ScanPlan& plan, void* ws, hipStream_t st) {
  switch (p.dstate) {
    case 1: return launch_typed<1, IO>(p, plan, ws, st);
    case 2: return launch_typed<2, IO>(p, plan, ws, st);
    case 4: return launch_typed<4, IO>(p, plan, ws, st);
    case 8: return launch_typed<8, IO>(p, plan, ws, st);
    case 16: return launch_typed<16, IO>(p, plan, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

ScanPlan plan_scan(int64_t batch, int64_t seqlen, int64_t dim, int dstate, int forced_segments) {
  ScanPlan plan{seqlen, 1, 0};
  const int64_t rows = batch * dim;
  if (rows <= 0 || seqlen <= 0) return plan;
  int64_t segs;
  if (forced_segments > 0) {
    segs = forced_segments;
  } else {
    // Aim for about two wave64s per SIMD (256 CUs x 4 SIMDs) when the rows
    // alone cannot provide them; keep segments at least 256 steps long.
    const int64_t target_lanes = 256LL * 4 * 64 * 2;
    segs = (target_lanes + rows - 1) / rows;
    const int64_t max_by_len = seqlen / 256 > 0 ? seqlen / 256 : 1;
    if (segs > max_by_len) segs = max_by_len;
  }
  if (segs > 4096) segs = 4096;
  if (segs > seqlen) segs = seqlen;
  if (segs < 1) segs = 1;
  int64_t seg_len = (seqlen + segs - 1) / segs;
  seg_len = (seg_len + kChunk - 1) / kChunk * kChunk;
  segs = (seqlen + seg_len - 1) / seg_len;
  plan.seg_len = seg_len;
  plan.segments = static_cast<int>(segs);
  if (segs > 1) {
    const size_t floats = static_cast<size_t>(segs - 1) * static_cast<size_t>(rows) *
                          static_cast<size_t>(dstate + 1);
    plan.workspace_bytes = (floats * sizeof(float) + 255) / 256 * 256;
  }
  return plan;
}

hipError_t launch_scan_fwd(const ScanProblem& p, const ScanPlan& plan, void* workspace,
                           hipStream_t stream) {
  if (p.batch == 0 || p.dim == 0) return hipSuccess;
  if (p.seqlen == 0) {
    if (p.last_state) {
      const int64_t n = p.batch * p.dim * p.dstate;
      hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((n + kBlock - 1) / kBlock)),
                         dim3(kBlock), 0, stream, p.last_state, n);
      return hipGetLastError();
    }
    return hipSuccess;
  }
  if (p.io == kIoBf16) return dispatch_n<Bf16Io>(p, plan, workspace, stream);
  return dispatch_n<F32Io>(p, plan, workspace, stream);
}

}  // namespace mscan
