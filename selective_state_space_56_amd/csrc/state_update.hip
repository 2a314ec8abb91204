// One-token decode (state update) on gfx950.
//
// Every sequence carries a D x N fp32 state that stays resident in HBM; one
// token advances it by exactly one step of the scan's recurrence and emits
// that step's output (erikxu.me notes "Mamba: Linear-Time Sequence Modeling
// with Selective State Spaces", section "State Space Models": constant work
// per generated token; "Mamba and selective state spaces, from first
// principles", section "A fixed state against a growing cache": decode is
// bound by memory traffic).
//
// The kernel is a single streaming pass over the state: each row's N states
// are split over N / 4 lanes that hold four consecutive states each, so one
// wave64 reads and writes a contiguous run of 64 x 16 bytes with 16-byte
// vector accesses. A thread keeps its channel's parameters (four states' A,
// D, bias) in registers and serves kDecodeRows batch rows in turn, so the
// per-channel parameters are read once per run of rows, not once per row. The
// per-row front-end (softplus, gate) is recomputed by each lane of the row;
// the C read-out is summed across the row's lanes with cross-lane shuffles.
#include "device_math.h"
#include "kernels.h"

namespace mscan {

namespace {

constexpr int kBlock = 256;
constexpr int kDecodeRows = 4;   // batch rows per thread (fewer rows, more workgroups: measured best)
constexpr int kGroupRows = 2;    // rows whose loads are in flight together

struct DecodeKernelArgs {
  float* state;
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* bias;
  void* out;
  int64_t batch;
  int64_t dim;
  int64_t ngroups;    // B and C: (batch, ngroups, N)
  int64_t group_dim;  // channels per group
  // elements between consecutive batch rows: x, Delta_raw, z, out, and B / C
  int64_t sx, sd, sz, so, sbc;
};

// Grid: x = (channel, lane-of-row) pairs, kBlock per workgroup; y = runs of
// kDecodeRows batch rows.
// ZOH: the input term takes the exact zero-order-hold weight instead of Delta.
template <int N, class IO, bool ZOH>
__global__ __launch_bounds__(kBlock) void state_update_kernel(DecodeKernelArgs a) {
  using raw = typename IO::raw;
  constexpr int SPL = N >= 4 ? 4 : N;  // states per lane
  constexpr int LPR = N / SPL;         // lanes per row (1, 2 or 4; a power of 2)
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t d_raw = gid / LPR;
  const int sub = static_cast<int>(gid % LPR);
  const bool active = d_raw < a.dim;
  // Inactive lanes of the last workgroup mirror the last channel so that the
  // cross-lane sum below sees full lane groups; they store nothing.
  const int64_t d = active ? d_raw : a.dim - 1;

  float A2[SPL];
  const float* Ad = a.A + d * N + sub * SPL;
#pragma unroll
  for (int k = 0; k < SPL; ++k) A2[k] = Ad[k] * kLog2e;
  const float bias = a.bias ? a.bias[d] : 0.0f;
  const float Dd = a.D ? a.D[d] : 0.0f;

  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * kDecodeRows;
  const int64_t b1 = b0 + kDecodeRows < a.batch ? b0 + kDecodeRows : a.batch;
  const raw* xp = static_cast<const raw*>(a.x);
  const raw* dp = static_cast<const raw*>(a.delta);
  const raw* zp = static_cast<const raw*>(a.z);
  // Rows are taken kGroupRows at a time: all of a group's loads are issued
  // before its rows are computed and stored (rows past the batch repeat the
  // last row and store nothing).
  for (int64_t g0 = b0; g0 < b1; g0 += kGroupRows) {
    float xf[kGroupRows], draw[kGroupRows], zf[kGroupRows], h[kGroupRows][SPL];
    float Bv[kGroupRows][SPL], Cv[kGroupRows][SPL];
#pragma unroll
    for (int r = 0; r < kGroupRows; ++r) {
      const int64_t b = g0 + r < b1 ? g0 + r : b1 - 1;
      const int64_t row = b * a.dim + d;
      xf[r] = IO::load(xp + b * a.sx + d);
      draw[r] = IO::load(dp + b * a.sd + d);
      zf[r] = a.z ? IO::load(zp + b * a.sz + d) : 0.0f;
      const float* hp = a.state + row * N + sub * SPL;
      if constexpr (SPL == 4) {
        const float4 v = *reinterpret_cast<const float4*>(hp);
        h[r][0] = v.x; h[r][1] = v.y; h[r][2] = v.z; h[r][3] = v.w;
      } else {
#pragma unroll
        for (int k = 0; k < SPL; ++k) h[r][k] = hp[k];
      }
      const int64_t bg = b * a.sbc + d / a.group_dim * N;  // (b, group of d)
      const raw* Bt = static_cast<const raw*>(a.B) + bg + sub * SPL;
      const raw* Ct = static_cast<const raw*>(a.C) + bg + sub * SPL;
#pragma unroll
      for (int k = 0; k < SPL; ++k) {
        Bv[r][k] = IO::load(Bt + k);
        Cv[r][k] = IO::load(Ct + k);
      }
    }
#pragma unroll
    for (int r = 0; r < kGroupRows; ++r) {
      const int64_t b = g0 + r;
      const float Delta = softplus_f(draw[r] + bias);
      const float dx = Delta * xf[r];
      float y = 0.0f;
#pragma unroll
      for (int k = 0; k < SPL; ++k) {
        const float v2 = Delta * A2[k];
        const float abar = hw_exp2(v2);
        const float bx = ZOH ? zoh_gain(v2, abar) * (dx * Bv[r][k]) : dx * Bv[r][k];
        h[r][k] = fmaf(abar, h[r][k], bx);
        y = fmaf(Cv[r][k], h[r][k], y);
      }
#pragma unroll
      for (int off = 1; off < LPR; off <<= 1) y += __shfl_xor(y, off);
      if (active && b < b1) {
        const int64_t row = b * a.dim + d;
        float* hp = a.state + row * N + sub * SPL;
        if constexpr (SPL == 4) {
          *reinterpret_cast<float4*>(hp) = make_float4(h[r][0], h[r][1], h[r][2], h[r][3]);
        } else {
#pragma unroll
          for (int k = 0; k < SPL; ++k) hp[k] = h[r][k];
        }
        if (sub == 0) {
          if (a.D) y = fmaf(Dd, xf[r], y);
          if (a.z) y *= silu_f(zf[r]);
          static_cast<raw*>(a.out)[b * a.so + d] = IO::from_f32(y);
        }
      }
    }
  }
}

template <int N, class IO>
hipError_t launch_typed(const DecodeProblem& p, hipStream_t stream) {
  constexpr int SPL = N >= 4 ? 4 : N;
  constexpr int LPR = N / SPL;
  DecodeKernelArgs a;
  a.state = p.state;
  a.x = p.x;
  a.delta = p.delta;
  a.A = p.A;
  a.B = p.B;
  a.C = p.C;
  a.D = p.D;
  a.z = p.z;
  a.bias = p.bias;
  a.out = p.out;
  a.batch = p.batch;
  a.dim = p.dim;
  a.ngroups = p.ngroups;
  a.group_dim = p.dim / p.ngroups;
  a.sx = p.sx;
  a.sd = p.sd;
  a.sz = p.sz;
  a.so = p.so;
  a.sbc = p.sbc;
  const int64_t threads = p.dim * LPR;
  const dim3 grid(static_cast<unsigned>((threads + kBlock - 1) / kBlock),
                  static_cast<unsigned>((p.batch + kDecodeRows - 1) / kDecodeRows));
  if (p.zoh)
    hipLaunchKernelGGL((state_update_kernel<N, IO, true>), grid, dim3(kBlock), 0, stream, a);
  else
    hipLaunchKernelGGL((state_update_kernel<N, IO, false>), grid, dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

template <class IO>
hipError_t dispatch_n(const DecodeProblem& p, hipStream_t st) {
  switch (p.dstate) {
    case 1: return launch_typed<1, IO>(p, st);
    case 2: return launch_typed<2, IO>(p, st);
    case 4: return launch_typed<4, IO>(p, st);
    case 8: return launch_typed<8, IO>(p, st);
    case 16: return launch_typed<16, IO>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_state_update(const DecodeProblem& p, hipStream_t stream) {
  if (p.batch == 0 || p.dim == 0) return hipSuccess;
  if (p.io == kIoBf16) return dispatch_n<Bf16Io>(p, stream);
  return dispatch_n<F32Io>(p, stream);
}

}  // namespace mscan
