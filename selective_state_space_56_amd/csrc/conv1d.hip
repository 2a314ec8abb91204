// Causal depthwise convolution of width W (1..4) followed by SiLU: the
// front-end of the SSM branch ("Mamba and selective state spaces, from first
// principles", section "The Mamba block": a causal depthwise convolution of
// width 4, then SiLU, then the selective SSM), over full sequences and as the
// one-token decode update.
//
//   v_t = bias[d] + sum_{j<W} weight[d, j] * xin[t - (W-1) + j, d]
//   out[t, d] = silu(v_t)
// The inputs before t = 0 come from the caller's state (the last W - 1 inputs
// of an earlier piece, oldest first), or are zero. The state after the
// sequence is its last W - 1 inputs.
//
// Streaming and bound by HBM (2 bytes read and 2 written per bf16 element):
// each thread owns 8 or 16 contiguous bytes of channels (4 bf16, or 4 fp32)
// of one batch row for a chunk of time steps, keeps the previous W - 1 inputs in
// registers (each input is read once, plus a W - 1 step halo per chunk), and
// moves its whole piece per load and store. Shapes whose rows are not whole
// pieces use one channel per thread. The one-token update moves 16-byte
// pieces (8 bf16 or 4 fp32).
#include "conv.h"
#include "device_math.h"

namespace mscan {

namespace {

constexpr int kConvThreads = 64;   // one wave per workgroup
constexpr int kConvChunk = 64;     // time steps per thread
constexpr int kGroup = 8;          // steps whose input loads are in flight together
constexpr int kUpdateThreads = 256;  // decode update: threads (channel groups) per workgroup
constexpr int kUpdateRows = 16;      // decode update: batch rows per thread

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// V consecutive io values <-> fp32
template <class IO, int V>
struct Vec;
template <>
struct Vec<Bf16Io, 8> {
  using raw_t = u32x4;
  static __device__ __forceinline__ raw_t load_raw(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
  }
  static __device__ __forceinline__ void widen(const raw_t& w, float (&f)[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = __uint_as_float(w[k] << 16);
      f[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void load(const void* p, float (&f)[8]) { widen(load_raw(p), f); }
  static __device__ __forceinline__ void store(void* p, const float (&f)[8]) {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = static_cast<uint32_t>(Bf16Io::from_f32(f[2 * k])) |
             (static_cast<uint32_t>(Bf16Io::from_f32(f[2 * k + 1])) << 16);
    *reinterpret_cast<u32x4*>(p) = w;
  }
};
// 4 bf16 in 8 bytes: the full-sequence kernel's piece for bf16 (see dispatch_vec)
template <>
struct Vec<Bf16Io, 4> {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  using raw_t = u32x2;
  static __device__ __forceinline__ raw_t load_raw(const void* p) {
    return *reinterpret_cast<const u32x2*>(p);
  }
  static __device__ __forceinline__ void widen(const raw_t& w, float (&f)[4]) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      f[2 * k] = __uint_as_float(w[k] << 16);
      f[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void load(const void* p, float (&f)[4]) { widen(load_raw(p), f); }
  static __device__ __forceinline__ void store(void* p, const float (&f)[4]) {
    u32x2 w;
#pragma unroll
    for (int k = 0; k < 2; ++k)
      w[k] = static_cast<uint32_t>(Bf16Io::from_f32(f[2 * k])) |
             (static_cast<uint32_t>(Bf16Io::from_f32(f[2 * k + 1])) << 16);
    *reinterpret_cast<u32x2*>(p) = w;
  }
};
template <>
struct Vec<F32Io, 4> {
  using raw_t = float4;
  static __device__ __forceinline__ raw_t load_raw(const void* p) {
    return *reinterpret_cast<const float4*>(p);
  }
  static __device__ __forceinline__ void widen(const raw_t& v, float (&f)[4]) {
    f[0] = v.x;
    f[1] = v.y;
    f[2] = v.z;
    f[3] = v.w;
  }
  static __device__ __forceinline__ void load(const void* p, float (&f)[4]) { widen(load_raw(p), f); }
  static __device__ __forceinline__ void store(void* p, const float (&f)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  }
};
template <class IO>
struct Vec<IO, 1> {
  using raw_t = typename IO::raw;
  static __device__ __forceinline__ raw_t load_raw(const void* p) {
    return *static_cast<const typename IO::raw*>(p);
  }
  static __device__ __forceinline__ void widen(const raw_t& v, float (&f)[1]) { f[0] = IO::to_f32(v); }
  static __device__ __forceinline__ void load(const void* p, float (&f)[1]) {
    f[0] = IO::to_f32(*static_cast<const typename IO::raw*>(p));
  }
  static __device__ __forceinline__ void store(void* p, const float (&f)[1]) {
    *static_cast<typename IO::raw*>(p) = IO::from_f32(f[0]);
  }
};

struct ConvArgs {
  const void* xin;
  const float* weight;
  const float* bias;
  const void* state_in;
  void* out;
  void* state_out;
  int64_t batch, seqlen, dim;
  int64_t groups;  // channel groups of V per batch row
  int chunks;      // time chunks per batch row
};

// Grid: x = channel groups (kConvThreads per workgroup), y = time chunk,
// z = batch row. Thread = V channels starting at channel c0 of batch row b.
template <class IO, int W, int V>
__global__ __launch_bounds__(kConvThreads) void conv1d_silu_kernel(ConvArgs a) {
  using raw = typename IO::raw;
  const int64_t grp = static_cast<int64_t>(blockIdx.x) * kConvThreads + threadIdx.x;
  if (grp >= a.groups) return;
  const int64_t b = blockIdx.z;
  const int64_t c0 = grp * V;
  const int nch = static_cast<int>(a.dim - c0 < V ? a.dim - c0 : V);  // V unless V == 1 tail
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kConvChunk;
  const int64_t t1 = t0 + kConvChunk < a.seqlen ? t0 + kConvChunk : a.seqlen;
  const raw* xin = static_cast<const raw*>(a.xin);
  const raw* sin = static_cast<const raw*>(a.state_in);

  float w[W][V], bias[V];
#pragma unroll
  for (int k = 0; k < V; ++k) {
    const int64_t d = c0 + (k < nch ? k : 0);
#pragma unroll
    for (int j = 0; j < W; ++j) w[j][k] = a.weight[d * W + j];
    bias[k] = a.bias ? a.bias[d] : 0.0f;
  }
  // input at time t (t >= -(W-1)) of this thread's channels
  auto input = [&](int64_t t, float (&f)[V]) {
    if (t >= 0) {
      Vec<IO, V>::load(xin + (b * a.seqlen + t) * a.dim + c0, f);
    } else {
#pragma unroll
      for (int k = 0; k < V; ++k)
        f[k] = sin ? IO::to_f32(sin[((b * a.dim + c0 + k) * (W - 1)) + (W - 1) + t]) : 0.0f;
    }
  };
  // win[j] = input at t - (W-1) + j for the next output time t
  float win[W > 1 ? W - 1 : 1][V];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) input(t0 - (W - 1) + j, win[j]);
  raw* out = static_cast<raw*>(a.out);
  // one output step from the window and the current input; the window moves
  auto step = [&](int64_t t, float (&cur)[V]) {
    float y[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
      float v = bias[k];
#pragma unroll
      for (int j = 0; j < W - 1; ++j) v = fmaf(w[j][k], win[j][k], v);
      v = fmaf(w[W - 1][k], cur[k], v);
      y[k] = silu_f(v);
    }
    Vec<IO, V>::store(out + (b * a.seqlen + t) * a.dim + c0, y);
#pragma unroll
    for (int j = 0; j + 1 < W - 1; ++j)
#pragma unroll
      for (int k = 0; k < V; ++k) win[j][k] = win[j + 1][k];
    if (W > 1)
#pragma unroll
      for (int k = 0; k < V; ++k) win[W - 2][k] = cur[k];
  };
  // groups of kGroup steps (t >= 0 here): the next group's loads are in
  // flight, kGroup per lane, while the current group is computed
  using RawV = typename Vec<IO, V>::raw_t;
  auto load_group = [&](int64_t tg, RawV (&r)[kGroup]) {
#pragma unroll
    for (int i = 0; i < kGroup; ++i) r[i] = Vec<IO, V>::load_raw(xin + (b * a.seqlen + tg + i) * a.dim + c0);
  };
  int64_t t = t0;
  if (t + kGroup <= t1) {
    RawV cur[kGroup];
    load_group(t, cur);
    for (; t + kGroup <= t1; t += kGroup) {
      RawV nxt[kGroup];
      const bool more = t + 2 * kGroup <= t1;
      if (more) load_group(t + kGroup, nxt);
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        float f[V];
        Vec<IO, V>::widen(cur[i], f);
        step(t + i, f);
      }
      if (more)
#pragma unroll
        for (int i = 0; i < kGroup; ++i) cur[i] = nxt[i];
    }
  }
  for (; t < t1; ++t) {
    float cur[V];
    input(t, cur);
    step(t, cur);
  }
  // the state after the sequence: its last W - 1 inputs (written once, by the
  // last time chunk)
  if (a.state_out && W > 1 && static_cast<int>(blockIdx.y) == a.chunks - 1) {
    raw* so = static_cast<raw*>(a.state_out);
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
      float f[V];
      input(a.seqlen - (W - 1) + j, f);
#pragma unroll
      for (int k = 0; k < V; ++k)
        if (k < nch) so[(b * a.dim + c0 + k) * (W - 1) + j] = IO::from_f32(f[k]);
    }
  }
}

// One token: out = silu(bias + sum_{j<W-1} w[j] state[j] + w[W-1] x), then the
// state shifts by one and takes x. Grid: x = channel groups of V
// (kUpdateThreads per workgroup), y = runs of kUpdateRows batch rows; each
// thread loads its V channels' taps and bias once and applies them to every
// batch row of its run. Its V channels' states in one row are V * (W - 1)
// contiguous values, moved as W - 1 16-byte pieces when V > 1.
template <class IO, int W, int V>
__global__ __launch_bounds__(kUpdateThreads) void conv1d_update_kernel(ConvArgs a) {
  using raw = typename IO::raw;
  constexpr int kS = W > 1 ? W - 1 : 1;
  const int64_t grp = static_cast<int64_t>(blockIdx.x) * kUpdateThreads + threadIdx.x;
  if (grp >= a.groups) return;
  const int64_t c0 = grp * V;  // V > 1 only when every row is whole groups
  float w[W][V], bias[V];
#pragma unroll
  for (int k = 0; k < V; ++k) {
#pragma unroll
    for (int j = 0; j < W; ++j) w[j][k] = a.weight[(c0 + k) * W + j];
    bias[k] = a.bias ? a.bias[c0 + k] : 0.0f;
  }
  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * kUpdateRows;
  const int64_t b1 = b0 + kUpdateRows < a.batch ? b0 + kUpdateRows : a.batch;
  for (int64_t b = b0; b < b1; ++b) {
    float x[V], y[V], sv[V * kS];
    Vec<IO, V>::load(static_cast<const raw*>(a.xin) + b * a.dim + c0, x);
    raw* st = W > 1 ? static_cast<raw*>(a.state_out) + (b * a.dim + c0) * (W - 1) : nullptr;
    if constexpr (W > 1) {
      if constexpr (V > 1) {
#pragma unroll
        for (int q = 0; q < W - 1; ++q) {
          float f[V];
          Vec<IO, V>::load(st + q * V, f);
#pragma unroll
          for (int k = 0; k < V; ++k) sv[q * V + k] = f[k];
        }
      } else {
#pragma unroll
        for (int j = 0; j < W - 1; ++j) sv[j] = IO::to_f32(st[j]);
      }
    }
#pragma unroll
    for (int k = 0; k < V; ++k) {
      float v = bias[k];
#pragma unroll
      for (int j = 0; j < W - 1; ++j) v = fmaf(w[j][k], sv[k * kS + j], v);
      v = fmaf(w[W - 1][k], x[k], v);
      y[k] = silu_f(v);
    }
    Vec<IO, V>::store(static_cast<raw*>(a.out) + b * a.dim + c0, y);
    if constexpr (W > 1) {
      // shift: each channel's values move one place towards the oldest; x enters
      float ns[V * kS];
#pragma unroll
      for (int k = 0; k < V; ++k) {
#pragma unroll
        for (int j = 0; j + 1 < W - 1; ++j) ns[k * kS + j] = sv[k * kS + j + 1];
        ns[k * kS + W - 2] = x[k];
      }
      if constexpr (V > 1) {
#pragma unroll
        for (int q = 0; q < W - 1; ++q) {
          float f[V];
#pragma unroll
          for (int k = 0; k < V; ++k) f[k] = ns[q * V + k];
          Vec<IO, V>::store(st + q * V, f);
        }
      } else {
#pragma unroll
        for (int j = 0; j < W - 1; ++j) st[j] = IO::from_f32(ns[j]);
      }
    }
  }
}

template <class IO, int W, int V>
hipError_t launch_conv(const ConvProblem& p, bool update, hipStream_t stream) {
  ConvArgs a;
  a.xin = p.xin;
  a.weight = p.weight;
  a.bias = p.bias;
  a.state_in = p.state_in;
  a.out = p.out;
  a.state_out = update ? p.state : p.state_out;
  a.batch = p.batch;
  a.seqlen = update ? 1 : p.seqlen;
  a.dim = p.dim;
  a.groups = (p.dim + V - 1) / V;
  a.chunks = update ? 1
                    : static_cast<int>(p.seqlen > 0 ? (p.seqlen + kConvChunk - 1) / kConvChunk : 1);
  if (update) {
    const dim3 ugrid(static_cast<unsigned>((a.groups + kUpdateThreads - 1) / kUpdateThreads),
                     static_cast<unsigned>((p.batch + kUpdateRows - 1) / kUpdateRows));
    hipLaunchKernelGGL((conv1d_update_kernel<IO, W, V>), ugrid, dim3(kUpdateThreads), 0, stream, a);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>((a.groups + kConvThreads - 1) / kConvThreads),
                  static_cast<unsigned>(a.chunks), static_cast<unsigned>(p.batch));
  hipLaunchKernelGGL((conv1d_silu_kernel<IO, W, V>), grid, dim3(kConvThreads), 0, stream, a);
  return hipGetLastError();
}

template <class IO, int W>
hipError_t dispatch_vec(const ConvProblem& p, bool update, hipStream_t s) {
  constexpr int eb = sizeof(typename IO::raw);
  constexpr int V = 16 / eb;
  // bf16 full sequences: 8-byte pieces (4 channels per thread). The kernel
  // then holds 88 vector registers instead of 160 and runs five waves per SIMD
  // (the 16-byte form: three, with 2.5 waves' worth of workgroups): on
  // 8 x 2048 x 5120 72.6-73.4 against 77.5-78.0 us per call in interleaved
  // timing, where a plain copy of the same bytes in this access pattern takes
  // about 58 us. 32 or 128 steps per thread, or 4 loads in flight, were slower.
  if constexpr (eb == 2) {
    if (!update) {
      const auto a8 = [](const void* q) { return q == nullptr || reinterpret_cast<uintptr_t>(q) % 8 == 0; };
      if ((p.dim * eb) % 8 == 0 && a8(p.xin) && a8(p.out))
        return launch_conv<IO, W, 4>(p, update, s);
      return launch_conv<IO, W, 1>(p, update, s);
    }
  }
  const auto a16 = [](const void* q) { return q == nullptr || reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  // 16-byte pieces: every row a whole number of them, tensors 16-byte aligned
  // (the update's state too: it is moved in 16-byte pieces)
  if ((p.dim * eb) % 16 == 0 && a16(p.xin) && a16(p.out) && a16(p.state))
    return launch_conv<IO, W, V>(p, update, s);
  return launch_conv<IO, W, 1>(p, update, s);
}

template <class IO>
hipError_t dispatch_width(const ConvProblem& p, bool update, hipStream_t s) {
  switch (p.width) {
    case 1: return dispatch_vec<IO, 1>(p, update, s);
    case 2: return dispatch_vec<IO, 2>(p, update, s);
    case 3: return dispatch_vec<IO, 3>(p, update, s);
    case 4: return dispatch_vec<IO, 4>(p, update, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_conv1d(const ConvProblem& p, hipStream_t stream) {
  if (p.batch == 0 || p.dim == 0) return hipSuccess;
  if (p.seqlen == 0 && (p.state_out == nullptr || p.width == 1)) return hipSuccess;
  if (p.io == kIoBf16) return dispatch_width<Bf16Io>(p, false, stream);
  return dispatch_width<F32Io>(p, false, stream);
}

hipError_t launch_conv1d_update(const ConvProblem& p, hipStream_t stream) {
  if (p.batch == 0 || p.dim == 0) return hipSuccess;
  if (p.io == kIoBf16) return dispatch_width<Bf16Io>(p, true, stream);
  return dispatch_width<F32Io>(p, true, stream);
}

}  // namespace mscan
