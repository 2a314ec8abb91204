// Backward of the full-sequence selective scan (S6) on gfx950: the gradients
// of a loss with respect to x, Delta_raw, A, B, C, D, z, the Delta bias and the
// initial state, given dLoss/dy and optionally dLoss/d(final state).
//
// The states are not kept from the forward pass; they are recomputed here from
// the inputs (erikxu.me notes "Mamba: Linear-Time Sequence Modeling with
// Selective State Spaces", section "GPU Memory Hierarchy"; "Mamba and
// selective state spaces, from first principles", section "The hardware-aware
// scan").
//
// Reverse-mode differentiation of h_t = abar_t h_{t-1} + Delta_t B_t x_t,
// abar_t = exp(Delta_t A), y_t = (C_t . h_t + D x_t) silu(z_t), per row (b, d)
// and state n:
//   ds_t     = dy_t silu(z_t)                        gradient of the pre-gate output
//   lam_t    = C_t ds_t + abar_{t+1} lam_{t+1},       lam_{L-1} = C_{L-1} ds_{L-1} + dlast
//   dA      += Delta_t lam_t abar_t h_{t-1}
//   dDelta_t = sum_n lam_t,n (A_n abar_t,n h_{t-1},n + B_t,n x_t)
//   dx_t     = D ds_t + Delta_t sum_n lam_t,n B_t,n
//   dB_t,n  += lam_t,n Delta_t x_t                   (summed over channels)
//   dC_t,n  += ds_t h_t,n                            (summed over channels)
//   dD      += ds_t x_t,   dz_t = dy_t (C_t . h_t + D x_t) silu'(z_t)
//   dDelta_raw_t = dDelta_t sigmoid(Delta_raw_t + bias),   dbias += dDelta_raw_t
//   dh0      = abar_0 lam_0
//
// Time is cut into segments as in the forward scan. Launches, in order:
//   0. state checkpoints: every segment scans forward from zero and stores its
//      state and Delta sum at every chunk start, and its end state; the
//      forward scan's combine turns the end states into carry-in states;
//   1. adjoint aggregate: every segment but the first runs the adjoint
//      recurrence backwards from zero and records abar at its first step times
//      the adjoint there, and its sum of Delta;
//   2. adjoint fold: a reverse fold over segments per (row, n), from dlast,
//      gives the adjoint that enters each segment from later time (the affine
//      pair combine of the forward scan run backwards: over a segment the
//      adjoint decays by exp(A_n sum Delta));
//   3. main: each segment walks its chunks of kChunk steps backwards: it
//      forms the state before the chunk from the checkpoint and the carry-in,
//      recomputes the chunk's states into registers and steps the adjoint back
//      through them, writing dx, dDelta_raw and dz and accumulating dA, dD and
//      dbias per lane; dB and dC of a step are summed over the wave's channels
//      with cross-lane exchanges, then over the workgroup's waves in LDS, and
//      stored per channel tile;
//   4. sums of the per-(segment, batch row) dA, dD, dbias partials and of the
//      per-tile dB, dC partials.
#include "device_math.h"
#include "kernels.h"
#include "tile_io.h"

namespace mscan {

namespace {

struct BwdDims {
  int64_t batch, seqlen, dim, rows, seg_len;
  int segments;
  unsigned tiles;
  int64_t ngroups, group_dim;  // B/C groups and channels per group
};

// Pointers of one backward call. carry_h / carry_hs: the end state from zero
// and the Delta sum of segment k in slot k, then (after the forward combine)
// the state entering segment s in slot s - 1; carry_a / carry_s: adjoint
// aggregates, then (after the fold) the adjoint entering segment s from later
// time in slot s; ck / ck_s: per chunk, the state before its first step from
// the segment's start from zero, and the Delta sum from the segment's start;
// pA, pDb, pBC: partial sums.
struct BwdPtrs {
  const void* x;
  const void* delta;
  const void* B;
  const void* C;
  const void* z;
  const void* dy;
  const float* A;
  const float* D;
  const float* bias;
  const float* h0;
  const float* dlast;
  void* dx;
  void* ddelta;
  void* dz;
  float* dh0;
  float* carry_h;  // segment end states from zero, then (after the combine) carry-in states
  float* carry_hs;  // segment sums of Delta
  float* carry_a;
  float* carry_s;
  float* ck;
  float* ck_s;
  float* pA;
  float* pDb;
  float* pBC;
  uint32_t* tile_flags;  // per channel tile: 1 = S4D-Real shaped
};

// |Delta x| floor of the rescaled form (the forward scan's value).
constexpr float kDxFloorBwd = 1e-20f;

__device__ __forceinline__ float sigmoid_f(float v) { return hw_rcp(1.0f + hw_exp2(-v * kLog2e)); }

// The value of lane l ^ 2^K: quad permutes (DPP) for K = 0, 1, otherwise a
// cross-lane read through the LDS crossbar.
template <int K>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (K == 0)
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false));
  else if constexpr (K == 1)
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xf, 0xf, false));
  else
    return __shfl_xor(v, 1 << K);
}

template <int M>
constexpr int log2_of() {
  int k = 0;
  while ((1 << k) < M) ++k;
  return k;
}

// Channel sums of dB and dC within a wave. Every lane holds, per step, N dB
// terms and N dC terms; the wave's 64 lanes are summed by recursive halving,
// each level leaving half of the values on each lane of a pair, so that at
// the end every value's total sits on some lane:
//   level 0, lane bit 5: v_permlane32_swap exchanges the upper half-wave of
//     the dB term with the lower half-wave of the dC term (per state, inline
//     in the step); the sum of the two results is the dB total over the lane
//     pair on lanes 0-31 and the dC total on lanes 32-63;
//   level 1, lane bit 4: v_permlane16_swap does the same between rows of 16
//     lanes for states n and n + N/2;
//   then, lane bits 0, 1, 2: lane l keeps one half of its values and adds the
//     other half of lane l ^ 2^k's (selected per lane);
//   the remaining lane bits add the one value left.
// The swap levels need no per-lane selection; they act where the most values
// are left.
template <int W, int K, int SZ>
__device__ __forceinline__ void sum_scatter_level(float (&v)[SZ], int lane) {
  if constexpr (W >= 2) {
    constexpr int H = W / 2;
    const bool hi = (lane >> K) & 1;
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const float keep = hi ? v[i + H] : v[i];
      const float send = hi ? v[i] : v[i + H];
      v[i] = keep + lane_xor<K>(send);
    }
    sum_scatter_level<H, K + 1>(v, lane);
  }
}

template <int N>
struct BcReduce {
  static constexpr int kW = N >= 2 ? N / 2 : 1;  // values left after the swap levels
  static constexpr int kSel = log2_of<kW>();     // select levels, lane bits 0 .. kSel - 1
  // lane bits summed at the end: kSel .. 3, and 4 when N == 1
  static constexpr int kRestMask = (0xf & ~((1 << kSel) - 1)) | (N == 1 ? 0x10 : 0);

  // value index (n for dB_n, N + n for dC_n) whose wave total lane ends with
  static __device__ __forceinline__ int index(int lane) {
    int e = ((lane >> 5) & 1) * N;
    if (N >= 2) e += ((lane >> 4) & 1) * (N / 2);
#pragma unroll
    for (int k = 0; k < kSel; ++k) e += ((lane >> k) & 1) * (kW >> (k + 1));
    return e;
  }
  // one lane per value stores its total
  static __device__ __forceinline__ bool writer(int lane) { return (lane & kRestMask) == 0; }

  // level 0 for one state: the dB and dC terms of state n
  static __device__ __forceinline__ float level0(float db, float dc) {
    const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(db), __float_as_uint(dc), false,
                                                    false);
    return __uint_as_float(w[0]) + __uint_as_float(w[1]);
  }
  // the remaining levels on the N level-0 results
  static __device__ __forceinline__ float rest(float (&t)[N], int lane) {
    if constexpr (N >= 2) {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        const auto w = __builtin_amdgcn_permlane16_swap(__float_as_uint(t[i]),
                                                        __float_as_uint(t[i + N / 2]), false, false);
        t[i] = __uint_as_float(w[0]) + __uint_as_float(w[1]);
      }
    }
    sum_scatter_level<kW, 0>(t, lane);
    float r = t[0];
    if constexpr ((kRestMask & 1) != 0) r += lane_xor<0>(r);
    if constexpr ((kRestMask & 2) != 0) r += lane_xor<1>(r);
    if constexpr ((kRestMask & 4) != 0) r += lane_xor<2>(r);
    if constexpr ((kRestMask & 8) != 0) r += lane_xor<3>(r);
    if constexpr ((kRestMask & 16) != 0) r += lane_xor<4>(r);
    return r;
  }
};

// LDS staging of one chunk: NIN input tiles (raw io values), the chunk's B and
// C widened to fp32, NOUT output tiles and the per-wave dB/dC sums (double
// buffered where a chunk is fetched or stored while another is computed).
template <int N, class IO, int NIN, int NOUT>
struct __align__(16) BwdStage {
  typename IO::raw in[2][NIN][kChunk][kBlock];
  float bc[2][kChunk][2 * N];
  typename IO::raw go[NOUT ? 2 : 1][NOUT ? NOUT : 1][NOUT ? kChunk : 1][kBlock];
  float red[NOUT ? kBlock / 64 : 1][NOUT ? kChunk : 1][2 * N];
  float dl[NOUT ? kChunk : 1][kBlock];  // Delta of the chunk's steps, per lane
  float dxs[NOUT ? kChunk : 1][kBlock];  // their floored Delta x (structured tiles)
};

// Addressing of one workgroup's channel tile within one time segment, shared
// by the adjoint aggregate and the main kernel.
template <int N, class IO, int CW>
struct TileCtx {
  using raw = typename IO::raw;
  static constexpr int eb = sizeof(raw);
  static constexpr int kTileElems = kChunk * 2 * N;
  static constexpr int kBcPer = (kTileElems + kBlock - 1) / kBlock;
  int64_t b, d0, d, row, row0, t_begin;
  uint32_t steps, row_bytes, ch_off, lane_off, bc_row;
  unsigned tile;
  int s, wv;
  bool active;
  const raw* Bp;
  const raw* Cp;
  BcOffsets bco[kBcPer];

  __device__ __forceinline__ TileCtx(const BwdDims& g, const void* B, const void* C, int seg) {
    const int tid = threadIdx.x;
    b = blockIdx.x / g.tiles;
    tile = blockIdx.x % g.tiles;
    d0 = static_cast<int64_t>(tile) * kBlock;
    active = d0 + tid < g.dim;
    // lanes past the last channel compute on channel dim - 1 and store nothing
    d = active ? d0 + tid : g.dim - 1;
    s = seg;
    t_begin = static_cast<int64_t>(s) * g.seg_len;
    const int64_t t_end = t_begin + g.seg_len < g.seqlen ? t_begin + g.seg_len : g.seqlen;
    steps = static_cast<uint32_t>(t_end - t_begin);
    row = b * g.dim + d;
    row0 = (b * g.seqlen + t_begin) * g.dim + d0;
    row_bytes = static_cast<uint32_t>(g.dim * eb);
    const int64_t left = g.dim - d0;
    const uint32_t valid_bytes = static_cast<uint32_t>((left < kBlock ? left : kBlock) * eb);
    ch_off = active ? tid * eb : kOffNone;
    lane_off = CW != 0 ? tile_lane_offset<IO, (CW != 0 ? CW : 4)>(row_bytes, valid_bytes) : 0u;
    wv = __builtin_amdgcn_readfirstlane(tid / 64);
    // the tile's group of B and C (every channel of a tile is in one group)
    const int64_t grp = d0 / g.group_dim;
    bc_row = static_cast<uint32_t>(g.ngroups * N);
    Bp = static_cast<const raw*>(B) + ((b * g.seqlen + t_begin) * g.ngroups + grp) * N;
    Cp = static_cast<const raw*>(C) + ((b * g.seqlen + t_begin) * g.ngroups + grp) * N;
#pragma unroll
    for (int r = 0; r < kBcPer; ++r) bco[r] = bc_offsets<N, IO>(tid + r * kBlock, bc_row);
  }

  // Start copying the tile rows of chunk step t1 of `count` tensors into the
  // consecutive tiles (kChunk x kBlock each) from `tiles` on (register-staged:
  // into regs[k], written by land()).
  static constexpr int kTile = kChunk * kBlock;
  template <int NT>
  __device__ __forceinline__ void fetch(const raw* const (&src)[NT], int count, uint32_t t1,
                                        raw* tiles, TileRegs<IO> (&regs)[NT]) const {
    const int64_t at = static_cast<int64_t>(t1) * (row_bytes / eb);
    const uint32_t left = steps - t1;
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      if (k < count) {
        if constexpr (CW != 0)
          dma_tile<IO, CW>(src[k] + at, left, row_bytes, tiles + k * kTile, wv, lane_off);
        else
          load_tile_regs<IO>(regs[k], src[k] + at, left, row_bytes, ch_off);
      }
    }
  }
  template <int NT>
  __device__ __forceinline__ void land(int count, raw* tiles, const TileRegs<IO> (&regs)[NT]) const {
    if constexpr (CW == 0) {
#pragma unroll
      for (int k = 0; k < NT; ++k)
        if (k < count) store_tile_regs<IO>(regs[k], tiles + k * kTile);
    }
  }
  __device__ __forceinline__ void fetch_bc(uint32_t t1, float (&bcv)[kBcPer]) const {
#pragma unroll
    for (int r = 0; r < kBcPer; ++r)
      bcv[r] = bc_elem<N, IO>(Bp + static_cast<int64_t>(t1) * bc_row,
                              Cp + static_cast<int64_t>(t1) * bc_row, steps - t1, bco[r], bc_row);
  }
  __device__ __forceinline__ void land_bc(const float (&bcv)[kBcPer], float (*bc)[2 * N]) const {
#pragma unroll
    for (int r = 0; r < kBcPer; ++r) {
      const int i = threadIdx.x + r * kBlock;
      if (i < kTileElems) bc[i / (2 * N)][i % (2 * N)] = bcv[r];
    }
  }
};

// Workgroups per CU: the adjoint aggregate as many as fit its LDS staging
// (bf16 tiles are half the size of fp32 ones); the main pass two with bf16
// tiles (a chunk of recomputed states, the adjoint and the dA sums take about
// 250 registers per lane: two waves per SIMD) and one with fp32 tiles (LDS).
// The launch bounds hold the compiler to the matching register budget.
template <class IO>
constexpr int kAggBlocksPerCU = sizeof(typename IO::raw) == 2 ? 4 : 3;
#ifndef MSCAN_BWD_BLOCKS
#define MSCAN_BWD_BLOCKS 2
#endif
template <class IO>
constexpr int kMainBlocksPerCU = sizeof(typename IO::raw) == 2 ? MSCAN_BWD_BLOCKS : 1;

// Decays abar_n = exp(Delta A[d, n]) of one step (A2 = A[d, :] log2 e), in
// order n = 0, 1, ...: on S4D-Real-shaped rows (A[d, n] = (n + 1) A[d, 0])
// the powers e^(n+1) of e = exp(Delta A[d, 0]), each the previous one times e
// (one value live at a time, at most N roundings); otherwise one exponential
// each.
template <int N, bool STRUCT>
struct Decays {
  float e, cur, Delta;
  __device__ __forceinline__ Decays(float delta, const float (&A2)[N]) : Delta(delta) {
    if constexpr (STRUCT) {
      e = hw_exp2(delta * A2[0]);
      cur = e;
    }
  }
  // abar_n; call for n = 0, 1, ... in turn
  __device__ __forceinline__ float next(int n, const float (&A2)[N]) {
    if constexpr (STRUCT) {
      const float v = cur;
      cur *= e;
      return v;
    } else {
      return hw_exp2(Delta * A2[n]);
    }
  }
};

// rho e^(n+1) for n = 0, 1, ... in turn, as one chain of multiplications (one
// value live besides e; N multiplications, against N + 1 and three live values
// for two interleaved chains: 16 vector instructions fewer per 8 steps of the
// main pass, 1,457-1,468 -> 1,456-1,462 us per call in interleaved timing).
template <int N>
struct PowerChains {
  float v, e;
  __device__ __forceinline__ PowerChains(float e_, float rho) {
    v = rho * e_;
    e = e_;
  }
  // call for n = 0, 1, ... in turn
  __device__ __forceinline__ float next(int) {
    const float r = v;
    v *= e;
    return r;
  }
};

// Whether every channel of the workgroup's tile is S4D-Real shaped (the same
// test as the forward scan); uniform over the workgroup.
template <int N>
__device__ __forceinline__ bool tile_is_structured(const float* A, int64_t d) {
  bool structured = true;
  const float a0 = A[d * N];
#pragma unroll
  for (int n = 1; n < N; ++n) structured = structured && (A[d * N + n] == (n + 1) * a0);
  return __syncthreads_and(structured);
}

// The decay path of a tile: the first launch of a call classifies the tile
// and the copy in batch row 0, segment 0 records it; later launches read it.
template <int N, bool CLASSIFY>
__device__ __forceinline__ bool tile_path(uint32_t* flags, const float* A, int64_t d, int64_t b,
                                          int s, unsigned tile) {
  if constexpr (CLASSIFY) {
    const bool structured = tile_is_structured<N>(A, d);
    if (b == 0 && s == 0 && threadIdx.x == 0) flags[tile] = structured ? 1u : 0u;
    return structured;
  } else {
    return flags[tile] != 0u;
  }
}

// Checkpoint layout: float[chunk][N / 4][rows][4] (N >= 4) or
// float[chunk][N][rows]: the state before the chunk's first step, for every
// chunk of kChunk steps of the sequence. Written once and read once, so the
// 16-byte accesses are non-temporal.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
template <int N>
__device__ __forceinline__ void ck_store(float* ck, int64_t chunk, int64_t rows, int64_t row,
                                         const float (&v)[N]) {
  float* base = ck + chunk * rows * N;
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int q = 0; q < N / 4; ++q)
      __builtin_nontemporal_store(f32x4_t{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]},
                                  reinterpret_cast<f32x4_t*>(base + (q * rows + row) * 4));
  } else {
#pragma unroll
    for (int n = 0; n < N; ++n) base[n * rows + row] = v[n];
  }
}

template <int N>
__device__ __forceinline__ void ck_load(const float* ck, int64_t chunk, int64_t rows, int64_t row,
                                        float (&v)[N]) {
  const float* base = ck + chunk * rows * N;
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const f32x4_t w =
          __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(base + (q * rows + row) * 4));
      v[4 * q] = w[0];
      v[4 * q + 1] = w[1];
      v[4 * q + 2] = w[2];
      v[4 * q + 3] = w[3];
    }
  } else {
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] = base[n * rows + row];
  }
}

// ---------------------------------------------------------------------------
// 0. State checkpoints. Grid: x = batch * channel tiles, y = segment. Scans
// segment blockIdx.y forward from zero; at the start of every chunk it stores
// the state and the Delta sum so far (the state there is this local state
// plus exp(A * Delta sum) times the segment's carry-in state: the affine-pair
// combine); every segment but the last also stores its end state and Delta
// sum for the forward combine. S4D-Real-shaped tiles run the rescaled form of
// the forward scan (g = h / (Delta x) and one exponential per step, with
// Delta x kept away from zero by at most 1e-20).
template <class IO>
constexpr int kCkBlocksPerCU = sizeof(typename IO::raw) == 2 ? 5 : 3;

template <int N, class IO, int CW, bool STRUCT>
__global__ __launch_bounds__(kBlock, kCkBlocksPerCU<IO>) void bwd_state_checkpoint_kernel(BwdPtrs a, BwdDims g) {
  using raw = typename IO::raw;
  __shared__ BwdStage<N, IO, 2, 0> st;  // x, Delta_raw
  const int tid = threadIdx.x;
  const TileCtx<N, IO, CW> tc(g, a.B, a.C, blockIdx.y);
  // the structured launch runs first and classifies the tiles
  if (tile_path<N, STRUCT>(a.tile_flags, a.A, tc.d, tc.b, tc.s, tc.tile) != STRUCT) return;
  float A2[N];
#pragma unroll
  for (int n = 0; n < N; ++n) A2[n] = a.A[tc.d * N + n] * kLog2e;
  const float bias = a.bias ? a.bias[tc.d] : 0.0f;
  const raw* const src[2] = {static_cast<const raw*>(a.x) + tc.row0,
                             static_cast<const raw*>(a.delta) + tc.row0};
  TileRegs<IO> regs[2];
  float bcv[TileCtx<N, IO, CW>::kBcPer];
  const int last = static_cast<int>((tc.steps + kChunk - 1) / kChunk) - 1;
  const int64_t ck0 = tc.t_begin / kChunk;

  float h[N];  // h, or g = h / dx_prev on structured tiles
#pragma unroll
  for (int n = 0; n < N; ++n) h[n] = 0.0f;
  float dx_prev = 1.0f;
  float S = 0.0f, S_c = 0.0f;  // Kahan-compensated sum of Delta
  tc.fetch(src, 2, 0, &st.in[0][0][0][0], regs);
  tc.fetch_bc(0, bcv);
  tc.land(2, &st.in[0][0][0][0], regs);
  tc.land_bc(bcv, st.bc[0]);
  wait_vmem();
  __syncthreads();
  for (int c = 0; c <= last; ++c) {
    const int buf = c & 1;
    if (c < last) {
      tc.fetch(src, 2, (c + 1) * kChunk, &st.in[buf ^ 1][0][0][0], regs);
      tc.fetch_bc((c + 1) * kChunk, bcv);
    }
    if (tc.active) {
      float hv[N];
#pragma unroll
      for (int n = 0; n < N; ++n) hv[n] = STRUCT ? h[n] * dx_prev : h[n];
      ck_store<N>(a.ck, ck0 + c, g.rows, tc.row, hv);
      a.ck_s[(ck0 + c) * g.rows + tc.row] = S;
    }
    const int valid = static_cast<int>(tc.steps) - c * kChunk;
    float dsum = 0.0f;
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      if (j < valid) {
        const float xf = IO::to_f32(st.in[buf][0][j][tid]);
        const float Delta = softplus_f(IO::to_f32(st.in[buf][1][j][tid]) + bias);
        const float* Br = &st.bc[buf][j][0];
        if constexpr (STRUCT) {
          const float dx = fmaf(Delta, xf, copysignf(kDxFloorBwd, xf));
          float p[N];
          scaled_powers<N>(hw_exp2(Delta * A2[0]), dx_prev * hw_rcp(dx), p);
          dx_prev = dx;
#pragma unroll
          for (int n = 0; n < N; ++n) h[n] = fmaf(p[n], h[n], Br[n]);
        } else {
          const float dxv = Delta * xf;
#pragma unroll
          for (int n = 0; n < N; ++n) h[n] = fmaf(hw_exp2(Delta * A2[n]), h[n], dxv * Br[n]);
        }
        dsum += Delta;
      }
    }
    const float v = dsum - S_c;
    const float tsum = S + v;
    S_c = (tsum - S) - v;
    S = tsum;
    if (c < last) {
      tc.land(2, &st.in[buf ^ 1][0][0][0], regs);
      tc.land_bc(bcv, st.bc[buf ^ 1]);
      wait_vmem();
    }
    __syncthreads();
  }
  if (!tc.active || tc.s + 1 >= g.segments) return;
  const int64_t slot = static_cast<int64_t>(tc.s) * g.rows + tc.row;
#pragma unroll
  for (int n = 0; n < N; ++n) a.carry_h[slot * N + n] = STRUCT ? h[n] * dx_prev : h[n];
  a.carry_hs[slot] = S;
}

// ---------------------------------------------------------------------------
// 1. Adjoint aggregate. Grid: x = batch * channel tiles, y = segment - 1.
// Runs the adjoint recurrence of segment blockIdx.y + 1 backwards from zero;
// stores abar at the segment's first step times the adjoint there, and the
// segment's sum of Delta, in slot blockIdx.y.
// STRUCT: the launch for S4D-Real-shaped channel tiles (the others leave at
// once), or for the general ones.
template <int N, class IO, bool GATE, int CW, bool STRUCT>
__global__ __launch_bounds__(kBlock, kAggBlocksPerCU<IO>) void bwd_adjoint_aggregate_kernel(BwdPtrs a, BwdDims g) {
  using raw = typename IO::raw;
  constexpr int kIn = GATE ? 3 : 2;  // Delta_raw, dy (, z)
  __shared__ BwdStage<N, IO, kIn, 0> st;
  const int tid = threadIdx.x;
  const TileCtx<N, IO, CW> tc(g, a.B, a.C, blockIdx.y + 1);
  if (tile_path<N, false>(a.tile_flags, a.A, tc.d, tc.b, tc.s, tc.tile) != STRUCT) return;

  float A2[N];
#pragma unroll
  for (int n = 0; n < N; ++n) A2[n] = a.A[tc.d * N + n] * kLog2e;
  const float bias = a.bias ? a.bias[tc.d] : 0.0f;

  const raw* const src[3] = {static_cast<const raw*>(a.delta) + tc.row0,
                             static_cast<const raw*>(a.dy) + tc.row0,
                             static_cast<const raw*>(GATE ? a.z : a.dy) + tc.row0};
  TileRegs<IO> regs[3];
  float bcv[TileCtx<N, IO, CW>::kBcPer];

  float m[N];  // abar_{t+1} lam_{t+1}
#pragma unroll
  for (int n = 0; n < N; ++n) m[n] = 0.0f;
  float S = 0.0f, S_c = 0.0f;  // Kahan-compensated sum of Delta

  const int last = static_cast<int>((tc.steps + kChunk - 1) / kChunk) - 1;
  {
    const int nb = last & 1;
    tc.fetch(src, kIn, last * kChunk, &st.in[nb][0][0][0], regs);
    tc.fetch_bc(last * kChunk, bcv);
    tc.land(kIn, &st.in[nb][0][0][0], regs);
    tc.land_bc(bcv, st.bc[nb]);
    wait_vmem();
    __syncthreads();
  }
  for (int c = last; c >= 0; --c) {
    const int buf = c & 1;
    if (c > 0) {
      tc.fetch(src, kIn, (c - 1) * kChunk, &st.in[buf ^ 1][0][0][0], regs);
      tc.fetch_bc((c - 1) * kChunk, bcv);
    }
    const int valid = static_cast<int>(tc.steps) - c * kChunk;
    float dsum = 0.0f;
#pragma unroll
    for (int jj = 0; jj < kChunk; ++jj) {
      const int j = kChunk - 1 - jj;
      if (j < valid) {
        const float Delta = softplus_f(IO::to_f32(st.in[buf][0][j][tid]) + bias);
        const float dyv = IO::to_f32(st.in[buf][1][j][tid]);
        const float ds = GATE ? dyv * silu_f(IO::to_f32(st.in[buf][kIn - 1][j][tid])) : dyv;
        const float* Cr = &st.bc[buf][j][N];
        Decays<N, STRUCT> ab(Delta, A2);
#pragma unroll
        for (int n = 0; n < N; ++n) m[n] = ab.next(n, A2) * fmaf(Cr[n], ds, m[n]);
        dsum += Delta;
      }
    }
    const float v = dsum - S_c;
    const float tsum = S + v;
    S_c = (tsum - S) - v;
    S = tsum;
    if (c > 0) {
      tc.land(kIn, &st.in[buf ^ 1][0][0][0], regs);
      tc.land_bc(bcv, st.bc[buf ^ 1]);
      wait_vmem();
    }
    __syncthreads();
  }
  if (!tc.active) return;
  const int64_t slot = static_cast<int64_t>(blockIdx.y) * g.rows + tc.row;
#pragma unroll
  for (int n = 0; n < N; ++n) a.carry_a[slot * N + n] = m[n];
  a.carry_s[slot] = S;
}

// ---------------------------------------------------------------------------
// 2. Adjoint fold over segments, per (row, n), from the last segment back:
// nu_{S-1} = dlast (or 0), nu_{s-1} = E_s + exp(A sum_s Delta) nu_s, where slot
// s - 1 holds (E_s, sum_s Delta) on entry and nu_{s-1} on exit.
constexpr int kFoldBlock = 8;

template <int N>
__global__ __launch_bounds__(kAuxBlock) void bwd_adjoint_fold_kernel(const float* __restrict__ A,
                                                                  float* __restrict__ ws_e,
                                                                  const float* __restrict__ ws_s,
                                                                  const float* __restrict__ dlast,
                                                                  int64_t rows, int64_t dim,
                                                                  int segments) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kAuxBlock + threadIdx.x;
  if (i >= rows * N) return;
  const int64_t row = i / N;
  const int n = static_cast<int>(i % N);
  const float a2 = A[(row % dim) * N + n] * kLog2e;
  float nu = dlast ? dlast[i] : 0.0f;
  for (int k0 = segments - 2; k0 >= 0; k0 -= kFoldBlock) {
    float ev[kFoldBlock], sv[kFoldBlock];
#pragma unroll
    for (int u = 0; u < kFoldBlock; ++u) {
      const int k = k0 - u >= 0 ? k0 - u : 0;
      ev[u] = ws_e[static_cast<int64_t>(k) * rows * N + i];
      sv[u] = ws_s[static_cast<int64_t>(k) * rows + row];
    }
#pragma unroll
    for (int u = 0; u < kFoldBlock; ++u) {
      if (k0 - u >= 0) {
        nu = fmaf(hw_exp2(a2 * sv[u]), nu, ev[u]);
        ws_e[static_cast<int64_t>(k0 - u) * rows * N + i] = nu;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. Main pass. Grid: x = batch * channel tiles, y = segment.
// STRUCT: the launch for S4D-Real-shaped channel tiles (the others leave at
// once), or for the general ones.
template <int N, class IO, bool GATE, int CW, bool STRUCT>
__global__ __launch_bounds__(kBlock, kMainBlocksPerCU<IO>) void scan_bwd_kernel(BwdPtrs a, BwdDims g) {
  using raw = typename IO::raw;
  constexpr int M = 2 * N;
  constexpr int kIn = GATE ? 4 : 3;   // x, Delta_raw, dy (, z)
  constexpr int kOut = GATE ? 3 : 2;  // dx, dDelta_raw (, dz)
  constexpr int iX = 0, iDl = 1, iDy = 2, iZ = 3;
  __shared__ BwdStage<N, IO, kIn, kOut> st;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const TileCtx<N, IO, CW> tc(g, a.B, a.C, blockIdx.y);
  if (tile_path<N, false>(a.tile_flags, a.A, tc.d, tc.b, tc.s, tc.tile) != STRUCT) return;
  const int s = tc.s;
  const bool active = tc.active;

  float A2[N];  // A[d, n] log2(e) (structured tiles use A2[0] only)
#pragma unroll
  for (int n = 0; n < N; ++n) A2[n] = a.A[tc.d * N + n] * kLog2e;
  const float Dd = a.D ? a.D[tc.d] : 0.0f;
  const float bias = a.bias ? a.bias[tc.d] : 0.0f;

  const raw* const src[4] = {static_cast<const raw*>(a.x) + tc.row0,
                             static_cast<const raw*>(a.delta) + tc.row0,
                             static_cast<const raw*>(a.dy) + tc.row0,
                             static_cast<const raw*>(GATE ? a.z : a.dy) + tc.row0};
  TileRegs<IO> regs[4];
  float bcv[TileCtx<N, IO, CW>::kBcPer];
  raw* const dst[3] = {static_cast<raw*>(a.dx) + tc.row0, static_cast<raw*>(a.ddelta) + tc.row0,
                       static_cast<raw*>(GATE && a.dz ? a.dz : a.dx) + tc.row0};
  const int n_out = GATE && a.dz ? 3 : 2;
  auto put = [&](int ob, uint32_t t1) {
    const int64_t at = static_cast<int64_t>(t1) * g.dim;
#pragma unroll
    for (int k = 0; k < kOut; ++k)
      if (k < n_out)
        store_tile<IO, CW>(dst[k] + at, tc.steps - t1, tc.row_bytes, &st.go[ob][k][0][0],
                           tc.lane_off, tc.ch_off);
  };
  // x and Delta_raw of step j of buffer buf; lanes past the last channel run
  // on zeros (finite values that add nothing to the channel sums).
  auto x_at = [&](int buf, int j) { return active ? IO::to_f32(st.in[buf][iX][j][tid]) : 0.0f; };
  auto u_at = [&](int buf, int j) {
    return (active ? IO::to_f32(st.in[buf][iDl][j][tid]) : 0.0f) + bias;
  };

  const int last = static_cast<int>((tc.steps + kChunk - 1) / kChunk) - 1;
  const int64_t ck0 = tc.t_begin / kChunk;  // sequence chunk index of the segment's chunk 0

  // carry-in state of the segment (null: zeros)
  const float* cin = s > 0 ? a.carry_h + (static_cast<int64_t>(s - 1) * g.rows + tc.row) * N
                           : (a.h0 ? a.h0 + tc.row * N : nullptr);

  // Reverse sweep over the chunks.
  float m[N];  // abar_{t+1} lam_{t+1}: the adjoint entering from later time
  // (zeros on lanes past the last channel, so that every term they add to the
  // channel sums of dB and dC is zero in both forms of the step below)
  if (!active) {
#pragma unroll
    for (int n = 0; n < N; ++n) m[n] = 0.0f;
  } else if (s + 1 < g.segments) {
    const float* ain = a.carry_a + (static_cast<int64_t>(s) * g.rows + tc.row) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) m[n] = ain[n];
  } else {
#pragma unroll
    for (int n = 0; n < N; ++n) m[n] = a.dlast ? a.dlast[tc.row * N + n] : 0.0f;
  }
  float dA[N];
#pragma unroll
  for (int n = 0; n < N; ++n) dA[n] = 0.0f;
  float dD = 0.0f, dbias = 0.0f;
  const int e_idx = BcReduce<N>::index(lane);
  const bool bc_writer = BcReduce<N>::writer(lane);
  float* pbc = a.pBC + ((static_cast<int64_t>(tc.tile) * g.batch + tc.b) * g.seqlen + tc.t_begin) * M;

  // The checkpoint of the chunk to be recomputed next (the first one's here,
  // the others' loaded early in the previous chunk's adjoint sweep, into the
  // registers of states it no longer needs, so that their latency is hidden).
  float hc[N];
  float cks = 0.0f;
#pragma unroll
  for (int n = 0; n < N; ++n) hc[n] = 0.0f;
  // (buffer loads: per chunk one resource in scalar registers, the tile's
  // first row as the scalar offset, the lane's 16 or 4 bytes as the vector
  // one; lanes past the last channel read zeros)
  const int64_t row_base = tc.b * g.dim + tc.d0;
  const uint32_t off16 = active ? static_cast<uint32_t>(tid) * 16u : kOffNone;
  const uint32_t off4 = active ? static_cast<uint32_t>(tid) * 4u : kOffNone;
  auto load_ck = [&](int cc) {
    const int64_t chunk = ck0 + cc;
    if constexpr (N % 4 == 0) {
      const auto r = make_rsrc(a.ck + chunk * g.rows * N);
#pragma unroll
      for (int q = 0; q < N / 4; ++q) {
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
            r, off16, static_cast<uint32_t>((q * g.rows + row_base) * 16), kNonTemporal);
#pragma unroll
        for (int k = 0; k < 4; ++k) hc[4 * q + k] = __uint_as_float(w[k]);
      }
    } else if (active) {
      ck_load<N>(a.ck, chunk, g.rows, tc.row, hc);
    }
    cks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        make_rsrc(a.ck_s + chunk * g.rows), off4, static_cast<uint32_t>(row_base * 4), 0));
  };
  load_ck(last);
  {
    const int nb = last & 1;
    tc.fetch(src, kIn, last * kChunk, &st.in[nb][0][0][0], regs);
    tc.fetch_bc(last * kChunk, bcv);
    tc.land(kIn, &st.in[nb][0][0][0], regs);
    tc.land_bc(bcv, st.bc[nb]);
    wait_vmem();
    __syncthreads();
  }
  for (int c = last; c >= 0; --c) {
    const int buf = c & 1;
    if (c < last) put(buf ^ 1, (c + 1) * kChunk);
    if (c > 0) {
      tc.fetch(src, kIn, (c - 1) * kChunk, &st.in[buf ^ 1][0][0][0], regs);
      tc.fetch_bc((c - 1) * kChunk, bcv);
    }
    const int valid = static_cast<int>(tc.steps) - c * kChunk;
    // recompute the chunk's states (from the checkpoint before its first
    // step; zeros on lanes past the last channel): h_t, or on S4D-Real-shaped
    // tiles g_t = h_t / dx_t with dx_t = Delta_t x_t kept away from zero by at
    // most 1e-20 (the forward scan's rescaled form: g_t = rho_t e^(n+1) g_{t-1}
    // + B_t with rho_t = dx_{t-1} / dx_t, and at the chunk's first step
    // g = e^(n+1) h / dx + B from the state h before it)
    float hist[kChunk][N];
    {
      if (active && cin) {
        // plus the carry-in decayed over the segment's steps before the chunk
        Decays<N, STRUCT> dk(cks, A2);
#pragma unroll
        for (int n = 0; n < N; ++n) hc[n] = fmaf(dk.next(n, A2), cin[n], hc[n]);
      }
      float dx_prev = 1.0f;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        if (j < valid) {
          const float Delta = softplus_f(u_at(buf, j));
          st.dl[j][tid] = Delta;
          const float xf = x_at(buf, j);
          const float* Br = &st.bc[buf][j][0];
          if constexpr (STRUCT) {
            const float dx = fmaf(Delta, xf, copysignf(kDxFloorBwd, xf));
            st.dxs[j][tid] = dx;
            const float rdx = hw_rcp(dx);
            PowerChains<N> pw(hw_exp2(Delta * A2[0]), j == 0 ? rdx : dx_prev * rdx);
            dx_prev = dx;
#pragma unroll
            for (int n = 0; n < N; ++n)
              hist[j][n] = fmaf(pw.next(n), j == 0 ? hc[n] : hist[j - 1][n], Br[n]);
          } else {
            const float dxv = Delta * xf;
            Decays<N, STRUCT> ab(Delta, A2);
#pragma unroll
            for (int n = 0; n < N; ++n)
              hist[j][n] = fmaf(ab.next(n, A2), j == 0 ? hc[n] : hist[j - 1][n], dxv * Br[n]);
          }
        }
      }
    }
    if constexpr (STRUCT) {
      // the adjoint enters the chunk's last step scaled like it: m dx there
      const float dx_top = st.dxs[valid < kChunk ? valid - 1 : kChunk - 1][tid];
#pragma unroll
      for (int n = 0; n < N; ++n) m[n] *= dx_top;
    }
    // step the adjoint back through them
#pragma unroll
    for (int jj = 0; jj < kChunk; ++jj) {
      const int j = kChunk - 1 - jj;
      if (c > 0 && jj == 1) load_ck(c - 1);
      if (j < valid) {
        const float xf = x_at(buf, j);
        const float u = u_at(buf, j);
        const float Delta = st.dl[j][tid];
        const float dyv = IO::to_f32(st.in[buf][iDy][j][tid]);
        float zf = 0.0f, sz = 0.0f, ds = dyv;
        if constexpr (GATE) {
          zf = IO::to_f32(st.in[buf][iZ][j][tid]);
          sz = sigmoid_f(zf);
          ds = dyv * (zf * sz);
        }
        ds = active ? ds : 0.0f;
        float bc[2 * N];
        read_bc<N>(st.bc[buf][j], bc, true);
        float sAq = 0.0f, sLB = 0.0f, ypre = Dd * xf;
        float r[N];  // dB / dC terms of this step after the first halving level
        if constexpr (STRUCT) {
          // Scaled adjoint l_t = lam_t dx_t: l_t = C_t ds_t dx_t + mu_{t+1},
          // mu_t = alpha_t l_t with the forward's alpha_t = rho_t e^(n+1)
          // (m holds mu_{t+1}). Then the dB term Delta_t x_t lam_t is
          // l_t Delta_t x_t / dx_t, ds_t h_t = ds_t dx_t g_t, and
          // abar_t lam_t h_{t-1} = mu_t g_{t-1}, or l_t (g_t - B_t) at the
          // chunk's first step, whose mu_t (rho = 1 / dx) is the unscaled
          // abar_t lam_t that enters the previous chunk.
          const float dx = st.dxs[j][tid];
          const float rdx = hw_rcp(dx);
          const float dsdx = ds * dx;
          const float kappa = Delta * xf * rdx;  // Delta x / dx: 1 but for the floor
          PowerChains<N> pw(hw_exp2(Delta * A2[0]),
                            j == 0 ? rdx : st.dxs[j > 0 ? j - 1 : 0][tid] * rdx);
          float sLBs = 0.0f, ypg = 0.0f;
#pragma unroll
          for (int n = 0; n < N; ++n) {
            // (mu last, so that it can take l's register, which is m's)
            const float l = fmaf(bc[N + n], dsdx, m[n]);
            sLBs = fmaf(l, bc[n], sLBs);
            ypg = fmaf(bc[N + n], hist[j][n], ypg);
            r[n] = BcReduce<N>::level0(l * kappa, dsdx * hist[j][n]);
            float q;
            if (j == 0) q = l * (hist[0][n] - bc[n]);
            m[n] = pw.next(n) * l;
            if (j != 0) q = m[n] * hist[j > 0 ? j - 1 : 0][n];
            dA[n] = fmaf(Delta, q, dA[n]);
            sAq = fmaf(static_cast<float>(n + 1), q, sAq);
          }
          sAq *= A2[0];
          sLB = sLBs * rdx;
          ypre = fmaf(dx, ypg, ypre);
        } else {
          const float dxv = Delta * xf;
          Decays<N, STRUCT> ab(Delta, A2);
#pragma unroll
          for (int n = 0; n < N; ++n) {
            const float lam = fmaf(bc[N + n], ds, m[n]);
            // abar_t h_{t-1} = h_t - Delta_t B_t x_t
            const float q = lam * fmaf(-dxv, bc[n], hist[j][n]);
            dA[n] = fmaf(Delta, q, dA[n]);
            sAq = fmaf(A2[n], q, sAq);
            sLB = fmaf(lam, bc[n], sLB);
            ypre = fmaf(bc[N + n], hist[j][n], ypre);
            r[n] = BcReduce<N>::level0(lam * dxv, ds * hist[j][n]);
            m[n] = ab.next(n, A2) * lam;
          }
        }
        const float tot = BcReduce<N>::rest(r, lane);
        if (bc_writer) st.red[tc.wv][j][e_idx] = tot;
        const float dDelta = fmaf(sAq, kLn2, xf * sLB);
        const float ddr = dDelta * sigmoid_f(u);
        dbias += ddr;
        dD = fmaf(ds, xf, dD);
        st.go[buf][0][j][tid] = IO::from_f32(fmaf(Dd, ds, Delta * sLB));
        st.go[buf][1][j][tid] = IO::from_f32(ddr);
        if constexpr (GATE) st.go[buf][kOut - 1][j][tid] = IO::from_f32(dyv * ypre * sz * fmaf(zf, 1.0f - sz, 1.0f));
      }
    }
    __syncthreads();
    // this chunk's dB / dC over the workgroup's channels
    {
      const auto rbc = make_rsrc(pbc + static_cast<int64_t>(c) * kChunk * M);
      for (int i = tid; i < (valid < kChunk ? valid : kChunk) * M; i += kBlock) {
        const int j = i / M, k = i % M;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kBlock / 64; ++w) sum += st.red[w][j][k];
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sum), rbc,
                                              static_cast<uint32_t>(i) * 4u, 0, 0);
      }
    }
    if (c > 0) {
      tc.land(kIn, &st.in[buf ^ 1][0][0][0], regs);
      tc.land_bc(bcv, st.bc[buf ^ 1]);
      wait_vmem();
    }
    __syncthreads();
  }
  put(0, 0);
  if (!active) return;
  if (s == 0 && a.dh0) {
#pragma unroll
    for (int n = 0; n < N; ++n) a.dh0[tc.row * N + n] = m[n];
  }
  const int64_t part = static_cast<int64_t>(s) * g.batch + tc.b;
#pragma unroll
  for (int n = 0; n < N; ++n) a.pA[(part * g.dim + tc.d) * N + n] = dA[n];
  a.pDb[(part * 2) * g.dim + tc.d] = dD;
  a.pDb[(part * 2 + 1) * g.dim + tc.d] = dbias;
}

// ---------------------------------------------------------------------------
// 4. Sums of the partials.
// sum_{k < count} p[k * stride] in four interleaved partial sums (their loads
// in flight together), added in a fixed order.
__device__ __forceinline__ float strided_sum(const float* __restrict__ p, int64_t stride,
                                            int64_t count) {
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
  int64_t k = 0;
  for (; k + 4 <= count; k += 4) {
    s0 += p[k * stride];
    s1 += p[(k + 1) * stride];
    s2 += p[(k + 2) * stride];
    s3 += p[(k + 3) * stride];
  }
  for (; k < count; ++k) s0 += p[k * stride];
  return (s0 + s1) + (s2 + s3);
}

// dA[d, n] = sum_p pA[p, d, n]; dD[d], dbias[d] likewise from pDb[p, 0 / 1, d].
template <int N>
__global__ __launch_bounds__(kAuxBlock) void bwd_param_sum_kernel(const float* __restrict__ pA,
                                                               const float* __restrict__ pDb,
                                                               float* __restrict__ dA,
                                                               float* __restrict__ dD,
                                                               float* __restrict__ dbias,
                                                               int64_t dim, int64_t parts) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kAuxBlock + threadIdx.x;
  const int64_t na = dim * N;
  if (i < na) {
    dA[i] = strided_sum(pA + i, na, parts);
  } else if (i < na + 2 * dim) {
    const int64_t j = i - na;
    const int64_t which = j / dim, d = j % dim;
    float* outp = which == 0 ? dD : dbias;
    if (outp) outp[d] = strided_sum(pDb + which * dim + d, 2 * dim, parts);
  }
}

// dB[b, t, g, n] = sum over the channel tiles of group g of pBC[tile, b, t, n],
// dC from n + N (tiles_per_group consecutive tiles per group).
template <int N>
__global__ __launch_bounds__(kAuxBlock) void bwd_bc_sum_kernel(const float* __restrict__ pBC,
                                                            float* __restrict__ dB,
                                                            float* __restrict__ dC,
                                                            int64_t tokens, int64_t ngroups,
                                                            unsigned tiles_per_group) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kAuxBlock + threadIdx.x;
  const int64_t total = tokens * ngroups * 2 * N;
  if (i >= total) return;
  const int k = static_cast<int>(i % (2 * N));
  const int64_t tg = i / (2 * N);  // token * ngroups + group
  const int64_t tok = tg / ngroups, grp = tg % ngroups;
  const int64_t tile_stride = tokens * 2 * N;  // one tile's partials
  const float acc = strided_sum(pBC + grp * tiles_per_group * tile_stride + tok * 2 * N + k,
                                tile_stride, tiles_per_group);
  if (k < N)
    dB[tg * N + k] = acc;
  else
    dC[tg * N + k - N] = acc;
}

// dst[i] = src[i], or 0 without src.
__global__ __launch_bounds__(kAuxBlock) void bwd_fill_kernel(float* dst, const float* src,
                                                             int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kAuxBlock + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}

hipError_t fill(float* dst, const float* src, int64_t n, hipStream_t stream) {
  if (!dst || n <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_fill_kernel, dim3(static_cast<unsigned>((n + kAuxBlock - 1) / kAuxBlock)),
                     dim3(kAuxBlock), 0, stream, dst, src, n);
  return hipGetLastError();
}

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

template <int N, class IO, bool GATE, int CW>
hipError_t launch_typed(const ScanBwdProblem& p, const ScanBwdPlan& plan, char* ws,
                        hipStream_t stream) {
  BwdDims g;
  g.batch = p.batch;
  g.seqlen = p.seqlen;
  g.dim = p.dim;
  g.rows = p.batch * p.dim;
  g.seg_len = plan.seg.seg_len;
  g.segments = plan.seg.segments;
  g.tiles = static_cast<unsigned>((p.dim + kBlock - 1) / kBlock);
  g.ngroups = p.ngroups;
  g.group_dim = p.dim / p.ngroups;
  BwdPtrs a;
  a.x = p.x;
  a.delta = p.delta;
  a.B = p.B;
  a.C = p.C;
  a.z = p.z;
  a.dy = p.dout;
  a.A = p.A;
  a.D = p.D;
  a.bias = p.bias;
  a.h0 = p.h0;
  a.dlast = p.dlast;
  a.dx = p.dx;
  a.ddelta = p.ddelta;
  a.dz = p.dz;
  a.dh0 = p.dh0;
  a.carry_h = reinterpret_cast<float*>(ws);
  a.carry_hs = a.carry_h + static_cast<int64_t>(g.segments > 1 ? g.segments - 1 : 0) * g.rows * N;
  a.carry_a = reinterpret_cast<float*>(ws + plan.adj_off);
  a.carry_s = a.carry_a + static_cast<int64_t>(g.segments > 1 ? g.segments - 1 : 0) * g.rows * N;
  a.ck = reinterpret_cast<float*>(ws + plan.ck_off);
  a.ck_s = reinterpret_cast<float*>(ws + plan.cks_off);
  a.pA = reinterpret_cast<float*>(ws + plan.pa_off);
  a.pDb = reinterpret_cast<float*>(ws + plan.pdb_off);
  a.pBC = reinterpret_cast<float*>(ws + plan.pbc_off);
  a.tile_flags = reinterpret_cast<uint32_t*>(ws + plan.flags_off);

  const unsigned blocks = g.tiles * static_cast<unsigned>(p.batch);
  hipLaunchKernelGGL((bwd_state_checkpoint_kernel<N, IO, CW, true>), dim3(blocks, g.segments),
                     dim3(kBlock), 0, stream, a, g);
  hipLaunchKernelGGL((bwd_state_checkpoint_kernel<N, IO, CW, false>), dim3(blocks, g.segments),
                     dim3(kBlock), 0, stream, a, g);
  if (g.segments > 1) {
    hipError_t e = launch_scan_combine(p.A, a.carry_h, a.carry_hs, p.h0, g.rows, p.dim, N,
                                       g.segments, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_adjoint_aggregate_kernel<N, IO, GATE, CW, true>),
                       dim3(blocks, g.segments - 1), dim3(kBlock), 0, stream, a, g);
    hipLaunchKernelGGL((bwd_adjoint_aggregate_kernel<N, IO, GATE, CW, false>),
                       dim3(blocks, g.segments - 1), dim3(kBlock), 0, stream, a, g);
    const int64_t work = g.rows * N;
    hipLaunchKernelGGL((bwd_adjoint_fold_kernel<N>),
                       dim3(static_cast<unsigned>((work + kAuxBlock - 1) / kAuxBlock)),
                       dim3(kAuxBlock), 0, stream, p.A, a.carry_a, a.carry_s, p.dlast, g.rows, p.dim,
                       g.segments);
  }
  hipLaunchKernelGGL((scan_bwd_kernel<N, IO, GATE, CW, true>), dim3(blocks, g.segments),
                     dim3(kBlock), 0, stream, a, g);
  hipLaunchKernelGGL((scan_bwd_kernel<N, IO, GATE, CW, false>), dim3(blocks, g.segments),
                     dim3(kBlock), 0, stream, a, g);
  const int64_t nparam = p.dim * N + 2 * p.dim;
  hipLaunchKernelGGL((bwd_param_sum_kernel<N>),
                     dim3(static_cast<unsigned>((nparam + kAuxBlock - 1) / kAuxBlock)),
                     dim3(kAuxBlock), 0, stream, a.pA, a.pDb, p.dA, p.dD, p.dbias, p.dim,
                     static_cast<int64_t>(g.segments) * p.batch);
  const int64_t tokens = p.batch * p.seqlen;
  const int64_t nbc = tokens * p.ngroups * 2 * N;
  hipLaunchKernelGGL((bwd_bc_sum_kernel<N>),
                     dim3(static_cast<unsigned>((nbc + kAuxBlock - 1) / kAuxBlock)),
                     dim3(kAuxBlock), 0, stream, a.pBC, p.dB, p.dC, tokens, p.ngroups,
                     static_cast<unsigned>(g.tiles / p.ngroups));
  return hipGetLastError();
}

// Copy width of the tile moves (see the forward scan): every tensor moved
// through a tile must allow it.
template <int N, class IO, bool GATE>
hipError_t launch_copy_width(const ScanBwdProblem& p, const ScanBwdPlan& plan, char* ws,
                             hipStream_t st) {
  constexpr int eb = sizeof(typename IO::raw);
  const void* ptrs[] = {p.x, p.delta, p.dout, p.z, p.dx, p.ddelta, p.dz};
  bool a16 = (p.dim * eb) % 16 == 0, a4 = (p.dim * eb) % 4 == 0;
  for (const void* q : ptrs) {
    if (!q) continue;
    a16 = a16 && reinterpret_cast<uintptr_t>(q) % 16 == 0;
    a4 = a4 && reinterpret_cast<uintptr_t>(q) % 4 == 0;
  }
  if (a16) return launch_typed<N, IO, GATE, 16>(p, plan, ws, st);
  if (a4) return launch_typed<N, IO, GATE, 4>(p, plan, ws, st);
  return launch_typed<N, IO, GATE, 0>(p, plan, ws, st);
}

template <class IO, bool GATE>
hipError_t dispatch_n(const ScanBwdProblem& p, const ScanBwdPlan& plan, char* ws, hipStream_t st) {
  switch (p.dstate) {
    case 1: return launch_copy_width<1, IO, GATE>(p, plan, ws, st);
    case 2: return launch_copy_width<2, IO, GATE>(p, plan, ws, st);
    case 4: return launch_copy_width<4, IO, GATE>(p, plan, ws, st);
    case 8: return launch_copy_width<8, IO, GATE>(p, plan, ws, st);
    case 16: return launch_copy_width<16, IO, GATE>(p, plan, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

ScanBwdPlan plan_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int dstate,
                          int forced_segments) {
  ScanBwdPlan plan{};
  const int64_t rows = batch * dim;
  int segs = forced_segments;
  if (segs <= 0 && rows > 0 && seqlen > 0) {
    // Cut the sequence into enough segments for about four rounds of the main
    // pass's resident workgroups, each at least 48 steps long. (On the
    // 8 x 2048 x 5120 layer: 12 segments, 1.49 ms per call against 1.55 ms with
    // two rounds; with two workgroups per compute unit the last, partly filled
    // round costs less when the rounds are short.)
    const int64_t blocks = batch * ((dim + kBlock - 1) / kBlock);
    const int64_t slots = static_cast<int64_t>(device_cu_count()) * kMainBlocksPerCU<Bf16Io>;
    int64_t v = 4 * slots / blocks;
    if (v > seqlen / 48) v = seqlen / 48;
    segs = static_cast<int>(v < 1 ? 1 : (v > 4096 ? 4096 : v));
  }
  plan.seg = plan_scan(batch, seqlen, dim, dstate, segs > 0 ? segs : 1, dim);
  if (rows <= 0 || seqlen <= 0) return plan;
  const size_t S = static_cast<size_t>(plan.seg.segments);
  const size_t N = static_cast<size_t>(dstate);
  const size_t R = static_cast<size_t>(rows);
  const size_t tiles = static_cast<size_t>((dim + kBlock - 1) / kBlock);
  const size_t chunks = static_cast<size_t>((seqlen + kChunk - 1) / kChunk);
  // segment end states and Delta sums (carries after the combine)
  size_t off = round256((S - 1) * R * (N + 1) * sizeof(float));
  plan.adj_off = off;
  off += round256((S - 1) * R * (N + 1) * sizeof(float));
  plan.ck_off = off;
  off += round256(chunks * R * N * sizeof(float));
  plan.cks_off = off;
  off += round256(chunks * R * sizeof(float));
  plan.pa_off = off;
  off += round256(S * R * N * sizeof(float));
  plan.pdb_off = off;
  off += round256(S * R * 2 * sizeof(float));
  plan.pbc_off = off;
  off += round256(tiles * static_cast<size_t>(batch) * static_cast<size_t>(seqlen) * 2 * N *
                  sizeof(float));
  plan.flags_off = off;
  off += round256(tiles * sizeof(uint32_t));
  plan.workspace_bytes = off;
  return plan;
}

hipError_t launch_scan_bwd(const ScanBwdProblem& p, const ScanBwdPlan& plan, void* workspace,
                           hipStream_t stream) {
  if (p.dim == 0) return hipSuccess;
  if (p.batch == 0 || p.seqlen == 0) {
    // no steps: the adjoint passes through unchanged, every sum is empty
    hipError_t e = fill(p.dA, nullptr, p.dim * p.dstate, stream);
    if (e == hipSuccess) e = fill(p.dD, nullptr, p.dim, stream);
    if (e == hipSuccess) e = fill(p.dbias, nullptr, p.dim, stream);
    if (e == hipSuccess) e = fill(p.dh0, p.dlast, p.batch * p.dim * p.dstate, stream);
    return e;
  }
  char* ws = static_cast<char*>(workspace);
  if (p.io == kIoBf16)
    return p.z ? dispatch_n<Bf16Io, true>(p, plan, ws, stream)
               : dispatch_n<Bf16Io, false>(p, plan, ws, stream);
  return p.z ? dispatch_n<F32Io, true>(p, plan, ws, stream)
             : dispatch_n<F32Io, false>(p, plan, ws, stream);
}

}  // namespace mscan
