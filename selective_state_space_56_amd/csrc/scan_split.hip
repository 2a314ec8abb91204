// Full-sequence selective scan (S6) on gfx950 with the N = 16 states of each
// channel row spread over four lanes, the whole sequence in one pass.
//
// The recurrence, its discretisation and the fused epilogue are those of the
// segmented scan ("Mamba and selective state spaces, from first principles",
// sections "Discretization" and "The hardware-aware scan"): per step
// Delta = softplus(Delta_raw + bias), h_n = exp(Delta A_n) h_n + Delta B_n x,
// y = (sum_n C_n h_n + D x) silu(z).
//
// Why four lanes per row: one lane per row leaves a layer of batch x dim rows
// (8 x 5120) with under one wave per SIMD, so the segmented scan cuts time
// into segments and pays for a second pass over every segment (aggregate,
// then output). Four lanes per row give the same layer 2.5 waves per SIMD
// with no segments, so every step is computed once. The per-step work that
// does not depend on the state (softplus, exponentials, the gate) is split
// over the four lanes of a row too: each computes it for two of every eight
// steps and shares it through LDS. The per-row read-out sum over n is a sum
// over the four lanes (two cross-lane adds within the quad).
//
// Structured rows (A[d, n] = (n + 1) A[d, 0], S4D-Real) keep the rescaled
// state g_n = h_n / dx_t of the segmented scan (dx_t = Delta_t x_t, kept away
// from zero): g_n,t = rho_t e_t^(n+1) g_n,t-1 + B_t,n with rho_t =
// dx_t-1 / dx_t and e_t = exp(Delta_t A[d, 0]); y_t = dx_t sum_n C_t,n g_n,t
// + D x_t. The front-end lane of a step writes, per lane q of the row, the
// decay of that lane's first state, rho e^(4q+1), and e; the lane forms its
// other three decays as successive products with e. General rows keep h and
// compute exp(Delta A_n) per state from Delta and dx.
//
// It runs only on request (MAMBA_SCAN_SPLIT_STATES): although it issues
// about 100 vector instructions per row-step against about 170 for the
// segmented scan's two passes, it keeps the vector units busy only about
// half the time and measured slower on the layers tried.
#include <type_traits>

#include "scan_split.h"
#include "tile_io.h"

namespace mscan {
namespace {

constexpr int kSplitState = 16;                           // N
constexpr int kSplitLanes = 4;                            // lanes per channel row
constexpr int kLaneStates = kSplitState / kSplitLanes;    // states per lane
constexpr int kSplitBlock = 256;                          // threads per workgroup
constexpr int kSplitRows = kSplitBlock / kSplitLanes;     // channel rows per workgroup
constexpr int kSplitChunk = kChunk;                       // steps per chunk (8)
constexpr int kFeSteps = kSplitChunk / kSplitLanes;       // front-end steps per lane per chunk
constexpr int kSplitWaves = kSplitBlock / 64;
constexpr int kBcPerLane = kSplitChunk * 2 * kSplitState / 64;  // B/C tile elements per lane
static_assert(kBcPerLane * 64 == kSplitChunk * 2 * kSplitState, "whole B/C tile per wave");
constexpr float kSplitDxFloor = 1e-20f;

// LDS record of one step: per row 8 floats, the (value, e) pairs of lanes
// q = 0..3 in two 16-byte halves (lanes 0, 1 | lanes 2, 3), plus 16 bytes of
// padding per step. The front-end lane of a step writes a row's two halves
// with two 16-byte stores; the four lanes of a quad write four different
// steps 2q + k, and lanes with odd q store the halves swapped: with the odd
// step stride (129 16-byte units) the eight lanes of two rows then reach
// eight different 16-byte bank groups in each store. Readers of step t undo
// the swap when t's front-end lane (t / 2) is odd.
constexpr int kRecStride = kSplitRows * 8 + 4;  // floats per step

struct SplitDims {
  int64_t seqlen, dim;
  int64_t sx, sd, sz, so, sbc;  // elements between consecutive steps
  int64_t group_dim;
  unsigned tiles;               // channel tiles of kSplitRows per batch row
};

// Inputs of one chunk held in registers between their loads and the front-end.
// (The B/C tile element arrives as two loads, one of them masked to 0, that
// are combined only in the front-end, so nothing waits for them earlier.)
template <class IO>
struct SplitLoads {
  typename IO::raw x[kFeSteps], d[kFeSteps], z[kFeSteps];
  typename IO::raw b[kBcPerLane], c[kBcPerLane];
};

// Lane permutations within a quad of lanes (DPP quad_perm).
template <int CTRL>
__device__ __forceinline__ float quad_perm(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
// v + v of the lane CTRL selects (one add with a DPP source operand)
template <int CTRL>
__device__ __forceinline__ float quad_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
constexpr int kSwap1 = 0xB1;  // lanes (1, 0, 3, 2)
constexpr int kSwap2 = 0x4E;  // lanes (2, 3, 0, 1)
constexpr int kRotate = 0x93; // lane q reads lane q - 1 (lane 0 reads lane 3)
constexpr int kLast = 0xFF;   // every lane reads lane 3

// Every LDS value a lane reads was written by a lane of its own wave (the
// records of a row by the row's four lanes, B and C by the wave's own copy),
// so the chunks need no workgroup barrier: the LDS executes one wave's
// instructions in order, and this keeps the compiler from moving LDS
// accesses across the point.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Grid: x = batch * channel tiles. Thread tid handles channel row
// d0 + tid / 4 and its states 4 (tid % 4) .. 4 (tid % 4) + 3.
template <class IO, bool GATE>
__global__ __launch_bounds__(kSplitBlock, 3) void scan_split_kernel(
    const typename IO::raw* __restrict__ x, const typename IO::raw* __restrict__ delta,
    const float* __restrict__ A, const typename IO::raw* __restrict__ B,
    const typename IO::raw* __restrict__ C, const float* __restrict__ D,
    const typename IO::raw* __restrict__ z, const float* __restrict__ bias_p,
    const float* __restrict__ h0, typename IO::raw* __restrict__ out,
    float* __restrict__ last_state, SplitDims g) {
  using raw = typename IO::raw;
  constexpr int eb = sizeof(raw);
  constexpr int Q = kLaneStates;
  // per (step, row, lane): structured rows (rho e^(4q+1), e), general rows
  // (Delta, dx); see kRecStride for the layout
  __shared__ __align__(16) float s_rec[2][kSplitChunk][kRecStride];
  // B and C of the chunk, one copy per wave: [wave][buffer][step][B_n, C_n]
  __shared__ __align__(16) float s_bc[kSplitWaves][2][kSplitChunk][2 * kSplitState];
  __shared__ float s_dx[kSplitRows];

  const int tid = threadIdx.x;
  const int r = tid / kSplitLanes, q = tid % kSplitLanes;
  const int64_t b = blockIdx.x / g.tiles;
  const int64_t d0 = static_cast<int64_t>(blockIdx.x % g.tiles) * kSplitRows;
  const bool active = d0 + r < g.dim;
  // rows past the last channel compute on channel dim - 1 and store nothing
  const int64_t d = active ? d0 + r : g.dim - 1;
  const int rc = static_cast<int>(d - d0);  // the row within the tile that is read
  const int64_t row = b * g.dim + d;
  const int64_t L = g.seqlen;

  // decay path of the workgroup: structured when every row of the tile is
  const float a0 = A[d * kSplitState];
  float A2[Q];  // A[d, n] log2(e) for this lane's states
  bool structured = true;
#pragma unroll
  for (int j = 0; j < Q; ++j) {
    const int n = q * Q + j;
    const float an = A[d * kSplitState + n];
    structured = structured && (an == (n + 1) * a0);
    A2[j] = an * kLog2e;
  }
  const bool tile_structured = __syncthreads_and(structured);
  const float a2_0 = a0 * kLog2e;
  const float Dd = D ? D[d] : 0.0f;
  const float bias = bias_p ? bias_p[d] : 0.0f;

  float h[Q];
#pragma unroll
  for (int j = 0; j < Q; ++j) h[j] = h0 ? h0[row * kSplitState + q * Q + j] : 0.0f;

  // Per-lane byte offsets within a chunk (fixed for the whole sequence): the
  // front-end steps 2q, 2q + 1 of row rc; the output uses kOffNone on
  // inactive rows so its stores are dropped.
  uint32_t off_x[kFeSteps], off_d[kFeSteps], off_z[kFeSteps], off_o[kFeSteps];
#pragma unroll
  for (int k = 0; k < kFeSteps; ++k) {
    const int64_t s = q * kFeSteps + k;
    off_x[k] = static_cast<uint32_t>((s * g.sx + rc) * eb);
    off_d[k] = static_cast<uint32_t>((s * g.sd + rc) * eb);
    off_z[k] = static_cast<uint32_t>((s * g.sz + rc) * eb);
    off_o[k] = active ? static_cast<uint32_t>((s * g.so + rc) * eb) : kOffNone;
  }
  const int64_t step0 = b * L;
  const raw* xb = x + step0 * g.sx + d0;
  const raw* db = delta + step0 * g.sd + d0;
  const raw* zb = GATE ? z + step0 * g.sz + d0 : xb;
  raw* ob = out + step0 * g.so + d0;
  const int64_t grp = d0 / g.group_dim;
  const raw* Bb = B + step0 * g.sbc + grp * kSplitState;
  const raw* Cb = C + step0 * g.sbc + grp * kSplitState;
  const uint32_t bc_row = static_cast<uint32_t>(g.sbc);
  // this lane's elements of the chunk's B/C tile (the wave loads all of it)
  const int lane = tid % 64, wv = tid / 64;
  BcOffsets bco[kBcPerLane];
#pragma unroll
  for (int i = 0; i < kBcPerLane; ++i) bco[i] = bc_offsets<kSplitState, IO>(lane + 64 * i, bc_row);

  // Loads of chunk c: buffer resources from the chunk's first step over its
  // valid steps (steps past the end read 0 and are never used). Chunks past
  // the last are loaded too, over 0 bytes (every load returns 0 and touches
  // no memory): with the same loads on every path the compiler's wait counts
  // stay exact, so the front-end never waits for a later chunk's loads.
  auto load = [&](SplitLoads<IO>& ld, int64_t c) {
    const int64_t t0 = c * kSplitChunk;
    const int64_t rows_left = L - t0 < kSplitChunk ? L - t0 : kSplitChunk;
    const uint32_t left = static_cast<uint32_t>(rows_left > 0 ? rows_left : 0);
    const auto rx = make_rsrc(xb + t0 * g.sx, static_cast<uint32_t>(left * g.sx * eb));
    const auto rd = make_rsrc(db + t0 * g.sd, static_cast<uint32_t>(left * g.sd * eb));
    const auto rz = make_rsrc(zb + t0 * g.sz, static_cast<uint32_t>(left * g.sz * eb));
#pragma unroll
    for (int k = 0; k < kFeSteps; ++k) {
      ld.x[k] = IO::bload(rx, off_x[k], 0);
      ld.d[k] = IO::bload(rd, off_d[k], 0);
      if (GATE) ld.z[k] = IO::bload(rz, off_z[k], 0);
    }
    const uint32_t bc_bytes = static_cast<uint32_t>(left * g.sbc * eb);
    const auto rb = make_rsrc(Bb + t0 * g.sbc, bc_bytes), rcc = make_rsrc(Cb + t0 * g.sbc, bc_bytes);
#pragma unroll
    for (int i = 0; i < kBcPerLane; ++i) {
      ld.b[i] = IO::bload(rb, bco[i].b, 0);
      ld.c[i] = IO::bload(rcc, bco[i].c, 0);
    }
  };

  // Epilogue values of this lane's front-end steps of the current chunk:
  // y = (f acc + Dx) gate, f = dx (structured) or 1.
  float ep_f[kFeSteps], ep_dx[kFeSteps], ep_g[kFeSteps];
  float yacc[kFeSteps];
  float carry = 1.0f;  // structured: dx of the step before the chunk (1 before step 0: g = h0)

  // State-free front-end of the chunk in `ld` into LDS buffer nb.
  auto front = [&](const SplitLoads<IO>& ld, int nb, auto struct_tag) {
    constexpr bool KS = decltype(struct_tag)::value;
    const int swap = (q & 1) * 4;  // floats: odd lanes store the halves swapped
    float dx[kFeSteps], rdx[kFeSteps], e[kFeSteps], Delta[kFeSteps];
#pragma unroll
    for (int k = 0; k < kFeSteps; ++k) {
      const float xf = IO::to_f32(ld.x[k]);
      Delta[k] = softplus_f(IO::to_f32(ld.d[k]) + bias);
      if (KS) {
        dx[k] = fmaf(Delta[k], xf, copysignf(kSplitDxFloor, xf));
        rdx[k] = hw_rcp(dx[k]);
        e[k] = hw_exp2(Delta[k] * a2_0);
        ep_f[k] = dx[k];
      } else {
        dx[k] = Delta[k] * xf;
        ep_f[k] = 1.0f;
      }
      ep_dx[k] = Dd * xf;
      ep_g[k] = GATE ? silu_f(IO::to_f32(ld.z[k])) : 1.0f;
    }
    if (KS) {
      // dx of the step before each front-end step: the previous lane's last
      // step, or for lane 0 the last step of the previous chunk
      const float prev_last = quad_perm<kRotate>(dx[kFeSteps - 1]);
      const float before = q == 0 ? carry : prev_last;
      carry = quad_perm<kLast>(dx[kFeSteps - 1]);
#pragma unroll
      for (int k = 0; k < kFeSteps; ++k) {
        const float rho = (k == 0 ? before : dx[k - 1]) * rdx[k];
        const float p0 = rho * e[k];
        const float e2 = e[k] * e[k];
        const float e4 = e2 * e2;
        const float p1 = p0 * e4, p2 = p1 * e4, p3 = p2 * e4;
        float* rec = &s_rec[nb][q * kFeSteps + k][r * 8];
        *reinterpret_cast<float4*>(rec + swap) = make_float4(p0, e[k], p1, e[k]);
        *reinterpret_cast<float4*>(rec + (4 ^ swap)) = make_float4(p2, e[k], p3, e[k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < kFeSteps; ++k) {
        float* rec = &s_rec[nb][q * kFeSteps + k][r * 8];
        *reinterpret_cast<float4*>(rec + swap) = make_float4(Delta[k], dx[k], Delta[k], dx[k]);
        *reinterpret_cast<float4*>(rec + (4 ^ swap)) = make_float4(Delta[k], dx[k], Delta[k], dx[k]);
      }
    }
#pragma unroll
    for (int i = 0; i < kBcPerLane; ++i)
      (&s_bc[wv][nb][0][0])[lane + 64 * i] = IO::to_f32(IO::bit_or(ld.b[i], ld.c[i]));
  };

  // State updates of the chunk in LDS buffer nb (`valid` steps).
  auto states = [&](int nb, int valid, auto struct_tag, auto full_tag) {
    constexpr bool KS = decltype(struct_tag)::value;
    constexpr bool FULL = decltype(full_tag)::value;
    // LDS reads ahead of their use: the chunk's eight decay records at once,
    // B and C two steps ahead (every slot of the buffer is readable; values
    // of steps past the end are never used)
    float2 pe_t[kSplitChunk];
    float4 Bt[kSplitChunk], Ct[kSplitChunk];
    auto read_bc = [&](int t) {
      Bt[t] = *reinterpret_cast<const float4*>(&s_bc[wv][nb][t][q * Q]);
      Ct[t] = *reinterpret_cast<const float4*>(&s_bc[wv][nb][t][kSplitState + q * Q]);
    };
#pragma unroll
    for (int t = 0; t < kSplitChunk; ++t) {
      const int qs = ((t / kFeSteps) & 1) ? (q ^ 2) : q;  // the writer's half swap
      pe_t[t] = *reinterpret_cast<const float2*>(&s_rec[nb][t][r * 8 + 2 * qs]);
    }
    read_bc(0);
    read_bc(1);
#pragma unroll
    for (int t = 0; t < kSplitChunk; ++t) {
      if (t + 2 < kSplitChunk) read_bc(t + 2);
      if (FULL || t < valid) {
        const float2 pe = pe_t[t];
        const float4 Bv = Bt[t];
        const float4 Cv = Ct[t];
        const float bv[Q] = {Bv.x, Bv.y, Bv.z, Bv.w};
        const float cv[Q] = {Cv.x, Cv.y, Cv.z, Cv.w};
        float acc = 0.0f;
        if (KS) {
          float a = pe.x;
#pragma unroll
          for (int j = 0; j < Q; ++j) {
            if (j > 0) a *= pe.y;
            h[j] = fmaf(a, h[j], bv[j]);
            acc = fmaf(cv[j], h[j], acc);
          }
        } else {
#pragma unroll
          for (int j = 0; j < Q; ++j) {
            h[j] = fmaf(hw_exp2(pe.x * A2[j]), h[j], pe.y * bv[j]);
            acc = fmaf(cv[j], h[j], acc);
          }
        }
        acc = quad_add<kSwap1>(acc);
        acc = quad_add<kSwap2>(acc);
        if (q == t / kFeSteps) yacc[t % kFeSteps] = acc;
      }
    }
  };

  // y of this lane's front-end steps of the chunk at t0 (rows past the end
  // and inactive rows are dropped by the resource range and kOffNone).
  auto epilogue = [&](int64_t t0) {
    const uint32_t left = static_cast<uint32_t>(L - t0 < kSplitChunk ? L - t0 : kSplitChunk);
    const auto ro = make_rsrc(ob + t0 * g.so, static_cast<uint32_t>(left * g.so * eb));
#pragma unroll
    for (int k = 0; k < kFeSteps; ++k) {
      float y = fmaf(ep_f[k], yacc[k], ep_dx[k]);
      if (GATE) y *= ep_g[k];
      IO::bstore(IO::from_f32(y), ro, off_o[k], 0);
    }
  };

  const int64_t n_chunks = (L + kSplitChunk - 1) / kSplitChunk;
  SplitLoads<IO> la, lb;

  auto run = [&](auto struct_tag) {
    load(la, 0);
    load(lb, 1);
    front(la, 0, struct_tag);
    wave_sync();
    // chunk c: loads of chunk c + 2 into the set the front-end of chunk c
    // has consumed, the states of chunk c, its outputs, then the front-end
    // of chunk c + 1 (loaded one chunk earlier) into the other LDS buffer
    auto chunk = [&](int64_t c, SplitLoads<IO>& mine, SplitLoads<IO>& next, auto nb_tag) {
      constexpr int NB = decltype(nb_tag)::value;  // c & 1
      load(mine, c + 2);
      __builtin_amdgcn_sched_barrier(0);
      const int64_t t0 = c * kSplitChunk;
      if (c + 1 < n_chunks) {
        // a full chunk and the next chunk's front-end in one straight-line
        // block, so the compiler can interleave the two (the front-end's
        // exponentials fill the waits on the state updates' LDS reads)
        states(NB, kSplitChunk, struct_tag, std::true_type{});
        epilogue(t0);
        front(next, NB ^ 1, struct_tag);
      } else {
        const int valid = static_cast<int>(L - t0);
        if (valid == kSplitChunk)
          states(NB, valid, struct_tag, std::true_type{});
        else
          states(NB, valid, struct_tag, std::false_type{});
        epilogue(t0);
      }
      wave_sync();
    };
    for (int64_t c = 0; c < n_chunks; c += 2) {
      chunk(c, la, lb, std::integral_constant<int, 0>{});
      if (c + 1 < n_chunks) chunk(c + 1, lb, la, std::integral_constant<int, 1>{});
    }
    if (decltype(struct_tag)::value && last_state) {
      // back from g to h: dx of the last step, held by its front-end lane
      const int j = static_cast<int>((L - 1) % kSplitChunk);
      if (q == j / kFeSteps) s_dx[r] = ep_f[j % kFeSteps];
      wave_sync();
      const float dxl = s_dx[r];
#pragma unroll
      for (int k = 0; k < Q; ++k) h[k] *= dxl;
    }
  };
  if (L > 0) {
    if (tile_structured)
      run(std::true_type{});
    else
      run(std::false_type{});
  }
  if (active && last_state) {
#pragma unroll
    for (int j = 0; j < Q; ++j) last_state[row * kSplitState + q * Q + j] = h[j];
  }
}

template <class IO>
hipError_t launch_split_typed(const ScanProblem& p, hipStream_t stream) {
  using raw = typename IO::raw;
  SplitDims g;
  g.seqlen = p.seqlen;
  g.dim = p.dim;
  g.sx = p.sx;
  g.sd = p.sd;
  g.sz = p.z ? p.sz : p.sx;
  g.so = p.so;
  g.sbc = p.sbc;
  g.group_dim = p.dim / p.ngroups;
  g.tiles = static_cast<unsigned>((p.dim + kSplitRows - 1) / kSplitRows);
  const dim3 grid(g.tiles * static_cast<unsigned>(p.batch));
  const raw* x = static_cast<const raw*>(p.x);
  const raw* dl = static_cast<const raw*>(p.delta);
  const raw* B = static_cast<const raw*>(p.B);
  const raw* C = static_cast<const raw*>(p.C);
  const raw* z = static_cast<const raw*>(p.z);
  raw* out = static_cast<raw*>(p.out);
  if (z)
    hipLaunchKernelGGL((scan_split_kernel<IO, true>), grid, dim3(kSplitBlock), 0, stream, x, dl,
                       p.A, B, C, p.D, z, p.bias, p.h0, out, p.last_state, g);
  else
    hipLaunchKernelGGL((scan_split_kernel<IO, false>), grid, dim3(kSplitBlock), 0, stream, x, dl,
                       p.A, B, C, p.D, z, p.bias, p.h0, out, p.last_state, g);
  return hipGetLastError();
}

}  // namespace

bool scan_split_fits(int64_t dstate, int64_t row_elems, int io) {
  const int64_t eb = io == kIoBf16 ? 2 : 4;
  // every in-chunk byte offset (kSplitChunk steps of the widest row) fits in 31 bits
  return dstate == kSplitState && row_elems * eb * (kSplitChunk + 1) < (int64_t(1) << 31);
}

hipError_t launch_scan_split(const ScanProblem& p, hipStream_t stream) {
  if (p.dstate != kSplitState || p.zoh) return hipErrorInvalidValue;
  if (p.io == kIoBf16) return launch_split_typed<Bf16Io>(p, stream);
  return launch_split_typed<F32Io>(p, stream);
}

}  // namespace mscan
