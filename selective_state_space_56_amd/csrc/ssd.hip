// Mamba-2 state space duality (SSD) layer on gfx950, by the chunked algorithm
// ("Mamba and selective state spaces, from first principles", section "Mamba-2:
// state space duality"): per head h, a_t = exp(Delta_t A_h) is a scalar, the
// head's P channels share a_t, B_t, C_t, and the state is an N x P matrix
//   S_t = a_t S_{t-1} + Delta_t B_t x_t^T,   y_t = S_t^T C_t + D_h x_t.
// Unrolled, Y = (L o C B^T)(Delta X) + D X with the decay mask
// L[t, s] = exp(ell_t - ell_s) for s <= t (ell: running sum of Delta A_h). The
// sequence is cut into chunks of kQ steps; inside a chunk the attention form
// runs on the matrix cores, across chunks the states are passed with the scalar
// recurrence, and each chunk adds the contribution of the state it inherits:
//   1. chunk state: S_c = sum_s exp(ell_end - ell_s) Delta_s B_s x_s^T
//      (one matrix product per chunk and head);
//   2. state pass: S_in(c + 1) = exp(ell_end(c)) S_in(c) + S_c (elementwise,
//      kQ times shorter than the sequence);
//   3. chunk scan: Y = (L o C B^T)(Delta X) + diag(exp(ell_t)) C S_in(c) + D X,
//      the scores C B^T formed once per chunk and group of heads.
// Products take bf16 operands and accumulate in fp32 (v_mfma_f32_32x32x16_bf16:
// 32 x 32 tiles, K = 16). Operand layouts of that instruction (wave64, lane l):
//   A (32 x 16): lane l holds row l % 32, k = 8 (l / 32) .. 8 (l / 32) + 7;
//   B (16 x 32): lane l holds column l % 32, the same k;
//   D (32 x 32): register r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4,
//                column l % 32.
#include "device_math.h"
#include "kernels.h"

namespace mscan {

namespace {

constexpr int kQ = 256;       // chunk length (steps)
constexpr int kP = 64;        // head dimension
constexpr int kN = 128;       // state size
constexpr int kThreads = 256; // four waves
constexpr int kSBlk = 64;     // steps per LDS block of the chunk-state product
constexpr int kPad = 8;       // bf16 padding of LDS rows (keeps rows 16-byte aligned, spreads banks)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t to_bf16(float v) {
  __bf16 b = static_cast<__bf16>(v);
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ float from_bf16(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Eight bf16 at p (16-byte aligned), as an MFMA operand.
__device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
}

struct SsdDims {
  int64_t batch, seqlen, nheads, ngroups;
  int chunks;
};

// Delta_t = softplus(dt + bias) of the workgroup's chunk, one step per thread
// (zero past the sequence's end), and ell_t = sum_{u <= t} Delta_u A_h, an
// inclusive prefix sum over the chunk (wave scans, then the wave totals).
__device__ __forceinline__ void chunk_decay(const uint16_t* __restrict__ dt, float bias, float A_h,
                                            const SsdDims& g, int64_t b, int64_t h, int c,
                                            float* s_delta, float* s_ell, float* s_wave) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int64_t t = static_cast<int64_t>(c) * kQ + tid;
  float Delta = 0.0f;
  if (t < g.seqlen) Delta = softplus_f(from_bf16(dt[(b * g.seqlen + t) * g.nheads + h]) + bias);
  float v = Delta * A_h;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) s_wave[wv] = v;
  __syncthreads();
  float base = 0.0f;
  for (int w = 0; w < wv; ++w) base += s_wave[w];
  s_delta[tid] = Delta;
  s_ell[tid] = base + v;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// 1. Chunk states. Grid (chunks, heads, batch). S_c[p][n] (fp32, [b][h][c][p][n])
// = sum_s w_s x_s[p] B_s[n], w_s = exp(ell_end - ell_s) Delta_s, as the product
// of (w o X)^T (P x Q) and B (Q x N), K = s. Both operands are transposed
// through LDS (s contiguous) one block of kSBlk steps at a time; w x is kept
// as a bf16 pair hi + lo (two products), so the weights lose no precision to
// the bf16 operands. Wave w owns the 32 states n of tile w and both
// 32-channel tiles of p.
__global__ __launch_bounds__(kThreads) void ssd_chunk_state_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ B, const float* __restrict__ dt_bias, float* __restrict__ Sc,
    float* __restrict__ ell_end, SsdDims g) {
  __shared__ float s_delta[kQ], s_ell[kQ], s_wave[4];
  __shared__ __align__(16) uint16_t s_xh[kP][kSBlk + kPad];  // (w o X)^T block, hi part
  __shared__ __align__(16) uint16_t s_xl[kP][kSBlk + kPad];  // lo part
  __shared__ __align__(16) uint16_t s_b[kN][kSBlk + kPad];   // B^T block
  const int c = blockIdx.x;
  const int64_t h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t grp = h / (g.nheads / g.ngroups);
  chunk_decay(dt, dt_bias ? dt_bias[h] : 0.0f, A[h], g, b, h, c, s_delta, s_ell, s_wave);
  const float ell_last = s_ell[kQ - 1];

  f32x16 acc[2] = {};
  for (int s0 = 0; s0 < kQ; s0 += kSBlk) {
    // stage: thread -> step s0 + tid / 4, a quarter of its channels / states
    {
      const int sl = tid >> 2, part = tid & 3;
      const int64_t t = static_cast<int64_t>(c) * kQ + s0 + sl;
      const bool in = t < g.seqlen;
      const float w = in ? hw_exp2((ell_last - s_ell[s0 + sl]) * kLog2e) * s_delta[s0 + sl] : 0.0f;
      u16x8 xv[2] = {}, bv[4] = {};
      if (in) {
        const u16x8* xr = reinterpret_cast<const u16x8*>(
            x + ((b * g.seqlen + t) * g.nheads + h) * kP + part * 16);
        const u16x8* br = reinterpret_cast<const u16x8*>(
            B + ((b * g.seqlen + t) * g.ngroups + grp) * kN + part * 32);
        xv[0] = xr[0];
        xv[1] = xr[1];
#pragma unroll
        for (int q = 0; q < 4; ++q) bv[q] = br[q];
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float v = from_bf16(xv[k / 8][k % 8]) * w;
        const uint16_t vh = to_bf16(v);
        s_xh[part * 16 + k][sl] = vh;
        s_xl[part * 16 + k][sl] = to_bf16(v - from_bf16(vh));
      }
#pragma unroll
      for (int k = 0; k < 32; ++k) s_b[part * 32 + k][sl] = bv[k / 8][k % 8];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kSBlk; kk += 16) {
      const int kofs = kk + 8 * (lane >> 5);
      const bf16x8 bop = load8(&s_b[wv * 32 + (lane & 31)][kofs]);
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
        acc[pt] = mfma(load8(&s_xh[pt * 32 + (lane & 31)][kofs]), bop, acc[pt]);
        acc[pt] = mfma(load8(&s_xl[pt * 32 + (lane & 31)][kofs]), bop, acc[pt]);
      }
    }
    __syncthreads();
  }
  float* out = Sc + (((b * g.nheads + h) * g.chunks + c) * kP) * kN;
#pragma unroll
  for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int p = pt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      out[p * kN + wv * 32 + (lane & 31)] = acc[pt][r];
    }
  }
  if (tid == 0) ell_end[(b * g.nheads + h) * g.chunks + c] = ell_last;
}

// ---------------------------------------------------------------------------
// 2. State pass. One thread per (b, h, p, n): the state entering each chunk,
// S_in(0) = h0 (or 0), S_in(c + 1) = exp(ell_end(c)) S_in(c) + S_c, written as
// a bf16 pair hi + lo, [b][h][c][p][n] each (the operand layout of the chunk
// scan); the final state (fp32, [b][h][n][p]) if asked for. The chunk loads are
// issued kPassAhead at a time.
constexpr int kPassAhead = 8;

__global__ __launch_bounds__(kThreads) void ssd_state_pass_kernel(
    const float* __restrict__ Sc, const float* __restrict__ ell_end, const float* __restrict__ h0,
    uint16_t* __restrict__ Sin_hi, uint16_t* __restrict__ Sin_lo, float* __restrict__ last_state,
    SsdDims g) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t per_head = static_cast<int64_t>(kP) * kN;
  if (i >= g.batch * g.nheads * per_head) return;
  const int64_t bh = i / per_head;
  const int pn = static_cast<int>(i % per_head);
  const int p = pn / kN, n = pn % kN;
  float s = h0 ? h0[bh * per_head + static_cast<int64_t>(n) * kP + p] : 0.0f;
  for (int c0 = 0; c0 < g.chunks; c0 += kPassAhead) {
    float sc[kPassAhead], dec[kPassAhead];
#pragma unroll
    for (int u = 0; u < kPassAhead; ++u) {
      const int c = c0 + u < g.chunks ? c0 + u : g.chunks - 1;
      sc[u] = Sc[(bh * g.chunks + c) * per_head + pn];
      dec[u] = ell_end[bh * g.chunks + c];
    }
#pragma unroll
    for (int u = 0; u < kPassAhead; ++u) {
      if (c0 + u < g.chunks) {
        const int64_t slot = (bh * g.chunks + c0 + u) * per_head + pn;
        const uint16_t hi = to_bf16(s);
        Sin_hi[slot] = hi;
        Sin_lo[slot] = to_bf16(s - from_bf16(hi));
        s = fmaf(hw_exp2(dec[u] * kLog2e), s, sc[u]);
      }
    }
  }
  if (last_state) last_state[bh * per_head + static_cast<int64_t>(n) * kP + p] = s;
}

// ---------------------------------------------------------------------------
// 3a. Chunk scores. Grid (chunks, groups, batch). The raw scores B_s . C_t of
// a chunk do not depend on the head, so they are formed once per (batch,
// chunk, group) for every head that shares the group: the kTiles
// lower-triangular 32 x 32 tiles (s tile j <= t tile i), K = n, each stored in
// the MFMA result layout (s as rows, t as columns) as [tile][register][lane]
// fp32, so that a wave reads it back with coalesced loads.
constexpr int kTiles = (kQ / 32) * (kQ / 32 + 1) / 2;  // 36

__device__ __forceinline__ int tile_index(int i, int j) { return i * (i + 1) / 2 + j; }

__global__ __launch_bounds__(kThreads) void ssd_chunk_scores_kernel(const uint16_t* __restrict__ B,
                                                                    const uint16_t* __restrict__ C,
                                                                    float* __restrict__ scores,
                                                                    SsdDims g) {
  const int c = blockIdx.x;
  const int64_t grp = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int lo = lane & 31, hi = lane >> 5;
  const int64_t t_base = static_cast<int64_t>(c) * kQ;
  auto frag = [&](const uint16_t* T, int64_t t, int kb) -> bf16x8 {
    if (t >= g.seqlen) return bf16x8{};
    return load8(T + ((b * g.seqlen + t) * g.ngroups + grp) * kN + 16 * kb + 8 * hi);
  };
  float* out = scores + ((b * g.chunks + c) * g.ngroups + grp) * (kTiles * 1024);
  // wave w forms tiles w, w + 4, ... in the flat lower-triangular order
  for (int tile = wv; tile < kTiles; tile += 4) {
    int i = 0;
    while (tile_index(i + 1, 0) <= tile) ++i;
    const int j = tile - tile_index(i, 0);
    f32x16 sc = {};
#pragma unroll
    for (int kb = 0; kb < kN / 16; ++kb)
      sc = mfma(frag(B, t_base + 32 * j + lo, kb), frag(C, t_base + 32 * i + lo, kb), sc);
#pragma unroll
    for (int r = 0; r < 16; ++r) out[(tile * 16 + r) * 64 + lane] = sc[r];
  }
}

// ---------------------------------------------------------------------------
// 3. Chunk scan. Grid (chunks, heads, batch). Wave w computes the output rows
// of the 32-step tiles w and 7 - w (the causal triangle split evenly) for both
// 32-channel tiles of p:
//   inherited part: C_t S_in (K = n; S_in as its bf16 pair hi + lo), rows
//     scaled by exp(ell_t);
//   diagonal part, per 32-step tile j <= i of earlier steps s: the chunk's
//     scores B_s . C_t (a 32 x 32 tile with s as rows, from 3a), masked
//     (s <= t) and scaled by exp(ell_t - ell_s) Delta_s, taken off the
//     diagonal as exp(ell_t - ell_ref) exp(ell_ref - ell_s) Delta_s with ell_ref
//     the value at the end of tile j (both factors at most 1; the second kept
//     per step in LDS) and formed directly on the diagonal tile, turned into
//     the A operand (t as rows, s as k) by exchanging
//     register halves across the half-waves, times X (K = s, from LDS);
//   then + D x and one bf16 store per element.
__global__ __launch_bounds__(kThreads, 2) void ssd_chunk_scan_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ B, const uint16_t* __restrict__ C, const float* __restrict__ D,
    const float* __restrict__ dt_bias, const uint16_t* __restrict__ Sin_hi,
    const uint16_t* __restrict__ Sin_lo, const float* __restrict__ scores, uint16_t* __restrict__ y,
    SsdDims g) {
  __shared__ float s_delta[kQ], s_ell[kQ], s_wave[4], s_v[kQ];
  __shared__ __align__(16) uint16_t s_x[kP][kQ + kPad];  // X^T of the chunk
  const int c = blockIdx.x;
  const int64_t h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int lo = lane & 31, hi = lane >> 5;
  const int64_t grp = h / (g.nheads / g.ngroups);
  const int64_t t_base = static_cast<int64_t>(c) * kQ;
  chunk_decay(dt, dt_bias ? dt_bias[h] : 0.0f, A[h], g, b, h, c, s_delta, s_ell, s_wave);
  // per step s: exp(ell_ref - ell_s) Delta_s, ell_ref at the end of the step's 32-step tile
  s_v[tid] = hw_exp2((s_ell[tid | 31] - s_ell[tid]) * kLog2e) * s_delta[tid];
  // X^T of the chunk into LDS: thread -> step tid, all 64 channels (16-byte loads)
  {
    const int64_t t = t_base + tid;
    const u16x8* xr = reinterpret_cast<const u16x8*>(x + ((b * g.seqlen + t) * g.nheads + h) * kP);
#pragma unroll
    for (int q = 0; q < kP / 8; ++q) {
      const u16x8 v = t < g.seqlen ? xr[q] : u16x8{};
#pragma unroll
      for (int k = 0; k < 8; ++k) s_x[8 * q + k][tid] = v[k];
    }
  }
  __syncthreads();
  const float Dh = D ? D[h] : 0.0f;
  const int64_t sin_off = (((b * g.nheads + h) * g.chunks + c) * kP) * kN;
  const uint16_t* sin_hi = Sin_hi + sin_off;
  const uint16_t* sin_lo = Sin_lo + sin_off;
  const float* tiles = scores + ((b * g.chunks + c) * g.ngroups + grp) * (kTiles * 1024);

  // the 8 bf16 at state offset 8 * hi + 16 kb of row t of B or C (zeros past the end)
  auto bc_frag = [&](const uint16_t* T, int64_t t, int kb) -> bf16x8 {
    if (t >= g.seqlen) return bf16x8{};
    return load8(T + ((b * g.seqlen + t) * g.ngroups + grp) * kN + 16 * kb + 8 * hi);
  };

#pragma unroll 1
  for (int which = 0; which < 2; ++which) {
    const int i = which == 0 ? wv : 7 - wv;  // this wave's 32-step tile
    const int64_t t_row = t_base + 32 * i + lo;  // the step of this lane's C row
    bf16x8 cf[kN / 16];
#pragma unroll
    for (int kb = 0; kb < kN / 16; ++kb) cf[kb] = bc_frag(C, t_row, kb);
    f32x16 acc[2] = {};
    // inherited state: C_t S_in
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
      for (int kb = 0; kb < kN / 16; ++kb) {
        const int64_t o = (pt * 32 + lo) * kN + 16 * kb + 8 * hi;
        acc[pt] = mfma(cf[kb], load8(sin_hi + o), acc[pt]);
        acc[pt] = mfma(cf[kb], load8(sin_lo + o), acc[pt]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[pt][r] *= hw_exp2(s_ell[32 * i + 8 * (r >> 2) + 4 * hi + (r & 3)] * kLog2e);
    }
    // diagonal blocks
    const int t_loc = 32 * i + lo;          // this lane's column step in the score tile
    const float ell_t = s_ell[t_loc];
    for (int j = 0; j <= i; ++j) {
      const float* tp = tiles + tile_index(i, j) * 1024 + lane;
      float sc[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = tp[r * 64];
      // mask and scale: element (s, t), s = 32 j + row(r)
      if (j < i) {
        // every s precedes every t: both factors are at most 1
        const float u_t = hw_exp2((ell_t - s_ell[32 * j + 31]) * kLog2e);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sc[r] *= u_t * s_v[32 * j + 8 * (r >> 2) + 4 * hi + (r & 3)];
      } else {
        // the diagonal tile: ell_t - ell_ref may be positive, so the weight is
        // formed directly
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int s_loc = 32 * j + 8 * (r >> 2) + 4 * hi + (r & 3);
          const float wgt = hw_exp2((ell_t - s_ell[s_loc]) * kLog2e) * s_delta[s_loc];
          sc[r] = s_loc <= t_loc ? sc[r] * wgt : 0.0f;
        }
      }
      // registers r and r + 4 swapped across the half-waves: lane l then holds
      // the eight consecutive s of k-half (l / 32) for step t = l % 32
      float e[16];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const auto w2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(sc[8 * q + r]),
                                                           __float_as_uint(sc[8 * q + r + 4]),
                                                           false, false);
          e[8 * q + r] = __uint_as_float(w2[0]);
          e[8 * q + r + 4] = __uint_as_float(w2[1]);
        }
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        u16x8 pk;
#pragma unroll
        for (int k = 0; k < 8; ++k) pk[k] = to_bf16(e[8 * q + k]);
        const bf16x8 aop = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
          acc[pt] = mfma(aop, load8(&s_x[pt * 32 + lo][32 * j + 16 * q + 8 * hi]), acc[pt]);
      }
    }
    // epilogue: + D x, store (rows past the sequence's end dropped)
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tl = 32 * i + 8 * (r >> 2) + 4 * hi + (r & 3);
        const int64_t t = t_base + tl;
        const int p = pt * 32 + lo;
        if (t < g.seqlen) {
          const float v = fmaf(Dh, from_bf16(s_x[p][tl]), acc[pt][r]);
          y[((b * g.seqlen + t) * g.nheads + h) * kP + p] = to_bf16(v);
        }
      }
    }
  }
}

}  // namespace

// Workspace: the chunk states (fp32), the chunks' decays (fp32), the states
// entering the chunks (two bf16 arrays), the chunks' score tiles (fp32), each
// 256-byte aligned.
struct SsdWs {
  size_t sc, ell, sin_hi, sin_lo, scores, total;
};
SsdWs ssd_ws_layout(int64_t batch, int64_t seqlen, int64_t nheads, int64_t ngroups) {
  const int64_t chunks = (seqlen + kQ - 1) / kQ;
  const size_t states = static_cast<size_t>(batch * nheads * chunks) * kP * kN;
  auto r256 = [](size_t v) { return (v + 255) / 256 * 256; };
  SsdWs w;
  w.sc = 0;
  w.ell = r256(states * sizeof(float));
  w.sin_hi = w.ell + r256(static_cast<size_t>(batch * nheads * chunks) * sizeof(float));
  w.sin_lo = w.sin_hi + r256(states * sizeof(uint16_t));
  w.scores = w.sin_lo + r256(states * sizeof(uint16_t));
  w.total = w.scores + r256(static_cast<size_t>(batch * chunks * ngroups) * kTiles * 1024 *
                           sizeof(float));
  return w;
}

size_t ssd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t ngroups) {
  return ssd_ws_layout(batch, seqlen, nheads, ngroups).total;
}

hipError_t launch_ssd_fwd(const SsdProblem& p, void* workspace, hipStream_t stream) {
  if (p.batch == 0 || p.nheads == 0) return hipSuccess;
  SsdDims g;
  g.batch = p.batch;
  g.seqlen = p.seqlen;
  g.nheads = p.nheads;
  g.ngroups = p.ngroups;
  g.chunks = static_cast<int>((p.seqlen + kQ - 1) / kQ);
  const int64_t per_head = static_cast<int64_t>(kP) * kN;
  if (p.seqlen == 0) {
    if (!p.last_state) return hipSuccess;
    // no steps: the final state is h0 (or 0); the state pass with no chunks
    const int64_t n = p.batch * p.nheads * per_head;
    hipLaunchKernelGGL(ssd_state_pass_kernel, dim3(static_cast<unsigned>((n + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, nullptr, nullptr, p.h0, nullptr, nullptr,
                       p.last_state, g);
    return hipGetLastError();
  }
  const SsdWs wl = ssd_ws_layout(p.batch, p.seqlen, p.nheads, p.ngroups);
  char* ws = static_cast<char*>(workspace);
  float* Sc = reinterpret_cast<float*>(ws + wl.sc);
  float* ell = reinterpret_cast<float*>(ws + wl.ell);
  uint16_t* Sin_hi = reinterpret_cast<uint16_t*>(ws + wl.sin_hi);
  uint16_t* Sin_lo = reinterpret_cast<uint16_t*>(ws + wl.sin_lo);
  float* scores = reinterpret_cast<float*>(ws + wl.scores);
  const auto* x = static_cast<const uint16_t*>(p.x);
  const auto* dt = static_cast<const uint16_t*>(p.dt);
  const auto* B = static_cast<const uint16_t*>(p.B);
  const auto* C = static_cast<const uint16_t*>(p.C);
  const dim3 grid(static_cast<unsigned>(g.chunks), static_cast<unsigned>(p.nheads),
                  static_cast<unsigned>(p.batch));
  hipLaunchKernelGGL(ssd_chunk_state_kernel, grid, dim3(kThreads), 0, stream, x, dt, p.A, B,
                     p.dt_bias, Sc, ell, g);
  const int64_t n = p.batch * p.nheads * per_head;
  hipLaunchKernelGGL(ssd_state_pass_kernel, dim3(static_cast<unsigned>((n + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, Sc, ell, p.h0, Sin_hi, Sin_lo, p.last_state, g);
  hipLaunchKernelGGL(ssd_chunk_scores_kernel,
                     dim3(static_cast<unsigned>(g.chunks), static_cast<unsigned>(p.ngroups),
                          static_cast<unsigned>(p.batch)),
                     dim3(kThreads), 0, stream, B, C, scores, g);
  hipLaunchKernelGGL(ssd_chunk_scan_kernel, grid, dim3(kThreads), 0, stream, x, dt, p.A, B, C, p.D,
                     p.dt_bias, Sin_hi, Sin_lo, scores, static_cast<uint16_t*>(p.out), g);
  return hipGetLastError();
}

}  // namespace mscan
