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
// Where k is the time step, the operands come from tiles kept in LDS in their
// HBM order (step-major rows written with 16-byte stores) and are read with the
// transposing LDS load of gfx950 (ds_read_b64_tr_b16), see lds_kmajor.
#include "device_math.h"
#include "kernels.h"

namespace mscan {

namespace {

constexpr int kQ = 256;       // chunk length (steps)
constexpr int kP = 64;        // head dimension
constexpr int kN = 128;       // state size
constexpr int kThreads = 256; // four waves, one step of a chunk per thread
static_assert(kThreads == kQ, "the chunk-state kernel scans one step per thread");
constexpr int kSBlk = 64;     // steps per LDS block of the chunk-state product
constexpr int kPad = 8;       // bf16 padding of LDS rows (keeps rows 16-byte aligned, spreads banks)
constexpr int kWidePad = 32;  // padding that puts the four rows of a transposing read on distinct banks

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two values rounded to bf16 (nearest even) in one register, a in the low
// half: one v_cvt_pk_bf16_f32 for both.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
// a and b each as a bf16 pair hi + lo (hi = bf16(v), lo = bf16(v - hi)),
// packed two values per register like pack_bf16; the same roundings as
// to_bf16 element by element, with half the conversions.
struct Bf16Pairs {
  uint32_t hi, lo;
};
__device__ __forceinline__ Bf16Pairs split_bf16_pair(float a, float b) {
  const uint32_t hi = pack_bf16(a, b);
  return {hi, pack_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u))};
}

// Eight bf16 at p (16-byte aligned), as an MFMA operand.
__device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
}

// The k-major MFMA operand from a row-major LDS tile T[k][col] (row stride ld
// elements, a multiple of 4; T 8-byte aligned): lane l receives
// T[8 (l / 32) + e][l % 32], e = 0..7, i.e. column (or row) l % 32 of the tile
// with k-half l / 32. ds_read_b64_tr_b16 works on groups of 16 lanes: lane q
// of a group names 4 consecutive elements of row q / 4 of a 4 x 16 block and
// receives column q of that block; two such reads give the 8 values of k.
__device__ __forceinline__ bf16x8 lds_kmajor(const uint16_t* T, int ld, int lane) {
  const int grp = lane >> 4, q = lane & 15;
  const uint16_t* p = T + (8 * (grp >> 1) + (q >> 2)) * ld + 16 * (grp & 1) + 4 * (q & 3);
  const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p));
  const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p + 4 * ld));
  const s16x8 v = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

struct SsdDims {
  int64_t batch, seqlen, nheads, ngroups;
  int chunks;
  // no initial state: the state entering chunk 0 is zero, so it is neither
  // handed over nor multiplied in
  bool zero_entry;
};

// Delta_t = softplus(dt + bias) of the workgroup's chunk, one step per thread
// of the first kQ (zero for steps past the sequence's end: `valid` false), and
// ell_t = sum_{u <= t} Delta_u A_h, an inclusive prefix sum over the chunk (wave
// scans, then the wave totals). s_wave holds one value per wave of the
// workgroup. `dt_raw` is this thread's dt value, loaded beforehand.
__device__ __forceinline__ void chunk_decay_from(float dt_raw, bool valid, float bias, float A_h,
                                                 float* s_delta, float* s_ell, float* s_wave) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const float Delta = valid ? softplus_f(dt_raw + bias) : 0.0f;
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
  if (tid < kQ) {
    s_delta[tid] = Delta;
    s_ell[tid] = base + v;
  }
  __syncthreads();
}

// The dt value of this thread's step of chunk c, and whether the step lies in
// the sequence.
__device__ __forceinline__ float load_dt(const uint16_t* __restrict__ dt, const SsdDims& g, int64_t b,
                                         int64_t h, int c, bool& valid) {
  const int64_t t = static_cast<int64_t>(c) * kQ + threadIdx.x;
  valid = threadIdx.x < kQ && t < g.seqlen;
  return valid ? from_bf16(dt[(b * g.seqlen + t) * g.nheads + h]) : 0.0f;
}

__device__ __forceinline__ void chunk_decay(const uint16_t* __restrict__ dt, float bias, float A_h,
                                            const SsdDims& g, int64_t b, int64_t h, int c,
                                            float* s_delta, float* s_ell, float* s_wave) {
  bool valid;
  const float raw = load_dt(dt, g, b, h, c, valid);
  chunk_decay_from(raw, valid, bias, A_h, s_delta, s_ell, s_wave);
}

// ---------------------------------------------------------------------------
// 1. Chunk states and their hand-off. Grid (heads, batch): one workgroup walks
// the chunks of one (batch, head) in order and keeps the state S (N x P, fp32)
// in registers. For chunk c it writes S_in(c) = S (fp32, [b][h][c][p][n]) for
// the chunk scan, forms the chunk's own contribution
//   S_c[p][n] = sum_s w_s x_s[p] B_s[n],   w_s = exp(ell_end - ell_s) Delta_s,
// as the product of (w o X)^T (P x Q) and B (Q x N), K = s, and passes the state
// on: S = exp(ell_end) S + S_c (ell_end: the chunk's total of Delta A_h). One
// block of kSBlk steps at a time, w x (as a bf16 pair hi + lo, two products, so
// the weights lose no precision to the bf16 operands) and B are stored
// step-major in LDS with 16-byte writes and read k-major by transposing loads;
// the next block's loads, and the next chunk's dt, are in flight meanwhile.
// Wave w owns the 32 states n of tile w and both 32-channel tiles of p. The
// final state (fp32, [b][h][n][p]) is written if asked for. No state of the
// sequence is passed between workgroups.
__global__ __launch_bounds__(kThreads, 3) void ssd_chunk_state_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ B, const float* __restrict__ dt_bias, const float* __restrict__ h0,
    float* __restrict__ Sin, float* __restrict__ last_state, SsdDims g) {
  constexpr int ldx = kP + kWidePad, ldb = kN + kWidePad;
  constexpr int kBlocks = kQ / kSBlk;
  constexpr int kXP = kSBlk * kP / 8 / kThreads, kBP = kSBlk * kN / 8 / kThreads;
  constexpr int64_t per_head = static_cast<int64_t>(kP) * kN;
  __shared__ float s_delta[kQ], s_ell[kQ], s_wave[kThreads / 64];
  __shared__ __align__(16) uint16_t s_xh[kSBlk][ldx];  // w o X block, hi part, [s][p]
  __shared__ __align__(16) uint16_t s_xl[kSBlk][ldx];  // lo part
  __shared__ __align__(16) uint16_t s_b[kSBlk][ldb];   // B block, [s][n]
  const int64_t h = blockIdx.x, b = blockIdx.y;
  const int64_t bh = b * g.nheads + h;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lo = lane & 31, hi = lane >> 5;
  const int64_t grp = h / (g.nheads / g.ngroups);
  const float bias = dt_bias ? dt_bias[h] : 0.0f, A_h = A[h];
  // register r of tile pt holds S[p][n], p = 32 pt + 8 (r / 4) + 4 hi + r % 4, n = 32 wv + lo
  auto p_of = [&](int pt, int r) { return pt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3); };
  const int n = wv * 32 + lo;
  f32x16 S[2];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      S[pt][r] = h0 ? h0[bh * per_head + static_cast<int64_t>(n) * kP + p_of(pt, r)] : 0.0f;

  // block k of chunk c into registers, 16-byte pieces with whole rows per group
  // of lanes: X rows (8 pieces), B rows (16 pieces); rows past the sequence's
  // end load its last row (no branch) and their B is zeroed (their weight is 0)
  u16x8 xv[kXP], bv[kBP];
  auto load_block = [&](int c, int k) {
#pragma unroll
    for (int q = 0; q < kXP; ++q) {
      const int id = tid + kThreads * q;
      const int64_t t = static_cast<int64_t>(c) * kQ + k * kSBlk + (id >> 3);
      const int64_t tr = t < g.seqlen ? t : g.seqlen - 1;
      xv[q] = *reinterpret_cast<const u16x8*>(x + ((b * g.seqlen + tr) * g.nheads + h) * kP + 8 * (id & 7));
    }
#pragma unroll
    for (int q = 0; q < kBP; ++q) {
      const int id = tid + kThreads * q;
      const int64_t t = static_cast<int64_t>(c) * kQ + k * kSBlk + (id >> 4);
      const int64_t tr = t < g.seqlen ? t : g.seqlen - 1;
      const u16x8 v = *reinterpret_cast<const u16x8*>(
          B + ((b * g.seqlen + tr) * g.ngroups + grp) * kN + 8 * (id & 15));
      bv[q] = t < g.seqlen ? v : u16x8{};
    }
  };
  bool dt_valid = false;
  float dt_raw = 0.0f;
  if (g.chunks > 0) {
    load_block(0, 0);
    dt_raw = load_dt(dt, g, b, h, 0, dt_valid);
  }
  for (int c = 0; c < g.chunks; ++c) {
    chunk_decay_from(dt_raw, dt_valid, bias, A_h, s_delta, s_ell, s_wave);
    if (c + 1 < g.chunks) dt_raw = load_dt(dt, g, b, h, c + 1, dt_valid);
    const float ell_last = s_ell[kQ - 1];
    // the state entering this chunk (the row offset of register r is a
    // constant); non-temporal (aux 2): it is read once, by the chunk scan, and
    // should not push the inputs read again out of the caches. A zero state
    // entering chunk 0 is not written (the chunk scan skips it).
    if (c > 0 || !g.zero_entry) {
      const auto rs = make_rsrc(Sin + (bh * g.chunks + c) * per_head, per_head * 4);
      const uint32_t voff = static_cast<uint32_t>((4 * hi * kN + n) * 4);
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[pt][r]), rs, voff,
                                                (pt * 32 + 8 * (r >> 2) + (r & 3)) * kN * 4, 2);
    }
    f32x16 acc[2] = {};
#pragma unroll
    for (int k = 0; k < kBlocks; ++k) {
      // stage block k (w o X as hi + lo, B) into LDS
#pragma unroll
      for (int q = 0; q < kXP; ++q) {
        const int id = tid + kThreads * q, row = id >> 3;
        const int64_t t = static_cast<int64_t>(c) * kQ + k * kSBlk + row;
        const float w = t < g.seqlen
                            ? hw_exp2((ell_last - s_ell[k * kSBlk + row]) * kLog2e) * s_delta[k * kSBlk + row]
                            : 0.0f;
        u32x4 vh, vl;
#pragma unroll
        for (int e = 0; e < 4; ++e)
        {
          const Bf16Pairs hl = split_bf16_pair(from_bf16(xv[q][2 * e]) * w, from_bf16(xv[q][2 * e + 1]) * w);
          vh[e] = hl.hi;
          vl[e] = hl.lo;
        }
        *reinterpret_cast<u32x4*>(&s_xh[row][8 * (id & 7)]) = vh;
        *reinterpret_cast<u32x4*>(&s_xl[row][8 * (id & 7)]) = vl;
      }
#pragma unroll
      for (int q = 0; q < kBP; ++q) {
        const int id = tid + kThreads * q;
        *reinterpret_cast<u16x8*>(&s_b[id >> 4][8 * (id & 15)]) = bv[q];
      }
      // the next block's loads go out before this block's products
      if (k + 1 < kBlocks)
        load_block(c, k + 1);
      else if (c + 1 < g.chunks)
        load_block(c + 1, 0);
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kSBlk; kk += 16) {
        const bf16x8 bop = lds_kmajor(&s_b[kk][wv * 32], ldb, lane);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          acc[pt] = mfma(lds_kmajor(&s_xh[kk][pt * 32], ldx, lane), bop, acc[pt]);
          acc[pt] = mfma(lds_kmajor(&s_xl[kk][pt * 32], ldx, lane), bop, acc[pt]);
        }
      }
      __syncthreads();
    }
    const float decay = hw_exp2(ell_last * kLog2e);
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int r = 0; r < 16; ++r) S[pt][r] = fmaf(decay, S[pt][r], acc[pt][r]);
  }
  if (last_state) {
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        last_state[bh * per_head + static_cast<int64_t>(n) * kP + p_of(pt, r)] = S[pt][r];
  }
}

// ---------------------------------------------------------------------------
// 3a. Chunk scores. Grid (chunks * kTiles / 4, groups, batch), one tile per
// wave. The raw scores B_s . C_t of a chunk do not depend on the head, so they
// are formed once per (batch, chunk, group) for every head that shares the
// group: the kTiles lower-triangular 32 x 32 tiles (s tile j <= t tile i),
// K = n, each kept in the MFMA result layout (s as rows, t as columns), fp32,
// stored as [tile][register / 4][lane][register % 4] so that a wave writes and
// reads a tile with 16-byte accesses, 1 KB contiguous per instruction.
constexpr int kTiles = (kQ / 32) * (kQ / 32 + 1) / 2;  // 36
constexpr int kScoreBlocks = kTiles / 4;

__device__ __forceinline__ int tile_index(int i, int j) { return i * (i + 1) / 2 + j; }

__global__ __launch_bounds__(kThreads) void ssd_chunk_scores_kernel(const uint16_t* __restrict__ B,
                                                                    const uint16_t* __restrict__ C,
                                                                    float* __restrict__ scores,
                                                                    SsdDims g) {
  const int c = blockIdx.x / kScoreBlocks;
  const int tile = (blockIdx.x % kScoreBlocks) * 4 + (threadIdx.x >> 6);
  const int64_t grp = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int lo = lane & 31, hi = lane >> 5;
  const int64_t t_base = static_cast<int64_t>(c) * kQ;
  int i = 0;
  while (tile_index(i + 1, 0) <= tile) ++i;
  const int j = tile - tile_index(i, 0);
  auto frag = [&](const uint16_t* T, int64_t t, int kb) -> bf16x8 {
    if (t >= g.seqlen) return bf16x8{};
    return load8(T + ((b * g.seqlen + t) * g.ngroups + grp) * kN + 16 * kb + 8 * hi);
  };
  f32x16 sc = {};
#pragma unroll
  for (int kb = 0; kb < kN / 16; ++kb)
    sc = mfma(frag(B, t_base + 32 * j + lo, kb), frag(C, t_base + 32 * i + lo, kb), sc);
  float* out = scores + (((b * g.chunks + c) * g.ngroups + grp) * kTiles + tile) * 1024;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4)
    *reinterpret_cast<f32x4*>(out + (r4 * 64 + lane) * 4) =
        f32x4{sc[4 * r4], sc[4 * r4 + 1], sc[4 * r4 + 2], sc[4 * r4 + 3]};
}

// ---------------------------------------------------------------------------
// 3. Chunk scan. Grid (chunks, heads, batch), eight waves. The chunk's X
// (step-major) and the state it inherits (S_in, split into a bf16 pair hi + lo,
// [p][n]) are staged in LDS once per workgroup. Each wave computes the output
// rows of one 32-step tile for both 32-channel tiles of p:
//   inherited part: C_t S_in (K = n; S_in as its pair hi + lo), rows scaled by
//     exp(ell_t);
//   diagonal part, per 32-step tile j <= i of earlier steps s: the chunk's
//     scores B_s . C_t (a 32 x 32 tile with s as rows, from 3a, the next tile's
//     load issued before the current one is used), masked (s <= t) and scaled
//     by exp(ell_t - ell_s) Delta_s, taken off the diagonal as
//     exp(ell_t - ell_ref) exp(ell_ref - ell_s) Delta_s with ell_ref the value
//     at the end of tile j (both factors at most 1; the second kept per step in
//     LDS) and formed directly on the diagonal tile, turned into the A operand
//     (t as rows, s as k) by exchanging register halves across the half-waves,
//     times X (K = s, transposing LDS reads);
//   then + D x; the 32 x 64 output tile leaves through LDS as 16-byte row
//   stores.
// Tile i takes i + 1 score tiles; waves are paired on SIMDs so that each SIMD
// gets 9, and two workgroups per compute unit fill the gaps.
constexpr int kScanThreads = 2 * kQ;

__global__ __launch_bounds__(kScanThreads, 2) void ssd_chunk_scan_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ B, const uint16_t* __restrict__ C, const float* __restrict__ D,
    const float* __restrict__ dt_bias, const float* __restrict__ Sin, const float* __restrict__ scores,
    uint16_t* __restrict__ y,
    SsdDims g) {
  constexpr int ldx = kP + kPad, ldsn = kN + kPad;
  __shared__ float s_delta[kQ], s_ell[kQ], s_wave[kScanThreads / 64], s_v[kQ];
  __shared__ __align__(16) uint16_t s_x[kQ][ldx];    // X of the chunk, [s][p]
  // S_in as a bf16 pair, [hi / lo][p][n]; once every wave has used it, the
  // space holds each wave's 32 x 64 output tile (bf16, [t][p])
  __shared__ __align__(16) uint16_t s_st[2][kP][ldsn];
  auto& s_sh = s_st[0];
  auto& s_sl = s_st[1];
  static_assert(kScanThreads / 64 * 32 * kP <= 2 * kP * ldsn, "output tiles fit the state space");
  const int c = blockIdx.x;
  const int64_t h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lo = lane & 31, hi = lane >> 5;
  const int64_t grp = h / (g.nheads / g.ngroups);
  const int64_t t_base = static_cast<int64_t>(c) * kQ;
  // staging loads first, in 16-byte pieces: X (eight per step; rows past the
  // sequence's end load the last row, no branch, and are zeroed) and S_in
  constexpr int kXPieces = kQ * kP / 8 / kScanThreads, kSPieces = kP * kN / 4 / kScanThreads;
  u16x8 xv[kXPieces];
  f32x4 sv[kSPieces];
#pragma unroll
  for (int k = 0; k < kXPieces; ++k) {
    const int id = tid + kScanThreads * k;
    const int64_t t = t_base + (id >> 3);
    const int64_t tr = t < g.seqlen ? t : g.seqlen - 1;
    xv[k] = *reinterpret_cast<const u16x8*>(x + ((b * g.seqlen + tr) * g.nheads + h) * kP + 8 * (id & 7));
    if (t >= g.seqlen) xv[k] = u16x8{};
  }
  const int64_t sin_off = (((b * g.nheads + h) * g.chunks + c) * kP) * kN;
  // whether a state enters this chunk (uniform over the workgroup)
  const bool inherit = c > 0 || !g.zero_entry;
  if (inherit) {
#pragma unroll
    for (int k = 0; k < kSPieces; ++k)
      sv[k] = __builtin_nontemporal_load(  // read once
          reinterpret_cast<const f32x4*>(Sin + sin_off + (tid + kScanThreads * k) * 4));
  }
  chunk_decay(dt, dt_bias ? dt_bias[h] : 0.0f, A[h], g, b, h, c, s_delta, s_ell, s_wave);
  // per step s: exp(ell_ref - ell_s) Delta_s, ell_ref at the end of the step's 32-step tile
  if (tid < kQ) s_v[tid] = hw_exp2((s_ell[tid | 31] - s_ell[tid]) * kLog2e) * s_delta[tid];
#pragma unroll
  for (int k = 0; k < kXPieces; ++k) {
    const int id = tid + kScanThreads * k;
    *reinterpret_cast<u16x8*>(&s_x[id >> 3][8 * (id & 7)]) = xv[k];
  }
  // S_in as a bf16 pair hi + lo (hi + lo = S_in to about 2^-17 relative)
#pragma unroll
  for (int k = 0; k < kSPieces && inherit; ++k) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const int id = tid + kScanThreads * k;
    u32x2 vh, vl;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const Bf16Pairs hl = split_bf16_pair(sv[k][2 * e], sv[k][2 * e + 1]);
      vh[e] = hl.hi;
      vl[e] = hl.lo;
    }
    *reinterpret_cast<u32x2*>(&s_sh[id >> 5][4 * (id & 31)]) = vh;
    *reinterpret_cast<u32x2*>(&s_sl[id >> 5][4 * (id & 31)]) = vl;
  }
  __syncthreads();
  const float Dh = D ? D[h] : 0.0f;
  const float* tiles = scores + ((b * g.chunks + c) * g.ngroups + grp) * (kTiles * 1024);

  // one 32-step tile of scores (16 values per lane) into registers
  auto load_tile = [&](f32x4* buf, const float* tp) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) buf[r4] = *reinterpret_cast<const f32x4*>(tp + r4 * 256);
  };

  {
    // this wave's 32-step tile: waves w and w + 4 share a SIMD, so they take
    // tiles w and 7 - w (9 score tiles per SIMD)
    const int i = wv < 4 ? wv : 11 - wv;
    const int64_t t_row = t_base + 32 * i + lo;  // the step of this lane's C row
    // C fragments: the 8 bf16 at state offset 8 * hi + 16 kb of row t (rows past
    // the end load the last row and are zeroed)
    bf16x8 cf[kN / 16];
    {
      const int64_t tr = t_row < g.seqlen ? t_row : g.seqlen - 1;
      const uint16_t* crow = C + ((b * g.seqlen + tr) * g.ngroups + grp) * kN + 8 * hi;
#pragma unroll
      for (int kb = 0; kb < kN / 16; ++kb) cf[kb] = load8(crow + 16 * kb);
      if (t_row >= g.seqlen) {
#pragma unroll
        for (int kb = 0; kb < kN / 16; ++kb) cf[kb] = bf16x8{};
      }
    }
    // score tiles (i, 0..i) are consecutive; the first one's load goes out now
    const float* trow = tiles + tile_index(i, 0) * 1024 + lane * 4;
    f32x4 bufA[4], bufB[4];
    load_tile(bufA, trow);
    // all of these loads are issued before any of them is used
    __builtin_amdgcn_sched_barrier(0);
    f32x16 acc[2] = {};
    // inherited state: C_t S_in
    if (inherit) {
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
        for (int kb = 0; kb < kN / 16; ++kb) {
          acc[pt] = mfma(cf[kb], load8(&s_sh[pt * 32 + lo][16 * kb + 8 * hi]), acc[pt]);
          acc[pt] = mfma(cf[kb], load8(&s_sl[pt * 32 + lo][16 * kb + 8 * hi]), acc[pt]);
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float f = hw_exp2(s_ell[32 * i + 8 * (r >> 2) + 4 * hi + (r & 3)] * kLog2e);
        acc[0][r] *= f;
        acc[1][r] *= f;
      }
    }
    // every wave is done with S_in: its space takes the output tiles from here on
    __syncthreads();
    // diagonal blocks
    const int t_loc = 32 * i + lo;          // this lane's column step in the score tile
    const float ell_t = s_ell[t_loc];
    // masked and scaled tile (s as rows) -> A operand (t as rows, s as k) -> times X
    auto apply = [&](float* sc, int j) {
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
      // the weights as a bf16 pair hi + lo (two products): one bf16 operand
      // would round each weight by up to 2^-9, and a long-memory head sums
      // hundreds of such terms into one output
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        u32x4 pk, pl;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const Bf16Pairs hl = split_bf16_pair(e[8 * q + 2 * k], e[8 * q + 2 * k + 1]);
          pk[k] = hl.hi;
          pl[k] = hl.lo;
        }
        const bf16x8 aop = __builtin_bit_cast(bf16x8, pk);
        const bf16x8 alo = __builtin_bit_cast(bf16x8, pl);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          const bf16x8 xop = lds_kmajor(&s_x[32 * j + 16 * q][pt * 32], ldx, lane);
          acc[pt] = mfma(aop, xop, acc[pt]);
          acc[pt] = mfma(alo, xop, acc[pt]);
        }
      }
    };
    // tile j < i: every s precedes every t, both factors are at most 1
    auto off_diag = [&](const f32x4* buf, int j) {
      const float u_t = hw_exp2((ell_t - s_ell[32 * j + 31]) * kLog2e);
      float sc[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sc[r] = buf[r >> 2][r & 3] * (u_t * s_v[32 * j + 8 * (r >> 2) + 4 * hi + (r & 3)]);
      apply(sc, j);
    };
    // tile i: ell_t - ell_ref may be positive, so the weight is formed directly
    auto diag = [&](const f32x4* buf) {
      float sc[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int s_loc = 32 * i + 8 * (r >> 2) + 4 * hi + (r & 3);
        const float wgt = hw_exp2(fminf(ell_t - s_ell[s_loc], 0.0f) * kLog2e) * s_delta[s_loc];
        sc[r] = (s_loc <= t_loc ? buf[r >> 2][r & 3] : 0.0f) * wgt;
      }
      apply(sc, i);
    };
    // two buffers in turn: the next tile's load is in flight while one is used
    int j = 0;
    for (; j + 1 < i; j += 2) {
      load_tile(bufB, trow + (j + 1) * 1024);
      __builtin_amdgcn_sched_barrier(0);
      off_diag(bufA, j);
      load_tile(bufA, trow + (j + 2) * 1024);
      __builtin_amdgcn_sched_barrier(0);
      off_diag(bufB, j + 1);
    }
    if (j < i) {
      load_tile(bufB, trow + i * 1024);
      __builtin_amdgcn_sched_barrier(0);
      off_diag(bufA, j);
      diag(bufB);
    } else {
      diag(bufA);
    }
    // epilogue: + D x into this wave's output tile in LDS, then 16-byte
    // non-temporal stores of whole rows through a buffer resource that ends
    // with the sequence (rows past its end are dropped)
    uint16_t* yt = &s_st[0][0][0] + wv * 32 * kP;
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tr = 8 * (r >> 2) + 4 * hi + (r & 3);
        yt[tr * kP + pt * 32 + lo] = to_bf16(fmaf(Dh, from_bf16(s_x[32 * i + tr][pt * 32 + lo]), acc[pt][r]));
      }
    }
    const int64_t t0 = t_base + 32 * i;
    const int64_t rows = g.seqlen - t0 < 32 ? g.seqlen - t0 : 32;
    const int64_t row_bytes = g.nheads * kP * 2;
    const auto rsrc = make_rsrc(y + ((b * g.seqlen + t0) * g.nheads + h) * kP,
                                rows > 0 ? static_cast<uint32_t>((rows - 1) * row_bytes + kP * 2) : 0u);
#pragma unroll
    for (int k = 0; k < 32 * kP / 8 / 64; ++k) {
      const int id = lane + 64 * k, row = id >> 3, col = 8 * (id & 7);
      const u16x8 v = *reinterpret_cast<const u16x8*>(yt + row * kP + col);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rsrc,
                                             static_cast<uint32_t>(row * row_bytes + col * 2), 0, 2);
    }
  }
}

}  // namespace

// Workspace: the states entering the chunks (fp32), then the chunks' score
// tiles (fp32), each 256-byte aligned.
struct SsdWs {
  size_t sin, scores, total;
};
SsdWs ssd_ws_layout(int64_t batch, int64_t seqlen, int64_t nheads, int64_t ngroups) {
  const int64_t chunks = (seqlen + kQ - 1) / kQ;
  const size_t states = static_cast<size_t>(batch * nheads * chunks) * kP * kN;
  auto r256 = [](size_t v) { return (v + 255) / 256 * 256; };
  SsdWs w;
  w.sin = 0;
  w.scores = r256(states * sizeof(float));
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
  g.zero_entry = p.h0 == nullptr;
  const auto* x = static_cast<const uint16_t*>(p.x);
  const auto* dt = static_cast<const uint16_t*>(p.dt);
  const auto* B = static_cast<const uint16_t*>(p.B);
  const auto* C = static_cast<const uint16_t*>(p.C);
  const dim3 heads(static_cast<unsigned>(p.nheads), static_cast<unsigned>(p.batch));
  if (p.seqlen == 0) {
    // no steps: the final state is h0 (or 0)
    if (!p.last_state) return hipSuccess;
    hipLaunchKernelGGL(ssd_chunk_state_kernel, heads, dim3(kThreads), 0, stream, x, dt, p.A, B,
                       p.dt_bias, p.h0, nullptr, p.last_state, g);
    return hipGetLastError();
  }
  const SsdWs wl = ssd_ws_layout(p.batch, p.seqlen, p.nheads, p.ngroups);
  char* ws = static_cast<char*>(workspace);
  float* Sin = reinterpret_cast<float*>(ws + wl.sin);
  float* scores = reinterpret_cast<float*>(ws + wl.scores);
  hipLaunchKernelGGL(ssd_chunk_state_kernel, heads, dim3(kThreads), 0, stream, x, dt, p.A, B,
                     p.dt_bias, p.h0, Sin, p.last_state, g);
  hipLaunchKernelGGL(ssd_chunk_scores_kernel,
                     dim3(static_cast<unsigned>(g.chunks * kScoreBlocks), static_cast<unsigned>(p.ngroups),
                          static_cast<unsigned>(p.batch)),
                     dim3(kThreads), 0, stream, B, C, scores, g);
  const dim3 grid(static_cast<unsigned>(g.chunks), static_cast<unsigned>(p.nheads),
                  static_cast<unsigned>(p.batch));
  hipLaunchKernelGGL(ssd_chunk_scan_kernel, grid, dim3(kScanThreads), 0, stream, x, dt, p.A, B, C, p.D,
                     p.dt_bias, Sin, scores, static_cast<uint16_t*>(p.out), g);
  return hipGetLastError();
}

}  // namespace mscan
