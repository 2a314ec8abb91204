// Channel-tile staging shared by the full-sequence scan kernels (forward and
// backward) on gfx950: tile geometry, global-to-LDS copies of input tiles
// through buffer resources, tile stores, and the B/C tile of a chunk.
#pragma once

#include "device_math.h"

namespace mscan {


#ifndef MSCAN_BLOCK
#define MSCAN_BLOCK 256
#endif
constexpr int kBlock = MSCAN_BLOCK;  // lanes (channels) per scan workgroup, a multiple of 64
static_assert(kBlock % 64 == 0 && kBlock <= 1024, "whole wave64s");
constexpr int kAuxBlock = 256;       // threads per workgroup of the small helper kernels
constexpr int kChunk = 8;     // time steps whose inputs are loaded together

// p[n] = rho e^(n+1) for n = 0..N-1 as two interleaved chains: rho e and
// rho e^2, then p[n] = p[n - 2] e^2 (N + 1 multiplications, at most N / 2 + 1
// deep; the states' own updates interleave with the two chains).
template <int N>
__device__ __forceinline__ void scaled_powers(float e, float rho, float (&p)[N]) {
  p[0] = rho * e;
  if constexpr (N > 1) {
    p[1] = p[0] * e;
    const float e2 = e * e;
#pragma unroll
    for (int n = 2; n < N; ++n) p[n] = p[n - 2] * e2;
  }
}

using lds_void = __attribute__((address_space(3))) void;

// A value every lane of the wave holds: taken from the first lane, so that
// the compiler keeps it (and what is built from it, like a buffer resource)
// in scalar registers instead of looping over lanes to make it uniform.
__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) {
  return __builtin_amdgcn_readfirstlane(v);
}

// Per-lane byte offset of a tile piece: a tile of kChunk rows (steps) by
// kBlock channels is moved S bytes per lane, lane i of instruction k taking
// the piece (k * kBlock + i) * S bytes into the tile; each instruction covers
// S / eb whole rows, so the offset within the instruction's rows is the same
// for every k. Pieces past the last channel get kOffNone.
template <class IO, int S>
__device__ __forceinline__ uint32_t tile_lane_offset(uint32_t row_bytes, uint32_t valid_bytes) {
  constexpr int eb = sizeof(typename IO::raw);
  const uint32_t flat = threadIdx.x * S;
  const uint32_t row = flat / (kBlock * eb), col = flat % (kBlock * eb);
  return col + S <= valid_bytes ? row * row_bytes + col : kOffNone;
}

// Cache policy of memory operations whose data is not read again by the
// library (buffer instructions' aux field, gfx950: non-temporal).
constexpr int kNonTemporal = 2;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One global-to-LDS copy instruction (buffer_load_dword{,x4} ... lds): lane i
// of the wave reads S bytes at `voff` in the buffer described by `rsrc` and
// writes them S * i bytes after `lds_base` (taken from M0).
//
// It is issued from inline assembly on purpose. The compiler tracks every
// LDS copy it emits itself and, unable to tell the two staging buffers apart,
// makes the next LDS access of any kind wait for all copies in flight
// (vmcnt(0)), which turns the prefetch of the next chunk into a full memory
// round trip at the start of every chunk. Copies it does not know about are
// not tracked; their callers order them explicitly instead: wait_vmem()
// (vmcnt(0)) and a workgroup barrier come between a copy and the first read
// of its bytes, and no lane reads or writes the target buffer while a copy is
// in flight. The instruction has no register results, so no register is
// left pending when the statement ends. The compiler's own counter waits stay
// correct: extra copies in flight only make them wait longer.
template <int S, int AUX>
__device__ __forceinline__ void lds_copy(u32x4 rsrc, uint32_t voff, uint32_t lds_base) {
  static_assert(S == 16 || S == 4, "copies are 16 or 4 bytes per lane");
  static_assert(AUX == 0 || AUX == kNonTemporal, "plain or non-temporal copies");
  if constexpr (S == 16 && AUX == 0)
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_base)
                 : "memory");
  else if constexpr (S == 16)
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc),
                 "{m0}"(lds_base)
                 : "memory");
  else if constexpr (AUX == 0)
    asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_base)
                 : "memory");
  else
    asm volatile("buffer_load_dword %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc),
                 "{m0}"(lds_base)
                 : "memory");
}

// Raw buffer descriptor words over `bytes` bytes from `base` (wave-uniform):
// base address, stride 0, record count, dword data format (as CDNA expects).
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32) & 0xffffu);
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = 0x00020000u;
  return r;
}

// Copy rows 0 .. kChunk - 1 (from `rows`, the tile's first element in the
// chunk's first step) of one input tensor's channel tile straight from global
// memory into LDS (no registers involved). Each copy instruction gets its own
// buffer descriptor, built in scalar registers, that starts at its first row
// and ends at the segment's end (`rows_left` rows from `rows`): rows past the
// segment read as zero, as do pieces past the last channel (`lane_off`); they
// are never used. Lane i of wave `wv` lands S * i bytes after the wave's LDS
// base. The caller waits for the copies (wait_vmem) and synchronises the
// workgroup before the tile is read (see lds_copy).
template <class IO, int S, int AUX = 0, int KC = kChunk>
__device__ __forceinline__ void dma_tile(const typename IO::raw* rows, uint32_t rows_left,
                                         uint32_t row_bytes, typename IO::raw* tile, int wv,
                                         uint32_t lane_off) {
  constexpr int eb = sizeof(typename IO::raw);
  constexpr int kTileBytes = KC * kBlock * eb;
  constexpr int kPerInstr = kBlock * S;
  constexpr int kRowsPerInstr = S / eb;
  static_assert(kTileBytes % kPerInstr == 0, "tile must be a whole number of copies");
#pragma unroll
  for (int k = 0; k < kTileBytes / kPerInstr; ++k) {
    const uint32_t r0 = k * kRowsPerInstr;
    const uint32_t left = uniform_u32(rows_left > r0 ? rows_left - r0 : 0u);
    const u32x4 r = rsrc_words(reinterpret_cast<const char*>(rows) + r0 * row_bytes, left * row_bytes);
    char* dst = reinterpret_cast<char*>(tile) + (k * kBlock + wv * 64) * S;
    const uint32_t lds_base = uniform_u32(static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(dst))));
    lds_copy<S, AUX>(r, lane_off, lds_base);
  }
}


// Write the y tile of one chunk from LDS to HBM in the pieces of dma_tile
// (same per-instruction resources, so rows past the segment are dropped;
// non-temporal: outputs are not read again here), or,
// with S == 0, each lane its own channel (`ch_off`, kOffNone past the last
// channel) row by row.
template <class IO, int S, int KC = kChunk>
__device__ __forceinline__ void store_tile(typename IO::raw* rows, uint32_t rows_left,
                                           uint32_t row_bytes, const typename IO::raw* tile,
                                           uint32_t lane_off, uint32_t ch_off) {
  constexpr int eb = sizeof(typename IO::raw);
  const int tid = threadIdx.x;
  if constexpr (S == 0) {
    const auto r = make_rsrc(rows);
#pragma unroll
    for (int j = 0; j < KC; ++j)
      if (static_cast<uint32_t>(j) < rows_left)
        IO::bstore(tile[j * kBlock + tid], r, ch_off, j * row_bytes);
  } else {
    constexpr int kTileBytes = KC * kBlock * eb;
    constexpr int kPerInstr = kBlock * S;
    constexpr int kRowsPerInstr = S / eb;
#pragma unroll
    for (int k = 0; k < kTileBytes / kPerInstr; ++k) {
      const uint32_t r0 = k * kRowsPerInstr;
      const uint32_t left = uniform_u32(rows_left > r0 ? rows_left - r0 : 0u);
      const auto r = make_rsrc(reinterpret_cast<char*>(rows) + r0 * row_bytes, left * row_bytes);
      const char* src = reinterpret_cast<const char*>(tile) + (k * kBlock + tid) * S;
      if constexpr (S == 16)
        __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(src), r, lane_off, 0,
                                               kNonTemporal);
      else
        __builtin_amdgcn_raw_buffer_store_b32(*reinterpret_cast<const uint32_t*>(src), r, lane_off, 0,
                                              kNonTemporal);
    }
  }
}

// Register-staged copy for tiles that are not a whole number of 32-bit words
// (an odd number of bf16 channels): each lane loads its own channel's value
// for every step of the chunk, and writes them to LDS after the current chunk
// has been computed.
template <class IO, int KC = kChunk>
struct TileRegs {
  typename IO::raw v[KC];
};

template <class IO, int KC>
__device__ __forceinline__ void load_tile_regs(TileRegs<IO, KC>& tr, const typename IO::raw* rows,
                                               uint32_t rows_left, uint32_t row_bytes,
                                               uint32_t ch_off) {
  const auto r = make_rsrc(rows);
#pragma unroll
  for (int j = 0; j < KC; ++j)
    tr.v[j] = IO::bload(r, static_cast<uint32_t>(j) < rows_left ? ch_off : kOffNone, j * row_bytes);
}

template <class IO, int KC>
__device__ __forceinline__ void store_tile_regs(const TileRegs<IO, KC>& tr, typename IO::raw* tile) {
#pragma unroll
  for (int j = 0; j < KC; ++j) tile[j * kBlock + threadIdx.x] = tr.v[j];
}

// Thread i < kChunk * 2N fetches element i of a chunk's B/C tile: B or C of
// step i / 2N, state i % 2N (C when i % 2N >= N). Its byte offsets into B and
// into C (kOffNone for the tensor it does not read, and for i past the tile);
// consecutive steps are row_elems elements apart (G * N with G groups).
struct BcOffsets {
  uint32_t b, c;
};
template <int N, class IO, int KC = kChunk>
__device__ __forceinline__ BcOffsets bc_offsets(int i, uint32_t row_elems) {
  constexpr int eb = sizeof(typename IO::raw);
  const int j = i / (2 * N), k = i % (2 * N);
  const bool in_tile = i < KC * 2 * N;
  return {in_tile && k < N ? static_cast<uint32_t>((j * row_elems + k) * eb) : kOffNone,
          in_tile && k >= N ? static_cast<uint32_t>((j * row_elems + k - N) * eb) : kOffNone};
}

// This thread's B/C tile element for the chunk whose first step is row 0 of
// Bc / Cc (`rows_left` steps to the segment's end; steps past it read 0 and are
// never used), widened to fp32.
template <int N, class IO>
__device__ __forceinline__ float bc_elem(const typename IO::raw* Bc, const typename IO::raw* Cc,
                                         uint32_t rows_left, BcOffsets o, uint32_t row_elems) {
  constexpr int eb = sizeof(typename IO::raw);
  const uint32_t bytes = rows_left * row_elems * eb;
  const auto rb = make_rsrc(Bc, bytes), rc = make_rsrc(Cc, bytes);
  return IO::to_f32(IO::bit_or(IO::bload(rb, o.b, 0), IO::bload(rc, o.c, 0)));
}

template <int N>
__device__ __forceinline__ void read_bc(const float* row, float (&bc)[2 * N], bool need_c) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int k = 0; k < 2 * N; k += 4) {
      if (k >= N && !need_c) break;
      const float4 q = *reinterpret_cast<const float4*>(row + k);
      bc[k] = q.x;
      bc[k + 1] = q.y;
      bc[k + 2] = q.z;
      bc[k + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 2 * N; ++k) bc[k] = (k < N || need_c) ? row[k] : 0.0f;
  }
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace mscan
