// Device-side element helpers shared by the scan and decode kernels (gfx950).
//
// Transcendentals use the gfx950 hardware instructions directly
// (v_exp_f32 = 2^x, v_log_f32 = log2 x, v_rcp_f32 = 1/x); softplus and silu are
// written from their definitions on top of them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mscan {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float hw_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float hw_log2(float v) { return __builtin_amdgcn_logf(v); }
__device__ __forceinline__ float hw_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

// Read-only memory that every lane of a wave reads at the same address (B_t,
// C_t): declaring it constant lets the compiler fetch it with scalar loads.
template <class T>
using const_ptr = const __attribute__((address_space(4))) T*;

template <class T>
__device__ __forceinline__ const_ptr<T> as_const(const T* p) {
  return (const_ptr<T>)(p);
}

// Buffer resource over a byte range that starts at `base` (wave-uniform). The
// record count is the largest positive 32-bit value: a lane offset of
// kOffNone is out of range, so its loads return 0 and its stores are dropped.
constexpr uint32_t kOffNone = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  // 0x00020000: raw (untyped) buffer, dword data format, as CDNA expects
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           0x7fffffff, 0x00020000);
}
// The same over `bytes` bytes from `base` (at most 0x7fffffff): offsets at or
// past the end read 0 and drop stores. With a wave-uniform base and size it is
// built in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// Storage types for the io tensors.
//   load_pair(p, k): elements 2k and 2k + 1 of a wave-uniform constant array,
//   widened to fp32.
struct F32Io {
  using raw = float;
  static __device__ __forceinline__ void load_pair(const_ptr<float> p, int k, float& a, float& b) {
    a = p[2 * k];
    b = p[2 * k + 1];
  }
  static __device__ __forceinline__ float load(const raw* p) { return *p; }
  static __device__ __forceinline__ raw bload(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
  }
  static __device__ __forceinline__ void bstore(raw v, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
  }
  static __device__ __forceinline__ float to_f32(raw v) { return v; }
  static __device__ __forceinline__ raw from_f32(float v) { return v; }
  // bitwise or of two raw values (one of them 0)
  static __device__ __forceinline__ raw bit_or(raw a, raw b) {
    return __uint_as_float(__float_as_uint(a) | __float_as_uint(b));
  }
};

struct Bf16Io {
  using raw = uint16_t;
  static __device__ __forceinline__ void load_pair(const_ptr<uint16_t> p, int k, float& a,
                                                   float& b) {
    const uint32_t w = ((const_ptr<uint32_t>)(p))[k];
    a = __uint_as_float(w << 16);
    b = __uint_as_float(w & 0xffff0000u);
  }
  static __device__ __forceinline__ float to_f32(raw v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
  }
  static __device__ __forceinline__ float load(const raw* p) { return to_f32(*p); }
  // bitwise or of two raw values (one of them 0)
  static __device__ __forceinline__ raw bit_or(raw a, raw b) { return static_cast<raw>(a | b); }
  static __device__ __forceinline__ raw bload(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
  }
  static __device__ __forceinline__ void bstore(raw v, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, soff, 0);
  }
  // Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
  static __device__ __forceinline__ raw from_f32(float v) {
    __bf16 b = static_cast<__bf16>(v);
    return __builtin_bit_cast(uint16_t, b);
  }
};

// softplus(u) = log(1 + e^u) = max(u, 0) + log(1 + e), e = e^-|u| in (0, 1].
// w = 1 + e is rounded; as w lies in [1, 2], w - 1 is exact and
// r = e - (w - 1) is the exact rounding error (1 + e = w + r). Then
// log(1 + e) = log(w) + r / w to first order; adding r instead of r / w moves
// the result by at most |r| (1 - 1/w) <= 2^-24 e, below 2^-23 of the result
// (log(1 + e) >= e ln 2 on (0, 1]). e never overflows, so large u needs no
// special case: the log term vanishes and max(u, 0) = u remains.
// max(u, 0) is formed as (u + |u|) / 2 (exact: 2u or 0, halved), one add with
// an operand modifier and the final fma, instead of a max (which gfx950
// issues at half the rate of adds and fmas). neg_log2e is -log2(e); a caller
// in a hot loop may pass it from a vector register, for the same reason.
__device__ __forceinline__ float softplus_f(float u, float neg_log2e = -kLog2e) {
  const float e = hw_exp2(fabsf(u) * neg_log2e);
  const float w = 1.0f + e;
  const float r = e - (w - 1.0f);
  return fmaf(0.5f, u + fabsf(u), fmaf(hw_log2(w), kLn2, r));
}

// silu(v) = v * sigmoid(v) = v / (1 + e^-v). For v -> -inf, e^-v = inf and the
// reciprocal gives 0.
__device__ __forceinline__ float silu_f(float v) {
  return v * hw_rcp(1.0f + hw_exp2(-v * kLog2e));
}

// Exact zero-order-hold input weight ("Mamba and selective state spaces, from
// first principles", section "Discretisation: zero-order hold"):
// Bbar_n = (exp(Delta A_n) - 1) / A_n B_n = Delta zoh_gain(Delta A_n) B_n with
// zoh_gain(v) = (e^v - 1) / v, given v2 = v log2(e) and e2 = 2^v2 = e^v. Near
// v = 0 the quotient is formed as (e - 1) / ln(e) from the rounded e (Kahan's
// form for expm1: the rounding of e cancels between numerator and
// denominator); for e < 1/2 the direct quotient has no cancellation (and stays
// right when e underflows); at e = 1 the gain is 1.
__device__ __forceinline__ float zoh_gain(float v2, float e2) {
  const float den = (e2 < 0.5f ? v2 : hw_log2(e2)) * kLn2;
  return e2 == 1.0f ? 1.0f : (e2 - 1.0f) * hw_rcp(den);
}

}  // namespace mscan
