// Device-side helpers shared by the scan and decode kernels (gfx950).
//
// Element functions of the selective scan, written for the CDNA4 VALU:
// exp and log go through the hardware base-2 transcendentals (v_exp_f32,
// v_log_f32, v_rcp_f32), which issue at half the FMA rate on gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace ssm {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(v), v = e^-|x| in (0, 1].
// log1p(v) is taken as log(w) + (v - (w - 1)) with w = fl(1 + v): w - 1 is
// exact, so the second term is the part of v lost when rounding 1 + v, and
// adding it restores log1p to first order (the term dropped, c * v / w with
// |c| <= half an ulp of w, is below 2^-24 v). Small v, the small-step regime,
// thus keeps full relative accuracy at two transcendentals.
__device__ __forceinline__ float softplus_f(float x) {
  const float v = exp2_hw(-fabsf(x) * kLog2e);
  const float w = 1.0f + v;
  const float lp = fmaf(log2_hw(w), kLn2, v - (w - 1.0f));
  return fmaxf(x, 0.0f) + lp;
}

// 1/a (correctly rounded), or 0 for a = 0.
__device__ __forceinline__ float inv_or_zero(float a) { return a != 0.0f ? 1.0f / a : 0.0f; }

// Input coefficient of the exact zero-order hold over one step of size dt,
// k = (e^(dt a) - 1) / a (the integral of e^(a s) over [0, dt]; k = dt at
// a = 0), given x2 = dt a log2(e), abar = 2^x2 and ia = 1/a (0 where a = 0).
// Away from x = 0, k = (abar - 1) ia, whose relative error is a few
// ulp(abar) / |x|: of order 2^-17 at |x| = ln(2)/64, smaller beyond. Closer to 0 (and at
// a = 0) the difference cancels, and k = dt (1 + x/2 + x^2/6) is used, the
// series of expm1(x)/x, whose first dropped term x^3/24 is below 2^-24 there.
__device__ __forceinline__ float zoh_coef(float dt, float x2, float abar, float ia) {
  constexpr float c1 = 0.5f * kLn2, c2 = kLn2 * kLn2 / 6.0f;  // x = x2 ln 2
  const float ks = fmaf(dt * x2, fmaf(x2, c2, c1), dt);
  const float kb = fmaf(abar, ia, -ia);
  return fabsf(x2) < 0x1p-6f ? ks : kb;
}

// Derivative of phi(x) = (e^x - 1) / x (so that the zero-order-hold
// coefficient k = dt phi(dt A) has dk/dA = dt^2 phi'(dt A)), given a = e^x:
// phi'(x) = (a (x - 1) + 1) / x^2 for |x| >= 0.3 (relative error near 2e-6
// there, from the rounding of a), else its Taylor series to x^6,
// sum_{n=1..7} n x^(n-1) / (n+1)!, whose first dropped term is below 1e-8.
__device__ __forceinline__ float zoh_dphi(float x, float a) {
  const float ser = fmaf(fmaf(fmaf(fmaf(fmaf(fmaf(x, 1.0f / 5760.0f, 1.0f / 840.0f), x, 1.0f / 144.0f), x,
                                          1.0f / 30.0f), x, 0.125f), x, 1.0f / 3.0f), x, 0.5f);
  const float closed = fmaf(a, x - 1.0f, 1.0f) * rcp_hw(x * x);
  return fabsf(x) < 0.3f ? ser : closed;
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z).
__device__ __forceinline__ float silu_f(float z) {
  return z * rcp_hw(1.0f + exp2_hw(-z * kLog2e));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  const __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if constexpr (BF16) {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

// Raw storage bits of element i (bf16 zero-extended, or the float32 pattern).
// Keeping the bits lets a prefetch stay in flight until the value is used.
template <bool BF16>
__device__ __forceinline__ uint32_t load_bits(const void* p, int64_t i) {
  if constexpr (BF16) {
    return static_cast<const uint16_t*>(p)[i];
  } else {
    return static_cast<const uint32_t*>(p)[i];
  }
}

template <bool BF16>
__device__ __forceinline__ float bits_to_f32(uint32_t v) {
  if constexpr (BF16) {
    return __uint_as_float(v << 16);
  } else {
    return __uint_as_float(v);
  }
}

template <bool BF16>
__device__ __forceinline__ void store_elem(void* p, int64_t i, float v) {
  if constexpr (BF16) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(v);
  } else {
    static_cast<float*>(p)[i] = v;
  }
}

// ---- raw buffer access (gfx9 family, untyped, stride 0)
//
// An access whose per-lane byte offset is at or beyond the descriptor's size
// is out of range: the load returns 0 and the store is dropped by the memory
// unit. Kernels use this to mask ragged edges without branching. The whole
// offset is passed per lane (the scalar offset is not range-checked).

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRawBufferFlags = 0x00020000;
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;

__device__ __forceinline__ rsrc_t raw_buffer(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           kRawBufferFlags);
}

// Storage bits of one element: uint16_t for bfloat16 (kept 16-bit so that a
// value carried across a loop needs no zero-extension), uint32_t for float32.
template <bool BF16>
using storage_t = std::conditional_t<BF16, uint16_t, uint32_t>;

// Cache policy of a buffer access: 0, or kNonTemporal for streams read or
// written once (the nt bit).
constexpr int kNonTemporal = 2;

template <bool BF16, int AUX = 0>
__device__ __forceinline__ storage_t<BF16> buffer_load_bits(rsrc_t r, uint32_t off) {
  if constexpr (BF16) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, AUX);
  } else {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
  }
}

template <bool BF16, int AUX = 0>
__device__ __forceinline__ void buffer_store_f32(float v, rsrc_t r, uint32_t off) {
  if constexpr (BF16) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(v), r, off, 0, AUX);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, AUX);
  }
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---- cross-lane moves (DPP): a lane reads another lane's value

// Every control used here (quad permutes, row_ror) reads a valid lane, so
// bound_ctrl changes no value; it is set because it lets the compiler fold
// the move into the instruction that consumes it (an add with a DPP source).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

constexpr int quad_perm(int a, int b, int c, int d) { return a | (b << 2) | (c << 4) | (d << 6); }

// Value of lane (this lane xor MASK) inside its quad.
template <int MASK>
__device__ __forceinline__ float quad_xor(float v) {
  static_assert(MASK == 1 || MASK == 2, "xor 1 or 2 inside a quad");
  if constexpr (MASK == 1) {
    return dpp_f<quad_perm(1, 0, 3, 2)>(v);
  } else {
    return dpp_f<quad_perm(2, 3, 0, 1)>(v);
  }
}

}  // namespace ssm
