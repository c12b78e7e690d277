// Device-side helpers shared by the dsfp8 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsfp8 {

constexpr int kBlock = 128;          // quantisation block (elements)
constexpr float kE4m3Max = 448.0f;   // largest finite e4m3fn magnitude
constexpr float kScaleFloor = 1e-4f; // lower clamp of a block's absolute maximum

// ---- bf16 <-> fp32 -----------------------------------------------------------

// The two bf16 values packed in a 32-bit word, widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two fp32 values to bf16 (nearest-even, v_cvt_pk_bf16_f32) and pack
// them, the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// SiLU(g) * u in fp32 with the hardware exponential and reciprocal (each
// within a few fp32 ulp, far below the bf16 rounding that follows), rounded
// to bf16 and widened back, so that a quantiser applied next sees exactly the
// bf16 value h (also returned in *hb).  For very negative g, e = inf and the
// reciprocal gives -0 as g / inf would.  The standalone gate kernel and the
// gated product's epilogue both use this one definition, so they agree bit
// for bit on the same bf16 inputs.
__device__ __forceinline__ float silu_mul_bf16(float g, float u, __bf16* hb) {
  const float e = __expf(-g);
  const float h = (g * __builtin_amdgcn_rcpf(1.0f + e)) * u;
  *hb = (__bf16)h;
  return (float)(*hb);
}

// ---- e4m3 --------------------------------------------------------------------

// Encode four fp32 values to e4m3fn bytes (nearest-even, v_cvt_pk_fp8_f32),
// packed little-endian.  The clamp to +-448 makes the conversion saturating:
// a quotient x/s can exceed 448 by one fp32 ulp when s = fl(amax/448) rounds
// down, and such values must encode to +-448 rather than NaN.  med3 passes a
// signed zero through unchanged.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -kE4m3Max, kE4m3Max);
  b = __builtin_amdgcn_fmed3f(b, -kE4m3Max, kE4m3Max);
  c = __builtin_amdgcn_fmed3f(c, -kE4m3Max, kE4m3Max);
  d = __builtin_amdgcn_fmed3f(d, -kE4m3Max, kE4m3Max);
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// ---- block scale ---------------------------------------------------------------

// Scale of a block from its absolute maximum: max(amax, 1e-4) / 448 as a
// correctly rounded fp32 division (any fp32 amax), optionally rounded up to a power of two
// (ue8m0).  The power-of-two rounding works on the bits: a positive normal
// value with a non-zero fraction moves to the next binade with a zero
// fraction, which is exactly the smallest power of two not below it.
__device__ __forceinline__ float block_scale(float amax, bool ue8m0) {
  float s = fmaxf(amax, kScaleFloor) / kE4m3Max;
  if (ue8m0) {
    uint32_t u = __float_as_uint(s);
    if (u & 0x007fffffu) u = (u + 0x00800000u) & 0xff800000u;
    s = __uint_as_float(u);
  }
  return s;
}

// The same scale for a block maximum that is a bf16 value (an activation, or
// the gate's bf16 output) with two fp32 operations fewer: max(amax, 1e-4) / 448
// as one multiply by RN(1/448) and one correction (div_by_scale below).  For
// every bf16 amax and the clamp constant this equals the correctly rounded
// division (an exact rational check over all bf16 significands on the CPU;
// every intermediate stays normal, so one binade covers all exponents).
__device__ __forceinline__ float block_scale_bf16(float amax, bool ue8m0);

// RN(1/s) for a scale produced by block_scale_bf16: the hardware reciprocal
// (within one ulp) refined by one Newton step with an fma residual,
// e = 1 - s*r0 and r = r0 + r0*e.  For every such s, and every r0 within two
// ulp of 1/s, the result is the correctly rounded reciprocal (exact rational
// check on the CPU over all reachable scale significands).
__device__ __forceinline__ float recip_rn(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, r0, 1.0f);
  return __builtin_fmaf(r0, e, r0);
}

// x / s, correctly rounded, given r = RN(1/s): q = RN(x*r), then one
// correction with the exact remainder t = q*s - x (formed by an fma), i.e.
// Markstein's final correction step for division (P. Markstein, "Computation
// of elementary functions on the IBM RISC System/6000 processor", IBM J. Res.
// Dev. 34(1), 1990).  The result equals the IEEE quotient for every pair
// (x, s) that act_quant can produce (bf16 x; s from a bf16 block maximum);
// this is checked by an exact rational computation over all bf16
// significands of x and all scale significands on the CPU.  Callers outside
// that domain (fp32 inputs) use the IEEE division instead.  The sign of a
// zero quotient is kept: for x = -0, q = -0 and t = +0, so
// fma(-t, r, q) = -0.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  float q = x * r;
  float t = __builtin_fmaf(q, s, -x);
  return __builtin_fmaf(-t, r, q);
}

__device__ __forceinline__ float block_scale_bf16(float amax, bool ue8m0) {
  constexpr float kRecip448 = 1.0f / kE4m3Max;  // RN(1/448), folded at compile time
  float s = div_by_scale(fmaxf(amax, kScaleFloor), kE4m3Max, kRecip448);
  if (ue8m0) {
    uint32_t u = __float_as_uint(s);
    if (u & 0x007fffffu) u = (u + 0x00800000u) & 0xff800000u;
    s = __uint_as_float(u);
  }
  return s;
}

// ---- division by a launch constant ------------------------------------------------

// n / d for 0 <= n < 2^31 by multiply and shift (Granlund and Montgomery's
// round-up method with N = 31): with l = ceil(log2 d) and
// m = floor(2^(31+l) / d) + 1 < 2^32, n / d == (n * m) >> (31 + l).
struct FastDiv {
  uint32_t d, m, shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while (((uint64_t)1 << l) < d) ++l;
  FastDiv f;
  f.d = d;
  f.m = (uint32_t)((((uint64_t)1) << (31 + l)) / d + 1);
  f.shift = 31 + l;
  return f;
}

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, const FastDiv& f) {
  return (uint32_t)(((uint64_t)n * f.m) >> f.shift);
}

// ---- cross-lane reductions -------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Maximum over each aligned group of 16 lanes (one DPP row).
__device__ __forceinline__ float max_row16(float v) {
  v = fmaxf(v, dpp_f32<0xb1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4e>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
  return v;
}

// Maximum over the whole wavefront (64 lanes), returned in every lane.
__device__ __forceinline__ float max_wave(float v) {
  v = max_row16(v);
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

}  // namespace dsfp8
