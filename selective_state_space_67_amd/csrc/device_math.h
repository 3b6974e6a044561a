// Device-side helpers shared by the scan and decode kernels (gfx950).
//
// Element access for the two input formats (float32 and bfloat16 bit
// patterns), the float32 step-size and gate functions, the conv window with
// reset visibility, and the DPP lane shift the scan's cross-lane accumulation
// uses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bfloat16 is stored as its 16-bit pattern; widening to float is a shift.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const bf16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i].bits) << 16);
}

__device__ __forceinline__ void store_elem(float* p, int64_t i, float v) { p[i] = v; }
// float -> bfloat16, round to nearest, ties to even.
__device__ __forceinline__ void store_elem(bf16_t* p, int64_t i, float v) {
  uint32_t b = __float_as_uint(v);
  b += 0x7FFFu + ((b >> 16) & 1u);
  p[i].bits = static_cast<uint16_t>(b >> 16);
}

// 2^x and log2(x) on the transcendental unit (v_exp_f32 / v_log_f32); both
// are within ~2 ulp of the correctly rounded value on gfx950.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = log(1 + e^x) with beta 1, evaluated as max(x, 0) + log1p(e^-|x|).
// log1p(e) for e in (0, 1] is log(1 + e) plus the rounding error of the sum
// 1 + e (recovered exactly by Sterbenz subtraction); without that term the
// result loses relative accuracy once e is small (x below about -3).
__device__ __forceinline__ float softplus_f32(float x) {
  const float e = fast_exp2(-fabsf(x) * kLog2e);
  const float s = 1.0f + e;
  const float lost = e - (s - 1.0f);
  return fmaxf(x, 0.0f) + __builtin_fmaf(fast_log2(s), kLn2, lost);
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z). For z -> -inf, e^-z -> inf and
// the reciprocal gives 0, so the result is a signed zero rather than NaN.
__device__ __forceinline__ float silu_f32(float z) {
  return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e));
}

// Input coefficient of the exact zero-order hold: Bbar = (e^{delta A} - 1) / A * B
// for a diagonal A ("Illustrated Mamba state space model", "Mathematical
// basis: structured SSM"). With x = delta A and abar = e^x already computed:
// for |x| >= 1/16 it is (abar - 1) / A (one FMA with the precomputed 1/A; the
// relative error of abar - 1 is at most ~2e-6 there); below that, where
// abar - 1 would cancel, the series delta (1 + x/2 + x^2/6 + x^3/24), whose
// truncation is below 1.3e-7 relative. A = 0 gives x = 0 and the series' delta.
__device__ __forceinline__ float zoh_coef(float delta, float x, float abar, float invA) {
  const float series = delta * __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 24.0f, 1.0f / 6.0f), 0.5f),
                                              1.0f);
  const float direct = __builtin_fmaf(abar, invA, -invA);
  return fabsf(x) < 0.0625f ? series : direct;
}

// Derivative of the zero-order-hold coefficient with respect to A, divided by
// delta^2: psi(x) = (x e^x - e^x + 1) / x^2 with x = delta A and abar = e^x.
// For |x| < 1/2 the series sum_k (k+1)/(k+2)! x^k through x^7 (truncation
// below 1e-8); above, the closed form, whose numerator no longer cancels.
__device__ __forceinline__ float zoh_psi(float x, float abar) {
  float s = __builtin_fmaf(x, 1.0f / 45360.0f, 1.0f / 5760.0f);
  s = __builtin_fmaf(x, s, 1.0f / 840.0f);
  s = __builtin_fmaf(x, s, 1.0f / 144.0f);
  s = __builtin_fmaf(x, s, 1.0f / 30.0f);
  s = __builtin_fmaf(x, s, 0.125f);
  s = __builtin_fmaf(x, s, 1.0f / 3.0f);
  s = __builtin_fmaf(x, s, 0.5f);
  const float direct = __builtin_fmaf(x, abar, 1.0f - abar) * fast_rcp(x * x);
  return fabsf(x) < 0.5f ? s : direct;
}

// Visibility of the conv window's inputs: the window of step Q covers
// Q-3 .. Q (taps 0..3, widths below 4 have leading zero taps); an input is
// hidden when a reset lies after it within the window (the document started
// later). r0, r1, r2 are the reset flags of Q, Q-1 and Q-2.
__device__ __forceinline__ float conv_pre(const float (&w)[4], float bias, float x0, float x1, float x2, float x3,
                                          bool r0, bool r1, bool r2) {
  float acc = __builtin_fmaf(w[3], x3, bias);
  if (!r0) {
    acc = __builtin_fmaf(w[2], x2, acc);
    if (!r1) {
      acc = __builtin_fmaf(w[1], x1, acc);
      if (!r2) acc = __builtin_fmaf(w[0], x0, acc);
    }
  }
  return acc;
}

// Value of the lane one below within the same row of 16 lanes (DPP
// row_shr:1); lane 0 of each row reads 0.
__device__ __forceinline__ float row_shr1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, true));
}

}  // namespace ssm
