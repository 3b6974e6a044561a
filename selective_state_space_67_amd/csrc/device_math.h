// Device-side helpers shared by the scan and decode kernels (gfx950).
//
// Element access for the two input formats (float32 and bfloat16 bit
// patterns), the float32 step-size and gate functions, the conv window with
// reset visibility, the DPP lane shift the scan's cross-lane accumulation
// uses, and for the decode kernels runs of consecutive elements loaded as one
// vector and sums over groups of lanes.
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
// Two floats as bfloat16 (same rounding as store_elem), lo in the low half.
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
  a += 0x7FFFu + ((a >> 16) & 1u);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (a >> 16) | (b & 0xFFFF0000u);
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

// Sum over each group of LR consecutive lanes, complete in the group's last
// lane only (DPP adds: row_shr inside 16-lane rows, then row_bcast across
// rows). Other lanes end with partial sums; each add's sources lie inside the
// last lane's own group. Measured on the 64 x 2048 x 128 decode step with the
// state from HBM: 32.2 -> 31.3 us against the all-lane butterfly of shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float y) {
  return y + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(y), CTRL, 0xF, 0xF, true));
}

template <int LR>
__device__ __forceinline__ float group_sum_last(float y) {
  if constexpr (LR >= 16) y = dpp_add<0x118>(y);
  if constexpr (LR >= 8) y = dpp_add<0x114>(y);
  if constexpr (LR >= 4) y = dpp_add<0x112>(y);
  if constexpr (LR >= 2) y = dpp_add<0x111>(y);
  if constexpr (LR >= 32) y = dpp_add<0x142>(y);   // row_bcast:15
  if constexpr (LR >= 64) y = dpp_add<0x143>(y);   // row_bcast:31
  return y;
}

// Raw words of a run of consecutive input elements, loaded with one vector
// load and kept as loaded until the arithmetic (converting at the load would
// make the load phase wait for each value in turn).
template <int BYTES>
struct Bits;
template <>
struct Bits<2> {
  using T = uint16_t;
};
template <>
struct Bits<4> {
  using T = uint32_t;
};
template <>
struct Bits<8> {
  using T = uint2;
};
template <>
struct Bits<16> {
  using T = uint4;
};

__device__ __forceinline__ uint32_t word(uint16_t v, int) { return v; }
__device__ __forceinline__ uint32_t word(uint32_t v, int) { return v; }
__device__ __forceinline__ uint32_t word(uint2 v, int k) { return k ? v.y : v.x; }
__device__ __forceinline__ uint32_t word(uint4 v, int k) { return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w; }

template <typename T, int R>
struct Run {
  using raw = typename Bits<R * static_cast<int>(sizeof(T))>::T;
  // `p` aligned to the run's size
  __device__ __forceinline__ static raw load(const T* p) { return *reinterpret_cast<const raw*>(p); }
  // element i (a compile-time constant after unrolling) as float
  __device__ __forceinline__ static float at(raw v, int i) {
    if constexpr (sizeof(T) == 2) {
      const uint32_t w = word(v, i >> 1);
      return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
    } else {
      return __uint_as_float(word(v, i));
    }
  }
};

// R consecutive outputs, one store (the run is aligned to its size).
template <int R>
__device__ __forceinline__ void store_run(float* p, const float (&v)[R]) {
  if constexpr (R == 4)
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  else if constexpr (R == 2)
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  else
    *p = v[0];
}
template <int R>
__device__ __forceinline__ void store_run(bf16_t* p, const float (&v)[R]) {
  if constexpr (R == 4)
    *reinterpret_cast<uint2*>(p) = make_uint2(bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3]));
  else if constexpr (R == 2)
    *reinterpret_cast<uint32_t*>(p) = bf16_pair(v[0], v[1]);
  else
    store_elem(p, 0, v[0]);
}

// h <- P[i] h + H[i] for i = 0 .. count - 1 in order: the affine aggregates
// of the pieces that precede a piece of a split sequence, `stride` elements
// apart. The loads go out eight pieces at a time; one piece at a time, every
// piece paid a full load latency before the next load was issued.
__device__ __forceinline__ float fold_aggregates(const float* P, const float* H, int count, int64_t stride, float h) {
  int i = 0;
  for (; i + 8 <= count; i += 8) {
    float p[8], q[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      p[k] = P[(i + k) * stride];
      q[k] = H[(i + k) * stride];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) h = __builtin_fmaf(p[k], h, q[k]);
  }
  for (; i < count; ++i) h = __builtin_fmaf(P[i * stride], h, H[i * stride]);
  return h;
}

// Placed in the body of a wave-uniform branch that is rarely taken (a reset
// somewhere in the wave): the body then stays behind the branch. Without it
// the compiler turns the branch and its selects into selects executed every
// step (measured: four extra VALU operations per step for two states per
// lane, two for one).
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// Wave priority from the share of a workgroup's work already done. The
// instruction arbiter of a SIMD favours its oldest waves, so of the
// workgroups sharing a CU the first-placed ones race ahead and the last one
// ends alone, with too few waves to hide latency. Dropping a wave's priority
// each time it passes another mark of its work lets the workgroups that are
// behind catch up, so that they end closer together. When the whole grid is
// resident at once the marks are at 1/2, 3/4 and 7/8 of the work (the spread
// at the end is what the last stretch lets accumulate); when later
// workgroups start as earlier ones end, at every quarter (a newcomer at the
// top priority would otherwise starve the workgroups about to finish).
class ProgressPriority {
 public:
  __device__ ProgressPriority(int total, bool all_resident)
      : q1_(all_resident ? total / 2 : total / 4),
        q2_(all_resident ? total - total / 4 : total / 2),
        q3_(all_resident ? total - total / 8 : total - total / 4) {}
  // `done`: units of work (chunks) completed so far, the same for every wave of the workgroup
  __device__ __forceinline__ void update(int done) const {
    if (done < q1_)
      __builtin_amdgcn_s_setprio(3);
    else if (done < q2_)
      __builtin_amdgcn_s_setprio(2);
    else if (done < q3_)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
  }

 private:
  int q1_, q2_, q3_;
};

}  // namespace ssm
