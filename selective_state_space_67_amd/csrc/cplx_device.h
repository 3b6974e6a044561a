// Device helpers of the complex-state kernels (scan_cplx.hip, scan_cplx_bwd.hip):
// the decay exp(delta A) of a complex A with an accurate angle, the per-state
// constants it needs, DPP row sums and loads of (re, im) pairs.
#pragma once

#include "device_math.h"

namespace ssm {
namespace cplx {

// 1 / (2 pi) as the sum of two floats (the second is the rounding error of the first).
constexpr float kInv2PiHi = 0.15915494f;
constexpr float kInv2PiLo = 0.15915494309189535 - static_cast<double>(0.15915494f);

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of a DPP row; every lane gets the total.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  return v;
}

// Polynomials for sin(w r) and cos(w r) in r (revolutions), |r| <= 1/8, with
// w = 2 pi rounded to float32: sin = r (S1 + S3 x + S5 x^2 + S7 x^3) and
// cos = 1 + x (C2 + C4 x + C6 x^2 + C8 x^3), x = r^2. The coefficients are
// weighted least-squares fits on Chebyshev nodes, reweighted toward equal
// ripple (relative error for sin, absolute for cos), done in float64 and
// rounded to float32 (rotation_coefficients.py beside this file computes them
// and checks the float32 evaluation). Fit error: below 3.3e-9 relative (sin)
// and 5.4e-11 (cos), under float32 rounding; S1 is w itself, so sine and
// cosine are of the same angle w r. Against Taylor series of degree 9 and 10
// this takes two fused multiply-adds fewer, with the same float32 error and a
// smaller mean bias of sin^2 + cos^2 (the decay's magnitude).
constexpr float kS1 = 6.2831854820251465f;
constexpr float kS3 = -41.3416633605957f;
constexpr float kS5 = 81.59234619140625f;
constexpr float kS7 = -75.39276123046875f;
constexpr float kC2 = -19.73921012878418f;
constexpr float kC4 = 64.9393310546875f;
constexpr float kC6 = -85.4437484741211f;
constexpr float kC8 = 59.24570083618164f;

// e (cos + i sin) of the angle delta (ai + ai_lo) revolutions. The product
// p = delta ai is split into p and its exact rounding error; p - rint(p) is
// exact and lies in [-1/2, 1/2]; k quarter turns are taken off exactly, and
// the small parts are added to the remainder r, |r| <= 1/8 revolution. Then
// sin and cos of 2 pi r by the polynomials above, and the k quarter turns as
// a product with i^k = (1 - |k|) + i k (2 - |k|), k in -2 .. 2, whose parts
// are 0 or +-1 (so the rotation is exact; e is folded into them first).
__device__ __forceinline__ void rotate_rev(float e, float delta, float ai, float ai_lo, float& re, float& im) {
  const float p = delta * ai;
  const float lo = __builtin_fmaf(delta, ai, -p) + delta * ai_lo;
  const float f = p - __builtin_rintf(p);
  const float k = __builtin_rintf(4.0f * f);  // -2 .. 2
  const float r = __builtin_fmaf(-0.25f, k, f) + lo;
  const float x = r * r;
  float sp = __builtin_fmaf(x, kS7, kS5);
  sp = __builtin_fmaf(x, sp, kS3);
  sp = __builtin_fmaf(x, sp, kS1);
  const float sn = r * sp;
  float cp = __builtin_fmaf(x, kC8, kC6);
  cp = __builtin_fmaf(x, cp, kC4);
  cp = __builtin_fmaf(x, cp, kC2);
  const float cs = __builtin_fmaf(x, cp, 1.0f);
  const float ak = fabsf(k);
  const float ec = e * (1.0f - ak), es = e * (k * (2.0f - ak));  // e i^k
  re = __builtin_fmaf(cs, ec, -sn * es);
  im = __builtin_fmaf(sn, ec, cs * es);
}

// Per-lane constants of one state: Re A log2(e) for the decay's magnitude,
// Im A / (2 pi) as ai + ai_lo (ai rounded, ai_lo the rest to within float32
// rounding) for its angle, and for the zero-order hold A and 1/A.
struct CState {
  float ar, ai, ai_lo;
  float re, im, ir, ii;
};

__device__ __forceinline__ CState make_cstate(float re, float im) {
  CState q;
  q.ar = re * kLog2e;
  q.ai = im * kInv2PiHi;
  q.ai_lo = __builtin_fmaf(im, kInv2PiHi, -q.ai) + im * kInv2PiLo;
  q.re = re;
  q.im = im;
  const float m = re * re + im * im;
  const float r = m > 0.0f ? 1.0f / m : 0.0f;  // 1/A = conj(A) / |A|^2; 0 for A = 0
  q.ir = re * r;
  q.ii = -im * r;
  return q;
}

// Constants of this lane's states n0 .. n0+NPL-1 (zero past N).
template <int NPL>
__device__ __forceinline__ void load_A(const float* A, int64_t d, int N, int n0, bool dvalid, CState (&q)[NPL]) {
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = n0 + j;
    const bool ok = dvalid && n < N;
    q[j] = make_cstate(ok ? A[2 * (d * N + n)] : 0.0f, ok ? A[2 * (d * N + n) + 1] : 0.0f);
  }
}

// exp(delta A) = 2^(delta Re A log2 e) (cos theta + i sin theta), theta = delta Im A.
__device__ __forceinline__ void decay(float dl, const CState& q, float& are, float& aim) {
  rotate_rev(fast_exp2(dl * q.ar), dl, q.ai, q.ai_lo, are, aim);
}

// The exact zero-order-hold input coefficient q = (e^{delta A} - 1)/A of one
// state, from its decay a = e^{delta A} = (are, aim): (a - 1) times the
// precomputed 1/A where |delta A| >= 1/16, and below that, where a - 1 would
// cancel, the series delta (1 + x/2 + x^2/6 + x^3/24), x = delta A
// (truncation below 1.3e-7). A = 0 gives delta.
__device__ __forceinline__ void zoh_coef_c(float dl, const CState& q, float are, float aim, float& qr, float& qi) {
  const float xr = dl * q.re, xi = dl * q.im;
  float pr = __builtin_fmaf(xr, 1.0f / 24.0f, 1.0f / 6.0f), pi = xi * (1.0f / 24.0f);
  const float tr = __builtin_fmaf(pr, xr, -pi * xi) + 0.5f, ti = __builtin_fmaf(pr, xi, pi * xr);
  pr = __builtin_fmaf(tr, xr, -ti * xi) + 1.0f;
  pi = __builtin_fmaf(tr, xi, ti * xr);
  const float mr = are - 1.0f, mi = aim;
  const bool small = xr * xr + xi * xi < 1.0f / 256.0f;
  qr = small ? dl * pr : __builtin_fmaf(mr, q.ir, -mi * q.ii);
  qi = small ? dl * pi : __builtin_fmaf(mr, q.ii, mi * q.ir);
}

// d q / dA for the zero-order hold, q as above: (delta a - q)/A for
// |delta A| >= 1/2, below that delta^2 sum_k (k+1)/(k+2)! x^k through x^7
// (truncation below 1e-8), x = delta A.
__device__ __forceinline__ void zoh_dq_dA(float dl, const CState& q, float are, float aim, float qr, float qi,
                                          float& kr, float& ki) {
  const float xr = dl * q.re, xi = dl * q.im;
  constexpr float c[8] = {0.5f, 1.0f / 3.0f, 0.125f, 1.0f / 30.0f, 1.0f / 144.0f, 1.0f / 840.0f, 1.0f / 5760.0f,
                          1.0f / 45360.0f};
  float sr = c[7], si = 0.0f;
#pragma unroll
  for (int k = 6; k >= 0; --k) {  // s <- s x + c_k
    const float nr = __builtin_fmaf(sr, xr, __builtin_fmaf(-si, xi, c[k]));
    const float ni = __builtin_fmaf(sr, xi, si * xr);
    sr = nr;
    si = ni;
  }
  const float d2 = dl * dl;
  const float er = __builtin_fmaf(dl, are, -qr), ei = __builtin_fmaf(dl, aim, -qi);  // delta a - q
  const bool small = xr * xr + xi * xi < 0.25f;
  kr = small ? d2 * sr : __builtin_fmaf(er, q.ir, -ei * q.ii);
  ki = small ? d2 * si : __builtin_fmaf(er, q.ii, ei * q.ir);
}

// One complex value stored as an (re, im) pair of the input type, widened.
// (hr, hi) <- P[i] (hr, hi) + H[i] (complex) for i = 0 .. count - 1 in
// order: the aggregates of the pieces before this one, `stride` floats
// apart, each an (re, im) pair. The loads go out eight pieces at a time.
// CONJ: conj(P[i]) in place of P[i] (the adjoint's fold over later segments).
template <bool CONJ = false>
__device__ __forceinline__ void fold_aggregates_c(const float* P, const float* H, int count, int64_t stride,
                                                  float& hr, float& hi) {
  auto one = [&](float pr, float pi, float gr, float gi) {
    if (CONJ) pi = -pi;
    const float nr = __builtin_fmaf(pr, hr, __builtin_fmaf(-pi, hi, gr));
    const float ni = __builtin_fmaf(pr, hi, __builtin_fmaf(pi, hr, gi));
    hr = nr;
    hi = ni;
  };
  int i = 0;
  for (; i + 8 <= count; i += 8) {
    float p[8][2], g[8][2];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t w = (i + k) * stride;
      p[k][0] = P[w];
      p[k][1] = P[w + 1];
      g[k][0] = H[w];
      g[k][1] = H[w + 1];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) one(p[k][0], p[k][1], g[k][0], g[k][1]);
  }
  for (; i < count; ++i) {
    const int64_t w = i * stride;
    one(P[w], P[w + 1], H[w], H[w + 1]);
  }
}

__device__ __forceinline__ float2 load_cpair(const float* p, int64_t n) {
  return *reinterpret_cast<const float2*>(p + 2 * n);
}
__device__ __forceinline__ float2 load_cpair(const bf16_t* p, int64_t n) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(p + 2 * n);
  return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u));
}

// Conv taps of channel d right-aligned in four slots (widths below 4 have
// leading zero taps) and its bias.
__device__ __forceinline__ void conv_taps(const float* conv_w, const float* conv_b, int64_t d, int K, float (&w)[4],
                                          float& cb) {
  for (int k = 0; k < 4; ++k) w[k] = 0.0f;
  for (int k = 0; k < K; ++k) w[4 - K + k] = conv_w[d * K + k];
  cb = conv_b ? conv_b[d] : 0.0f;
}

// silu(causal depthwise conv) of a row's input at absolute step P: x_row and
// rs_row point at the row's step 0; inputs before the sequence come from the
// row's conv state st_row (K - 1 values, oldest first; zeros without one);
// inputs hidden by a later reset within the window count as 0.
template <typename InT, bool HAS_RESET>
__device__ __forceinline__ float conv_silu_at(const float (&w)[4], float cb, const InT* x_row, const uint8_t* rs_row,
                                              const float* st_row, int K, int64_t P) {
  float x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t pos = P - 3 + j;
    x[j] = pos >= 0 ? load_elem(x_row, pos) : (st_row && pos >= 1 - K ? st_row[pos + K - 1] : 0.0f);
  }
  const bool r0 = HAS_RESET && rs_row[P] != 0;
  const bool r1 = HAS_RESET && P >= 1 && rs_row[P - 1] != 0;
  const bool r2 = HAS_RESET && P >= 2 && rs_row[P - 2] != 0;
  return silu_f32(conv_pre(w, cb, x[0], x[1], x[2], x[3], r0, r1, r2));
}

// Entry kk of a row's final conv state: input L - (K - 1) + kk, 0 when a
// later reset hides it (a reset at that step itself starts a document there).
template <typename InT, bool HAS_RESET>
__device__ __forceinline__ float conv_state_at_end(const InT* x_row, const uint8_t* rs_row, const float* st_row, int K,
                                                   int64_t L, int kk) {
  const int64_t pos = L - (K - 1) + kk;
  if (HAS_RESET)
    for (int64_t q = pos + 1 > 0 ? pos + 1 : 0; q < L; ++q)
      if (rs_row[q]) return 0.0f;
  if (pos >= 0) return load_elem(x_row, pos);
  return st_row ? st_row[pos + K - 1] : 0.0f;
}

}  // namespace cplx
}  // namespace ssm
