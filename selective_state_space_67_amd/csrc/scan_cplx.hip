// Selective scan with a complex diagonal state (the S4D-Lin variant) for
// gfx950: the full-sequence forward and the single-token decode step.
//
// The pages give this variant's initialisation, A = -1/2 + i n, and say a
// complex state keeps phase information ("Technical analysis: Mamba selective
// state spaces", sections 4.1 and 5.3). The recurrence is the real one with
// complex A, B, C and h, real delta and u, and the real part of the read-out:
//
//   h[n] = exp(delta A[d,n]) h[n] + delta B[t,n] u
//   out  = (Re sum_n C[t,n] h[n] + D[d] u) * silu(z)
//
// exp(delta A) = exp(delta Re A) (cos(delta Im A) + i sin(delta Im A)). The
// angle is kept in revolutions: Im A / (2 pi) is held as an unevaluated sum
// of two floats and its product with delta is formed with an exact FMA
// remainder, so the angle reduced to [-1/2, 1/2] carries no rounding of the
// product or of 1/(2 pi), only delta's own. Sine and cosine come from Taylor
// polynomials on the quarter-turn-reduced angle (|theta| <= pi/4), accurate to
// about an ulp and without bias. The hardware v_sin_f32 / v_cos_f32 are not
// used: measured on gfx950, the cosine of small angles is low by about one
// ulp on average and the sine of small angles is off by up to 1e-6 relative
// (4.5e-5 for negative ones), and a biased decay compounds over the thousands
// of steps a slowly decaying state remembers. What is left grows with the
// angle: a relative error of a few float32 ulps in delta turns into a phase
// error of that size times |delta Im A|.
//
// Mapping. A DPP row of 16 lanes owns one channel (b, d) and lane k holds the
// NPL consecutive states k NPL .. k NPL + NPL - 1, so each lane reads its B
// and C values as contiguous (re, im) pairs. All lanes of a row run the same
// step together; the read-out is summed over the row with four DPP steps,
// after which every lane holds it. A workgroup of 4 waves covers 16 channels
// of one batch row, and B and C of each 16-step chunk are staged in LDS once
// for all of them.
//
// Chunk items. Thread (channel c, lane k) stages step k of its channel's chunk
// (delta with a reset flag in its sign bit, delta u) and keeps D u and
// silu(z); after the chunk the same lane holds the read-out of that step
// (selected while the steps go by) and writes the output. Lanes run their
// recurrences in lockstep, so the row needs no skew.
#include <algorithm>
#include <type_traits>

#include "cplx_device.h"
#include "kernels.h"

namespace ssm {
namespace {

using namespace cplx;

constexpr int kThreads = 256;
constexpr int kCPW = 16;  // channels per workgroup (one per DPP row)
constexpr int kT = 16;    // steps per chunk (one per lane of a row)

struct CplxArgs {
  int64_t B, D, L, N;
  int out_bf16;
  const void* u;
  const void* dt;
  const void* z;
  const void* Bm;  // (B, L, N, 2)
  const void* Cm;  // (B, L, N, 2)
  const float* dt_bias;
  const float* A;  // (D, N, 2)
  const float* Dskip;
  const float* h0;  // (B, D, N, 2) or null
  const uint8_t* reset;
  void* out;
  float* h_last;  // (B, D, N, 2) or null
  int n_dgroups;
  int64_t seg_len;  // steps per piece when the sequence is split (the last may be shorter)
  int nseg;
  float* ws_P;  // (nseg - 1, B, D, N, 2): the decay product of pieces 0 .. nseg-2
  float* ws_H;  // (nseg - 1, B, D, N, 2): their end states from a zero start
  // causal conv1d + SiLU on u (CONV kernels only)
  const float* conv_w;         // (D, conv_k)
  const float* conv_b;         // (D) or null
  const float* conv_state_in;  // (B, D, conv_k - 1) or null
  float* conv_state_out;       // (B, D, conv_k - 1) or null
  int conv_k;
};

// One step of a state: h = exp(delta A) h + q u B with the input coefficient
// q = delta, or with the zero-order hold q = (exp(delta A) - 1) / A
// (zoh_coef_c); returns Re(C h). dv is delta u (or u with the zero-order hold).
template <bool ZOH>
__device__ __forceinline__ float cplx_step(float dl, float dv, const CState& q, float2 Bv, float2 Cv, float& hr,
                                           float& hi) {
  float are, aim;
  decay(dl, q, are, aim);
  float br = Bv.x * dv, bi = Bv.y * dv;
  if constexpr (ZOH) {
    float qr, qi;
    zoh_coef_c(dl, q, are, aim, qr, qi);
    br = dv * __builtin_fmaf(qr, Bv.x, -qi * Bv.y);
    bi = dv * __builtin_fmaf(qr, Bv.y, qi * Bv.x);
  }
  const float nr = __builtin_fmaf(are, hr, __builtin_fmaf(-aim, hi, br));
  const float ni = __builtin_fmaf(are, hi, __builtin_fmaf(aim, hr, bi));
  hr = nr;
  hi = ni;
  return __builtin_fmaf(Cv.x, nr, -Cv.y * ni);
}

// Long sequences with few channels are split into pieces like the real scan:
// a first launch (AGG) runs each piece from a zero state and keeps only its
// affine aggregate, the decay product P = exp(A sum delta) (0 after a reset)
// and the end state H; the full launch folds the aggregates of the preceding
// pieces into its starting state, h <- P h + H, and runs its piece.
template <int NPL, typename InT, bool HAS_RESET, bool AGG, bool ZOH, bool CONV>
__global__ __launch_bounds__(kThreads) void cplx_scan_kernel(const CplxArgs a) {
  constexpr int NPAD = 16 * NPL;
  const int g = blockIdx.x % a.n_dgroups;
  const int rest = blockIdx.x / a.n_dgroups;
  const int b = rest % static_cast<int>(a.B);
  const int sp = rest / static_cast<int>(a.B);  // piece
  const int64_t t_seg = static_cast<int64_t>(sp) * a.seg_len;
  const int Lseg = static_cast<int>(min(a.seg_len, a.L - t_seg));
  const int N = static_cast<int>(a.N);
  const int tid = threadIdx.x;
  const int k = tid & 15;
  const int c = tid >> 4;  // channel within the workgroup = DPP row
  const int64_t d = static_cast<int64_t>(g) * kCPW + c;
  const bool dvalid = d < a.D;
  const int n0 = k * NPL;

  // (B, C) of the chunk's steps per state, as (B.re, B.im, C.re, C.im); states
  // past N stay zero.
  __shared__ __align__(16) float4 s_bc[kT * NPAD];
  // (delta, delta u), or (delta, u) with the zero-order hold; delta negated on a reset step
  __shared__ __align__(8) float2 s_du[kCPW * kT];
  // Read-out partials of a chunk, [channel][step][lane]; the lane that owns a
  // step adds its row's 16 partials after the chunk. Channels are kYS floats
  // apart so that the four rows of a wave write to different banks.
  constexpr int kYS = kT * 16 + 16;
  __shared__ __align__(16) float s_y[AGG ? 4 : kCPW * kYS];

  CState cq[NPL];
  float hr[NPL], hi[NPL];
  load_A<NPL>(a.A, d, N, n0, dvalid, cq);
  const int64_t row = static_cast<int64_t>(b) * a.D + d;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int64_t e = 2 * (row * N + n0 + j);
    const bool ok = !AGG && dvalid && n0 + j < N;
    hr[j] = ok && a.h0 ? a.h0[e] : 0.0f;
    hi[j] = ok && a.h0 ? a.h0[e + 1] : 0.0f;
    if (ok)  // h <- P h + H for the preceding pieces
      fold_aggregates_c(a.ws_P + e, a.ws_H + e, sp, a.B * a.D * N * 2, hr[j], hi[j]);
  }
  for (int i = tid; i < kT * NPAD; i += kThreads) s_bc[i] = make_float4(0.f, 0.f, 0.f, 0.f);

  const InT* __restrict__ u = static_cast<const InT*>(a.u) + row * a.L + t_seg;
  const InT* __restrict__ dt = static_cast<const InT*>(a.dt) + row * a.L + t_seg;
  const InT* __restrict__ z = a.z ? static_cast<const InT*>(a.z) + row * a.L + t_seg : nullptr;
  const InT* __restrict__ Bb = static_cast<const InT*>(a.Bm) + (static_cast<int64_t>(b) * a.L + t_seg) * N * 2;
  const InT* __restrict__ Cb = static_cast<const InT*>(a.Cm) + (static_cast<int64_t>(b) * a.L + t_seg) * N * 2;
  const uint8_t* __restrict__ rs = HAS_RESET ? a.reset + static_cast<int64_t>(b) * a.L + t_seg : nullptr;
  // AGG: this lane's compensated (Kahan) sum of delta over its steps, and whether one of them resets
  float dsum = 0.0f, dcomp = 0.0f;
  bool cleared = false;
  const float bias = dvalid && a.dt_bias ? a.dt_bias[d] : 0.0f;
  const float dsk = dvalid && a.Dskip ? a.Dskip[d] : 0.0f;
  // conv stage: taps, and the row's input, resets and initial conv state from step 0
  float cw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cb = 0.0f;
  if (CONV && dvalid) conv_taps(a.conv_w, a.conv_b, d, a.conv_k, cw, cb);
  const InT* __restrict__ u_row = u - t_seg;
  const uint8_t* __restrict__ rs_row = HAS_RESET ? rs - t_seg : nullptr;
  const float* __restrict__ cst = CONV && a.conv_state_in ? a.conv_state_in + row * (a.conv_k - 1) : nullptr;

  const ProgressPriority prio((Lseg + kT - 1) / kT, false);
  for (int t0 = 0; t0 < Lseg; t0 += kT) {
    prio.update(t0 / kT);
    const int steps = min(kT, Lseg - t0);
    __syncthreads();  // the previous chunk's readers are done
    // B and C of steps t0 .. t0+steps-1: contiguous (steps, N, 2) blocks (the
    // aggregate pass reads no C: Cm may be null there)
    for (int i = tid; i < steps * N; i += kThreads) {
      const int tl = i / N, n = i - tl * N;
      const int64_t e = (static_cast<int64_t>(t0 + tl) * N + n) * 2;
      s_bc[tl * NPAD + n] = make_float4(load_elem(Bb, e), load_elem(Bb, e + 1), AGG ? 0.0f : load_elem(Cb, e),
                                        AGG ? 0.0f : load_elem(Cb, e + 1));
    }
    // this lane's row item: step t0 + k of channel d
    const int t = t0 + k;
    const bool live = dvalid && k < steps;
    float dl = 0.0f, uu = 0.0f, gate = 1.0f;
    if (live) {
      uu = CONV ? conv_silu_at<InT, HAS_RESET>(cw, cb, u_row, rs_row, cst, a.conv_k, t_seg + t) : load_elem(u, t);
      dl = softplus_f32(load_elem(dt, t) + bias);
      if (!AGG && z) gate = silu_f32(load_elem(z, t));
      if constexpr (AGG) {
        const float yk = dl - dcomp;
        const float tk = dsum + yk;
        dcomp = (tk - dsum) - yk;
        dsum = tk;
      }
      if (HAS_RESET && rs[t]) {
        dl = -dl;
        cleared = true;
      }
    }
    s_du[c * kT + k] = make_float2(dl, ZOH ? uu : fabsf(dl) * uu);
    __syncthreads();

    float ymine = 0.0f;
    // (one step at a time for 16 states per lane: their registers leave no room to unroll)
#pragma unroll (NPL >= 16 ? 1 : 4)
    for (int tl = 0; tl < kT; ++tl) {
      const float2 du = s_du[c * kT + tl];
      float dlt = du.x;
      if (HAS_RESET) {
        const bool rs = __float_as_int(dlt) < 0;
        if (__builtin_amdgcn_ballot_w64(rs)) {
          keep_branch();
#pragma unroll
          for (int j = 0; j < NPL; ++j) {
            hr[j] = rs ? 0.0f : hr[j];
            hi[j] = rs ? 0.0f : hi[j];
          }
        }
        dlt = fabsf(dlt);
      }
      float p = 0.0f;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const float4 bc = s_bc[tl * NPAD + n0 + j];
        p += cplx_step<ZOH>(dlt, du.y, cq[j], make_float2(bc.x, bc.y), make_float2(bc.z, bc.w), hr[j], hi[j]);
      }
      if constexpr (!AGG) s_y[c * kYS + tl * 16 + k] = p;
    }
    if constexpr (!AGG) {
      // the row's lanes wrote the partials; lane k adds those of step k
      __builtin_amdgcn_wave_barrier();
      const float4* yr = reinterpret_cast<const float4*>(s_y + c * kYS + k * 16);
      const float4 y0 = yr[0], y1 = yr[1], y2 = yr[2], y3 = yr[3];
      ymine = ((y0.x + y0.y) + (y0.z + y0.w)) + ((y1.x + y1.y) + (y1.z + y1.w)) +
              (((y2.x + y2.y) + (y2.z + y2.w)) + ((y3.x + y3.y) + (y3.z + y3.w)));
      __builtin_amdgcn_wave_barrier();
    }
    if (!AGG && live) {
      const float v = (ymine + dsk * uu) * gate;
      const int64_t o = row * a.L + t_seg + t;
      if (a.out_bf16)
        store_elem(static_cast<bf16_t*>(a.out), o, v);
      else
        store_elem(static_cast<float*>(a.out), o, v);
    }
  }
  if constexpr (AGG) {
    // The piece's decay product exp(A S), S = its sum of delta (0 after a reset).
    const float S = row_sum16(dsum) - row_sum16(dcomp);
    const bool any_reset = __builtin_amdgcn_ballot_w64(cleared) & (0xFFFFull << (16 * ((tid >> 4) & 3)));
    if (dvalid) {
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        if (n0 + j >= N) continue;
        const int64_t w = static_cast<int64_t>(sp) * a.B * a.D * N * 2 + 2 * (row * N + n0 + j);
        float pr, pi;
        rotate_rev(any_reset ? 0.0f : fast_exp2(S * cq[j].ar), S, cq[j].ai, cq[j].ai_lo, pr, pi);
        a.ws_P[w] = pr;
        a.ws_P[w + 1] = pi;
        a.ws_H[w] = hr[j];
        a.ws_H[w + 1] = hi[j];
      }
    }
    return;
  }
  if (CONV && a.conv_state_out && sp == a.nseg - 1 && tid < kCPW * 3) {  // final conv state
    const int cc = tid / 3, kk = tid % 3;
    const int64_t dd = static_cast<int64_t>(g) * kCPW + cc;
    if (dd < a.D && kk < a.conv_k - 1) {
      const int64_t rr = static_cast<int64_t>(b) * a.D + dd;
      a.conv_state_out[rr * (a.conv_k - 1) + kk] = conv_state_at_end<InT, HAS_RESET>(
          static_cast<const InT*>(a.u) + rr * a.L, HAS_RESET ? a.reset + static_cast<int64_t>(b) * a.L : nullptr,
          a.conv_state_in ? a.conv_state_in + rr * (a.conv_k - 1) : nullptr, a.conv_k, a.L, kk);
    }
  }
  if (a.h_last && dvalid && sp == a.nseg - 1) {
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      if (n0 + j < N) {
        a.h_last[2 * (row * N + n0 + j)] = hr[j];
        a.h_last[2 * (row * N + n0 + j) + 1] = hi[j];
      }
    }
  }
}

struct CplxUpdateArgs {
  int64_t B, D, N;
  int out_bf16;
  float* h;  // (B, D, N, 2), in place
  const void* u;
  const void* dt;
  const void* z;
  const float* dt_bias;
  const float* A;  // (D, N, 2)
  const float* Dskip;
  const void* Bm;  // (B, N, 2)
  const void* Cm;
  void* out;
  float* conv_state;    // (B, D, conv_k - 1), updated in place; null without a conv stage
  const float* conv_w;  // (D, conv_k)
  const float* conv_b;  // (D) or null
  int conv_k;
  int dtiles;  // channel tiles per batch-row tile (cplx_update_tile)
  int stream;  // cplx_update_tile: read the state with nontemporal loads
};

// Decode: one (b, d) row per DPP row of 16 lanes, 16 rows per workgroup. Lane
// k holds states k, k + 16, k + 32, ..., so for each j the 16 lanes of a row
// read 16 consecutive (re, im) pairs of h, A, B and C: coalesced accesses to
// the state, which is what the step moves.
// STREAM: the state is read with nontemporal loads (states larger than the
// L2, which a model's decode reads from HBM; as in the real decode step).
template <int NPL, typename InT, bool ZOH, bool STREAM>
__global__ __launch_bounds__(kThreads) void cplx_update_kernel(const CplxUpdateArgs a) {
  const int tid = threadIdx.x;
  const int k = tid & 15;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kCPW + (tid >> 4);
  if (row >= a.B * a.D) return;  // whole DPP rows leave together
  const int64_t b = row / a.D, d = row % a.D;
  const int N = static_cast<int>(a.N);
  const InT* __restrict__ Bb = static_cast<const InT*>(a.Bm) + b * N * 2;
  const InT* __restrict__ Cb = static_cast<const InT*>(a.Cm) + b * N * 2;
  const float* __restrict__ Ad = a.A + d * N * 2;
  float* __restrict__ h = a.h + row * N * 2;
  // States past N read state N - 1 (always in bounds) and are zeroed after
  // the load, so every load is an unconditional global load.
  float2 hv[NPL], av[NPL], bv[NPL], cv[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = k + 16 * j;
    const bool ok = n < N;
    const int nc = ok ? n : N - 1;
    if constexpr (STREAM) {
      typedef float v2f __attribute__((ext_vector_type(2)));
      const v2f t = __builtin_nontemporal_load(reinterpret_cast<const v2f*>(h + 2 * nc));
      hv[j] = make_float2(t.x, t.y);
    } else {
      hv[j] = *reinterpret_cast<const float2*>(h + 2 * nc);
    }
    av[j] = *reinterpret_cast<const float2*>(Ad + 2 * nc);
    bv[j] = load_cpair(Bb, nc);
    cv[j] = load_cpair(Cb, nc);
    if (!ok) {
      hv[j] = make_float2(0.0f, 0.0f);
      av[j] = hv[j];
      bv[j] = hv[j];
      cv[j] = hv[j];
    }
  }
  const float x = load_elem(static_cast<const InT*>(a.u), row);
  float uu = x;
  float* cst = nullptr;
  if (a.conv_w) {  // u' = silu(conv over the row's conv state and this input)
    const int K = a.conv_k;
    cst = a.conv_state + row * (K - 1);
    float pre = __builtin_fmaf(a.conv_w[d * K + K - 1], x, a.conv_b ? a.conv_b[d] : 0.0f);
    for (int q = 0; q < K - 1; ++q) pre = __builtin_fmaf(a.conv_w[d * K + q], cst[q], pre);
    uu = silu_f32(pre);
  }
  const float dl = softplus_f32(load_elem(static_cast<const InT*>(a.dt), row) + (a.dt_bias ? a.dt_bias[d] : 0.0f));
  const float dv = ZOH ? uu : dl * uu;
  float p = 0.0f;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = k + 16 * j;
    float hr = hv[j].x, hi = hv[j].y;
    p += cplx_step<ZOH>(dl, dv, make_cstate(av[j].x, av[j].y), bv[j], cv[j], hr, hi);
    if (n < N) *reinterpret_cast<float2*>(h + 2 * n) = make_float2(hr, hi);
  }
  p = row_sum16(p);
  if (k == 0) {
    if (cst) {  // shift the conv state by this input (the row's lanes have all read it)
      for (int q = 0; q + 1 < a.conv_k - 1; ++q) cst[q] = cst[q + 1];
      if (a.conv_k > 1) cst[a.conv_k - 2] = x;
    }
    float v = p + (a.Dskip ? a.Dskip[d] : 0.0f) * uu;
    if (a.z) v *= silu_f32(load_elem(static_cast<const InT*>(a.z), row));
    if (a.out_bf16)
      store_elem(static_cast<bf16_t*>(a.out), row, v);
    else
      store_elem(static_cast<float*>(a.out), row, v);
  }
}

// Tiled decode for N = 8 .. 128, a power of two: LR = N / 2 lanes per row,
// each lane two consecutive complex states, so every state access is 16
// bytes. As in the real decode step, a thread holds a tile of RD consecutive
// channels by RB batch rows of its state pair: its A values (and the
// constants derived from them) serve RB rows, its B and C values RD rows, and
// u, dt_raw, z, dt_bias and D come as runs of RD elements. Every load of the
// tile is issued before any arithmetic; batch rows past the end of a ragged
// last tile repeat the last row's loads and skip every store.
template <typename InT, int LR, int RD, int RB, bool ZOH>
__global__ __launch_bounds__(kThreads) void cplx_update_tile(const CplxUpdateArgs a) {
  constexpr int SLOTS = kThreads / LR;
  const int li = threadIdx.x % LR;
  const int bt = blockIdx.x / a.dtiles;
  const int d0 = ((blockIdx.x - bt * a.dtiles) * SLOTS + static_cast<int>(threadIdx.x) / LR) * RD;
  // Whole slots only (LR divides 64): an inactive slot takes no part in the
  // other slots' cross-lane adds.
  if (d0 >= a.D) return;
  const int D = static_cast<int>(a.D), N = static_cast<int>(a.N);
  const int b0 = bt * RB;
  const int nb = min(RB, static_cast<int>(a.B) - b0);
  const int n0 = li * 2;
  using RunIn = Run<InT, RD>;
  using Run4 = Run<InT, 4>;
  using RunF = Run<float, RD>;
  const InT* u_in = static_cast<const InT*>(a.u);
  const InT* dt_in = static_cast<const InT*>(a.dt);
  const InT* z_in = static_cast<const InT*>(a.z);

  int bj[RB];
  int64_t rowj[RB];
  float4 hv[RB][RD];  // (re, im) of states n0 and n0 + 1
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    bj[j] = min(b0 + j, static_cast<int>(a.B) - 1);
    rowj[j] = static_cast<int64_t>(bj[j]) * D + d0;
#pragma unroll
    for (int i = 0; i < RD; ++i) {
      const float* p = a.h + ((rowj[j] + i) * N + n0) * 2;
      if (a.stream) {  // a state larger than the L2: nontemporal loads
        typedef float v4f __attribute__((ext_vector_type(4)));
        const v4f t = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
        hv[j][i] = make_float4(t.x, t.y, t.z, t.w);
      } else {
        hv[j][i] = *reinterpret_cast<const float4*>(p);
      }
    }
  }
  float4 Av[RD];
#pragma unroll
  for (int i = 0; i < RD; ++i)
    Av[i] = *reinterpret_cast<const float4*>(a.A + (static_cast<int64_t>(d0 + i) * N + n0) * 2);
  typename Run4::raw Bv[RB], Cv[RB];
  typename RunIn::raw uv[RB], xv[RB], zv[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int64_t bn = (static_cast<int64_t>(bj[j]) * N + n0) * 2;
    Bv[j] = Run4::load(static_cast<const InT*>(a.Bm) + bn);
    Cv[j] = Run4::load(static_cast<const InT*>(a.Cm) + bn);
    uv[j] = RunIn::load(u_in + rowj[j]);
    xv[j] = RunIn::load(dt_in + rowj[j]);
    zv[j] = z_in ? RunIn::load(z_in + rowj[j]) : typename RunIn::raw{};
  }
  const typename RunF::raw biasv = a.dt_bias ? RunF::load(a.dt_bias + d0) : typename RunF::raw{};
  const typename RunF::raw dskv = a.Dskip ? RunF::load(a.Dskip + d0) : typename RunF::raw{};

  CState q0[RD], q1[RD];
#pragma unroll
  for (int i = 0; i < RD; ++i) {
    q0[i] = make_cstate(Av[i].x, Av[i].y);
    q1[i] = make_cstate(Av[i].z, Av[i].w);
  }
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const float2 B0 = make_float2(Run4::at(Bv[j], 0), Run4::at(Bv[j], 1));
    const float2 B1 = make_float2(Run4::at(Bv[j], 2), Run4::at(Bv[j], 3));
    const float2 C0 = make_float2(Run4::at(Cv[j], 0), Run4::at(Cv[j], 1));
    const float2 C1 = make_float2(Run4::at(Cv[j], 2), Run4::at(Cv[j], 3));
    float o[RD];
#pragma unroll
    for (int i = 0; i < RD; ++i) {
      const int64_t row = rowj[j] + i;
      const float x = RunIn::at(uv[j], i);
      float uu = x;
      if (a.conv_w) {  // u' = silu(conv over the row's conv state and this input)
        const int K = a.conv_k, d = d0 + i;
        const float* cst = a.conv_state + row * (K - 1);
        float pre = __builtin_fmaf(a.conv_w[d * K + K - 1], x, a.conv_b ? a.conv_b[d] : 0.0f);
        for (int q = 0; q < K - 1; ++q) pre = __builtin_fmaf(a.conv_w[d * K + q], cst[q], pre);
        uu = silu_f32(pre);
      }
      const float dl = softplus_f32(RunIn::at(xv[j], i) + RunF::at(biasv, i));
      const float dv = ZOH ? uu : dl * uu;
      float4 h = hv[j][i];
      float p = cplx_step<ZOH>(dl, dv, q0[i], B0, C0, h.x, h.y);
      p += cplx_step<ZOH>(dl, dv, q1[i], B1, C1, h.z, h.w);
      if (j < nb) *reinterpret_cast<float4*>(a.h + (row * N + n0) * 2) = h;
      p = group_sum_last<LR>(p);
      if (a.Dskip) p += RunF::at(dskv, i) * uu;
      o[i] = z_in ? p * silu_f32(RunIn::at(zv[j], i)) : p;
    }
    if (li == LR - 1 && j < nb) {
      if (a.out_bf16)
        store_run<RD>(static_cast<bf16_t*>(a.out) + rowj[j], o);
      else
        store_run<RD>(static_cast<float*>(a.out) + rowj[j], o);
      if (a.conv_w && a.conv_k > 1) {  // shift the conv states by this input (the row's lanes have all read them)
#pragma unroll
        for (int i = 0; i < RD; ++i) {
          float* cst = a.conv_state + (rowj[j] + i) * (a.conv_k - 1);
          for (int q = 0; q + 1 < a.conv_k - 1; ++q) cst[q] = cst[q + 1];
          cst[a.conv_k - 2] = RunIn::at(uv[j], i);
        }
      }
    }
  }
}

// States per lane: the smallest power of two with 16 NPL >= N.
template <typename Fn>
hipError_t with_npl(int64_t N, Fn&& fn) {
  if (N <= 16) return fn(std::integral_constant<int, 1>{});
  if (N <= 32) return fn(std::integral_constant<int, 2>{});
  if (N <= 64) return fn(std::integral_constant<int, 4>{});
  if (N <= 128) return fn(std::integral_constant<int, 8>{});
  return fn(std::integral_constant<int, 16>{});
}

}  // namespace

// Pieces of the sequence. Splitting costs an aggregate pass nearly as long
// as the scan itself (the rotation dominates both), so it pays only where the
// channels leave CUs idle or short of the waves that hide latency: aim for
// about 4 / NPL workgroups per CU (at least one), split only when the
// channels fill less than half of that, and keep pieces >= 128 steps and a
// multiple of 16 (the rotation makes every step costly enough that a piece's
// start-up is small against it: with a 512-step floor 1 x 256 x 8192 took
// 171 us in 16 pieces, 81 us in 64). With several states per lane (N > 32)
// one workgroup per CU already has the independent work it needs.
void plan_cplx_segments(int64_t B, int64_t D, int64_t L, int64_t N, int requested, int* nseg, int64_t* seg_len) {
  int64_t want;
  if (requested > 0) {
    want = requested;
  } else {
    const int64_t npl = N <= 16 ? 1 : N <= 32 ? 2 : 4;
    const int64_t blocks = B * ((D + kCPW - 1) / kCPW);
    const int64_t round = 256 * std::max<int64_t>(1, 4 / npl);
    want = 2 * blocks >= round ? 1 : round / blocks;
    want = std::min<int64_t>(want, std::max<int64_t>(1, L / 128));
  }
  want = std::max<int64_t>(1, std::min<int64_t>(want, (L + 15) / 16));
  int64_t len = (L + want - 1) / want;
  len = (len + 15) / 16 * 16;
  *seg_len = len;
  *nseg = static_cast<int>((L + len - 1) / len);
}

size_t cplx_workspace_bytes(int64_t B, int64_t D, int64_t N, int nseg) {
  if (nseg <= 1) return 0;
  return static_cast<size_t>(2) * static_cast<size_t>(nseg - 1) * static_cast<size_t>(B) * static_cast<size_t>(D) *
         static_cast<size_t>(N) * 2 * sizeof(float);
}

int64_t cplx_scan_grid_blocks(int64_t B, int64_t D, int nseg) { return B * ((D + kCPW - 1) / kCPW) * nseg; }

namespace {

CplxArgs cplx_args(const ScanPlan& p) {
  CplxArgs a{};
  a.B = p.B;
  a.D = p.D;
  a.L = p.L;
  a.N = p.N;
  a.out_bf16 = p.out_bf16;
  a.u = p.u;
  a.dt = p.dt;
  a.z = p.z;
  a.Bm = p.Bm;
  a.Cm = p.Cm;
  a.dt_bias = p.dt_bias;
  a.A = p.A;
  a.Dskip = p.Dskip;
  a.h0 = p.h0;
  a.reset = p.reset;
  a.out = p.out;
  a.h_last = p.h_last;
  a.n_dgroups = static_cast<int>((p.D + kCPW - 1) / kCPW);
  a.nseg = p.nseg;
  a.seg_len = p.seg_len;
  a.conv_w = p.conv_w;
  a.conv_b = p.conv_b;
  a.conv_state_in = p.conv_state_in;
  a.conv_state_out = p.conv_state_out;
  a.conv_k = p.conv_k;
  return a;
}

// Aggregates of pieces 0 .. agg_pieces-1 into a.ws_P / a.ws_H, then (when
// full) the full pass over every piece.
hipError_t launch_cplx(const ScanPlan& p, const CplxArgs& a, int agg_pieces, bool full, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(cplx_scan_grid_blocks(p.B, p.D, p.nseg)));
  const dim3 grid_agg(static_cast<unsigned>(cplx_scan_grid_blocks(p.B, p.D, agg_pieces)));
  return with_npl(p.N, [&](auto npl) {
    constexpr int NPL = decltype(npl)::value;
    auto run = [&](auto in_t, auto has_reset, auto zoh, auto conv) {
      using InT = decltype(in_t);
      constexpr bool R = decltype(has_reset)::value, Z = decltype(zoh)::value, C = decltype(conv)::value;
      if (agg_pieces > 0) {
        SSM_LOG("launch cplx_scan_kernel<%d> aggregate: %s in, reset %d, zoh %d, conv %d; grid %u x %d threads "
                "(%d channels per workgroup), %d pieces of %lld steps",
                NPL, sizeof(InT) == 2 ? "bf16" : "f32", R, Z, C, grid_agg.x, kThreads, kCPW, agg_pieces,
                static_cast<long long>(p.seg_len));
        hipLaunchKernelGGL((cplx_scan_kernel<NPL, InT, R, true, Z, C>), grid_agg, dim3(kThreads), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess || !full) return e;
      }
      if (!full) return hipSuccess;
      SSM_LOG("launch cplx_scan_kernel<%d> full: %s in, reset %d, zoh %d, conv %d; grid %u x %d threads "
              "(%d channels per workgroup), %d pieces of %lld steps",
              NPL, sizeof(InT) == 2 ? "bf16" : "f32", R, Z, C, grid.x, kThreads, kCPW, p.nseg,
              static_cast<long long>(p.seg_len));
      hipLaunchKernelGGL((cplx_scan_kernel<NPL, InT, R, false, Z, C>), grid, dim3(kThreads), 0, stream, a);
      return hipGetLastError();
    };
    auto with_conv = [&](auto in_t, auto has_reset, auto zoh) {
      return p.conv_w ? run(in_t, has_reset, zoh, std::true_type{}) : run(in_t, has_reset, zoh, std::false_type{});
    };
    auto with_zoh = [&](auto in_t, auto has_reset) {
      return p.zoh ? with_conv(in_t, has_reset, std::true_type{}) : with_conv(in_t, has_reset, std::false_type{});
    };
    if (p.in_bf16)
      return p.reset ? with_zoh(bf16_t{}, std::true_type{}) : with_zoh(bf16_t{}, std::false_type{});
    return p.reset ? with_zoh(float{}, std::true_type{}) : with_zoh(float{}, std::false_type{});
  });
}

// Folds the pieces' complex aggregates in order: P = prod_s P_s, H <- P_s H + H_s.
__global__ __launch_bounds__(256) void cplx_aggregate_fold_kernel(const float2* wsP, const float2* wsH, int nseg,
                                                                  int64_t count, float2* P, float2* H) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= count) return;
  float pr = 1.0f, pi = 0.0f, hr = 0.0f, hi = 0.0f;
  for (int s = 0; s < nseg; ++s) {
    const float2 q = wsP[s * count + i], g = wsH[s * count + i];
    const float nr = __builtin_fmaf(q.x, hr, __builtin_fmaf(-q.y, hi, g.x));
    const float ni = __builtin_fmaf(q.x, hi, __builtin_fmaf(q.y, hr, g.y));
    hr = nr;
    hi = ni;
    const float mr = __builtin_fmaf(q.x, pr, -q.y * pi);
    const float mi = __builtin_fmaf(q.x, pi, q.y * pr);
    pr = mr;
    pi = mi;
  }
  P[i] = make_float2(pr, pi);
  H[i] = make_float2(hr, hi);
}

}  // namespace

hipError_t launch_scan_cplx(const ScanPlan& p, hipStream_t stream, bool aggregates_only) {
  CplxArgs a = cplx_args(p);
  if (p.nseg > 1) {
    const size_t half = cplx_workspace_bytes(p.B, p.D, p.N, p.nseg) / 2 / sizeof(float);
    a.ws_P = p.ws;
    a.ws_H = p.ws + half;
  }
  // the last piece's aggregate is never needed
  return launch_cplx(p, a, p.nseg - 1, !aggregates_only, stream);
}

hipError_t launch_aggregate_cplx(const ScanPlan& p, float* P, float* H, hipStream_t stream) {
  CplxArgs a = cplx_args(p);
  const int64_t count = p.B * p.D * p.N;  // complex values
  a.ws_P = p.nseg > 1 ? p.ws : P;
  a.ws_H = p.nseg > 1 ? p.ws + 2 * static_cast<size_t>(p.nseg) * count : H;
  hipError_t e = launch_cplx(p, a, p.nseg, false, stream);
  if (e != hipSuccess || p.nseg == 1) return e;
  SSM_LOG("launch cplx_aggregate_fold_kernel: %lld states, %d pieces; grid %lld x 256 threads",
          static_cast<long long>(count), p.nseg, static_cast<long long>((count + 255) / 256));
  hipLaunchKernelGGL(cplx_aggregate_fold_kernel, dim3(static_cast<unsigned>((count + 255) / 256)), dim3(256), 0,
                     stream, reinterpret_cast<const float2*>(a.ws_P), reinterpret_cast<const float2*>(a.ws_H),
                     p.nseg, count, reinterpret_cast<float2*>(P), reinterpret_cast<float2*>(H));
  return hipGetLastError();
}

hipError_t launch_state_update_cplx(const UpdatePlan& p, hipStream_t stream) {
  CplxUpdateArgs a{};
  a.B = p.B;
  a.D = p.D;
  a.N = p.N;
  a.out_bf16 = p.out_bf16;
  a.h = p.h;
  a.u = p.u;
  a.dt = p.dt;
  a.z = p.z;
  a.dt_bias = p.dt_bias;
  a.A = p.A;
  a.Dskip = p.Dskip;
  a.Bm = p.Bm;
  a.Cm = p.Cm;
  a.out = p.out;
  a.conv_state = p.conv_state;
  a.conv_w = p.conv_w;
  a.conv_b = p.conv_b;
  a.conv_k = p.conv_k;
  const bool streamed = p.B * p.D * p.N * 2 * static_cast<int64_t>(sizeof(float)) > (int64_t{32} << 20);
  // The tiled kernel: N = 8 .. 128 a power of two, 16-byte state and A rows,
  // runs of two channels (D even, the (B, D) and (D) tensors aligned to them),
  // two or more batch rows and fewer than 2^31 rows.
  const auto al = [](const void* q, size_t n) { return reinterpret_cast<uintptr_t>(q) % n == 0; };
  const size_t s_in = p.in_bf16 ? 2 : 4;
  const bool tile_ok = p.N >= 8 && p.N <= 128 && (p.N & (p.N - 1)) == 0 && p.B >= 2 && p.D % 2 == 0 &&
                       p.B * p.D < (int64_t{1} << 31) && al(p.h, 16) && al(p.A, 16) && al(p.Bm, 4 * s_in) &&
                       al(p.Cm, 4 * s_in) && al(p.u, 2 * s_in) && al(p.dt, 2 * s_in) && (!p.z || al(p.z, 2 * s_in)) &&
                       al(p.out, p.out_bf16 ? 4 : 8) && (!p.dt_bias || al(p.dt_bias, 8)) && (!p.Dskip || al(p.Dskip, 8));
  if (tile_ok) {
    a.stream = streamed;
    auto tile = [&](auto lr, auto zoh) {
      constexpr int LR = decltype(lr)::value;
      constexpr bool Z = decltype(zoh)::value;
      constexpr int kChannels = kThreads / LR * 2;
      a.dtiles = static_cast<int>((p.D + kChannels - 1) / kChannels);
      const dim3 grid(static_cast<unsigned>(a.dtiles * ((p.B + 1) / 2)));
      SSM_LOG("launch cplx_update_tile<%d lanes per row, 2 channels x 2 batch rows per thread>: %s in, zoh %d, "
              "streamed state %d; grid %u x %d threads",
              LR, p.in_bf16 ? "bf16" : "f32", Z, static_cast<int>(streamed), grid.x, kThreads);
      if (p.in_bf16)
        hipLaunchKernelGGL((cplx_update_tile<bf16_t, LR, 2, 2, Z>), grid, dim3(kThreads), 0, stream, a);
      else
        hipLaunchKernelGGL((cplx_update_tile<float, LR, 2, 2, Z>), grid, dim3(kThreads), 0, stream, a);
      return hipGetLastError();
    };
    auto with_lr = [&](auto zoh) {
      switch (p.N) {
        case 8: return tile(std::integral_constant<int, 4>{}, zoh);
        case 16: return tile(std::integral_constant<int, 8>{}, zoh);
        case 32: return tile(std::integral_constant<int, 16>{}, zoh);
        case 64: return tile(std::integral_constant<int, 32>{}, zoh);
        default: return tile(std::integral_constant<int, 64>{}, zoh);
      }
    };
    return p.zoh ? with_lr(std::true_type{}) : with_lr(std::false_type{});
  }
  const dim3 grid(static_cast<unsigned>((p.B * p.D + kCPW - 1) / kCPW));
  auto go = [&](auto npl, auto zoh, auto st) {
    constexpr int NPL = decltype(npl)::value;
    constexpr bool Z = decltype(zoh)::value, S = decltype(st)::value;
    SSM_LOG("launch cplx_update_kernel<%d>: %s in, zoh %d, streamed state %d; grid %u x %d threads", NPL,
            p.in_bf16 ? "bf16" : "f32", Z, S, grid.x, kThreads);
    if (p.in_bf16)
      hipLaunchKernelGGL((cplx_update_kernel<NPL, bf16_t, Z, S>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((cplx_update_kernel<NPL, float, Z, S>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
  };
  using T = std::true_type;
  using F = std::false_type;
  return with_npl(p.N, [&](auto npl) {
    if (p.zoh) return streamed ? go(npl, T{}, T{}) : go(npl, T{}, F{});
    return streamed ? go(npl, F{}, T{}) : go(npl, F{}, F{});
  });
}

}  // namespace ssm
