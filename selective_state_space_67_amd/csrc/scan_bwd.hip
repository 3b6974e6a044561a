// Backward pass of the selective scan for gfx950 (MI355X): the reverse sweep
// and the final reduction.
//
// The forward keeps no intermediate states and the backward recomputes them
// ("Technical analysis: Mamba selective state spaces", section 2.2, item 3,
// gradient recomputation). The gradients are the chain rule through the
// recurrence of the forward kernel (softplus step, h_t = a_t h_{t-1} +
// delta_t B_t u_t with a_t = exp(delta_t A), y_t = C_t h_t + D u_t, SiLU gate),
// run in reverse time with the adjoint g_t of h_t:
//
//   g_t  = a_{t+1} g_{t+1} + dy_t C_t,   dy_t = dout_t silu(z_t)
//   dB[t,n] += g_t[n] delta_t u_t          dC[t,n] += dy_t h_t[n]
//   dA[n]   += g_t[n] a_t[n] h_{t-1}[n] delta_t
//   du_t     = dy_t D + delta_t S1_t,      S1_t = sum_n g_t[n] B_t[n]
//   d dt_t   = (S2_t + u_t S1_t) sigmoid(x_t),  S2_t = sum_n A[n] g_t[n] a_t[n] h_{t-1}[n]
//   dz_t     = dout_t (Y_t + D u_t) silu'(z_t),  Y_t = sum_n C_t[n] h_t[n]
//
// Three launches make up the pass:
//  1. the checkpoint sweep (scan_fwd.hip, kCheckpoint): the forward recurrence
//     in lockstep, writing the state entering every 16-step chunk, and for
//     every backward segment the product of its a_t and its adjoint from a
//     zero start (accumulated in forward order as sum (prod a) dy C);
//  2. the reverse sweep (this file): one workgroup per (batch row, channel
//     group, segment). It folds the later segments' aggregates into the
//     adjoint entering its segment, then walks the segment's 16-step chunks
//     backwards: recompute the chunk's states from its checkpoint (kept in
//     registers), then run the adjoint through the chunk;
//  3. the reduction (this file): the shared gradients summed over channel
//     groups (dB, dC) and over batch rows and segments (dA, dD, d dt_bias).
//
// Layout of the reverse sweep. Each lane holds four consecutive states of one
// channel; a channel spans LPC lanes (LPC = N/4 rounded up to a power of two,
// at least 4). The sums over n (S1, S2, Y) are butterflies of DPP adds over
// those LPC lanes (two for N <= 16), so four states share every cross-lane
// operation. Lanes step in lockstep. After each step the lane whose index
// matches the step (mod 4) keeps the three sums; every four steps those lanes
// compute du, d dt_raw and dz for four steps at once. The sums over channels
// (dB, dC) go through a per-wave LDS buffer (a wave adds up its channels for
// two steps at a time into its own totals); the waves' totals are added in a
// fixed order and written as one partial per channel group, so every sum has
// a fixed order and repeated calls give identical bits.
#include <algorithm>

#include "device_math.h"
#include "kernels.h"

namespace ssm {
namespace {

constexpr int kK = 16;                 // steps per chunk (the checkpoint spacing)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kNPL = 4;                // states per lane

template <int LPC_>
struct BwdTile {
  static constexpr int LPC = LPC_;               // lanes per channel
  static constexpr int NPADC = LPC * kNPL;       // states covered per channel
  static constexpr int CPWAVE = 64 / LPC;        // channels per wave
  static constexpr int CPW = kWaves * CPWAVE;    // channels per workgroup
  // Per-wave buffer for the channel sums: [type][channel][step parity][state],
  // padded so that the 16-byte writes and the 4-byte reads spread over banks.
  // A write pass covers 16 lanes, 16 / LPC channels of LPC x 4 floats each:
  // with fewer than 16 lanes per channel the channel stride QS is an odd
  // multiple (3) of 4 x LPC, so those channels start in different bank
  // groups (2 x NPADC + 4 put two of every four channels on the same banks).
  static constexpr int QS = LPC >= 16 ? 2 * NPADC + 4 : 12 * LPC;
  static constexpr int TS = CPWAVE * QS + 32;
  // Steps per flush of the dB / dC totals: each wave keeps its own totals
  // (2 x FP x NPADC floats) and the flush adds the waves in a fixed order, so
  // the result does not depend on timing. FP x NPADC <= 1024 bounds the LDS.
  static constexpr int FP = NPADC <= 64 ? 16 : 1024 / NPADC;
};

struct BwdArgs {
  int64_t B, D, L, N, seg_steps, n_ck;
  int nsegb, n_dgroups, nblocks, grad_bf16;
  const void* u;
  const void* dt;
  const void* z;
  const void* Bm;
  const void* Cm;
  const void* dout;
  const float* dt_bias;
  const float* A;
  const float* Dskip;
  const uint8_t* reset;
  const float* dh_last;
  const float* ckpt;
  const float* seg_P;
  const float* seg_G;
  void* du;
  void* ddt;
  void* dz;
  float* dh0;
  float* partB;     // (G, B, L, N)
  float* partC;     // (G, B, L, N)
  float* partA;     // (B, nsegb, D, N)
  float* partD;     // (B, nsegb, D)
  float* partBias;  // (B, nsegb, D)
  const float* uconv;  // conv stage: the scan input u' (B, D, L), read in place of u
  float* du_conv;      // conv stage: the gradient of u' (B, D, L), written in place of du
};

// Zero-order hold (ZOH kernels): the input term is phi B u with
// phi = (e^{delta A} - 1) / A in place of delta, so
//   d phi / d delta = abar (the decay before any reset masking),
//   d phi / d A     = delta^2 psi(delta A),
// du = dy D + sum_n g phi B, d delta = S2 + u sum_n g B abar, and dA gains
// g B u delta^2 psi; dB is g u phi.

// DPP lane permutation within rows of 16 (control word CTRL).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the LPC lanes of a channel; every lane of the group gets the total.
template <int LPC>
__device__ __forceinline__ float chan_sum(float v) {
  if constexpr (LPC >= 2) v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (LPC >= 4) v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (LPC >= 8) v += dpp_f<0x141>(v);   // row_half_mirror: the other quad of each 8
  if constexpr (LPC >= 16) v += dpp_f<0x140>(v);  // row_mirror: the other 8 of each row
  // Across rows: v_permlane16_swap / v_permlane32_swap exchange rows between
  // the two operands (a VALU operation, where a shuffle would go through the
  // LDS); with both operands v, the two results are this row's value and the
  // partner row's, so their sum is the pair's total in every lane.
  if constexpr (LPC >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (LPC >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return v;
}


__device__ __forceinline__ void store_grad(const BwdArgs& a, void* p, int64_t i, float v) {
  if (a.grad_bf16)
    store_elem(static_cast<bf16_t*>(p), i, v);
  else
    store_elem(static_cast<float*>(p), i, v);
}

// Two waves per SIMD; the zero-order-hold variant's extra per-state terms need
// more registers than that allows without spilling, so it runs at one.
template <typename TL, typename InT, bool HAS_RESET, bool ZOH>
__global__ __launch_bounds__(kThreads, ZOH ? 1 : 2) void scan_bwd_kernel(const BwdArgs a) {
  constexpr int LPC = TL::LPC, NPADC = TL::NPADC, CPWAVE = TL::CPWAVE, CPW = TL::CPW;
  constexpr int QS = TL::QS, TS = TL::TS, FP = TL::FP;
  static_assert(kK % FP == 0 && FP % 2 == 0, "flush period");
  constexpr int BCI = kK * NPADC / kThreads;  // (step, state) staging items per thread
  static_assert(BCI >= 1 && (kK * NPADC) % kThreads == 0, "B/C staging split");

  // (delta, delta*u, dy, 0) per (channel, step); delta negated on a reset.
  // Channel rows are RS = 17 float4 apart (an odd number of 16-byte units),
  // so the channels of a wave read their rows from different banks.
  constexpr int RS = kK + 1;
  __shared__ __align__(16) float4 s_rec[CPW * RS];
  __shared__ __align__(16) float s_B[kK * NPADC];
  __shared__ __align__(16) float s_C[kK * NPADC];
  __shared__ __align__(16) float s_w[kWaves * 2 * TS];
  // Per-wave totals of the dB and dC terms: [wave][type][step][state], the
  // type halves 32 floats apart in banks.
  constexpr int AT = FP * NPADC + 32;   // floats per type
  constexpr int AW = 2 * AT;            // floats per wave
  __shared__ float s_acc[kWaves * AW];
  // The input gradients (du or the conv stage's du', d dt_raw, dz) of a pair
  // of chunks, [gradient][channel][step]: written out together once the pair
  // is done, as whole rows of 32 steps (128 bytes in float32) rather than the
  // 4 steps the finalizing lanes of a channel hold at a time, so that the L2
  // does not write back partially filled lines. Layouts with few channels per
  // workgroup (N > 64) store directly: there the dB/dC partials dominate the
  // traffic, and staging measured slower (2x2048x4096x128: 4.70 -> 4.82 ms).
  constexpr bool STAGE_OUT = LPC <= 16;
  constexpr int OS = 2 * kK + 4;        // floats per (gradient, channel) row
  __shared__ __align__(16) float s_out[STAGE_OUT ? 3 * CPW * OS : 4];

  int idx = blockIdx.x;
  if ((a.nblocks & 7) == 0) idx = (idx & 7) * (a.nblocks >> 3) + (idx >> 3);
  const int g = idx % a.n_dgroups;
  const int rest = idx / a.n_dgroups;
  const int b = rest % static_cast<int>(a.B);
  const int s = rest / static_cast<int>(a.B);
  const int64_t t_seg = static_cast<int64_t>(s) * a.seg_steps;
  const int64_t pend = min(t_seg + a.seg_steps, a.L);
  const int nchunks = static_cast<int>((pend - t_seg + kK - 1) / kK);
  const int N = static_cast<int>(a.N);
  const int64_t d0 = static_cast<int64_t>(g) * CPW;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int cw = lane / LPC;       // channel within the wave
  const int c = w * CPWAVE + cw;   // channel within the workgroup
  const int l = lane % LPC;        // lane within the channel
  const int64_t d = d0 + c;
  const bool dvalid = d < a.D;
  const int n0 = l * kNPL;
  const bool fin = l < 4;          // finalize / staging lane: owns steps l, l+4, l+8, l+12 of a chunk

  const InT* __restrict__ u_in = static_cast<const InT*>(a.u);
  const InT* __restrict__ dt_in = static_cast<const InT*>(a.dt);
  const InT* __restrict__ z_in = static_cast<const InT*>(a.z);
  const InT* __restrict__ go_in = static_cast<const InT*>(a.dout);
  const InT* __restrict__ B_in = static_cast<const InT*>(a.Bm);
  const InT* __restrict__ C_in = static_cast<const InT*>(a.Cm);
  const int64_t rowbase = (static_cast<int64_t>(b) * a.D + (dvalid ? d : 0)) * a.L;
  const int64_t bdn = (static_cast<int64_t>(b) * a.D + d) * N;

  // Per-lane parameters, gradient accumulators and the adjoint entering this
  // segment: dh_last folded through the aggregates of every later segment,
  // g <- P g + G (the later segments' affine maps, last one first).
  float Av[kNPL], A2[kNPL], gv[kNPL], dA[kNPL], invA[ZOH ? kNPL : 1];
#pragma unroll
  for (int j = 0; j < kNPL; ++j) {
    const int n = n0 + j;
    const bool ok = dvalid && n < N;
    Av[j] = ok ? a.A[d * N + n] : 0.0f;
    A2[j] = Av[j] * kLog2e;
    if constexpr (ZOH) invA[j] = Av[j] != 0.0f ? 1.0f / Av[j] : 0.0f;
    dA[j] = 0.0f;
    float gg = ok && a.dh_last ? a.dh_last[bdn + n] : 0.0f;
    if (ok) {
      // the later segments, last one first (stride back one segment)
      const int64_t wl = ((static_cast<int64_t>(b) * a.nsegb + a.nsegb - 1) * a.D + d) * N + n;
      gg = fold_aggregates(a.seg_P + wl, a.seg_G + wl, a.nsegb - 1 - s, -a.D * N, gg);
    }
    gv[j] = gg;
  }
  const float bias = dvalid && a.dt_bias ? a.dt_bias[d] : 0.0f;
  const float dsk = dvalid && a.Dskip ? a.Dskip[d] : 0.0f;
  float dD_acc = 0.0f, dbias_acc = 0.0f;

  struct Raw {
    InT b[BCI], c[BCI], dt[4], z[4], go[4];
    uint32_t u[4];  // raw bits: a float (f32 input or the conv stage's u'), or a bf16 in the low half
    uint8_t rs[4];
  };
  struct Out {
    float u[4], sig[4], gz[4];
  };

  auto load = [&](int J, Raw& r) {
    const int64_t tc = t_seg + static_cast<int64_t>(J) * kK;
#pragma unroll
    for (int q = 0; q < BCI; ++q) {
      const int it = tid + q * kThreads;
      const int t = it / NPADC, n = it % NPADC;
      const bool ok = n < N && tc + t < pend;
      const int64_t off = (static_cast<int64_t>(b) * a.L + tc + t) * N + n;
      r.b[q] = ok ? B_in[off] : InT{};
      r.c[q] = ok ? C_in[off] : InT{};
    }
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const int t = l + 4 * G;
      const bool ok = fin && dvalid && tc + t < pend;
      const int64_t off = rowbase + tc + t;
      // kept as loaded and converted at staging: a conversion here would wait for the load
      if constexpr (sizeof(InT) == 2)
        r.u[G] = ok ? (a.uconv ? __float_as_uint(a.uconv[off]) : static_cast<uint32_t>(u_in[off].bits)) : 0u;
      else
        r.u[G] = ok ? __float_as_uint(a.uconv ? a.uconv[off] : load_elem(u_in, off)) : 0u;
      r.dt[G] = ok ? dt_in[off] : InT{};
      r.z[G] = ok && z_in ? z_in[off] : InT{};
      r.go[G] = ok ? go_in[off] : InT{};
      r.rs[G] = HAS_RESET && ok ? a.reset[static_cast<int64_t>(b) * a.L + tc + t] : 0;
    }
  };

  // Per-step parameters of chunk J into LDS; the finalize factors stay in the
  // staging lane's registers (it finalizes the same steps).
  auto store = [&](int J, const Raw& r, Out& o) {
    const int64_t tc = t_seg + static_cast<int64_t>(J) * kK;
#pragma unroll
    for (int q = 0; q < BCI; ++q) {
      const int it = tid + q * kThreads;
      s_B[it] = load_elem(&r.b[q], 0);
      s_C[it] = load_elem(&r.c[q], 0);
    }
    if (!fin) return;
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const int t = l + 4 * G;
      const bool ok = dvalid && tc + t < pend;
      const float x = load_elem(&r.dt[G], 0) + bias;
      float dl = ok ? softplus_f32(x) : 0.0f;
      const float uu = __uint_as_float(sizeof(InT) == 2 && !a.uconv ? r.u[G] << 16 : r.u[G]);
      const float go = load_elem(&r.go[G], 0);
      float dy = go, gz = 0.0f;
      if (z_in) {
        const float zz = load_elem(&r.z[G], 0);
        const float sg = fast_rcp(1.0f + fast_exp2(-zz * kLog2e));
        dy = go * (zz * sg);
        gz = go * (sg * __builtin_fmaf(zz, 1.0f - sg, 1.0f));
      }
      const float dv = ZOH ? uu : dl * uu;  // ZOH keeps u: its coefficient depends on the state's A
      if (HAS_RESET && r.rs[G]) dl = -dl;  // sign bit: the state is cleared before this step
      s_rec[c * RS + t] = make_float4(dl, dv, dy, 0.0f);
      o.u[G] = uu;
      o.sig[G] = fast_rcp(1.0f + fast_exp2(-x * kLog2e));
      o.gz[G] = gz;
    }
  };

  float* const wbuf = s_w + w * 2 * TS;
  float* const wacc = s_acc + w * AW;

  // The workgroup's dB / dC terms of steps [t0, t0 + FP) of the chunk at tc:
  // the waves' totals added in order, one partial per channel group.
  // Items (type, step, state) are spread over the threads in a fixed pattern
  // (2 x FP x NPADC is a multiple of the thread count), and the address of
  // each item is a 32-bit offset from one base per flush. The loop stays
  // rolled: unrolled inside the unrolled steps it spilled (N = 128).
  constexpr int FLUSH_ITEMS = 2 * FP * NPADC;
  static_assert(FLUSH_ITEMS % kThreads == 0, "flush items per thread");
  const int64_t part_row = (static_cast<int64_t>(g) * a.B + b) * a.L * N;  // this group's (b, 0, 0)
  const int64_t part_type = static_cast<int64_t>(a.B) * a.L * N * a.n_dgroups;  // partC - partB
  auto flush = [&](int64_t tc, int t0) {
    const int64_t t_first = tc + t0;
    float* const base = a.partB + part_row + t_first * N;
    const int limit = static_cast<int>(min<int64_t>(FP, pend - t_first));  // steps of this period in the segment
#pragma unroll 1
    for (int q = 0; q < FLUSH_ITEMS / kThreads; ++q) {
      const int i = tid + q * kThreads;
      const int type = i / (FP * NPADC);
      const int tt = (i / NPADC) % FP;
      const int n = i % NPADC;
      if (n < N && tt < limit) {
        const int k = type * AT + tt * NPADC + n;
        float sum = s_acc[k];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) sum += s_acc[ww * AW + k];
        __builtin_nontemporal_store(sum, base + (type ? part_type : 0) + tt * N + n);
      }
    }
  };

  // Chunk J: recompute its states from the checkpoint, then the adjoint
  // backwards through it.
  // The checkpoint (state entering chunk J), loaded one chunk ahead.
  auto load_ckpt = [&](int J, float (&hs)[kNPL]) {
    const int64_t tc = t_seg + static_cast<int64_t>(J) * kK;
    const int64_t ci = ((static_cast<int64_t>(b) * a.n_ck + tc / kK) * a.D + d) * N;
#pragma unroll
    for (int j = 0; j < kNPL; ++j) hs[j] = dvalid && n0 + j < N ? __builtin_nontemporal_load(a.ckpt + ci + n0 + j) : 0.0f;
  };

  // The chunk pair (J, J + 1) of input gradients from s_out to memory: one
  // item per (gradient, channel, 4 steps), 16-byte stores (8-byte in bf16)
  // where the 4 steps are complete and aligned.
  auto flush_out = [&](int J) {
    constexpr int GROUPS = 2 * kK / 4;
    const int64_t t0 = t_seg + static_cast<int64_t>(J) * kK;
    const int steps = static_cast<int>(min<int64_t>(2 * kK, pend - t0));
    for (int i = tid; i < 3 * CPW * GROUPS; i += kThreads) {
      const int q = i % GROUPS, cc = (i / GROUPS) % CPW, kind = i / (GROUPS * CPW);
      const int64_t dd = d0 + cc;
      const int s0 = 4 * q;
      if (dd >= a.D || s0 >= steps || (kind == 2 && !a.dz)) continue;
      const float4 v = *reinterpret_cast<const float4*>(s_out + (kind * CPW + cc) * OS + s0);
      const float e[4] = {v.x, v.y, v.z, v.w};
      const int cnt = min(4, steps - s0);
      const int64_t at = (static_cast<int64_t>(b) * a.D + dd) * a.L + t0 + s0;
      const bool f32 = (kind == 0 && a.du_conv) || !a.grad_bf16;
      void* const dst = kind == 0 ? (a.du_conv ? static_cast<void*>(a.du_conv) : a.du) : kind == 1 ? a.ddt : a.dz;
      if (f32) {
        float* p = static_cast<float*>(dst) + at;
        if (cnt == 4 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
          typedef float v4f __attribute__((ext_vector_type(4)));
          __builtin_nontemporal_store(v4f{v.x, v.y, v.z, v.w}, reinterpret_cast<v4f*>(p));
        } else {
          for (int k = 0; k < cnt; ++k) p[k] = e[k];
        }
      } else {
        bf16_t* p = static_cast<bf16_t*>(dst) + at;
        if (cnt == 4 && (reinterpret_cast<uintptr_t>(p) & 7) == 0) {
          typedef uint32_t v2u __attribute__((ext_vector_type(2)));
          __builtin_nontemporal_store(v2u{bf16_pair(e[0], e[1]), bf16_pair(e[2], e[3])}, reinterpret_cast<v2u*>(p));
        } else {
          for (int k = 0; k < cnt; ++k) store_elem(p, k, e[k]);
        }
      }
    }
  };

  auto chunk = [&](int J, const Out& o, const float (&hs)[kNPL]) {
    const int64_t tc = t_seg + static_cast<int64_t>(J) * kK;
    // States of the chunk: the checkpoint hs, then h_t of every odd step in
    // registers; an even step's state is rebuilt from its odd predecessor in
    // the reverse pass (one FMA with the a_t that pass computes anyway).
    float hist[kK / 2][kNPL];
    __syncthreads();  // this chunk's LDS parameters are complete

    float h[kNPL];
#pragma unroll
    for (int j = 0; j < kNPL; ++j) h[j] = hs[j];
#pragma unroll
    for (int t = 0; t < kK; ++t) {
      const float4 r = s_rec[c * RS + t];
      const float4 bv = *reinterpret_cast<const float4*>(s_B + t * NPADC + n0);
      const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
      float dl = r.x;
      if (HAS_RESET) {
        const bool rs = __float_as_int(dl) < 0;
        if (__builtin_amdgcn_ballot_w64(rs)) {
          keep_branch();
#pragma unroll
          for (int j = 0; j < kNPL; ++j) h[j] = rs ? 0.0f : h[j];
        }
        dl = fabsf(dl);
      }
#pragma unroll
      for (int j = 0; j < kNPL; ++j) {
        const float abar = fast_exp2(dl * A2[j]);
        if constexpr (ZOH)
          h[j] = __builtin_fmaf(abar, h[j], (bb[j] * r.y) * zoh_coef(dl, dl * Av[j], abar, invA[j]));
        else
          h[j] = __builtin_fmaf(abar, h[j], bb[j] * r.y);
        if (t & 1) hist[t >> 1][j] = h[j];
      }
    }

    // The next chunk's loads (issued before this chunk) have landed by now:
    // wait for them here, before this chunk issues its gradient stores, so
    // that the loop does not wait at its end for those stores to complete.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    float F1 = 0.0f, F2 = 0.0f, FY = 0.0f, F3 = 0.0f;  // this lane's step sums in the current group of four

    // One reverse step: av = a_t (0 on a reset), hp = h_{t-1}, ht = h_t.
    // av = a_t masked by a reset, au = e^{delta A} unmasked (ZOH's d phi / d delta).
    auto rstep = [&](const int t, const float4 r, const float (&bb)[4], const float (&cc)[4],
                     const float (&av)[kNPL], const float (&au)[kNPL], const float (&hp)[kNPL],
                     const float (&ht)[kNPL]) {
      const float dl = fabsf(r.x), dv = r.y, dy = r.z;
      float s1 = 0.0f, s2 = 0.0f, s3 = 0.0f, yy = 0.0f, p3[kNPL], p4[kNPL];
#pragma unroll
      for (int j = 0; j < kNPL; ++j) {
        gv[j] = __builtin_fmaf(dy, cc[j], gv[j]);  // adjoint of h_t
        const float gq = gv[j] * (av[j] * hp[j]);
        if constexpr (ZOH) {
          const float x = dl * Av[j];
          const float phi = zoh_coef(dl, x, au[j], invA[j]);
          const float gb = gv[j] * bb[j];
          s1 = __builtin_fmaf(gb, phi, s1);    // for du
          s3 = __builtin_fmaf(gb, au[j], s3);  // for d delta
          dA[j] = __builtin_fmaf(gq, dl, dA[j]);
          dA[j] = __builtin_fmaf(gb * dv, (dl * dl) * zoh_psi(x, au[j]), dA[j]);
          p3[j] = (gv[j] * dv) * phi;
        } else {
          s1 = __builtin_fmaf(gv[j], bb[j], s1);
          dA[j] = __builtin_fmaf(gq, dl, dA[j]);
          p3[j] = gv[j] * dv;
        }
        s2 = __builtin_fmaf(gq, Av[j], s2);
        yy = __builtin_fmaf(cc[j], ht[j], yy);
        p4[j] = dy * ht[j];
        gv[j] = av[j] * gv[j];  // carried to step t-1
      }
      s1 = chan_sum<LPC>(s1);
      s2 = chan_sum<LPC>(s2);
      yy = chan_sum<LPC>(yy);
      if constexpr (ZOH) s3 = chan_sum<LPC>(s3);
      const bool mine = (l & 3) == (t & 3);
      F1 = mine ? s1 : F1;
      F2 = mine ? s2 : F2;
      FY = mine ? yy : FY;
      if constexpr (ZOH) F3 = mine ? s3 : F3;

      // dB / dC terms of this step into the wave buffer (slot t & 1).
      *reinterpret_cast<float4*>(wbuf + cw * QS + (t & 1) * NPADC + n0) = make_float4(p3[0], p3[1], p3[2], p3[3]);
      *reinterpret_cast<float4*>(wbuf + TS + cw * QS + (t & 1) * NPADC + n0) =
          make_float4(p4[0], p4[1], p4[2], p4[3]);
      if ((t & 1) == 0) {
        // Steps t and t+1 are in the buffer: add up the wave's channels into
        // the wave's totals.
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int it = 0; it < 4 * NPADC / 64; ++it) {
          const int item = lane + 64 * it;
          const int type = item / (2 * NPADC);
          const int par = (item / NPADC) & 1;
          const int n = item % NPADC;
          const float* src = wbuf + type * TS + par * NPADC + n;
          float sum = src[0];
#pragma unroll
          for (int q = 1; q < CPWAVE; ++q) sum += src[q * QS];
          wacc[type * AT + ((t + par) % FP) * NPADC + n] = sum;
        }
        __builtin_amdgcn_wave_barrier();
        if (t % FP == 0 && t > 0) {
          __syncthreads();  // every wave's totals of steps [t, t + FP) are in LDS
          flush(tc, t);
          __syncthreads();  // read before the next period overwrites them
        }
      }

      if ((t & 3) == 0 && fin) {
        // Steps t .. t+3 are complete: lane l finalizes step t + l.
        const int G = t / 4;
        const int tf = t + l;
        const int64_t tg = tc + tf;
        const float4 rf = s_rec[c * RS + tf];
        if (dvalid && tg < pend) {
          const float dlf = fabsf(rf.x), dyf = rf.z;
          const float du = __builtin_fmaf(dyf, dsk, ZOH ? F1 : dlf * F1);
          const float dx = __builtin_fmaf(o.u[G], ZOH ? F3 : F1, F2) * o.sig[G];
          const float dz = o.gz[G] * __builtin_fmaf(dsk, o.u[G], FY);
          if constexpr (STAGE_OUT) {
            const int tl = (J & 1) * kK + tf;  // step within the chunk pair
            s_out[c * OS + tl] = du;
            s_out[(CPW + c) * OS + tl] = dx;
            s_out[(2 * CPW + c) * OS + tl] = dz;
          } else {
            if (a.du_conv)
              a.du_conv[rowbase + tg] = du;  // the conv backward takes it from here
            else
              store_grad(a, a.du, rowbase + tg, du);
            store_grad(a, a.ddt, rowbase + tg, dx);
            if (a.dz) store_grad(a, a.dz, rowbase + tg, dz);
          }
          dD_acc = __builtin_fmaf(dyf, o.u[G], dD_acc);
          dbias_acc += dx;
        }
      }
    };

    // Steps in pairs (t odd, t - 1 even), last pair first.
#pragma unroll
    for (int t = kK - 1; t >= 1; t -= 2) {
      const float4 r1 = s_rec[c * RS + t], r0 = s_rec[c * RS + t - 1];
      const float4 b1v = *reinterpret_cast<const float4*>(s_B + t * NPADC + n0);
      const float4 b0v = *reinterpret_cast<const float4*>(s_B + (t - 1) * NPADC + n0);
      const float4 c1v = *reinterpret_cast<const float4*>(s_C + t * NPADC + n0);
      const float4 c0v = *reinterpret_cast<const float4*>(s_C + (t - 1) * NPADC + n0);
      const float b1[4] = {b1v.x, b1v.y, b1v.z, b1v.w}, b0[4] = {b0v.x, b0v.y, b0v.z, b0v.w};
      const float c1[4] = {c1v.x, c1v.y, c1v.z, c1v.w}, c0[4] = {c0v.x, c0v.y, c0v.z, c0v.w};
      const bool rs1 = HAS_RESET && __float_as_int(r1.x) < 0;
      const bool rs0 = HAS_RESET && __float_as_int(r0.x) < 0;
      float a1[kNPL], a0[kNPL], u1[kNPL], u0[kNPL], hodd[kNPL], hev[kNPL], hpp[kNPL];
#pragma unroll
      for (int j = 0; j < kNPL; ++j) {
        u1[j] = fast_exp2(fabsf(r1.x) * A2[j]);
        u0[j] = fast_exp2(fabsf(r0.x) * A2[j]);
        a1[j] = u1[j];
        a0[j] = u0[j];
      }
      // a_t = 0 at a reset (every lane of a workgroup sees its batch row's resets at the same step)
      if (HAS_RESET && __builtin_amdgcn_ballot_w64(rs1 || rs0)) {
        keep_branch();
#pragma unroll
        for (int j = 0; j < kNPL; ++j) {
          a1[j] = rs1 ? 0.0f : a1[j];
          a0[j] = rs0 ? 0.0f : a0[j];
        }
      }
#pragma unroll
      for (int j = 0; j < kNPL; ++j) {
        hpp[j] = t >= 3 ? hist[(t - 2) >> 1][j] : hs[j];  // h_{t-2}
        // h_{t-1}, as the forward computed it
        if constexpr (ZOH)
          hev[j] = __builtin_fmaf(a0[j], hpp[j],
                                  (b0[j] * r0.y) * zoh_coef(fabsf(r0.x), fabsf(r0.x) * Av[j], u0[j], invA[j]));
        else
          hev[j] = __builtin_fmaf(a0[j], hpp[j], b0[j] * r0.y);
        hodd[j] = hist[t >> 1][j];  // h_t
      }
      rstep(t, r1, b1, c1, a1, u1, hev, hodd);
      rstep(t - 1, r0, b0, c0, a0, u0, hpp, hev);
      // Keep the scheduler from hoisting later pairs' reads and exponentials
      // above this one: that costs registers the wave needs for occupancy.
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();  // totals of the chunk's first period complete; LDS parameters free
    flush(tc, 0);
    if constexpr (STAGE_OUT) {
      if ((J & 1) == 0) flush_out(J);
    }
  };

  Raw r;
  Out o;
  float hs[kNPL];
  load(nchunks - 1, r);
  load_ckpt(nchunks - 1, hs);
  const ProgressPriority prio(nchunks, false);
  for (int J = nchunks - 1; J >= 0; --J) {
    prio.update(nchunks - 1 - J);
    store(J, r, o);
    float hs_next[kNPL];
    if (J > 0) {
      load(J - 1, r);
      load_ckpt(J - 1, hs_next);
    }
    chunk(J, o, hs);
#pragma unroll
    for (int j = 0; j < kNPL; ++j) hs[j] = hs_next[j];
  }

  // Per-(b, segment) partials of dA, dD and d dt_bias; dh0 from the first segment.
#pragma unroll
  for (int j = 0; j < kNPL; ++j) {
    const int n = n0 + j;
    if (!dvalid || n >= N) continue;
    a.partA[((static_cast<int64_t>(b) * a.nsegb + s) * a.D + d) * N + n] = dA[j];
    if (s == 0 && a.dh0) a.dh0[bdn + n] = gv[j];
  }
  dD_acc = chan_sum<4>(dD_acc);
  dbias_acc = chan_sum<4>(dbias_acc);
  if (l == 0 && dvalid) {
    const int64_t pi = (static_cast<int64_t>(b) * a.nsegb + s) * a.D + d;
    a.partD[pi] = dD_acc;
    a.partBias[pi] = dbias_acc;
  }
}

struct RedArgs {
  int64_t bln, dn, D, groups, bs;  // groups: channel groups; bs: batch rows x segments
  const float* partB;
  const float* partC;
  const float* partA;
  const float* partD;
  const float* partBias;
  float* dB;
  float* dC;
  float* dA;
  float* dD;
  float* dbias;
  int batch8;  // issue the loads of eight partial sets at a time
};

// Shared gradients: sums of the partials in a fixed order. One thread owns
// four consecutive outputs (float4 loads and stores where the range allows).
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const RedArgs r) {
  const int64_t n4_bc = (r.bln + 3) / 4, n4_a = (r.dn + 3) / 4, n4_d = (r.D + 3) / 4;
  const int64_t total = 2 * n4_bc + n4_a + 2 * n4_d;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const float* src;
    float* dst;
    int64_t e, len, stride, count;
    if (i < 2 * n4_bc) {
      const bool isC = i >= n4_bc;
      e = (isC ? i - n4_bc : i) * 4;
      src = isC ? r.partC : r.partB;
      dst = isC ? r.dC : r.dB;
      len = r.bln;
      stride = r.bln;
      count = r.groups;
    } else if (i < 2 * n4_bc + n4_a) {
      e = (i - 2 * n4_bc) * 4;
      src = r.partA;
      dst = r.dA;
      len = r.dn;
      stride = r.dn;
      count = r.bs;
    } else {
      const int64_t k = i - 2 * n4_bc - n4_a;
      const bool isBias = k >= n4_d;
      e = (isBias ? k - n4_d : k) * 4;
      src = isBias ? r.partBias : r.partD;
      dst = isBias ? r.dbias : r.dD;
      len = r.D;
      stride = r.D;
      count = r.bs;
      if (!dst) continue;
    }
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // 16-byte accesses only where every row of src and dst is 16-byte aligned
    const bool vec = e + 4 <= len && (stride % 4) == 0 && (reinterpret_cast<uintptr_t>(src) % 16) == 0 &&
                     (reinterpret_cast<uintptr_t>(dst) % 16) == 0;
    if (vec) {
      // batch8: the loads of eight partial sets at a time, added in the same
      // order as one at a time.
      const float* p = src + e;
      int64_t q = 0;
      if (r.batch8)
        for (; q + 8 <= count; q += 8) {
          float4 v[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) v[k] = *reinterpret_cast<const float4*>(p + (q + k) * stride);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            acc[0] += v[k].x;
            acc[1] += v[k].y;
            acc[2] += v[k].z;
            acc[3] += v[k].w;
          }
        }
      for (; q < count; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(p + q * stride);
        acc[0] += v.x;
        acc[1] += v.y;
        acc[2] += v.z;
        acc[3] += v.w;
      }
      *reinterpret_cast<float4*>(dst + e) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    } else {
      for (int64_t q = 0; q < count; ++q) {
        const float* p = src + q * stride + e;
        for (int k = 0; k < 4 && e + k < len; ++k) acc[k] += p[k];
      }
      for (int k = 0; k < 4 && e + k < len; ++k) dst[e + k] = acc[k];
    }
  }
}

// ---- backward of the causal conv1d + SiLU input stage ----
//
// Given du' (the gradient of the scan input u' = silu(pre)), with
//   pre_t = conv_b + sum_{k<4} w[k] x_{t-3+k}   (taps right-aligned: widths
//           below 4 have leading zero taps; inputs hidden by a later reset
//           within the window count as 0),
// the chain rule gives dpre_t = du'_t silu'(pre_t) and
//   dx_s      = sum_k w[k] dpre_{s+3-k}       (over taps that see x_s)
//   dw[k]    += dpre_t x_{t-3+k};  dconv_b += dpre_t;  the terms of s < 0 go to
//   the initial conv state.
// One workgroup covers kConvTile steps of one (b, d) row; each thread owns four
// consecutive steps and recomputes pre for them and the three that follow.
constexpr int kConvTile = 1024;

struct ConvBwdArgs {
  int64_t B, D, L;
  int K, ntiles, grad_bf16;
  const void* x;
  const uint8_t* reset;
  const float* w;
  const float* bias;
  const float* state_in;
  const float* du_conv;
  void* dx;
  float* dstate;
  float* part;  // (B, D, ntiles, 5): four taps and the bias
};

template <typename InT>
__global__ __launch_bounds__(256) void conv_bwd_kernel(const ConvBwdArgs a) {
  const int64_t row = blockIdx.x / a.ntiles;  // b * D + d
  const int tile = blockIdx.x % a.ntiles;
  const int64_t d = row % a.D, b = row / a.D;
  const int K = a.K;
  float wp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k = 0; k < K; ++k) wp[4 - K + k] = a.w[d * K + k];
  const float cb = a.bias ? a.bias[d] : 0.0f;
  const InT* xr = static_cast<const InT*>(a.x) + row * a.L;
  const float* dur = a.du_conv + row * a.L;
  const uint8_t* rs = a.reset ? a.reset + b * a.L : nullptr;
  const int64_t t0 = static_cast<int64_t>(tile) * kConvTile + 4 * threadIdx.x;

  // x_{t0-3} .. x_{t0+6} and the reset flags of t0-3 .. t0+6
  float xv[10];
  bool rv[10];
#pragma unroll
  for (int j = 0; j < 10; ++j) {
    const int64_t pos = t0 - 3 + j;
    float v = 0.0f;
    if (pos >= 0 && pos < a.L)
      v = load_elem(xr, pos);
    else if (pos < 0 && a.state_in && pos >= 1 - K)
      v = a.state_in[row * (K - 1) + (pos + K - 1)];
    xv[j] = v;
    rv[j] = rs && pos >= 0 && pos < a.L && rs[pos];
  }
  // tap k of step t0 + i reads x_{t0+i-3+k} = xv[i + k]; it is visible unless a
  // reset lies in (that input, t0 + i], i.e. at xv indices i+k+1 .. i+3.
  auto vis = [&](int i, int k) {
    bool v = true;
#pragma unroll
    for (int q = 1; q <= 3; ++q)
      if (q > k) v = v && !rv[i + q];  // reset flags of t0+i-3+q for q in k+1 .. 3
    return v;
  };
  float dpre[7];
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    const int64_t t = t0 + i;
    float p = cb;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (vis(i, k)) p = __builtin_fmaf(wp[k], xv[i + k], p);
    const float sg = fast_rcp(1.0f + fast_exp2(-p * kLog2e));
    const float g = t < a.L ? dur[t] : 0.0f;
    dpre[i] = g * (sg * __builtin_fmaf(p, 1.0f - sg, 1.0f));
  }
  float dw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, db = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t s = t0 + i;  // the step this thread owns: dx_s and the sums of dpre_s
    if (s >= a.L) break;
    float acc = 0.0f;
    // dpre_{s+3-k} reaches x_s through tap k when x_s is visible from s+3-k
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (vis(i + 3 - k, k)) acc = __builtin_fmaf(wp[k], dpre[i + 3 - k], acc);
    if (a.grad_bf16)
      store_elem(static_cast<bf16_t*>(a.dx) + row * a.L, s, acc);
    else
      store_elem(static_cast<float*>(a.dx) + row * a.L, s, acc);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (vis(i, k)) dw[k] = __builtin_fmaf(dpre[i], xv[i + k], dw[k]);
    db += dpre[i];
  }
  // the initial conv state: inputs x_{-3..-1} feed steps 0..2
  if (t0 == 0 && a.dstate) {
    for (int j = 0; j < K - 1; ++j) {
      const int pos = j - (K - 1);  // -K+1 .. -1
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < 3; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (i - 3 + k == pos && vis(i, k) && i < a.L) acc = __builtin_fmaf(wp[k], dpre[i], acc);
      a.dstate[row * (K - 1) + j] = acc;
    }
  }
  // workgroup sums of the tap and bias gradients, in a fixed order
  __shared__ float red[5][256];
#pragma unroll
  for (int k = 0; k < 4; ++k) red[k][threadIdx.x] = dw[k];
  red[4][threadIdx.x] = db;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off)
#pragma unroll
      for (int j = 0; j < 5; ++j) red[j][threadIdx.x] += red[j][threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x < 5) a.part[(row * a.ntiles + tile) * 5 + threadIdx.x] = red[threadIdx.x][0];
}

// dconv_w[d, k] and dconv_b[d]: the tiles' sums over batch rows and tiles, in order.
__global__ __launch_bounds__(256) void conv_param_reduce_kernel(int64_t B, int64_t D, int K, int ntiles,
                                                                const float* part, float* dw, float* db) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= D * 5) return;
  const int64_t d = i / 5;
  const int j = static_cast<int>(i % 5);
  float acc = 0.0f;
  for (int64_t b = 0; b < B; ++b)
    for (int t = 0; t < ntiles; ++t) acc += part[((b * D + d) * ntiles + t) * 5 + j];
  if (j < 4) {
    if (dw && j >= 4 - K) dw[d * K + (j - (4 - K))] = acc;
  } else if (db) {
    db[d] = acc;
  }
}

int bwd_lpc(int64_t N) {
  if (N <= 16) return 4;
  if (N <= 32) return 8;
  if (N <= 64) return 16;
  if (N <= 128) return 32;
  return 64;
}

template <typename Fn>
hipError_t with_bwd_tile(int64_t N, Fn&& fn) {
  switch (bwd_lpc(N)) {
    case 4: return fn(BwdTile<4>{});
    case 8: return fn(BwdTile<8>{});
    case 16: return fn(BwdTile<16>{});
    case 32: return fn(BwdTile<32>{});
    default: return fn(BwdTile<64>{});
  }
}

}  // namespace

int bwd_channels_per_block(int64_t N) { return kWaves * 64 / bwd_lpc(N); }

// Reverse-sweep workgroups resident on the whole chip: 256 CUs x workgroups
// per CU. The kernels need 200-250 VGPRs (two waves per SIMD, two 4-wave
// workgroups per CU); the N > 128 layout's 84 KB of LDS allows one, and so
// does the zero-order-hold variant's register budget.
int64_t bwd_resident_blocks(int64_t N, bool zoh) { return 256 * (bwd_lpc(N) >= 64 || zoh ? 1 : 2); }

void plan_bwd_segments(int64_t B, int64_t D, int64_t L, int64_t N, bool zoh, int* nsegb, int64_t* seg_steps) {
  // Segments of whole 16-step chunks. Workgroups run in rounds of the
  // resident count, each as long as its segment, so pick the count that
  // minimises rounds x chunks per segment (the fewest segments on a tie).
  const int64_t groups = B * ((D + bwd_channels_per_block(N) - 1) / bwd_channels_per_block(N));
  const int64_t chunks = (L + kK - 1) / kK;
  const int64_t resident = bwd_resident_blocks(N, zoh);
  int64_t best = 1, best_cost = -1;
  const int64_t max_seg = std::min<int64_t>(chunks, 4096);
  for (int64_t ns = 1; ns <= max_seg; ++ns) {
    // an even number of chunks per segment keeps the reverse sweep's chunk
    // pairs (its 32-step output rows) aligned to 32 steps of the sequence
    int64_t per = (chunks + ns - 1) / ns;
    per = std::min(per + (per & 1), chunks);
    const int64_t used = (chunks + per - 1) / per;  // segments actually needed at this length
    const int64_t cost = (groups * used + resident - 1) / resident * per;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = per;
    }
  }
  *seg_steps = best * kK;
  *nsegb = static_cast<int>((chunks + best - 1) / best);
}

size_t bwd_partial_floats(int64_t B, int64_t D, int64_t L, int64_t N, int nsegb) {
  const int64_t groups = (D + bwd_channels_per_block(N) - 1) / bwd_channels_per_block(N);
  return static_cast<size_t>(2 * groups * B * L * N + B * nsegb * D * N + 2 * B * nsegb * D);
}

size_t bwd_conv_partial_floats(int64_t B, int64_t D, int64_t L) {
  return static_cast<size_t>(B * D * ((L + kConvTile - 1) / kConvTile) * 5);
}

int64_t bwd_grid_blocks(int64_t B, int64_t D, int64_t N, int nsegb) {
  return B * ((D + bwd_channels_per_block(N) - 1) / bwd_channels_per_block(N)) * nsegb;
}

hipError_t launch_bwd_reduce(const float* partB, const float* partC, const float* partA, const float* partD,
                             const float* partBias, float* dB, float* dC, float* dA, float* dD, float* dbias,
                             int64_t bln, int64_t dn, int64_t D, int64_t groups, int64_t bs, hipStream_t stream) {
  RedArgs r{};
  r.bln = bln;
  r.dn = dn;
  r.D = D;
  r.groups = groups;
  r.bs = bs;
  r.partB = partB;
  r.partC = partC;
  r.partA = partA;
  r.partD = partD;
  r.partBias = partBias;
  r.dB = dB;
  r.dC = dC;
  r.dA = dA;
  r.dD = dD;
  r.dbias = dbias;
  const int64_t total = 2 * ((r.bln + 3) / 4) + (r.dn + 3) / 4 + 2 * ((r.D + 3) / 4);
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 8192);
  // With fewer threads than the GPU holds at once (256 CUs x 2048), one load
  // in flight per thread leaves the kernel latency-bound: at 8 x 1536 x 2048,
  // N = 16 (24 partial sets, 53 MB) it took 35 us; the loads then go out
  // eight sets at a time. A full grid keeps enough loads in flight already,
  // and batching measured 1.6% slower on the whole backward there (2 x 2048
  // x 4096, N = 128: 256 sets, 2.1 GB).
  r.batch8 = total < int64_t{256} * 2048;
  SSM_LOG("launch bwd_reduce_kernel: %lld partial sets of dB/dC over %lld (b, l, n), %lld of dA/dD/dbias; "
          "grid %lld x 256 threads, loads %s",
          static_cast<long long>(groups), static_cast<long long>(bln), static_cast<long long>(bs),
          static_cast<long long>(blocks), r.batch8 ? "eight sets at a time" : "one set at a time");
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, r);
  return hipGetLastError();
}

hipError_t launch_scan_bwd(const BwdPlan& pl, hipStream_t stream) {
  const int cpw = bwd_channels_per_block(pl.N);
  const int64_t groups = (pl.D + cpw - 1) / cpw;
  BwdArgs a{};
  a.B = pl.B;
  a.D = pl.D;
  a.L = pl.L;
  a.N = pl.N;
  a.seg_steps = pl.seg_steps;
  a.n_ck = pl.n_ck;
  a.nsegb = pl.nsegb;
  a.n_dgroups = static_cast<int>(groups);
  a.nblocks = static_cast<int>(pl.B * groups * pl.nsegb);
  a.grad_bf16 = pl.grad_bf16;
  a.u = pl.u;
  a.dt = pl.dt;
  a.z = pl.z;
  a.Bm = pl.Bm;
  a.Cm = pl.Cm;
  a.dout = pl.dout;
  a.dt_bias = pl.dt_bias;
  a.A = pl.A;
  a.Dskip = pl.Dskip;
  a.reset = pl.reset;
  a.dh_last = pl.dh_last;
  a.ckpt = pl.ckpt;
  a.seg_P = pl.seg_P;
  a.seg_G = pl.seg_G;
  a.du = pl.du;
  a.ddt = pl.ddt;
  a.dz = pl.dz;
  a.dh0 = pl.dh0;
  a.uconv = pl.conv_w ? pl.uconv : nullptr;
  a.du_conv = pl.conv_w ? pl.du_conv : nullptr;
  const int64_t bln = pl.B * pl.L * pl.N;
  a.partB = pl.part;
  a.partC = pl.part + groups * bln;
  a.partA = pl.part + 2 * groups * bln;
  a.partD = a.partA + pl.B * pl.nsegb * pl.D * pl.N;
  a.partBias = a.partD + pl.B * pl.nsegb * pl.D;
  const bool reset = pl.reset != nullptr;
  hipError_t e = with_bwd_tile(pl.N, [&](auto tile) {
    using TL = decltype(tile);
    const dim3 grid(static_cast<unsigned>(a.nblocks)), block(kThreads);
    SSM_LOG("launch scan_bwd_kernel<BwdTile<%d>>: %s in, reset %d, zoh %d; grid %d x %d threads (%d channels x "
            "%d states per workgroup), %d reverse segments of %lld steps",
            TL::LPC, pl.in_bf16 ? "bf16" : "f32", reset, pl.zoh, a.nblocks, kThreads, TL::CPW, TL::NPADC,
            pl.nsegb, static_cast<long long>(pl.seg_steps));
    if (pl.zoh) {
      if (pl.in_bf16) {
        if (reset)
          hipLaunchKernelGGL((scan_bwd_kernel<TL, bf16_t, true, true>), grid, block, 0, stream, a);
        else
          hipLaunchKernelGGL((scan_bwd_kernel<TL, bf16_t, false, true>), grid, block, 0, stream, a);
      } else {
        if (reset)
          hipLaunchKernelGGL((scan_bwd_kernel<TL, float, true, true>), grid, block, 0, stream, a);
        else
          hipLaunchKernelGGL((scan_bwd_kernel<TL, float, false, true>), grid, block, 0, stream, a);
      }
    } else if (pl.in_bf16) {
      if (reset)
        hipLaunchKernelGGL((scan_bwd_kernel<TL, bf16_t, true, false>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((scan_bwd_kernel<TL, bf16_t, false, false>), grid, block, 0, stream, a);
    } else {
      if (reset)
        hipLaunchKernelGGL((scan_bwd_kernel<TL, float, true, false>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((scan_bwd_kernel<TL, float, false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;

  e = launch_bwd_reduce(a.partB, a.partC, a.partA, a.partD, a.partBias, pl.dB, pl.dC, pl.dA, pl.dD, pl.dbias, bln,
                        pl.D * pl.N, pl.D, groups, pl.B * pl.nsegb, stream);
  if (e != hipSuccess || !pl.conv_w) return e;
  return launch_conv_bwd(pl, stream);
}

hipError_t launch_conv_bwd(const BwdPlan& pl, hipStream_t stream) {
  ConvBwdArgs c{};
  c.B = pl.B;
  c.D = pl.D;
  c.L = pl.L;
  c.K = pl.conv_k;
  c.ntiles = static_cast<int>((pl.L + kConvTile - 1) / kConvTile);
  c.grad_bf16 = pl.grad_bf16;
  c.x = pl.u;
  c.reset = pl.reset;
  c.w = pl.conv_w;
  c.bias = pl.conv_b;
  c.state_in = pl.conv_state_in;
  c.du_conv = pl.du_conv;
  c.dx = pl.du;
  c.dstate = pl.dconv_state;
  c.part = pl.conv_part;
  const dim3 cgrid(static_cast<unsigned>(pl.B * pl.D * c.ntiles));
  SSM_LOG("launch conv_bwd_kernel: width %d, %d tiles of %d steps; grid %u x 256 threads", c.K, c.ntiles, kConvTile,
          cgrid.x);
  if (pl.in_bf16)
    hipLaunchKernelGGL(conv_bwd_kernel<bf16_t>, cgrid, dim3(256), 0, stream, c);
  else
    hipLaunchKernelGGL(conv_bwd_kernel<float>, cgrid, dim3(256), 0, stream, c);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SSM_LOG("launch conv_param_reduce_kernel: grid %lld x 256 threads", static_cast<long long>((pl.D * 5 + 255) / 256));
  hipLaunchKernelGGL(conv_param_reduce_kernel, dim3(static_cast<unsigned>((pl.D * 5 + 255) / 256)), dim3(256), 0,
                     stream, pl.B, pl.D, pl.conv_k, c.ntiles, static_cast<const float*>(pl.conv_part), pl.dconv_w,
                     pl.dconv_b);
  return hipGetLastError();
}

}  // namespace ssm
