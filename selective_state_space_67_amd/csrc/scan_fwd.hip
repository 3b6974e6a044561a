// Selective-scan forward kernels for gfx950 (MI355X).
//
// What is computed (the recurrence of the selective SSM with a diagonal state
// matrix; "Illustrated Mamba state space model", sections "Mathematical basis:
// structured SSM" and step 1; "Mamba SSM core theory and Keras/TensorFlow
// implementation", SelectiveSSM layer and its scan step):
//
//   delta = softplus(dt_raw + dt_bias)
//   h[n]  = exp(delta A[d,n]) h[n] + delta B[t,n] u        (h := 0 first on a reset)
//   out   = (sum_n C[t,n] h[n] + D[d] u) * silu(z)
//
// The pages describe one fused kernel that keeps the recurrence on chip and
// writes back only the result ("Technical analysis: Mamba selective state
// spaces", sections 1 and 2.2). This is that kernel for CDNA4, designed around
// what binds on gfx950: the recurrence needs one exponential and four other
// float32 operations per (b, d, t, n), while it moves well under one byte of
// HBM traffic per element, so the vector ALU -- not HBM -- is the limit.
//
// Mapping. A workgroup owns 16 channels of one batch row (4 waves, 4 channels
// per wave). Within a wave each channel occupies one DPP row of 16 lanes and
// lane k of that row holds states n = k*NPL .. k*NPL+NPL-1 in registers. Every
// lane runs the recurrence sequentially in time for its own states, so no
// per-element work is spent on a parallel scan; the (b, d, n) recurrences
// already give each launch thousands of waves.
//
// Skewed pipeline. Lane k processes step t at iteration m = t + k. The partial
// output sum_n C h of lane k is added to the running sum that lane k-1
// produced for the same step one iteration earlier (one DPP row_shr:1 add), so
// after lane 15 the row holds the full dot product over n. This costs one add
// per lane-step instead of a log2(16)-level reduction.
//
// Staging. Per chunk of T steps the workgroup
//  - loads dt_raw, u, z along L (consecutive threads read consecutive steps)
//    and computes delta, delta*u, D*u and silu(z) once per (channel, step);
//  - loads B_t, C_t once and shares them through LDS with all 16 channels.
// Rings of two chunks in LDS let lanes that lag by up to 15 steps still read
// the previous chunk. The layouts make every per-lane LDS read a 16-byte,
// 16-byte-aligned load:
//  - (delta, delta*u) pairs are kept in two copies shifted by one step; lane k
//    reads the copy that aligns its window (k odd or even);
//  - (B, C) of state n is stored in row n at column t + n/NPL, which cancels
//    the lane's skew, so lane k's window starts at a multiple of 16.
// Lane 15 of each row writes the finished sums into an LDS ring; after the
// next chunk the workgroup applies D*u and the gate and stores `out` along L.
//
// Long sequences with few channels (L split into pieces): a first launch
// computes each piece's affine aggregate (product of the decays and the end
// state from a zero start); the second launch folds the aggregates of the
// preceding pieces into the starting state of each piece and runs the full
// recurrence. The two-level composition is the associative combine of affine
// maps (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2).
//
// Resets: the step's delta is stored with its sign bit set; the lane clears
// its states before that step (a wave-uniform branch, taken only when some
// lane of the wave meets a reset).
#include <algorithm>

#include "device_math.h"
#include "kernels.h"

namespace ssm {
namespace {

constexpr int kThreads = 256;
constexpr int kChannels = kScanChannelsPerBlock;  // 16 = 4 waves x 4 rows

enum Mode { kFull = 0, kAggregate = 1 };

template <int NPL>
struct Tile {
  static constexpr int NPAD = 16 * NPL;          // states covered by one row
  static constexpr int T = NPL <= 2 ? 32 : 16;   // steps per chunk
  static constexpr int RING = 2 * T;             // steps kept in LDS
  static_assert((RING & (RING - 1)) == 0, "ring length must be a power of two");
  static_assert(T % 16 == 0 && T >= 16, "chunk must hold whole 16-step blocks");
};

struct ScanArgs {
  int64_t B, D, L, N;
  int64_t seg_len;
  int nseg;
  int n_dgroups;
  int nblocks;
  int in_bf16;
  int out_bf16;
  const void* u;
  const void* dt;
  const void* z;
  const void* Bm;
  const void* Cm;
  const float* dt_bias;
  const float* A;
  const float* Dskip;
  const float* h0;
  const uint8_t* reset;
  void* out;
  float* h_last;
  float* ws_P;  // decay products of pieces 0..nseg-2, (nseg-1, B, D, N)
  float* ws_H;  // end states of pieces 0..nseg-2 from a zero start
};

template <int NPL, typename InT, bool HAS_RESET, int MODE>
__global__ __launch_bounds__(kThreads) void scan_kernel(const ScanArgs a) {
  using TL = Tile<NPL>;
  constexpr int T = TL::T, RING = TL::RING, NPAD = TL::NPAD;
  constexpr int MASK = RING - 1;
  // (delta, delta*u) rows carry a 16-entry mirror of their first 16 slots so a
  // lane's 16-step window never wraps; (B, C) windows start at multiples of 16
  // and cannot wrap.
  constexpr int DU_STRIDE = RING + 16 + 2;
  constexpr int BC_STRIDE = RING + 2;
  constexpr bool FULL = MODE == kFull;
  constexpr int BC_ITEMS = T * NPAD / kThreads;       // (step, state) items per thread per chunk
  constexpr int ROW_ITEMS = kChannels * T / kThreads; // (channel, step) items per thread per chunk
  static_assert(BC_ITEMS >= 1 && (T * NPAD) % kThreads == 0, "B/C staging split");
  static_assert(ROW_ITEMS >= 1 && (kChannels * T) % kThreads == 0, "row staging split");

  __shared__ __align__(16) float2 s_du[2][kChannels][DU_STRIDE];   // (delta, delta*u), two shifted copies
  __shared__ __align__(16) float2 s_bc[NPAD][BC_STRIDE];           // (B, C) per state, diagonal layout
  __shared__ __align__(16) float s_y[FULL ? kChannels : 1][RING];  // finished sum_n C h per step
  __shared__ __align__(16) float2 s_g[FULL ? kChannels : 1][RING]; // (D*u, silu(z)) per step

  // Workgroup -> (piece, batch row, channel group). Consecutive logical tiles
  // share a batch row and therefore B and C; hardware dispatches consecutive
  // workgroup ids to different XCDs, so tiles are renumbered to keep a batch
  // row's tiles on one XCD and its B/C in that XCD's L2.
  int idx = blockIdx.x;
  if ((a.nblocks & 7) == 0) idx = (idx & 7) * (a.nblocks >> 3) + (idx >> 3);
  const int g = idx % a.n_dgroups;
  const int rest = idx / a.n_dgroups;
  const int b = rest % static_cast<int>(a.B);
  const int s = rest / static_cast<int>(a.B);
  const int64_t t_seg = static_cast<int64_t>(s) * a.seg_len;
  const int Lseg = static_cast<int>(min(a.seg_len, a.L - t_seg));
  const InT* __restrict__ u_in = static_cast<const InT*>(a.u);
  const InT* __restrict__ dt_in = static_cast<const InT*>(a.dt);
  const InT* __restrict__ z_in = static_cast<const InT*>(a.z);
  const InT* __restrict__ B_in = static_cast<const InT*>(a.Bm);
  const InT* __restrict__ C_in = static_cast<const InT*>(a.Cm);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int k = lane & 15;                        // lane within the channel's row
  const int c = (tid >> 6) * 4 + (lane >> 4);     // channel within the workgroup
  const int64_t d = static_cast<int64_t>(g) * kChannels + c;
  const bool dvalid = d < a.D;

  // Per-lane parameters and state.
  float A2[NPL], h[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = k * NPL + j;
    const bool ok = dvalid && n < a.N;
    A2[j] = ok ? a.A[d * a.N + n] * kLog2e : 0.0f;
    h[j] = 0.0f;
    if (FULL && ok) {
      const int64_t hi = (static_cast<int64_t>(b) * a.D + d) * a.N + n;
      float hv = a.h0 ? a.h0[hi] : 0.0f;
      // Fold the aggregates of the preceding pieces: h <- P h + H.
      for (int sp = 0; sp < s; ++sp) {
        const int64_t wi = (static_cast<int64_t>(sp) * a.B + b) * a.D * a.N + d * a.N + n;
        hv = __builtin_fmaf(a.ws_P[wi], hv, a.ws_H[wi]);
      }
      h[j] = hv;
    }
  }

  // Empty rings: steps before the start (read by lagging lanes) are identity
  // steps (delta = 0, delta*u = 0, B = C = 0).
  for (int i = tid; i < 2 * kChannels * DU_STRIDE; i += kThreads) (&s_du[0][0][0])[i] = make_float2(0.f, 0.f);
  for (int i = tid; i < NPAD * BC_STRIDE; i += kThreads) (&s_bc[0][0])[i] = make_float2(0.f, 0.f);

  const int nchunks = (Lseg + 18 + T - 1) / T;  // lane 15 finishes step L-1 by iteration L+17
  const int p = k & 1;

  float yreg[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) yreg[i] = 0.0f;
  float sum_delta = 0.0f;
  bool cleared = false;

  // Channel parameters of this thread's staging items (the channel of an item
  // does not change from chunk to chunk).
  float bias_r[ROW_ITEMS], dskip_r[ROW_ITEMS];
#pragma unroll
  for (int r = 0; r < ROW_ITEMS; ++r) {
    const int64_t dd = static_cast<int64_t>(g) * kChannels + (tid + r * kThreads) / T;
    const bool ok = dd < a.D;
    bias_r[r] = ok && a.dt_bias ? a.dt_bias[dd] : 0.0f;
    dskip_r[r] = ok && a.Dskip ? a.Dskip[dd] : 0.0f;
  }

  // ---- raw inputs of one chunk, loaded a chunk ahead of their use ----
  InT pb[BC_ITEMS], pc[BC_ITEMS], pu[ROW_ITEMS], pdt[ROW_ITEMS], pz[ROW_ITEMS];
  uint8_t prs[ROW_ITEMS];
  auto load_chunk = [&](int J) {
    const int tau0 = J * T;
#pragma unroll
    for (int r = 0; r < BC_ITEMS; ++r) {
      const int q = tid + r * kThreads;
      const int tau = tau0 + q / NPAD, n = q % NPAD;
      pb[r] = InT{};
      pc[r] = InT{};
      if (tau < Lseg && n < a.N) {
        const int64_t gi = (static_cast<int64_t>(b) * a.L + t_seg + tau) * a.N + n;
        pb[r] = B_in[gi];
        if (FULL) pc[r] = C_in[gi];
      }
    }
#pragma unroll
    for (int r = 0; r < ROW_ITEMS; ++r) {
      const int q = tid + r * kThreads;
      const int tau = tau0 + q % T;
      const int64_t dd = static_cast<int64_t>(g) * kChannels + q / T;
      pu[r] = InT{};
      pdt[r] = InT{};
      pz[r] = InT{};
      prs[r] = 0;
      if (tau < Lseg && dd < a.D) {
        const int64_t t = t_seg + tau;
        const int64_t gi = (static_cast<int64_t>(b) * a.D + dd) * a.L + t;
        pu[r] = u_in[gi];
        pdt[r] = dt_in[gi];
        if (FULL && z_in) pz[r] = z_in[gi];
        if (HAS_RESET) prs[r] = a.reset[static_cast<int64_t>(b) * a.L + t];
      }
    }
  };

  // ---- chunk J into the rings: per-step parameters computed once ----
  auto store_chunk = [&](int J) {
    const int tau0 = J * T;
#pragma unroll
    for (int r = 0; r < BC_ITEMS; ++r) {
      const int q = tid + r * kThreads;
      const int tau = tau0 + q / NPAD, n = q % NPAD;
      s_bc[n][(tau + n / NPL) & MASK] = make_float2(load_elem(&pb[r], 0), FULL ? load_elem(&pc[r], 0) : 0.0f);
    }
#pragma unroll
    for (int r = 0; r < ROW_ITEMS; ++r) {
      const int q = tid + r * kThreads;
      const int cc = q / T;
      const int tau = tau0 + q % T;
      const int64_t dd = static_cast<int64_t>(g) * kChannels + cc;
      float dl = 0.0f, dv = 0.0f, dskip = 0.0f, gate = 1.0f;
      if (tau < Lseg && dd < a.D) {
        const float uu = load_elem(&pu[r], 0);
        dl = softplus_f32(load_elem(&pdt[r], 0) + bias_r[r]);
        dv = dl * uu;
        if (FULL) {
          dskip = dskip_r[r] * uu;
          if (z_in) gate = silu_f32(load_elem(&pz[r], 0));
        }
        if (HAS_RESET && prs[r]) dl = -dl;  // sign bit: clear the state before this step
      }
      const float2 v = make_float2(dl, dv);
      const int s0 = tau & MASK, s1 = (tau + 1) & MASK;
      s_du[0][cc][s0] = v;
      if (s0 < 16) s_du[0][cc][s0 + RING] = v;
      s_du[1][cc][s1] = v;
      if (s1 < 16) s_du[1][cc][s1 + RING] = v;
      if (FULL) s_g[cc][s0] = make_float2(dskip, gate);
    }
  };

  // ---- the finished outputs of chunk J: out = (y + D u) silu(z) ----
  auto finalize = [&](int J) {
#pragma unroll
    for (int r = 0; r < ROW_ITEMS; ++r) {
      const int q = tid + r * kThreads;
      const int cc = q / T;
      const int tau = J * T + q % T;
      const int64_t dd = static_cast<int64_t>(g) * kChannels + cc;
      if (tau < Lseg && dd < a.D) {
        const float2 gg = s_g[cc][tau & MASK];
        const float o = (s_y[cc][tau & MASK] + gg.x) * gg.y;
        const int64_t gi = (static_cast<int64_t>(b) * a.D + dd) * a.L + t_seg + tau;
        if (a.out_bf16)
          store_elem(static_cast<bf16_t*>(a.out), gi, o);
        else
          store_elem(static_cast<float*>(a.out), gi, o);
      }
    }
  };

  // ---- one recurrence step of this lane (unrolled position i in a 16-step block) ----
  auto step = [&](const int i, const int m0, float dl, const float dv, const float (&Bv)[NPL],
                  const float (&Cv)[NPL]) {
    if (HAS_RESET) {
      const bool rs = __float_as_int(dl) < 0;
      if (__builtin_amdgcn_ballot_w64(rs)) {
#pragma unroll
        for (int j = 0; j < NPL; ++j) h[j] = rs ? 0.0f : h[j];
      }
      if (!FULL) cleared = cleared || rs;
      dl = fabsf(dl);
    }
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const float abar = fast_exp2(dl * A2[j]);
      h[j] = __builtin_fmaf(abar, h[j], Bv[j] * dv);
      if (FULL) part = j == 0 ? Cv[j] * h[j] : __builtin_fmaf(Cv[j], h[j], part);
    }
    if (FULL) {
      yreg[i] = row_shr1(yreg[(i + 15) & 15]) + part;
      if ((i & 3) == 2 && k == 15) {
        // steps m0+i-18 .. m0+i-15 are complete in this row: one aligned 16-byte store
        *reinterpret_cast<float4*>(&s_y[c][(m0 + i - 18) & MASK]) =
            make_float4(yreg[(i - 3) & 15], yreg[(i - 2) & 15], yreg[(i - 1) & 15], yreg[i]);
      }
    } else {
      sum_delta += dl;
    }
  };

  load_chunk(0);
  __syncthreads();  // rings are empty before the first chunk is stored
  for (int J = 0; J < nchunks; ++J) {
    store_chunk(J);
    if (J + 1 < nchunks) load_chunk(J + 1);  // in flight during this chunk's recurrence
    __syncthreads();
    for (int blk = 0; blk < T / 16; ++blk) {
      const int m0 = J * T + blk * 16;
      // This lane's 16-step window of (delta, delta*u) pairs, pair-aligned in copy p.
      const float2* du_win = &s_du[p][c][(m0 - k + p) & MASK];
      const float2* bc_win = &s_bc[k * NPL][m0 & MASK];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float4 dd = *reinterpret_cast<const float4*>(du_win + i);
        float B0[NPL], C0[NPL], B1[NPL], C1[NPL];
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          const float4 v = *reinterpret_cast<const float4*>(bc_win + j * BC_STRIDE + i);
          B0[j] = v.x;
          C0[j] = v.y;
          B1[j] = v.z;
          C1[j] = v.w;
        }
        step(i, m0, dd.x, dd.y, B0, C0);
        step(i + 1, m0, dd.z, dd.w, B1, C1);
      }
    }
    __syncthreads();
    if (FULL && J >= 1) finalize(J - 1);
  }
  if (FULL && (nchunks - 1) * T < Lseg) finalize(nchunks - 1);

  // ---- results that leave the workgroup ----
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = k * NPL + j;
    if (!dvalid || n >= a.N) continue;
    if (FULL) {
      if (a.h_last && s == a.nseg - 1) a.h_last[(static_cast<int64_t>(b) * a.D + d) * a.N + n] = h[j];
    } else {
      const int64_t wi = (static_cast<int64_t>(s) * a.B + b) * a.D * a.N + d * a.N + n;
      a.ws_H[wi] = h[j];
      a.ws_P[wi] = cleared ? 0.0f : fast_exp2(A2[j] * sum_delta);
    }
  }
}

template <int NPL, typename InT, bool HAS_RESET>
hipError_t launch_tile(const ScanArgs& args, int nblocks_full, int nblocks_agg, hipStream_t stream) {
  if (args.nseg > 1) {
    ScanArgs agg = args;
    agg.nblocks = nblocks_agg;
    hipLaunchKernelGGL((scan_kernel<NPL, InT, HAS_RESET, kAggregate>), dim3(nblocks_agg), dim3(kThreads), 0,
                       stream, agg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ScanArgs full = args;
  full.nblocks = nblocks_full;
  hipLaunchKernelGGL((scan_kernel<NPL, InT, HAS_RESET, kFull>), dim3(nblocks_full), dim3(kThreads), 0, stream,
                     full);
  return hipGetLastError();
}

template <typename InT, bool HAS_RESET>
hipError_t launch_npl(int npl, const ScanArgs& args, int nf, int na, hipStream_t stream) {
  switch (npl) {
    case 1: return launch_tile<1, InT, HAS_RESET>(args, nf, na, stream);
    case 2: return launch_tile<2, InT, HAS_RESET>(args, nf, na, stream);
    case 4: return launch_tile<4, InT, HAS_RESET>(args, nf, na, stream);
    case 8: return launch_tile<8, InT, HAS_RESET>(args, nf, na, stream);
    default: return launch_tile<16, InT, HAS_RESET>(args, nf, na, stream);
  }
}

template <typename InT>
hipError_t launch_dtype(int npl, bool reset, const ScanArgs& args, int nf, int na, hipStream_t stream) {
  return reset ? launch_npl<InT, true>(npl, args, nf, na, stream) : launch_npl<InT, false>(npl, args, nf, na, stream);
}

}  // namespace

void plan_segments(int64_t B, int64_t D, int64_t L, int64_t N, int requested, int* nseg,
                   int64_t* seg_len) {
  (void)N;
  int64_t want;
  if (requested > 0) {
    want = requested;
  } else {
    // About four workgroups per CU (256 CUs) keeps every SIMD busy; split the
    // sequence only when the channels alone give far fewer, and keep pieces
    // long enough (>= 512 steps) that the extra aggregate pass stays small.
    const int64_t blocks = B * ((D + kChannels - 1) / kChannels);
    want = blocks >= 512 ? 1 : (1024 + blocks - 1) / blocks;
    want = std::min<int64_t>(want, std::max<int64_t>(1, L / 512));
  }
  want = std::max<int64_t>(1, std::min<int64_t>(want, (L + 15) / 16));
  int64_t len = (L + want - 1) / want;
  len = (len + 15) / 16 * 16;
  *seg_len = len;
  *nseg = static_cast<int>((L + len - 1) / len);
}

size_t scan_workspace_bytes(int64_t B, int64_t D, int64_t N, int nseg) {
  if (nseg <= 1) return 0;
  return static_cast<size_t>(2) * static_cast<size_t>(nseg - 1) * static_cast<size_t>(B) *
         static_cast<size_t>(D) * static_cast<size_t>(N) * sizeof(float);
}

int64_t scan_grid_blocks(int64_t B, int64_t D, int nseg) {
  return static_cast<int64_t>(nseg) * B * ((D + kChannels - 1) / kChannels);
}

hipError_t launch_scan(const ScanPlan& pl, hipStream_t stream) {
  ScanArgs a{};
  a.B = pl.B;
  a.D = pl.D;
  a.L = pl.L;
  a.N = pl.N;
  a.seg_len = pl.seg_len;
  a.nseg = pl.nseg;
  a.n_dgroups = static_cast<int>((pl.D + kChannels - 1) / kChannels);
  a.in_bf16 = pl.in_bf16;
  a.out_bf16 = pl.out_bf16;
  a.u = pl.u;
  a.dt = pl.dt;
  a.z = pl.z;
  a.Bm = pl.Bm;
  a.Cm = pl.Cm;
  a.dt_bias = pl.dt_bias;
  a.A = pl.A;
  a.Dskip = pl.Dskip;
  a.h0 = pl.h0;
  a.reset = pl.reset;
  a.out = pl.out;
  a.h_last = pl.h_last;
  const size_t per = static_cast<size_t>(pl.nseg > 1 ? pl.nseg - 1 : 0) * pl.B * pl.D * pl.N;
  a.ws_P = pl.ws;
  a.ws_H = pl.ws ? pl.ws + per : nullptr;
  const int per_piece = static_cast<int>(pl.B) * a.n_dgroups;
  const int nf = per_piece * pl.nseg;
  const int na = per_piece * (pl.nseg - 1);
  int npl = 1;
  while (npl * 16 < pl.N) npl *= 2;
  return pl.in_bf16 ? launch_dtype<bf16_t>(npl, pl.reset != nullptr, a, nf, na, stream)
                    : launch_dtype<float>(npl, pl.reset != nullptr, a, nf, na, stream);
}

}  // namespace ssm
