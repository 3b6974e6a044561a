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
  constexpr bool FULL = MODE == kFull;
  // LDS geometry, in float2 units.
  //  (delta, delta*u): two copies x 16 channel rows. Each row carries a
  //  16-entry mirror of its first 16 slots so a lane's 16-step window never
  //  wraps. Row stride and copy offset were chosen by measurement on gfx950:
  //  with a row stride of RING + 16 float2 and copy 1 offset by 16 float2
  //  beyond copy 0's rows, the skewed 16-byte window reads of a wave are free
  //  of bank conflicts.
  constexpr int DU_STRIDE = RING + 16;
  constexpr int DU_COPY = kChannels * DU_STRIDE + 16;
  //  (B, C): one row per state; windows start at multiples of 16 and never wrap.
  constexpr int BC_STRIDE = RING + 2;
  constexpr int RI = kChannels * T / kThreads;   // consecutive steps per thread in row staging
  constexpr int BC_ITEMS = T * NPAD / kThreads;  // (step, state) items per thread per chunk
  static_assert(RI == 1 || RI == 2, "row staging handles one or two steps per thread");
  static_assert(BC_ITEMS >= 1 && (T * NPAD) % kThreads == 0, "B/C staging split");

  __shared__ __align__(16) float2 s_du[DU_COPY + kChannels * DU_STRIDE];
  __shared__ __align__(16) float2 s_bc[NPAD * BC_STRIDE];
  __shared__ __align__(16) float s_y[FULL ? kChannels * RING : 4];  // finished sum_n C h per step

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
  const int L = static_cast<int>(a.L);
  const int N = static_cast<int>(a.N);
  const int64_t d0 = static_cast<int64_t>(g) * kChannels;
  const bool group_full = d0 + kChannels <= a.D;

  // Workgroup-uniform bases; per-thread offsets below stay in 32 bits
  // (channel * L + step < 16 L, and L < 2^27 is checked by the front end).
  const int64_t row0 = (static_cast<int64_t>(b) * a.D + d0) * a.L + t_seg;
  const InT* __restrict__ u_wg = static_cast<const InT*>(a.u) + row0;
  const InT* __restrict__ dt_wg = static_cast<const InT*>(a.dt) + row0;
  const InT* __restrict__ z_wg = a.z ? static_cast<const InT*>(a.z) + row0 : nullptr;
  const int64_t bc0 = (static_cast<int64_t>(b) * a.L + t_seg) * a.N;
  const InT* __restrict__ B_wg = static_cast<const InT*>(a.Bm) + bc0;
  const InT* __restrict__ C_wg = static_cast<const InT*>(a.Cm) + bc0;
  const uint8_t* __restrict__ rs_wg = HAS_RESET ? a.reset + static_cast<int64_t>(b) * a.L + t_seg : nullptr;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int k = lane & 15;                        // lane within the channel's row
  const int c = (tid >> 6) * 4 + (lane >> 4);     // channel within the workgroup
  const int64_t d = d0 + c;
  const bool dvalid = d < a.D;

  // Per-lane parameters and state.
  float A2[NPL], h[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = k * NPL + j;
    const bool ok = dvalid && n < N;
    A2[j] = ok ? a.A[d * N + n] * kLog2e : 0.0f;
    h[j] = 0.0f;
    if (FULL && ok) {
      const int64_t hi = (static_cast<int64_t>(b) * a.D + d) * N + n;
      float hv = a.h0 ? a.h0[hi] : 0.0f;
      // Fold the aggregates of the preceding pieces: h <- P h + H.
      for (int sp = 0; sp < s; ++sp) {
        const int64_t wi = (static_cast<int64_t>(sp) * a.B + b) * a.D * N + d * N + n;
        hv = __builtin_fmaf(a.ws_P[wi], hv, a.ws_H[wi]);
      }
      h[j] = hv;
    }
  }

  // Empty rings: steps before the start (read by lagging lanes) are identity
  // steps (delta = 0, delta*u = 0, B = C = 0).
  for (int i = tid; i < DU_COPY + kChannels * DU_STRIDE; i += kThreads) s_du[i] = make_float2(0.f, 0.f);
  for (int i = tid; i < NPAD * BC_STRIDE; i += kThreads) s_bc[i] = make_float2(0.f, 0.f);

  const int nchunks = (Lseg + 18 + T - 1) / T;  // lane 15 finishes step L-1 by iteration L+17
  const int p = k & 1;

  float yreg[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) yreg[i] = 0.0f;
  float sum_delta = 0.0f;
  bool cleared = false;

  // Row-staging items of this thread: RI consecutive steps of one channel.
  const int sc = tid / 16;              // channel
  const int stl = (tid % 16) * RI;      // first step within the chunk
  const unsigned srow = static_cast<unsigned>(sc * L + stl);  // offset from the workgroup base
  const bool sc_valid = d0 + sc < a.D;
  const float s_bias = sc_valid && a.dt_bias ? a.dt_bias[d0 + sc] : 0.0f;
  const float s_dskip = sc_valid && a.Dskip ? a.Dskip[d0 + sc] : 0.0f;

  // (step, state) staging items of this thread; offsets are chunk-invariant.
  unsigned bc_off[BC_ITEMS];
  int bc_tl[BC_ITEMS];
  bool bc_ok[BC_ITEMS];
#pragma unroll
  for (int r = 0; r < BC_ITEMS; ++r) {
    const int q = tid + r * kThreads;
    bc_tl[r] = q / NPAD;
    bc_ok[r] = q % NPAD < N;
    bc_off[r] = static_cast<unsigned>(bc_tl[r] * N + q % NPAD);
  }

  // Raw inputs of one chunk (loaded two chunks ahead of their use) and the
  // per-step output factors D*u and silu(z) kept until the chunk is finished.
  struct Raw {
    InT b[BC_ITEMS], c[BC_ITEMS], u[RI], dt[RI], z[RI];
    uint8_t rs[RI];
  };
  struct Out {
    float dsk[RI], gate[RI];
  };

  // Interior chunks of a full channel group take the unmasked path; the last
  // chunks and partial groups mask each item (masked items load nothing and
  // stay zero).
  auto load_chunk = [&](int J, Raw& r) {
    const int tau0 = J * T;
    const InT* __restrict__ Bj = B_wg + static_cast<int64_t>(tau0) * N;
    const InT* __restrict__ Cj = C_wg + static_cast<int64_t>(tau0) * N;
    const InT* __restrict__ uj = u_wg + tau0;
    const InT* __restrict__ dtj = dt_wg + tau0;
    const InT* __restrict__ zj = z_wg ? z_wg + tau0 : nullptr;
    const uint8_t* __restrict__ rsj = HAS_RESET ? rs_wg + tau0 : nullptr;
    if (group_full && tau0 + T <= Lseg) {
#pragma unroll
      for (int q = 0; q < BC_ITEMS; ++q) {
        r.b[q] = bc_ok[q] ? Bj[bc_off[q]] : InT{};
        r.c[q] = FULL && bc_ok[q] ? Cj[bc_off[q]] : InT{};
      }
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        r.u[i] = uj[srow + i];
        r.dt[i] = dtj[srow + i];
        r.z[i] = FULL && zj ? zj[srow + i] : InT{};
        r.rs[i] = HAS_RESET ? rsj[stl + i] : 0;
      }
    } else {
#pragma unroll
      for (int q = 0; q < BC_ITEMS; ++q) {
        const bool ok = bc_ok[q] && tau0 + bc_tl[q] < Lseg;
        r.b[q] = ok ? Bj[bc_off[q]] : InT{};
        r.c[q] = FULL && ok ? Cj[bc_off[q]] : InT{};
      }
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        const bool ok = sc_valid && tau0 + stl + i < Lseg;
        r.u[i] = ok ? uj[srow + i] : InT{};
        r.dt[i] = ok ? dtj[srow + i] : InT{};
        r.z[i] = FULL && zj && ok ? zj[srow + i] : InT{};
        r.rs[i] = HAS_RESET && ok ? rsj[stl + i] : 0;
      }
    }
  };

  // ---- chunk J (ring half `par` = J & 1) into LDS: per-step parameters computed once ----
  auto store_chunk = [&](int J, const int par, const Raw& r, Out& o) {
    const int tau0 = J * T;
#pragma unroll
    for (int q = 0; q < BC_ITEMS; ++q) {
      const int n = (tid + q * kThreads) % NPAD;
      s_bc[n * BC_STRIDE + ((par * T + bc_tl[q] + n / NPL) & MASK)] =
          make_float2(load_elem(&r.b[q], 0), FULL ? load_elem(&r.c[q], 0) : 0.0f);
    }
    float dl[RI], dv[RI];
#pragma unroll
    for (int i = 0; i < RI; ++i) {
      // Items past the end carry zeros, which make identity steps (delta = 0).
      const float uu = load_elem(&r.u[i], 0);
      dl[i] = softplus_f32(load_elem(&r.dt[i], 0) + s_bias);
      if (!sc_valid || tau0 + stl + i >= Lseg) dl[i] = 0.0f;
      dv[i] = dl[i] * uu;
      if (FULL) {
        o.dsk[i] = s_dskip * uu;
        o.gate[i] = z_wg ? silu_f32(load_elem(&r.z[i], 0)) : 1.0f;
      }
      if (HAS_RESET && r.rs[i]) dl[i] = -dl[i];  // sign bit: clear the state before this step
    }
    const int s0 = par * T + stl;                       // ring slot of this thread's first step
    float2* du0 = s_du + sc * DU_STRIDE;                // copy 0: step tau at slot tau
    float2* du1 = s_du + DU_COPY + sc * DU_STRIDE;      // copy 1: step tau at slot tau + 1
    if (RI == 2) {
      const float4 v = make_float4(dl[0], dv[0], dl[RI - 1], dv[RI - 1]);
      *reinterpret_cast<float4*>(du0 + s0) = v;
      if (s0 < 16) *reinterpret_cast<float4*>(du0 + s0 + RING) = v;
    } else {
      du0[s0] = make_float2(dl[0], dv[0]);
      if (s0 < 16) du0[s0 + RING] = make_float2(dl[0], dv[0]);
    }
#pragma unroll
    for (int i = 0; i < RI; ++i) {
      const int s1 = (s0 + 1 + i) & MASK;
      du1[s1] = make_float2(dl[i], dv[i]);
      if (s1 < 16) du1[s1 + RING] = make_float2(dl[i], dv[i]);
    }
  };

  // ---- the finished outputs of chunk J: out = (y + D u) silu(z) ----
  auto finalize = [&](int J, const int par, const Out& o) {
    const int tau0 = J * T;
    const int s0 = par * T + stl;
    float y[RI];
    if (RI == 2) {
      const float2 yy = *reinterpret_cast<const float2*>(s_y + sc * RING + s0);
      y[0] = yy.x;
      y[RI - 1] = yy.y;
    } else {
      y[0] = s_y[sc * RING + s0];
    }
    const int64_t o0 = row0 + tau0 + srow;  // element index of this thread's first output
#pragma unroll
    for (int i = 0; i < RI; ++i) {
      if (sc_valid && tau0 + stl + i < Lseg) {
        const float v = (y[i] + o.dsk[i]) * o.gate[i];
        if (a.out_bf16)
          store_elem(static_cast<bf16_t*>(a.out), o0 + i, v);
        else
          store_elem(static_cast<float*>(a.out), o0 + i, v);
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
        *reinterpret_cast<float4*>(s_y + c * RING + ((m0 + i - 18) & MASK)) =
            make_float4(yreg[(i - 3) & 15], yreg[(i - 2) & 15], yreg[(i - 1) & 15], yreg[i]);
      }
    } else {
      sum_delta += dl;
    }
  };

  const float2* du_row = s_du + p * DU_COPY + c * DU_STRIDE;
  const float2* bc_row = s_bc + (k * NPL) * BC_STRIDE;

  // ---- the recurrence over chunk J (ring half `par`) ----
  auto compute = [&](const int par) {
#pragma unroll 1
    for (int blk = 0; blk < T / 16; ++blk) {
      const int m0 = par * T + blk * 16;  // ring position of the block (step offsets cancel mod RING)
      // This lane's 16-step window of (delta, delta*u) pairs, pair-aligned in copy p.
      const float2* du_win = du_row + ((m0 - k + p) & MASK);
      const float2* bc_win = bc_row + m0;
      float4 dd[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) dd[i] = *reinterpret_cast<const float4*>(du_win + 2 * i);
      float4 bcb[NPL == 1 ? 8 : 1];
      if (NPL == 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) bcb[NPL == 1 ? i : 0] = *reinterpret_cast<const float4*>(bc_win + 2 * i);
      }
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        float B0[NPL], C0[NPL], B1[NPL], C1[NPL];
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          const float4 v = NPL == 1 ? bcb[NPL == 1 ? i / 2 : 0]
                                    : *reinterpret_cast<const float4*>(bc_win + j * BC_STRIDE + i);
          B0[j] = v.x;
          C0[j] = v.y;
          B1[j] = v.z;
          C1[j] = v.w;
        }
        step(i, m0, dd[i / 2].x, dd[i / 2].y, B0, C0);
        step(i + 1, m0, dd[i / 2].z, dd[i / 2].w, B1, C1);
      }
    }
  };

  Raw r0, r1;
  Out o0, o1;
  load_chunk(0, r0);
  if (nchunks > 1) load_chunk(1, r1);
  __syncthreads();  // rings are empty before the first chunk is stored
  for (int J = 0; J < nchunks; J += 2) {
    // even chunk: ring half 0, register sets r0 / o0
    store_chunk(J, 0, r0, o0);
    if (J + 2 < nchunks) load_chunk(J + 2, r0);
    __syncthreads();
    compute(0);
    __syncthreads();
    if (FULL && J >= 1) finalize(J - 1, 1, o1);
    if (J + 1 >= nchunks) break;
    // odd chunk: ring half 1, register sets r1 / o1
    store_chunk(J + 1, 1, r1, o1);
    if (J + 3 < nchunks) load_chunk(J + 3, r1);
    __syncthreads();
    compute(1);
    __syncthreads();
    if (FULL) finalize(J, 0, o0);
  }
  if (FULL && (nchunks - 1) * T < Lseg) {
    if ((nchunks - 1) & 1)
      finalize(nchunks - 1, 1, o1);
    else
      finalize(nchunks - 1, 0, o0);
  }

  // ---- results that leave the workgroup ----
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = k * NPL + j;
    if (!dvalid || n >= N) continue;
    if (FULL) {
      if (a.h_last && s == a.nseg - 1) a.h_last[(static_cast<int64_t>(b) * a.D + d) * N + n] = h[j];
    } else {
      const int64_t wi = (static_cast<int64_t>(s) * a.B + b) * a.D * N + d * N + n;
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
