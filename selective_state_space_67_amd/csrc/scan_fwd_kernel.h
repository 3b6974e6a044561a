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
// Mapping. A workgroup owns CPW channels of one batch row. Each channel
// occupies RPC DPP rows of 16 lanes (RPC = 1, 2 or 4 by state size, so that
// even N = 128 launches four waves per SIMD), and lane k of slice s holds
// states n = (16 s + k) * NPL .. + NPL - 1 in registers. Every lane runs the
// recurrence sequentially in time for its own states, so no per-element work
// is spent on a parallel scan; the (b, d, n) recurrences already give each
// launch thousands of waves.
//
// Skewed pipeline. Lane k processes step t at iteration m = t + k. The partial
// output sum_n C h of lane k is added to the running sum that lane k-1
// produced for the same step one iteration earlier (one DPP row_shr:1 add), so
// after lane 15 the row holds the dot product over its slice of n. This costs
// one add per lane-step instead of a log2(16)-level reduction; the RPC slice
// sums of a channel are added when the output is written.
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
// Lane 15 of each row writes the finished slice sums into an LDS ring; after
// the next chunk the workgroup adds the slices, applies D*u and the gate and
// stores `out` along L.
//
// Long sequences with few channels (L split into pieces): a first launch
// computes each piece's affine aggregate (product of the decays and the end
// state from a zero start); the second launch folds the aggregates of the
// preceding pieces into the starting state of each piece and runs the full
// recurrence. The two-level composition is the associative combine of affine
// maps (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2). The aggregate launch writes
// no output, so its lanes run in lockstep without the skew (one copy of the
// (delta, delta*u) ring, broadcast reads), and the sum of delta that gives the
// decay product is taken by the staging threads, once per (channel, step).
//
// Resets: the step's delta is stored with its sign bit set; the lane clears
// its states before that step (a wave-uniform branch, taken only when some
// lane of the wave meets a reset).
#pragma once

#include <algorithm>

#include "device_math.h"
#include "kernels.h"

namespace ssm {
namespace fwd {

// kFull: the scan itself. kAggregate: per-piece affine aggregates of a split
// scan. kCheckpoint: the forward sweep of the backward pass (states every 16
// steps and per-segment adjoint aggregates; see the kernel).
enum Mode { kFull = 0, kAggregate = 1, kCheckpoint = 2 };

// Work layout of one kernel instance, fixed at compile time.
template <int NPL_, int RPC_>
struct Tile {
  static constexpr int NPL = NPL_;                  // states per lane
  static constexpr int RPC = RPC_;                  // DPP rows (slices) per channel
  static constexpr int WAVES = RPC >= 4 ? 8 : 4;    // waves per workgroup
  static constexpr int THREADS = 64 * WAVES;
  // Register budget for the occupancy the layout relies on (waves per SIMD).
  static constexpr int MIN_WAVES_PER_SIMD = NPL >= 4 ? 2 : RPC >= 4 ? 4 : 3;
  static constexpr int CPW = WAVES * 4 / RPC;       // channels per workgroup
  static constexpr int NPAD = 16 * NPL * RPC;       // states covered per channel
  static constexpr int T = NPAD <= 32 ? 32 : 16;    // steps per chunk
  static constexpr int RING = 2 * T;                // steps kept in LDS
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
  // kCheckpoint only
  const void* dout;   // (B, D, L), the gradient of out
  float* ckpt;        // (B, n_ck, D, N): the state entering every 16-step chunk
  float* seg_P;       // (B, nsegb, D, N): product of a_t over each backward segment
  float* seg_G;       // (B, nsegb, D, N): sum of (prod a) dy C over each segment
  int64_t seg_steps;  // backward segment length (a multiple of 16 dividing seg_len)
  int64_t n_ck;
  int nsegb;
  // causal conv1d + SiLU on u (CONV kernels only)
  const float* conv_w;         // (D, conv_k)
  const float* conv_b;         // (D) or null
  const float* conv_state_in;  // (B, D, conv_k - 1) or null
  float* conv_state_out;       // (B, D, conv_k - 1) or null
  int conv_k;                  // 1 .. 4
  float* uconv_out;            // kCheckpoint with a conv stage: the scan input u' (B, D, L), f32
  int zoh;                     // exact zero-order hold input coefficient (ZOH kernels)
};

// Final conv state of a workgroup's channels d0 .. d0 + cpw - 1 of batch row
// b: the last conv_k - 1 inputs of the sequence, oldest first, zeros for those
// hidden by a later reset; threads tid < 3 cpw write one value each. Called
// by the workgroups of the last piece.
template <typename InT, bool HAS_RESET>
__device__ __forceinline__ void write_final_conv_state(const ScanArgs& a, int b, int64_t d0, int cpw, int tid) {
  if (tid >= cpw * 3) return;
  const int cc = tid / 3, kk = tid % 3;
  const int64_t dd = d0 + cc;
  if (dd >= a.D || kk >= a.conv_k - 1) return;
  const int64_t pos = a.L - (a.conv_k - 1) + kk;
  bool vis = true;  // no reset after pos (a reset at pos itself starts a document there)
  if (HAS_RESET)
    for (int64_t q = max(pos + 1, int64_t{0}); q < a.L; ++q) vis = vis && !a.reset[static_cast<int64_t>(b) * a.L + q];
  float v = 0.0f;
  if (vis) {
    if (pos >= 0)
      v = load_elem(static_cast<const InT*>(a.u), (static_cast<int64_t>(b) * a.D + dd) * a.L + pos);
    else if (a.conv_state_in)
      v = a.conv_state_in[(static_cast<int64_t>(b) * a.D + dd) * (a.conv_k - 1) + (pos + a.conv_k - 1)];
  }
  a.conv_state_out[(static_cast<int64_t>(b) * a.D + dd) * (a.conv_k - 1) + kk] = v;
}

// Register budget (waves per SIMD) of one kernel instance. The checkpoint
// sweep keeps more per-state values live (the segment's decay product and
// adjoint sum), so with several states per lane it gets two waves. The plain
// full pass with one state per lane fits in 128 VGPRs when its LDS reads are
// single-buffered, and runs at four waves: the fourth wave hides the read
// latency better than the second register set did (measured 1-5% faster on
// N = 16 shapes); its conv and zero-order-hold variants would spill there.
template <typename TL, int MODE, bool CONV, bool ZOH>
constexpr int kernel_waves_per_simd() {
  if (MODE == kCheckpoint && TL::NPL >= 2) return 2;
  if (MODE == kFull && !CONV && !ZOH && TL::NPL == 1 && TL::RPC == 1) return 4;
  return TL::MIN_WAVES_PER_SIMD;
}

// One chunk's B or C rows through a buffer descriptor: the base (the chunk's
// first element) and the range move with the chunk in scalar registers, so a
// staging item keeps one fixed 32-bit byte offset for the whole kernel. (With
// plain pointers the compiler strength-reduces every item's address into its
// own 64-bit pointer, advanced by a 64-bit vector add per chunk.) The range is
// the bytes from the base to the end of the tensor, clamped to [0, 2^31 - 1]
// (0 for the trailing chunks the full pass runs past a piece, whose items are
// all masked off); every item a chunk loads lies inside it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           static_cast<int>(max(int64_t{0}, min(bytes, int64_t{0x7FFFFFFF}))),
                                           0x00020000);
}
__device__ __forceinline__ bf16_t buffer_elem(__amdgpu_buffer_rsrc_t r, uint32_t item, bf16_t) {
  return bf16_t{__builtin_amdgcn_raw_buffer_load_b16(r, item * 2u, 0, 0)};
}
__device__ __forceinline__ float buffer_elem(__amdgpu_buffer_rsrc_t r, uint32_t item, float) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, item * 4u, 0, 0));
}

template <typename TL, typename InT, bool HAS_RESET, int MODE, bool CONV, bool ZOH>
__global__ __launch_bounds__(TL::THREADS, (kernel_waves_per_simd<TL, MODE, CONV, ZOH>())) void scan_kernel(
    const ScanArgs a) {
  constexpr int NPL = TL::NPL, RPC = TL::RPC, CPW = TL::CPW, THREADS = TL::THREADS;
  constexpr int T = TL::T, RING = TL::RING, NPAD = TL::NPAD;
  constexpr int MASK = RING - 1;
  constexpr bool FULL = MODE == kFull;
  constexpr bool CKPT = MODE == kCheckpoint;
  // LDS geometry, in float2 units.
  //  (delta, delta*u): two copies x CPW channel rows. Each row carries a
  //  16-entry mirror of its first 16 slots so a lane's 16-step window never
  //  wraps. Row stride and copy offset were chosen by measurement on gfx950:
  //  with a row stride of RING + 16 float2 and copy 1 offset by 16 float2
  //  beyond copy 0's rows, the skewed 16-byte window reads of a wave are free
  //  of bank conflicts. The lockstep aggregate pass reads one address per row;
  //  a row stride of RING + 8 float2 (144 dwords at RING = 64) puts the four
  //  rows of a wave in different banks.
  constexpr int DU_STRIDE = FULL ? RING + 16 : RING + 8;
  constexpr int DU_COPY = CPW * DU_STRIDE + 16;
  //  (B, C): one row per state; windows start at multiples of 16 and never wrap.
  constexpr int BC_STRIDE = RING + 2;
  //  The lockstep passes (aggregate, checkpoint) read B (and the checkpoint
  //  sweep C) as floats: one row per lane, holding the NPL states of that
  //  lane side by side for every step, row stride RING * NPL + 4 floats. A
  //  lane's values of consecutive steps are then one contiguous 16-byte read,
  //  and consecutive lanes' reads start 4 banks apart, so the 16 lanes of a
  //  read pass cover the 64 banks once. (A row per state puts the rows of
  //  lanes with two states 2 x (RING + 4) floats apart, all in 8 banks.)
  constexpr int LS_STRIDE = RING * NPL + 4;
  constexpr int C_OFF = (NPAD / NPL) * LS_STRIDE;  // the checkpoint sweep's C rows follow the B rows
  constexpr int BC_FLOATS = CKPT ? 2 * C_OFF : 2 * NPAD * BC_STRIDE;
  static_assert(CKPT || C_OFF <= 2 * NPAD * BC_STRIDE, "aggregate B rows fit the (B, C) buffer");
  //  dy (the gate-weighted output gradient) per (channel, step).
  constexpr int DY_STRIDE = RING + 4;
  // Row staging: CPW x T (channel, step) items per chunk, RI consecutive steps
  // per thread, handled by the first ROW_THREADS threads.
  constexpr int ROW_ITEMS = CPW * T;
  constexpr int RI = ROW_ITEMS >= 2 * THREADS ? 2 : 1;
  constexpr int ROW_THREADS = ROW_ITEMS / RI;
  constexpr int BC_ITEMS = T * NPAD / THREADS;  // (step, state) items per thread per chunk
  static_assert(ROW_THREADS <= THREADS && ROW_ITEMS % RI == 0, "row staging split");
  static_assert(BC_ITEMS >= 1 && (T * NPAD) % THREADS == 0, "B/C staging split");

  __shared__ __align__(16) float2 s_du[DU_COPY + CPW * DU_STRIDE];
  __shared__ __align__(16) float s_bcf[BC_FLOATS];
  float2* const s_bc = reinterpret_cast<float2*>(s_bcf);
  __shared__ __align__(16) float s_dy[CKPT ? CPW * DY_STRIDE : 4];
  __shared__ __align__(16) float s_y[FULL ? CPW * RPC * RING : 4];  // finished slice sums per step
  __shared__ float s_sum[FULL ? 1 : CPW];                              // aggregate pass: sum of delta

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
  const int64_t d0 = static_cast<int64_t>(g) * CPW;
  const bool group_full = d0 + CPW <= a.D;

  // Workgroup-uniform bases; per-thread offsets below stay in 32 bits
  // (channel * L + step < CPW L <= 16 L, and L < 2^27 is checked by the front end).
  const int64_t row0 = (static_cast<int64_t>(b) * a.D + d0) * a.L + t_seg;
  const InT* __restrict__ u_wg = static_cast<const InT*>(a.u) + row0;
  const InT* __restrict__ dt_wg = static_cast<const InT*>(a.dt) + row0;
  const InT* __restrict__ z_wg = a.z ? static_cast<const InT*>(a.z) + row0 : nullptr;
  const int64_t bc0 = (static_cast<int64_t>(b) * a.L + t_seg) * a.N;
  const InT* __restrict__ B_wg = static_cast<const InT*>(a.Bm) + bc0;
  const InT* __restrict__ C_wg = static_cast<const InT*>(a.Cm) + bc0;
  const int64_t bc_total = a.B * a.L * a.N;  // elements of B (and of C)
  const uint8_t* __restrict__ rs_wg = HAS_RESET ? a.reset + static_cast<int64_t>(b) * a.L + t_seg : nullptr;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int k = lane & 15;                          // lane within its DPP row
  const int grow = (tid >> 6) * 4 + (lane >> 4);    // DPP row within the workgroup
  const int c = grow / RPC;                         // channel within the workgroup
  const int slice = grow % RPC;                     // slice of the channel's states
  const int64_t d = d0 + c;
  const bool dvalid = d < a.D;
  const int nbase = (slice * 16 + k) * NPL;         // first state of this lane

  // Per-lane parameters and state. With ZOH also A and 1/A (0 for A = 0).
  float A2[NPL], h[NPL], Aj[ZOH ? NPL : 1], invA[ZOH ? NPL : 1];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = nbase + j;
    const bool ok = dvalid && n < N;
    A2[j] = ok ? a.A[d * N + n] * kLog2e : 0.0f;
    if constexpr (ZOH) {
      Aj[j] = ok ? a.A[d * N + n] : 0.0f;
      invA[j] = Aj[j] != 0.0f ? 1.0f / Aj[j] : 0.0f;
    }
    h[j] = 0.0f;
    if ((FULL || CKPT) && ok) {
      const int64_t hi = (static_cast<int64_t>(b) * a.D + d) * N + n;
      float hv = a.h0 ? a.h0[hi] : 0.0f;
      // Fold the aggregates of the preceding pieces: h <- P h + H.
      const int64_t w0 = (static_cast<int64_t>(b) * a.D + d) * N + n;
      h[j] = fold_aggregates(a.ws_P + w0, a.ws_H + w0, s, a.B * a.D * N, hv);
    }
  }

  // Empty rings: steps before the start (read by lagging lanes) are identity
  // steps (delta = 0, delta*u = 0, B = C = 0).
  for (int i = tid; i < DU_COPY + CPW * DU_STRIDE; i += THREADS) s_du[i] = make_float2(0.f, 0.f);
  for (int i = tid; i < BC_FLOATS; i += THREADS) s_bcf[i] = 0.0f;

  // Full pass: lane 15 finishes step L-1 by iteration L+17. The aggregate pass
  // needs no cross-lane sum, so its lanes run in lockstep without the skew.
  const int nchunks = FULL ? (Lseg + 18 + T - 1) / T : (Lseg + T - 1) / T;
  const int p = FULL ? k & 1 : 0;

  float yreg[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) yreg[i] = 0.0f;
  // Aggregate pass: sum of delta over this staging thread's steps, and whether
  // one of them resets (then the piece's decay product is 0).
  float sum_delta = 0.0f;
  bool cleared = false;
  // Checkpoint sweep: running decay product and adjoint sum of the current
  // backward segment.
  float segP[NPL], segG[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    segP[j] = 1.0f;
    segG[j] = 0.0f;
  }
  // ... and where the current backward segment ends, and its index (a piece
  // starts on a segment boundary: seg_steps divides seg_len). Tracked as the
  // sweep advances: a 64-bit remainder every 16 steps cost more scalar and
  // vector instructions than the step arithmetic between them.
  int64_t seg_end = CKPT ? t_seg + a.seg_steps : 0;
  int64_t seg_idx = CKPT ? t_seg / a.seg_steps : 0;
  // This lane's checkpoint slot for the piece's first 16-step block (the
  // piece starts on a block boundary); block k of the piece is k x D x N
  // floats further, a scalar offset, where the full index cost a chain of
  // 64-bit multiplies per write.
  float* const ck_lane =
      CKPT ? a.ckpt + ((static_cast<int64_t>(b) * a.n_ck + t_seg / 16) * a.D + (dvalid ? d : 0)) * N + nbase
           : nullptr;
  const int64_t ck_block = a.D * N;
  const InT* __restrict__ go_wg = CKPT ? static_cast<const InT*>(a.dout) + row0 : nullptr;

  // Row-staging items of this thread: RI consecutive steps of one channel.
  const bool row_thread = tid < ROW_THREADS;
  const int sc = (tid / (T / RI)) % CPW;   // channel (threads past ROW_THREADS repeat, unused)
  const int stl = (tid % (T / RI)) * RI;   // first step within the chunk
  const unsigned srow = static_cast<unsigned>(sc * L + stl);  // offset from the workgroup base
  const bool sc_valid = row_thread && d0 + sc < a.D;
  const float s_bias = sc_valid && a.dt_bias ? a.dt_bias[d0 + sc] : 0.0f;
  const float s_dskip = sc_valid && a.Dskip ? a.Dskip[d0 + sc] : 0.0f;
  // Conv taps of this staging thread's channel, right-aligned in 4 slots.
  float s_cw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float s_cb = 0.0f;
  if (CONV && sc_valid) {
    for (int k = 0; k < a.conv_k; ++k) s_cw[4 - a.conv_k + k] = a.conv_w[(d0 + sc) * a.conv_k + k];
    s_cb = a.conv_b ? a.conv_b[d0 + sc] : 0.0f;
  }

  // (step, state) staging item q of this thread: step q_tl within the chunk,
  // state q_n (NPAD is a power of two, so these are a shift and a mask).
  auto bc_tl = [&](int q) { return (tid + q * THREADS) / NPAD; };
  auto bc_n = [&](int q) { return (tid + q * THREADS) % NPAD; };

  // Raw inputs of one chunk (loaded two chunks ahead of their use) and the
  // per-step output factors D*u and silu(z) kept until the chunk is finished.
  struct Raw {
    InT b[BC_ITEMS], c[BC_ITEMS], u[RI], dt[RI], z[RI], go[RI];
    uint8_t rs[RI];
    float xh[CONV ? 3 : 1];    // conv inputs of the three steps before the thread's first step
    uint8_t rh[CONV ? 2 : 1];  // reset flags of the two steps before it
  };
  struct Out {
    float dsk[RI], gate[RI];
  };

  // Interior chunks of a full channel group take the unmasked path; the last
  // chunks and partial groups mask each item (masked items load nothing and
  // stay zero).
  auto load_chunk = [&](int J, Raw& r) {
    const int tau0 = J * T;
    // B and C of the chunk: in the full pass and the checkpoint sweep through
    // descriptors based at its first element (item offsets below T * N stay
    // fixed; see chunk_rsrc). The aggregate pass, which loads only B, keeps
    // plain loads: there the descriptors measured 2% slower (long-genomics).
    const int64_t bc_left = (bc_total - bc0 - static_cast<int64_t>(tau0) * N) * static_cast<int64_t>(sizeof(InT));
    const InT* __restrict__ Bp = B_wg + static_cast<int64_t>(tau0) * N;
    const __amdgpu_buffer_rsrc_t Bj = chunk_rsrc(Bp, bc_left);
    const __amdgpu_buffer_rsrc_t Cj = chunk_rsrc(C_wg + static_cast<int64_t>(tau0) * N, bc_left);
    auto bc_at = [&](__amdgpu_buffer_rsrc_t r, unsigned item) {
      if constexpr (MODE == kAggregate)
        return Bp[item];  // only B is read in this mode
      else
        return buffer_elem(r, item, InT{});
    };
    const InT* __restrict__ uj = u_wg + tau0;
    const InT* __restrict__ dtj = dt_wg + tau0;
    const InT* __restrict__ zj = z_wg ? z_wg + tau0 : nullptr;
    const InT* __restrict__ goj = CKPT ? go_wg + tau0 : nullptr;
    const uint8_t* __restrict__ rsj = HAS_RESET ? rs_wg + tau0 : nullptr;
    // Conv halo: the conv inputs of steps T0-3 .. T0-1 (T0 = this thread's
    // first step) and the reset flags of T0-2, T0-1. Steps before the sequence
    // come from the initial conv state (zeros without one).
    if constexpr (CONV) {
      const int64_t T0 = t_seg + tau0 + stl;
      const int64_t dch = d0 + sc;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int64_t pos = T0 - 3 + j;
        float v = 0.0f;
        if (sc_valid && pos < L) {
          if (pos >= 0)
            v = load_elem(uj, static_cast<int64_t>(srow) - 3 + j);
          else if (a.conv_state_in && pos >= 1 - a.conv_k)
            v = a.conv_state_in[(static_cast<int64_t>(b) * a.D + dch) * (a.conv_k - 1) + (pos + a.conv_k - 1)];
        }
        r.xh[j] = v;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t pos = T0 - 2 + j;
        r.rh[j] = HAS_RESET && sc_valid && pos >= 0 && pos < L ? a.reset[static_cast<int64_t>(b) * L + pos] : 0;
      }
    }
    if (group_full && tau0 + T <= Lseg) {
#pragma unroll
      for (int q = 0; q < BC_ITEMS; ++q) {
        const bool ok = bc_n(q) < N;
        const unsigned off = static_cast<unsigned>(bc_tl(q) * N + bc_n(q));
        r.b[q] = ok ? bc_at(Bj, off) : InT{};
        r.c[q] = (FULL || CKPT) && ok ? bc_at(Cj, off) : InT{};
      }
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        r.u[i] = row_thread ? uj[srow + i] : InT{};
        r.dt[i] = row_thread ? dtj[srow + i] : InT{};
        r.z[i] = (FULL || CKPT) && zj && row_thread ? zj[srow + i] : InT{};
        r.go[i] = CKPT && row_thread ? goj[srow + i] : InT{};
        r.rs[i] = HAS_RESET && row_thread ? rsj[stl + i] : 0;
      }
    } else {
#pragma unroll
      for (int q = 0; q < BC_ITEMS; ++q) {
        const bool ok = bc_n(q) < N && tau0 + bc_tl(q) < Lseg;
        const unsigned off = static_cast<unsigned>(bc_tl(q) * N + bc_n(q));
        r.b[q] = ok ? bc_at(Bj, off) : InT{};
        r.c[q] = (FULL || CKPT) && ok ? bc_at(Cj, off) : InT{};
      }
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        const bool ok = sc_valid && tau0 + stl + i < Lseg;
        r.u[i] = ok ? uj[srow + i] : InT{};
        r.dt[i] = ok ? dtj[srow + i] : InT{};
        r.z[i] = (FULL || CKPT) && zj && ok ? zj[srow + i] : InT{};
        r.go[i] = CKPT && ok ? goj[srow + i] : InT{};
        r.rs[i] = HAS_RESET && ok ? rsj[stl + i] : 0;
      }
    }
  };

  // ---- chunk J (ring half `par` = J & 1) into LDS: per-step parameters computed once ----
  auto store_chunk = [&](int J, const int par, const Raw& r, Out& o) {
    const int tau0 = J * T;
#pragma unroll
    for (int q = 0; q < BC_ITEMS; ++q) {
      const int n = bc_n(q);
      if (FULL)
        s_bc[n * BC_STRIDE + ((par * T + bc_tl(q) + (n / NPL) % 16) & MASK)] =
            make_float2(load_elem(&r.b[q], 0), load_elem(&r.c[q], 0));
      else
        s_bcf[(n / NPL) * LS_STRIDE + (par * T + bc_tl(q)) * NPL + n % NPL] = load_elem(&r.b[q], 0);
      if (CKPT) s_bcf[C_OFF + (n / NPL) * LS_STRIDE + (par * T + bc_tl(q)) * NPL + n % NPL] = load_elem(&r.c[q], 0);
    }
    if (!row_thread) return;
    float dl[RI], dv[RI];
    float xw[3 + RI];   // conv window inputs x_{T0-3} .. x_{T0+RI-1}
    bool rr[2 + RI];    // reset flags of T0-2 .. T0+RI-1
    if constexpr (CONV) {
#pragma unroll
      for (int j = 0; j < 3; ++j) xw[j] = r.xh[j];
      rr[0] = r.rh[0];
      rr[1] = r.rh[1];
#pragma unroll
      for (int i = 0; i < RI; ++i) {
        xw[3 + i] = load_elem(&r.u[i], 0);
        rr[2 + i] = r.rs[i];
      }
    }
#pragma unroll
    for (int i = 0; i < RI; ++i) {
      // Items past the end carry zeros, which make identity steps (delta = 0).
      float uu = load_elem(&r.u[i], 0);
      if constexpr (CONV) {  // the scan input is silu(causal conv of u) at step T0 + i
        uu = silu_f32(conv_pre(s_cw, s_cb, xw[i], xw[i + 1], xw[i + 2], xw[i + 3], rr[i + 2], rr[i + 1], rr[i]));
        if (CKPT && a.uconv_out && sc_valid && tau0 + stl + i < Lseg) a.uconv_out[row0 + tau0 + srow + i] = uu;
      }
      dl[i] = softplus_f32(load_elem(&r.dt[i], 0) + s_bias);
      if (!sc_valid || tau0 + stl + i >= Lseg) dl[i] = 0.0f;
      dv[i] = ZOH ? uu : dl[i] * uu;  // ZOH keeps u: its coefficient depends on the state's A
      if (FULL) {
        o.dsk[i] = s_dskip * uu;
        o.gate[i] = z_wg ? silu_f32(load_elem(&r.z[i], 0)) : 1.0f;
      }
      if (MODE == kAggregate) {
        sum_delta += dl[i];
        cleared = cleared || (HAS_RESET && r.rs[i]);
      }
      if (CKPT) {
        // dy = dout * silu(z): the gradient reaching y (zero past the end,
        // where dout was not loaded)
        const float go = load_elem(&r.go[i], 0);
        s_dy[sc * DY_STRIDE + par * T + stl + i] = z_wg ? go * silu_f32(load_elem(&r.z[i], 0)) : go;
      }
      if (HAS_RESET && r.rs[i]) dl[i] = -dl[i];  // sign bit: clear the state before this step
    }
    const int s0 = par * T + stl;                       // ring slot of this thread's first step
    if (!FULL) {
      // Lockstep lanes read slot tau itself: one copy, no mirror.
      float2* du = s_du + sc * DU_STRIDE + s0;
      if (RI == 2)
        *reinterpret_cast<float4*>(du) = make_float4(dl[0], dv[0], dl[RI - 1], dv[RI - 1]);
      else
        du[0] = make_float2(dl[0], dv[0]);
      return;
    }
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

  // ---- the finished outputs of chunk J: out = (sum of slices + D u) silu(z) ----
  auto finalize = [&](int J, const int par, const Out& o) {
    if (!row_thread) return;
    const int tau0 = J * T;
    const int s0 = par * T + stl;
    float y[RI];
#pragma unroll
    for (int i = 0; i < RI; ++i) y[i] = 0.0f;
#pragma unroll
    for (int sl = 0; sl < RPC; ++sl) {
      const float* yrow = s_y + (sc * RPC + sl) * RING + s0;
      if (RI == 2) {
        const float2 yy = *reinterpret_cast<const float2*>(yrow);
        y[0] += yy.x;
        y[RI - 1] += yy.y;
      } else {
        y[0] += yrow[0];
      }
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
  float* const yslot = s_y + grow * RING;  // this row's slice sums
  auto step = [&](const int i, const int m0, float dl, const float dv, const float (&Bv)[NPL],
                  const float (&Cv)[NPL]) {
    if (HAS_RESET) {
      const bool rs = __float_as_int(dl) < 0;
      if (__builtin_amdgcn_ballot_w64(rs)) {
        keep_branch();
#pragma unroll
        for (int j = 0; j < NPL; ++j) h[j] = rs ? 0.0f : h[j];
      }
      dl = fabsf(dl);
    }
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const float abar = fast_exp2(dl * A2[j]);
      if constexpr (ZOH)
        h[j] = __builtin_fmaf(abar, h[j], (Bv[j] * dv) * zoh_coef(dl, dl * Aj[j], abar, invA[j]));
      else
        h[j] = __builtin_fmaf(abar, h[j], Bv[j] * dv);
      if (FULL) part = j == 0 ? Cv[j] * h[j] : __builtin_fmaf(Cv[j], h[j], part);
    }
    if (FULL) {
      yreg[i] = row_shr1(yreg[(i + 15) & 15]) + part;
      if ((i & 3) == 2 && k == 15) {
        // steps m0+i-18 .. m0+i-15 are complete in this row: one aligned 16-byte store
        *reinterpret_cast<float4*>(yslot + ((m0 + i - 18) & MASK)) =
            make_float4(yreg[(i - 3) & 15], yreg[(i - 2) & 15], yreg[(i - 1) & 15], yreg[i]);
      }
    }
  };

  const float2* du_row = s_du + p * DU_COPY + c * DU_STRIDE;
  const float2* bc_row = s_bc + nbase * BC_STRIDE;

  // ---- one step of the checkpoint sweep ----
  // h as in the scan; segP = product of a_t since the segment start (0 after a
  // reset, where a_t counts as 0); segG += segP dy C, the segment's adjoint
  // from a zero start, accumulated in forward order. `seg` (a std::bool_constant)
  // false leaves out (segP, segG): the first backward segment's are never read,
  // since the reverse sweep folds only the segments after its own.
  auto step_ck = [&](auto seg, float dl, const float dv, const float dy, const float (&Bv)[NPL],
                     const float (&Cv)[NPL]) {
    bool rs = false;
    if (HAS_RESET) {
      rs = __float_as_int(dl) < 0;
      if (__builtin_amdgcn_ballot_w64(rs)) {
        keep_branch();
#pragma unroll
        for (int j = 0; j < NPL; ++j) h[j] = rs ? 0.0f : h[j];
      }
      dl = fabsf(dl);
    }
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const float abar = fast_exp2(dl * A2[j]);
      if constexpr (ZOH)
        h[j] = __builtin_fmaf(abar, h[j], (Bv[j] * dv) * zoh_coef(dl, dl * Aj[j], abar, invA[j]));
      else
        h[j] = __builtin_fmaf(abar, h[j], Bv[j] * dv);
      if constexpr (decltype(seg)::value) {
        segP[j] = rs ? 0.0f : segP[j] * abar;
        segG[j] = __builtin_fmaf(segP[j] * dy, Cv[j], segG[j]);
      }
    }
    (void)rs;
    (void)dy;
  };

  // ---- the recurrence over chunk J (ring half `par`) ----
  // One lane-step reads one (delta, delta*u) pair and NPL (B, C) pairs. With
  // one state per lane, the reads of each 8-step half block are issued while
  // the previous half block computes (two register sets, alternating
  // statically) at three waves per SIMD; at four waves (the plain full pass)
  // one register set, the other waves covering the read latency.
  auto compute = [&](const int J, const int par) {
    if constexpr (CKPT) {
      // Lockstep, like the aggregate pass, plus C and dy per step. The state
      // entering every 16-step chunk is written out, and each backward
      // segment's (segP, segG) at its last step.
      const float* b_row = s_bcf + (nbase / NPL) * LS_STRIDE;
      const float* c_row = b_row + C_OFF;
      const float* dy_row = s_dy + c * DY_STRIDE;
      const int64_t tchunk = t_seg + static_cast<int64_t>(J) * T;  // step held in slot par * T
      const int64_t pend = t_seg + Lseg;
      auto sweep = [&](auto seg) {
#pragma unroll
      for (int i = 0; i < T; i += 4) {
        const int m = par * T + i;
        if (i % 16 == 0 && tchunk + i < pend) {
          float* const ck = ck_lane + static_cast<int64_t>((J * T + i) >> 4) * ck_block;
#pragma unroll
          for (int j = 0; j < NPL; ++j)
            if (dvalid && nbase + j < N) ck[j] = h[j];
        }
        if constexpr (NPL == 1) {
          const float4 d01 = *reinterpret_cast<const float4*>(du_row + m);
          const float4 d23 = *reinterpret_cast<const float4*>(du_row + m + 2);
          const float4 dy4 = *reinterpret_cast<const float4*>(dy_row + m);
          float B0[NPL], B1[NPL], B2[NPL], B3[NPL], C0[NPL], C1[NPL], C2[NPL], C3[NPL];
#pragma unroll
          for (int j = 0; j < NPL; ++j) {
            const float4 vb = *reinterpret_cast<const float4*>(b_row + m);
            const float4 vc = *reinterpret_cast<const float4*>(c_row + m);
            B0[j] = vb.x;
            B1[j] = vb.y;
            B2[j] = vb.z;
            B3[j] = vb.w;
            C0[j] = vc.x;
            C1[j] = vc.y;
            C2[j] = vc.z;
            C3[j] = vc.w;
          }
          step_ck(seg, d01.x, d01.y, dy4.x, B0, C0);
          step_ck(seg, d01.z, d01.w, dy4.y, B1, C1);
          step_ck(seg, d23.x, d23.y, dy4.z, B2, C2);
          step_ck(seg, d23.z, d23.w, dy4.w, B3, C3);
        } else {
          // Several states per lane: two steps per group of reads, so that
          // fewer B and C values are live at once (no spills at the register
          // budget of two waves per SIMD).
#pragma unroll
          for (int i2 = 0; i2 < 4; i2 += 2) {
            const float4 d01 = *reinterpret_cast<const float4*>(du_row + m + i2);
            const float2 dy2 = *reinterpret_cast<const float2*>(dy_row + m + i2);
            // steps m + i2 and m + i2 + 1, the lane's NPL states each: 2 x NPL
            // consecutive floats of B and of C
            float bt[2 * NPL], ct[2 * NPL];
#pragma unroll
            for (int q = 0; q < 2 * NPL; q += 4) {
              const float4 vb = *reinterpret_cast<const float4*>(b_row + (m + i2) * NPL + q);
              const float4 vc = *reinterpret_cast<const float4*>(c_row + (m + i2) * NPL + q);
              bt[q] = vb.x;
              bt[q + 1] = vb.y;
              bt[q + 2] = vb.z;
              bt[q + 3] = vb.w;
              ct[q] = vc.x;
              ct[q + 1] = vc.y;
              ct[q + 2] = vc.z;
              ct[q + 3] = vc.w;
            }
            float B0[NPL], B1[NPL], C0[NPL], C1[NPL];
#pragma unroll
            for (int j = 0; j < NPL; ++j) {
              B0[j] = bt[j];
              B1[j] = bt[NPL + j];
              C0[j] = ct[j];
              C1[j] = ct[NPL + j];
            }
            step_ck(seg, d01.x, d01.y, dy2.x, B0, C0);
            step_ck(seg, d01.z, d01.w, dy2.y, B1, C1);
            // keep the next group's reads from being hoisted above this one
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (i % 16 == 12) {
          const int64_t tend = tchunk + i + 4;  // end of this 16-step block
          if (tend - 16 < pend && (tend == seg_end || tend >= pend)) {
            const int64_t si = ((static_cast<int64_t>(b) * a.nsegb + seg_idx) * a.D + d) * N;
            seg_end += a.seg_steps;
            ++seg_idx;
#pragma unroll
            for (int j = 0; j < NPL; ++j) {
              if (dvalid && nbase + j < N) {
                a.seg_P[si + nbase + j] = segP[j];
                a.seg_G[si + nbase + j] = segG[j];
              }
              segP[j] = 1.0f;
              segG[j] = 0.0f;
            }
          }
        }
      }
      };
      // Chunks that end within the first backward segment skip (segP, segG):
      // what the sweep writes for that segment (P = 1, G = 0) is never read.
      // Only with two states per lane and no conv stage or zero-order hold:
      // with four states, the conv stage or the zero-order hold the second copy
      // of the loop spills, and with one state per lane the sweep gained nothing
      // (its step is not held by VALU issue there; 1-2% slower from the extra
      // registers), while packed N = 128 documents went from 4.56 to 4.38 ms.
      if constexpr (NPL == 2 && !CONV && !ZOH) {
        if (tchunk + T > a.seg_steps)
          sweep(std::true_type{});
        else
          sweep(std::false_type{});
      } else {
        sweep(std::true_type{});
      }
    } else if constexpr (!FULL) {
      // Lockstep: every lane is at step m. Per four steps a lane reads two
      // (delta, delta*u) float4s (broadcast within its DPP row) and one B
      // float4 per state (shared by the rows of a wave). Nothing is stored,
      // so the compiler may issue the reads of the whole chunk early.
      const float* b_row = reinterpret_cast<const float*>(s_bc) + (nbase / NPL) * LS_STRIDE;
#pragma unroll
      for (int i = 0; i < T; i += 4) {
        const int m = par * T + i;
        const float4 d01 = *reinterpret_cast<const float4*>(du_row + m);
        const float4 d23 = *reinterpret_cast<const float4*>(du_row + m + 2);
        // steps m .. m + 3, the lane's NPL states each: 4 x NPL consecutive floats
        float bt[4 * NPL];
#pragma unroll
        for (int q = 0; q < 4 * NPL; q += 4) {
          const float4 v = *reinterpret_cast<const float4*>(b_row + m * NPL + q);
          bt[q] = v.x;
          bt[q + 1] = v.y;
          bt[q + 2] = v.z;
          bt[q + 3] = v.w;
        }
        float B0[NPL], B1[NPL], B2[NPL], B3[NPL];
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          B0[j] = bt[j];
          B1[j] = bt[NPL + j];
          B2[j] = bt[2 * NPL + j];
          B3[j] = bt[3 * NPL + j];
        }
        step(i, m, d01.x, d01.y, B0, B0);  // C is not used by the aggregate pass
        step(i + 1, m, d01.z, d01.w, B1, B1);
        step(i + 2, m, d23.x, d23.y, B2, B2);
        step(i + 3, m, d23.z, d23.w, B3, B3);
      }
    } else if constexpr (NPL == 1 && RPC <= 2) {
      constexpr int HB = T / 8;
      float4 dA[4], bA[NPL][4], dB[4], bB[NPL][4];
      auto fetch = [&](const int hb, float4 (&dd)[4], float4 (&bb)[NPL][4]) {
        const int m0 = par * T + (hb >> 1) * 16;
        const float2* du_win = du_row + ((m0 - k + p) & MASK) + (hb & 1) * 8;
        const float2* bc_win = bc_row + m0 + (hb & 1) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dd[i] = *reinterpret_cast<const float4*>(du_win + 2 * i);
#pragma unroll
          for (int j = 0; j < NPL; ++j) bb[j][i] = *reinterpret_cast<const float4*>(bc_win + j * BC_STRIDE + 2 * i);
        }
      };
      auto run = [&](const int hb, const float4 (&dd)[4], const float4 (&bb)[NPL][4]) {
        const int m0 = par * T + (hb >> 1) * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int st = (hb & 1) * 8 + 2 * i;
          float B0[NPL], C0[NPL], B1[NPL], C1[NPL];
#pragma unroll
          for (int j = 0; j < NPL; ++j) {
            B0[j] = bb[j][i].x;
            C0[j] = bb[j][i].y;
            B1[j] = bb[j][i].z;
            C1[j] = bb[j][i].w;
          }
          step(st, m0, dd[i].x, dd[i].y, B0, C0);
          step(st + 1, m0, dd[i].z, dd[i].w, B1, C1);
        }
      };
      if constexpr (kernel_waves_per_simd<TL, MODE, CONV, ZOH>() >= 4) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          fetch(hb, dA, bA);
          run(hb, dA, bA);
        }
      } else {
        fetch(0, dA, bA);
#pragma unroll
        for (int hb = 0; hb < HB; hb += 2) {
          fetch(hb + 1, dB, bB);
          run(hb, dA, bA);
          if (hb + 2 < HB) fetch(hb + 2, dA, bA);
          run(hb + 1, dB, bB);
        }
      }
    } else {
#pragma unroll 1
      for (int blk = 0; blk < T / 16; ++blk) {
        const int m0 = par * T + blk * 16;  // ring position of the block
        // This lane's 16-step window of (delta, delta*u) pairs, pair-aligned in copy p.
        const float2* du_win = du_row + ((m0 - k + p) & MASK);
        const float2* bc_win = bc_row + m0;
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
    }
  };

  Raw r0, r1;
  Out o0, o1;
  load_chunk(0, r0);
  if (nchunks > 1) load_chunk(1, r1);
  __syncthreads();  // rings are empty before the first chunk is stored
  // workgroups resident per CU at the occupancy bound: 4 SIMDs x waves per SIMD / waves per workgroup
  constexpr int kResidentPerCU = 4 * kernel_waves_per_simd<TL, MODE, CONV, ZOH>() / TL::WAVES;
  const ProgressPriority prio(nchunks, a.nblocks <= 256 * kResidentPerCU);
  for (int J = 0; J < nchunks; J += 2) {
    prio.update(J);
    // even chunk: ring half 0, register sets r0 / o0
    store_chunk(J, 0, r0, o0);
    if (J + 2 < nchunks) load_chunk(J + 2, r0);
    __syncthreads();
    compute(J, 0);
    __syncthreads();
    if (FULL && J >= 1) finalize(J - 1, 1, o1);
    if (J + 1 >= nchunks) break;
    // odd chunk: ring half 1, register sets r1 / o1
    store_chunk(J + 1, 1, r1, o1);
    if (J + 3 < nchunks) load_chunk(J + 3, r1);
    __syncthreads();
    compute(J + 1, 1);
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
  if (MODE == kAggregate) {
    // Per-channel totals from the T / RI staging threads of each channel
    // (consecutive threads within one wave).
    constexpr int G = T / RI;
    int clr = cleared ? 1 : 0;
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) {
      sum_delta += __shfl_xor(sum_delta, off, G);
      clr |= __shfl_xor(clr, off, G);
    }
    if (row_thread && stl == 0) s_sum[sc] = clr ? -1.0f : sum_delta;  // delta >= 0, so -1 marks a reset
    __syncthreads();
    sum_delta = s_sum[c];
  }
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int n = nbase + j;
    if (!dvalid || n >= N) continue;
    if (FULL) {
      if (a.h_last && s == a.nseg - 1) a.h_last[(static_cast<int64_t>(b) * a.D + d) * N + n] = h[j];
    } else if (MODE == kAggregate) {
      const int64_t wi = (static_cast<int64_t>(s) * a.B + b) * a.D * N + d * N + n;
      a.ws_H[wi] = h[j];
      a.ws_P[wi] = sum_delta < 0.0f ? 0.0f : fast_exp2(A2[j] * sum_delta);
    }
  }

  if constexpr (FULL && CONV) {
    if (a.conv_state_out && s == a.nseg - 1) write_final_conv_state<InT, HAS_RESET>(a, b, d0, CPW, tid);
  }
}

template <typename TL, typename InT>
void log_tile_launch(const char* mode, const ScanArgs& a, int nblocks, bool reset, bool conv, bool zoh) {
  SSM_LOG("launch scan_kernel<Tile<%d,%d>> %s: %s in, reset %d, conv %d, zoh %d; grid %d x %d threads "
          "(%d channels x %d states per workgroup, %d-step chunks), %d pieces of %lld steps",
          TL::NPL, TL::RPC, mode, sizeof(InT) == 2 ? "bf16" : "f32", reset, conv, zoh, nblocks, TL::THREADS,
          TL::CPW, TL::NPAD, TL::T, a.nseg, static_cast<long long>(a.seg_len));
}

template <typename TL, typename InT, bool HAS_RESET, bool CONV, bool ZOH>
hipError_t launch_tile(const ScanArgs& args, int nblocks_full, int nblocks_agg, bool checkpoint,
                       hipStream_t stream) {
  // nblocks_agg workgroups of piece aggregates (none when the sequence is one
  // piece), then nblocks_full of the full pass (none for aggregates only)
  if (nblocks_agg > 0) {
    ScanArgs agg = args;
    agg.nblocks = nblocks_agg;
    log_tile_launch<TL, InT>("aggregate", agg, nblocks_agg, HAS_RESET, CONV, ZOH);
    hipLaunchKernelGGL((scan_kernel<TL, InT, HAS_RESET, kAggregate, CONV, ZOH>), dim3(nblocks_agg),
                       dim3(TL::THREADS), 0, stream, agg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (nblocks_full == 0) return hipSuccess;
  ScanArgs full = args;
  full.nblocks = nblocks_full;
  log_tile_launch<TL, InT>(checkpoint ? "checkpoint" : "full", full, nblocks_full, HAS_RESET, CONV, ZOH);
  if (checkpoint)
    hipLaunchKernelGGL((scan_kernel<TL, InT, HAS_RESET, kCheckpoint, CONV, ZOH>), dim3(nblocks_full),
                       dim3(TL::THREADS), 0, stream, full);
  else
    hipLaunchKernelGGL((scan_kernel<TL, InT, HAS_RESET, kFull, CONV, ZOH>), dim3(nblocks_full), dim3(TL::THREADS),
                       0, stream, full);
  return hipGetLastError();
}

template <typename TL, typename InT, bool HAS_RESET>
hipError_t launch_conv(const ScanArgs& a, int nf, int na, bool ck, hipStream_t stream) {
  if (a.zoh)
    return a.conv_w ? launch_tile<TL, InT, HAS_RESET, true, true>(a, nf, na, ck, stream)
                    : launch_tile<TL, InT, HAS_RESET, false, true>(a, nf, na, ck, stream);
  return a.conv_w ? launch_tile<TL, InT, HAS_RESET, true, false>(a, nf, na, ck, stream)
                  : launch_tile<TL, InT, HAS_RESET, false, false>(a, nf, na, ck, stream);
}

// Layout by state size: (states per lane, rows per channel).
//   N <= 16: (1, 1)   N <= 32: (1, 2)   N <= 64: (1, 4)   N <= 128: (2, 4)   N <= 256: (4, 4)
template <typename Fn>
hipError_t with_tile(int64_t N, Fn&& fn) {
  if (N <= 16) return fn(Tile<1, 1>{});
  if (N <= 32) return fn(Tile<1, 2>{});
  if (N <= 64) return fn(Tile<1, 4>{});
  if (N <= 128) return fn(Tile<2, 4>{});
  return fn(Tile<4, 4>{});
}

inline int channels_per_block(int64_t N) {
  int cpw = 0;
  (void)with_tile(N, [&](auto tile) {
    cpw = decltype(tile)::CPW;
    return hipSuccess;
  });
  return cpw;
}

// Workgroups of the full pass that are resident at once on the whole chip
// (256 CUs x 4 SIMDs x the kernel's waves per SIMD / waves per workgroup);
// `plain`: the plain full pass (no conv stage, delta B coefficient).
inline int resident_blocks(int64_t N, bool plain) {
  int r = 0;
  (void)with_tile(N, [&](auto tile) {
    using TL = decltype(tile);
    const int waves = plain ? kernel_waves_per_simd<TL, kFull, false, false>() : TL::MIN_WAVES_PER_SIMD;
    r = 256 * 4 * waves / TL::WAVES;
    return hipSuccess;
  });
  return r;
}

// Every (tile, mode, conv) kernel of one input type and reset setting. The
// four combinations are instantiated in their own translation units
// (scan_fwd_<type>_<reset>.hip) so that they compile in parallel.
template <typename InT, bool HAS_RESET>
hipError_t launch_variant(const ScanArgs& a, int nf, int na, bool ck, hipStream_t stream) {
  return with_tile(a.N, [&](auto tile) {
    using TL = decltype(tile);
    return launch_conv<TL, InT, HAS_RESET>(a, nf, na, ck, stream);
  });
}

extern template hipError_t launch_variant<float, false>(const ScanArgs&, int, int, bool, hipStream_t);
extern template hipError_t launch_variant<float, true>(const ScanArgs&, int, int, bool, hipStream_t);
extern template hipError_t launch_variant<bf16_t, false>(const ScanArgs&, int, int, bool, hipStream_t);
extern template hipError_t launch_variant<bf16_t, true>(const ScanArgs&, int, int, bool, hipStream_t);

// The 16-state full pass (scan_fwd_n16.hip): whether it takes a launch, and
// the launch (the pieces' aggregates, when split, through launch_variant).
bool n16_eligible(const ScanArgs& a, bool checkpoint);
hipError_t launch_n16(const ScanArgs& a, int nblocks_full, int nblocks_agg, hipStream_t stream);

}  // namespace fwd
}  // namespace ssm
