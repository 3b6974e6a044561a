// The full pass of the selective scan for 16 states per channel on gfx950,
// output written (the "Mamba-130M/2.8B-shaped" layer scans and the
// long-sequence scan), with the delta B input coefficient or (template flag
// ZOH) the exact zero-order hold (e^{delta A} - 1) / A B of "Illustrated Mamba
// state space model", "Mathematical basis: structured SSM", and optionally
// (template flag CONV) the causal depthwise conv1d + SiLU on u.
//
// What is computed is the same as scan_kernel's kFull mode in
// scan_fwd_kernel.h (the recurrence of "Illustrated Mamba state space model",
// "Mathematical basis: structured SSM" and step 1, with the read-out and D
// term of "Mamba SSM core theory and Keras/TensorFlow implementation", scan
// step, and the SiLU gate). The mapping is that kernel's one-state-per-lane
// layout: a workgroup owns 16 channels of one batch row, a channel is one DPP
// row of 16 lanes, lane k holds state k, and lane k runs step t at iteration
// t + k so that the read-out sum over the row is one row_shr:1 move and one
// FMA per lane-step. This instance trims everything around that recurrence,
// which is what decides its speed: the vector ALU is the limit, and per
// (b, d, t, n) the recurrence itself needs a multiply, the exponential (two
// issue slots), a multiply, the state FMA, the DPP move and the read-out FMA.
//  - Inputs are read as pairs of consecutive elements through buffer
//    descriptors whose base moves with the chunk in scalar registers, so the
//    per-lane offsets stay fixed for the whole kernel and no load needs a
//    64-bit address, a bounds branch or a zero fill: the descriptor's range
//    turns reads past the end of a tensor into zeros, and the chunks that
//    reach past the piece (or a partial channel group) mask their steps in
//    one uniform branch.
//  - Each staging thread owns two consecutive steps of one channel, and the
//    outputs of those steps are written as one pair.
// The per-chunk structure (LDS rings, skew, mirrors, finishing order) is
// scan_kernel's; see the layout notes there.
#include <type_traits>

#include "scan_fwd_kernel.h"


namespace ssm {
namespace fwd {

namespace {

// Raw buffer descriptor: base, no stride, `bytes` of range (reads beyond read
// as 0, writes beyond are dropped). The third word selects 32-bit data on gfx9.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Bytes from element `start` to the end of a tensor of `total` elements,
// capped at 2^31 - 1; 0 once the start lies past the end, so that every read
// then returns 0. Every offset a workgroup uses (its 16 rows of L elements
// plus the chunk advance) stays below the cap where this kernel is used.
__device__ __forceinline__ int bytes_left(int64_t total, int64_t start, int elem) {
  const int64_t left = start < total ? (total - start) * elem : 0;
  return static_cast<int>(min(left, int64_t{0x7FFFFFFF}));
}

// A pair of consecutive input elements, as loaded.
template <typename InT>
struct Pair;

template <>
struct Pair<bf16_t> {
  using raw = uint32_t;
  __device__ __forceinline__ static raw load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  __device__ __forceinline__ static float lo(raw v) { return __uint_as_float(v << 16); }
  __device__ __forceinline__ static float hi(raw v) { return __uint_as_float(v & 0xFFFF0000u); }
  __device__ __forceinline__ static raw zero() { return 0u; }
};

template <>
struct Pair<float> {
  using raw = uint32_t __attribute__((ext_vector_type(2)));
  __device__ __forceinline__ static raw load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  }
  __device__ __forceinline__ static float lo(raw v) { return __uint_as_float(v.x); }
  __device__ __forceinline__ static float hi(raw v) { return __uint_as_float(v.y); }
  __device__ __forceinline__ static raw zero() { return raw{0u, 0u}; }
};

}  // namespace

// Waves per SIMD the kernel is built for: four in bf16 (128 registers), three
// in float32 and where the conv stage and the zero-order hold come together
// (they would spill at 128); five for the compact-LDS layout below.
template <typename InT, bool ZOH, bool CONV, bool FIVE>
constexpr int n16_waves_per_simd() {
  return FIVE ? 5 : sizeof(InT) == 2 && !(ZOH && CONV) ? 4 : 3;
}

// FIVE: the compact-LDS layout (29 KB instead of 37 KB per workgroup, so that
// five workgroups fit a CU where four do otherwise): a two-part (B, C) ring,
// which costs a second barrier per chunk, and the read-out sums kept in the
// (delta, delta*u) slots of copy 0 once no lane reads them any more. It is
// used where five workgroups per CU save a round of the grid.
template <typename InT, bool HAS_RESET, bool ZOH, bool CONV, bool FIVE>
__global__ __launch_bounds__(256, (n16_waves_per_simd<InT, ZOH, CONV, FIVE>())) void scan16_kernel(
    const ScanArgs a) {
  using P = Pair<InT>;
  constexpr int N = 16, T = 32, RING = 2 * T, MASK = RING - 1, CPW = 16, THREADS = 256;
  constexpr int S_IN = sizeof(InT);
  // LDS (float2 units unless noted), as in scan_kernel's full pass:
  //  (delta, delta*u) in two copies, copy 1 shifted by one step, each row with
  //  a 16-entry mirror of its first slots; (B, C) of state n in row n at
  //  column t + n; the finished read-out sums per channel and step (floats).
  constexpr int DU_STRIDE = RING + 16;
  constexpr int DU_COPY = CPW * DU_STRIDE + 16;
  //  The (B, C) ring has three chunk parts where the (delta, delta*u) ring has
  //  two: a chunk's (B, C) spill over into the next part (the skewed columns
  //  t + n run past the chunk), so with two parts store_chunk(J + 1) would
  //  overwrite the part compute(J) reads. With three, the one barrier per
  //  chunk (after store_chunk) orders every cross-wave use of the ring; the
  //  compact layout has two parts and a second barrier before each staging.
  constexpr int BC_PARTS = FIVE ? 2 : 3;
  constexpr int BC_RING = BC_PARTS * T;
  constexpr int BC_STRIDE = BC_RING + 2;
  __shared__ __align__(16) float2 s_du[DU_COPY + CPW * DU_STRIDE];
  __shared__ __align__(16) float2 s_bc[N * BC_STRIDE];
  __shared__ __align__(16) float s_y[FIVE ? 4 : CPW * RING];

  // Workgroup -> (piece, batch row, channel group), renumbered so that a batch
  // row's workgroups (which share B and C) run on one XCD.
  int idx = blockIdx.x;
  if ((a.nblocks & 7) == 0) idx = (idx & 7) * (a.nblocks >> 3) + (idx >> 3);
  const int g = idx % a.n_dgroups;
  const int rest = idx / a.n_dgroups;
  const int b = rest % static_cast<int>(a.B);
  const int s = rest / static_cast<int>(a.B);
  const int64_t t_seg = static_cast<int64_t>(s) * a.seg_len;
  const int Lseg = static_cast<int>(min(a.seg_len, a.L - t_seg));
  const int64_t d0 = static_cast<int64_t>(g) * CPW;
  const bool group_full = d0 + CPW <= a.D;

  const int64_t row0 = (static_cast<int64_t>(b) * a.D + d0) * a.L + t_seg;  // element of (b, d0, t_seg)
  const int64_t n_rows = a.B * a.D * a.L;                                    // elements of u, dt_raw, z, out
  const int64_t bc0 = (static_cast<int64_t>(b) * a.L + t_seg) * N;
  const int64_t n_bc = a.B * a.L * N;
  const InT* __restrict__ u_g = static_cast<const InT*>(a.u);
  const InT* __restrict__ dt_g = static_cast<const InT*>(a.dt);
  const InT* __restrict__ z_g = static_cast<const InT*>(a.z);
  const InT* __restrict__ B_g = static_cast<const InT*>(a.Bm);
  const InT* __restrict__ C_g = static_cast<const InT*>(a.Cm);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int k = lane & 15;  // state of this lane
  const int c = tid >> 4;   // channel of this lane's DPP row; also the staging channel of this thread
  const int64_t d = d0 + c;
  const bool dvalid = d < a.D;

  // Per-lane parameter and starting state (h0, then the preceding pieces' aggregates folded in).
  const float A2 = dvalid ? a.A[d * N + k] * kLog2e : 0.0f;
  // zero-order hold: A and 1/A of this lane's state (0 for A = 0)
  const float Aj = ZOH && dvalid ? a.A[d * N + k] : 0.0f;
  const float invA = ZOH && Aj != 0.0f ? 1.0f / Aj : 0.0f;
  float h = 0.0f;
  if (dvalid) {
    const int64_t hi = (static_cast<int64_t>(b) * a.D + d) * N + k;
    h = a.h0 ? a.h0[hi] : 0.0f;
    const int64_t w0 = (static_cast<int64_t>(b) * a.D + d) * N + k;
    h = fold_aggregates(a.ws_P + w0, a.ws_H + w0, s, a.B * a.D * N, h);
  }

  // Steps before the start are identity steps (delta = 0, delta*u = 0, B = C = 0).
  for (int i = tid; i < DU_COPY + CPW * DU_STRIDE; i += THREADS) s_du[i] = make_float2(0.f, 0.f);
  for (int i = tid; i < N * BC_STRIDE; i += THREADS) s_bc[i] = make_float2(0.f, 0.f);

  // Lane 15 finishes step Lseg - 1 by iteration Lseg + 17.
  const int nchunks = (Lseg + 18 + T - 1) / T;

  // Staging roles: steps stl, stl + 1 of channel c (the row pair), and states
  // bn, bn + 1 of step bt (the B/C pair).
  const int stl = (tid & 15) * 2;
  const int bt = tid >> 3;
  const int bn = (tid & 7) * 2;
  const uint32_t row_off = static_cast<uint32_t>(c * a.L + stl) * S_IN;  // < 16 L S_IN, checked by the caller
  const uint32_t bc_off = static_cast<uint32_t>(bt * N + bn) * S_IN;
  const float s_bias = dvalid && a.dt_bias ? a.dt_bias[d] : 0.0f;
  const float s_dskip = dvalid && a.Dskip ? a.Dskip[d] : 0.0f;
  const bool has_z = a.z != nullptr;
  // Conv stage: the taps of channel d right-aligned in four slots (widths
  // below 4 have leading zero taps) and its bias.
  float s_cw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float s_cb = 0.0f;
  if (CONV && dvalid) {
    for (int q = 0; q < a.conv_k; ++q) s_cw[4 - a.conv_k + q] = a.conv_w[d * a.conv_k + q];
    s_cb = a.conv_b ? a.conv_b[d] : 0.0f;
  }

  // uh0, uh1: with the conv stage, the inputs of steps stl - 4 .. stl - 1 (two
  // pairs) and rsh the reset flags of stl - 2, stl - 1: the conv window of the
  // thread's two steps reaches three steps back.
  struct Raw {
    typename P::raw u, dt, z, bb, cc;
    typename P::raw uh0, uh1;
    uint32_t rs, rsh;
  };
  struct Out {
    float u0, u1, g0, g1;
  };

  // One descriptor per tensor from this workgroup's first element; a chunk
  // adds its advance to the per-lane offsets.
  const int64_t rs0 = static_cast<int64_t>(b) * a.L + t_seg;
  const int left_rows = bytes_left(n_rows, row0, S_IN);
  const int left_bc = bytes_left(n_bc, bc0, S_IN);
  const __amdgpu_buffer_rsrc_t rsrc_u = make_rsrc(u_g + row0, left_rows);
  const __amdgpu_buffer_rsrc_t rsrc_dt = make_rsrc(dt_g + row0, left_rows);
  const __amdgpu_buffer_rsrc_t rsrc_z = make_rsrc(has_z ? z_g + row0 : u_g, has_z ? left_rows : 0);
  const __amdgpu_buffer_rsrc_t rsrc_B = make_rsrc(B_g + bc0, left_bc);
  const __amdgpu_buffer_rsrc_t rsrc_C = make_rsrc(C_g + bc0, left_bc);
  const __amdgpu_buffer_rsrc_t rsrc_rs =
      make_rsrc(HAS_RESET ? a.reset + rs0 : nullptr, HAS_RESET ? bytes_left(a.B * a.L, rs0, 1) : 0);
  // The conv window's earlier inputs through descriptors based 4 elements (2
  // reset bytes) before the workgroup's first one. Inputs before the sequence
  // (the first chunk of the first piece) are never loaded: they come from the
  // initial conv state. The base is formed as an integer, since it can lie
  // before the tensor; every address read through it lies inside.
  const __amdgpu_buffer_rsrc_t rsrc_uh =
      CONV ? make_rsrc(reinterpret_cast<const void*>(reinterpret_cast<uintptr_t>(u_g + row0) - 4 * S_IN),
                       static_cast<int>(min(int64_t{left_rows} + 4 * S_IN, int64_t{0x7FFFFFFF})))
           : rsrc_u;
  const __amdgpu_buffer_rsrc_t rsrc_rsh =
      CONV && HAS_RESET ? make_rsrc(reinterpret_cast<const void*>(reinterpret_cast<uintptr_t>(a.reset + rs0) - 2),
                                    static_cast<int>(min(int64_t{bytes_left(a.B * a.L, rs0, 1)} + 2,
                                                         int64_t{0x7FFFFFFF})))
                        : rsrc_rs;
  // whether this thread's window reaches before the sequence in chunk 0
  const bool head0 = CONV && t_seg == 0 && stl < 4;

  auto load_chunk = [&](int J, Raw& r) {
    const uint32_t tau0 = static_cast<uint32_t>(J * T);
    const uint32_t ro = row_off + tau0 * S_IN;
    r.u = P::load(rsrc_u, ro);
    r.dt = P::load(rsrc_dt, ro);
    r.z = has_z ? P::load(rsrc_z, ro) : P::zero();
    const uint32_t bo = bc_off + tau0 * (N * S_IN);
    r.bb = P::load(rsrc_B, bo);
    r.cc = P::load(rsrc_C, bo);
    if (HAS_RESET) r.rs = __builtin_amdgcn_raw_buffer_load_b16(rsrc_rs, stl + tau0, 0, 0);
    if constexpr (CONV) {
      r.uh0 = r.uh1 = P::zero();
      r.rsh = 0;
      if (J > 0 || !head0) {
        r.uh0 = P::load(rsrc_uh, ro);
        r.uh1 = P::load(rsrc_uh, ro + 2 * S_IN);
        if (HAS_RESET) r.rsh = __builtin_amdgcn_raw_buffer_load_b16(rsrc_rsh, stl + tau0, 0, 0);
      } else if (stl == 2) {
        r.uh1 = P::load(rsrc_uh, ro + 2 * S_IN);  // steps 0, 1
        if (HAS_RESET) r.rsh = __builtin_amdgcn_raw_buffer_load_b16(rsrc_rsh, stl + tau0, 0, 0);
      }
    }
  };

  auto store_chunk = [&](int J, const int par, const int bpart, const Raw& r, Out& o) {
    const int tau0 = J * T;
    float b0 = P::lo(r.bb), b1 = P::hi(r.bb), c0 = P::lo(r.cc), c1 = P::hi(r.cc);
    float u0 = P::lo(r.u), u1 = P::hi(r.u);
    if constexpr (CONV) {
      // the scan input is silu(causal conv of u) over steps stl - 3 .. stl + 1
      float x3 = P::hi(r.uh0), x2 = P::lo(r.uh1), x1 = P::hi(r.uh1);  // steps stl - 3, stl - 2, stl - 1
      if (J == 0 && head0) {
        // steps before the sequence: the initial conv state (oldest first), or zeros
        const int K = a.conv_k;
        auto before = [&](int pos) {
          return a.conv_state_in && pos >= 1 - K && dvalid
                     ? a.conv_state_in[(static_cast<int64_t>(b) * a.D + d) * (K - 1) + (pos + K - 1)]
                     : 0.0f;
        };
        x3 = before(stl - 3);
        if (stl == 0) {
          x2 = before(-2);
          x1 = before(-1);
        }
      }
      const bool rq0 = HAS_RESET && (r.rs & 0xFFu), rq1 = HAS_RESET && (r.rs & 0xFF00u);
      const bool rm1 = HAS_RESET && (r.rsh & 0xFF00u), rm2 = HAS_RESET && (r.rsh & 0xFFu);
      const float x0 = u0;
      u0 = silu_f32(conv_pre(s_cw, s_cb, x3, x2, x1, x0, rq0, rm1, rm2));
      u1 = silu_f32(conv_pre(s_cw, s_cb, x2, x1, x0, u1, rq1, rq0, rm1));
    }
    float dl0 = softplus_f32(P::lo(r.dt) + s_bias);
    float dl1 = softplus_f32(P::hi(r.dt) + s_bias);
    if (!group_full || tau0 + T > Lseg) {
      // steps past the piece and channels past D are identity steps (their
      // loads may have read the next row or piece, so u, B and C are zeroed too)
      if (!dvalid || tau0 + stl >= Lseg) dl0 = u0 = 0.0f;
      if (!dvalid || tau0 + stl + 1 >= Lseg) dl1 = u1 = 0.0f;
      if (tau0 + bt >= Lseg) b0 = b1 = c0 = c1 = 0.0f;
    }
    // the input term's factor: delta u, or u itself with the zero-order hold
    // (its coefficient depends on the state's A and is formed per state)
    const float dv0 = ZOH ? u0 : dl0 * u0, dv1 = ZOH ? u1 : dl1 * u1;
    o.u0 = u0;
    o.u1 = u1;
    o.g0 = has_z ? silu_f32(P::lo(r.z)) : 1.0f;
    o.g1 = has_z ? silu_f32(P::hi(r.z)) : 1.0f;
    if (HAS_RESET) {
      // a reset is carried as the sign bit of delta (delta >= 0); none past the piece
      const bool r0 = (r.rs & 0xFFu) != 0 && tau0 + stl < Lseg;
      const bool r1 = (r.rs & 0xFF00u) != 0 && tau0 + stl + 1 < Lseg;
      dl0 = r0 ? -dl0 : dl0;
      dl1 = r1 ? -dl1 : dl1;
    }
    // (B, C) of states bn, bn + 1 at step bt: row n, column (part slot + n) mod BC_RING
    const int col = bpart * T + bt;
    const int c0i = col + bn, c1i = col + bn + 1;
    s_bc[bn * BC_STRIDE + (c0i >= BC_RING ? c0i - BC_RING : c0i)] = make_float2(b0, c0);
    s_bc[(bn + 1) * BC_STRIDE + (c1i >= BC_RING ? c1i - BC_RING : c1i)] = make_float2(b1, c1);
    // (delta, delta*u): copy 0 at slots s0, s0 + 1 (one 16-byte store), copy 1 one slot later
    const int s0 = par * T + stl;
    float2* du0 = s_du + c * DU_STRIDE;
    float2* du1 = s_du + DU_COPY + c * DU_STRIDE;
    const float4 v = make_float4(dl0, dv0, dl1, dv1);
    *reinterpret_cast<float4*>(du0 + s0) = v;
    if (s0 < 16) *reinterpret_cast<float4*>(du0 + s0 + RING) = v;
    const int s1 = (s0 + 1) & MASK, s2 = (s0 + 2) & MASK;
    du1[s1] = make_float2(dl0, dv0);
    du1[s2] = make_float2(dl1, dv1);
    if (s1 < 16) du1[s1 + RING] = make_float2(dl0, dv0);
    if (s2 < 16) du1[s2 + RING] = make_float2(dl1, dv1);
  };

  const int s_out = a.out_bf16 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t rsrc_out =
      make_rsrc(static_cast<char*>(a.out) + row0 * s_out, bytes_left(n_rows, row0, s_out));
  const uint32_t out_off = static_cast<uint32_t>(c * a.L + stl) * s_out;

  // The compact layout keeps the read-out sum of step slot m in copy 0's
  // (delta, delta*u) entry of slot m, float 2m of the channel's row: lane 15
  // writes it at least 15 iterations after lane 14, the last lane that reads
  // copy 0 there, and the wave that owns the channel does both, in order.
  float* const yrow0 = reinterpret_cast<float*>(s_du + c * DU_STRIDE);
  auto finalize = [&](int J, const int par, const Out& o) {
    const int tau0 = J * T;
    const int ys = par * T + stl;
    const float2 yy = FIVE ? make_float2(yrow0[2 * ys], yrow0[2 * ys + 2])
                           : *reinterpret_cast<const float2*>(s_y + c * RING + ys);
    const float o0 = __builtin_fmaf(s_dskip, o.u0, yy.x) * o.g0;
    const float o1 = __builtin_fmaf(s_dskip, o.u1, yy.y) * o.g1;
    const uint32_t off = out_off + static_cast<uint32_t>(tau0 * s_out);
    if (group_full && tau0 + T <= Lseg) {
      if (a.out_bf16) {
        uint32_t p0 = __float_as_uint(o0), p1 = __float_as_uint(o1);
        p0 += 0x7FFFu + ((p0 >> 16) & 1u);
        p1 += 0x7FFFu + ((p1 >> 16) & 1u);
        __builtin_amdgcn_raw_buffer_store_b32((p0 >> 16) | (p1 & 0xFFFF0000u), rsrc_out, off, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b64(Pair<float>::raw{__float_as_uint(o0), __float_as_uint(o1)}, rsrc_out,
                                              off, 0, 0);
      }
    } else {
      const int64_t oi = row0 + tau0 + static_cast<int64_t>(c) * a.L + stl;
      const bool ok0 = dvalid && tau0 + stl < Lseg, ok1 = dvalid && tau0 + stl + 1 < Lseg;
      if (a.out_bf16) {
        if (ok0) store_elem(static_cast<bf16_t*>(a.out), oi, o0);
        if (ok1) store_elem(static_cast<bf16_t*>(a.out), oi + 1, o1);
      } else {
        if (ok0) store_elem(static_cast<float*>(a.out), oi, o0);
        if (ok1) store_elem(static_cast<float*>(a.out), oi + 1, o1);
      }
    }
  };

  // ---- one recurrence step of this lane (position i of a 16-step block at ring slot m0) ----
  float yreg[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) yreg[i] = 0.0f;
  float* const yslot = s_y + (FIVE ? 0 : c * RING);
  auto step = [&](const int i, const int m0, float dl, const float dv, const float Bv, const float Cv) {
    if (HAS_RESET) {
      const bool rs = __float_as_int(dl) < 0;
      if (__builtin_amdgcn_ballot_w64(rs)) {
        keep_branch();
        h = rs ? 0.0f : h;
      }
      dl = fabsf(dl);
    }
    const float abar = fast_exp2(dl * A2);
    if constexpr (ZOH)
      h = __builtin_fmaf(abar, h, (Bv * dv) * zoh_coef(dl, dl * Aj, abar, invA));
    else
      h = __builtin_fmaf(abar, h, Bv * dv);
    yreg[i] = __builtin_fmaf(Cv, h, row_shr1(yreg[(i + 15) & 15]));
    if ((i & 3) == 2 && k == 15) {
      // steps m0+i-18 .. m0+i-15 are complete in this row: one aligned 16-byte store
      const int ym = (m0 + i - 18) & MASK;
      if constexpr (FIVE) {
        yrow0[2 * ym] = yreg[(i - 3) & 15];
        yrow0[2 * ym + 2] = yreg[(i - 2) & 15];
        yrow0[2 * ym + 4] = yreg[(i - 1) & 15];
        yrow0[2 * ym + 6] = yreg[i];
      } else {
        *reinterpret_cast<float4*>(yslot + ym) =
            make_float4(yreg[(i - 3) & 15], yreg[(i - 2) & 15], yreg[(i - 1) & 15], yreg[i]);
      }
    }
  };

  const int p = k & 1;
  const float2* du_row = s_du + p * DU_COPY + c * DU_STRIDE;
  const float2* bc_row = s_bc + k * BC_STRIDE;

  // ---- the recurrence over chunk J (ring half `par`), two steps per LDS read pair ----
  // Each pair of steps needs one 16-byte read of (delta, delta*u) and one of
  // (B, C). The reads run PF pairs ahead of their use and are issued one pair
  // at a time between the steps' arithmetic: issued in bursts, they fill the
  // LDS command queue and the waves stall at issue.
  constexpr int PF = 4;
  auto read_pair = [&](const int par, const int bpart, const int q, float4& dd, float4& bc) {
    const int m0 = par * T + (q >> 3) * 16;
    dd = *reinterpret_cast<const float4*>(du_row + ((m0 - k + p) & MASK) + (q & 7) * 2);
    bc = *reinterpret_cast<const float4*>(bc_row + bpart * T + (q >> 3) * 16 + (q & 7) * 2);
  };
  auto compute = [&](const int par, const int bpart) __attribute__((always_inline)) {
    float4 dd[T / 2], bc[T / 2];
#pragma unroll
    for (int q = 0; q < PF; ++q) read_pair(par, bpart, q, dd[q], bc[q]);
#pragma unroll
    for (int q = 0; q < T / 2; ++q) {
      if (q + PF < T / 2) read_pair(par, bpart, q + PF, dd[q + PF], bc[q + PF]);
      const int m0 = par * T + (q >> 3) * 16;
      const int st = (q & 7) * 2;
      step(st, m0, dd[q].x, dd[q].y, bc[q].x, bc[q].y);
      step(st + 1, m0, dd[q].z, dd[q].w, bc[q].z, bc[q].w);
      // one pair of reads, then this pair's arithmetic
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
    }
  };

  Raw r0, r1;
  Out o0, o1;
  load_chunk(0, r0);
  if (nchunks > 1) load_chunk(1, r1);
  __syncthreads();  // rings are empty before the first chunk is stored
  // workgroups resident per CU: one wave per SIMD each, as many as the occupancy bound allows
  const ProgressPriority prio(nchunks, a.nblocks <= 256 * n16_waves_per_simd<InT, ZOH, CONV, FIVE>());
  // One barrier per chunk. The (B, C) ring is the only LDS data shared across
  // waves; the barrier after store_chunk(J) makes part J mod 3 visible, and a
  // wave past it knows that every wave has finished compute(J - 1), whose
  // part the next staging, store_chunk(J + 1), starts to overwrite (its
  // spill-over lands in that part's first columns; store_chunk(J + 2) fills
  // the rest after the next barrier). The (delta, delta*u) rows and the read-out slots of a
  // channel are written and read only by the wave that owns the channel
  // (channel = tid / 16 in staging, compute and finalize alike), in program
  // order.
  // The compact layout's second barrier: before store_chunk(J + 1) every wave
  // has finished compute(J), whose part the staging's spill-over reaches.
  int bpart = 0;  // J mod BC_PARTS
  for (int J = 0; J < nchunks; J += 2) {
    prio.update(J);
    const int bpart1 = bpart == BC_PARTS - 1 ? 0 : bpart + 1;
    if (FIVE && J > 0) __syncthreads();
    store_chunk(J, 0, bpart, r0, o0);
    if (J + 2 < nchunks) load_chunk(J + 2, r0);
    __syncthreads();
    compute(0, bpart);
    if (J >= 1) finalize(J - 1, 1, o1);
    if (J + 1 >= nchunks) break;
    if (FIVE) __syncthreads();
    store_chunk(J + 1, 1, bpart1, r1, o1);
    if (J + 3 < nchunks) load_chunk(J + 3, r1);
    __syncthreads();
    compute(1, bpart1);
    finalize(J, 0, o0);
    bpart = bpart1 == BC_PARTS - 1 ? 0 : bpart1 + 1;
  }
  if ((nchunks - 1) * T < Lseg) {
    if ((nchunks - 1) & 1)
      finalize(nchunks - 1, 1, o1);
    else
      finalize(nchunks - 1, 0, o0);
  }

  if (dvalid && a.h_last && s == a.nseg - 1) a.h_last[(static_cast<int64_t>(b) * a.D + d) * N + k] = h;
  if constexpr (CONV) {
    if (a.conv_state_out && s == a.nseg - 1) write_final_conv_state<InT, HAS_RESET>(a, b, d0, CPW, tid);
  }
}

// Whether the 16-state full pass takes this launch: 16 states, not the
// checkpoint sweep, an even L (element pairs stay aligned) and buffer ranges
// within 31 bits (17 rows of L elements plus a chunk).
bool n16_eligible(const ScanArgs& a, bool checkpoint) {
  const int64_t s_in = a.in_bf16 ? 2 : 4;
  return a.N == 16 && !checkpoint && a.L % 2 == 0 && (17 * a.L + 256) * s_in < (int64_t{1} << 31);
}

hipError_t launch_n16(const ScanArgs& args, int nblocks_full, int nblocks_agg, hipStream_t stream) {
  const bool reset = args.reset != nullptr;
  if (nblocks_agg > 0) {
    // the pieces' aggregates come from scan_kernel's aggregate pass (no full pass: 0 workgroups)
    hipError_t e = args.in_bf16 ? (reset ? launch_variant<bf16_t, true>(args, 0, nblocks_agg, false, stream)
                                         : launch_variant<bf16_t, false>(args, 0, nblocks_agg, false, stream))
                                : (reset ? launch_variant<float, true>(args, 0, nblocks_agg, false, stream)
                                         : launch_variant<float, false>(args, 0, nblocks_agg, false, stream));
    if (e != hipSuccess) return e;
  }
  ScanArgs full = args;
  full.nblocks = nblocks_full;
  // The compact-LDS layout (bf16 inputs without resets, conv stage or
  // zero-order hold: the others would spill at five waves per SIMD) where five
  // workgroups per CU need fewer rounds of the grid than four.
  const int64_t per4 = 256 * 4, per5 = 256 * 5;
  const bool five = args.in_bf16 && !reset && !args.zoh && !args.conv_w &&
                    (nblocks_full + per5 - 1) / per5 < (nblocks_full + per4 - 1) / per4;
  SSM_LOG("launch scan16_kernel full: %s in, reset %d, zoh %d, conv %d; grid %d x 256 threads (16 channels x 16 "
          "states per workgroup, 32-step chunks), %d pieces of %lld steps, %s LDS layout",
          args.in_bf16 ? "bf16" : "f32", reset, args.zoh, args.conv_w != nullptr, nblocks_full, args.nseg,
          static_cast<long long>(args.seg_len), five ? "compact (five workgroups per CU)" : "standard");
  auto go = [&](auto in_t, auto has_reset, auto zoh, auto conv) {
    using InT = decltype(in_t);
    constexpr bool R = decltype(has_reset)::value, Z = decltype(zoh)::value, C = decltype(conv)::value;
    if constexpr (sizeof(InT) == 2 && !R && !Z && !C) {
      if (five) {
        hipLaunchKernelGGL((scan16_kernel<InT, R, Z, C, true>), dim3(nblocks_full), dim3(256), 0, stream, full);
        return;
      }
    }
    hipLaunchKernelGGL((scan16_kernel<InT, R, Z, C, false>), dim3(nblocks_full), dim3(256), 0, stream, full);
  };
  auto with_conv = [&](auto in_t, auto has_reset, auto zoh) {
    if (args.conv_w)
      go(in_t, has_reset, zoh, std::true_type{});
    else
      go(in_t, has_reset, zoh, std::false_type{});
  };
  auto with_zoh = [&](auto in_t, auto has_reset) {
    if (args.zoh)
      with_conv(in_t, has_reset, std::true_type{});
    else
      with_conv(in_t, has_reset, std::false_type{});
  };
  if (args.in_bf16) {
    if (reset)
      with_zoh(bf16_t{}, std::true_type{});
    else
      with_zoh(bf16_t{}, std::false_type{});
  } else {
    if (reset)
      with_zoh(float{}, std::true_type{});
    else
      with_zoh(float{}, std::false_type{});
  }
  return hipGetLastError();
}

}  // namespace fwd
}  // namespace ssm
