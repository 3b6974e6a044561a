// The selective-scan forward as a chunked two-level associative scan: the
// layout the library keeps for comparison with its sequential-in-lane
// kernels (scan_fwd_n16.hip, scan_fwd_kernel.h), for 16 real states.
//
// What is computed is the forward of ssm_scan_fwd with the delta B input
// coefficient: the recurrence of "Illustrated Mamba state space model",
// "Mathematical basis: structured SSM" and step 1, the read-out and D term of
// "Mamba SSM core theory and Keras/TensorFlow implementation", scan step, the
// SiLU gate, and resets at document boundaries ("Technical analysis: Mamba
// selective state spaces", 3.2). The parallel-scan idea is the one that page
// names in 2.2 (a Blelloch scan over the sequence in place of the serial
// recursion); here it takes its wavefront form.
//
// Layout: one wave per (batch row, channel); lane i holds step t0 + i of a
// 64-step chunk and all 16 states of it. Per chunk:
//  - every lane forms the affine pair of its step for each state,
//    a = exp(delta A[n]) (0 on a reset) and b = delta B[t, n] u;
//  - an inclusive scan of the pairs over the 64 lanes composes them,
//    (a, b) after (a', b') = (a a', a b' + b): four DPP row_shr levels inside
//    each row of 16 lanes, then row_bcast:15 and row_bcast:31 across rows;
//  - the carry from the previous chunk (the state after its last step, read
//    from lane 63 into scalar registers) gives h_t = A_t carry + B_t;
//  - the read-out sum over n is in-lane, and the output is written once.
// Per element this costs the pair (multiply, exponential, multiply), two
// operations per scan level (six levels), the carry FMA and the read-out FMA,
// against the sequential lane's multiply, exponential, multiply, FMA and
// read-out FMA plus one DPP move.
#include "device_math.h"
#include "kernels.h"

namespace ssm {
namespace {

constexpr int kN = 16;     // states per channel
constexpr int kT = 64;     // steps per chunk, one per lane
constexpr int kWaves = 4;  // channels per workgroup, one wave each

struct WaveArgs {
  int64_t B, D, L;
  int in_bf16, out_bf16;
  int nblocks;
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
};

// One level of the scan for eight states: each pair (a, b) composed after the
// pair CTRL selects (row_shr:s, or a row broadcast limited to the rows in the
// row mask), a <- a a', b <- a b' + b, as one v_fmac_f32_dpp (b first: it
// reads this lane's a before the update) and one v_mul_f32_dpp. Without
// bound_ctrl, lanes with no source lane and rows outside the mask are not
// written: they keep their own pair, as if composed with the identity (1, 0).
// The compiler folds no DPP move into a float multiply or FMA, so the level
// is written out here, and the compiler's hazard checks do not see the DPP
// inside the block: the leading s_nop gives the two wait states gfx9 requires
// between a VALU write of a register and a DPP read of it, and the chunk's
// first block waits five, the requirement after a write of EXEC (the
// prefetch's per-lane branch precedes the scan). Inside the blocks a state's
// registers are read by DPP only in the next level's block, 14 instructions
// or more after their last write.
#define SSM_WF_PAIR(A, B, CTRL) "v_fmac_f32_dpp " B ", " B ", " A " " CTRL "\n\tv_mul_f32_dpp " A ", " A ", " A " " CTRL "\n\t"
#define SSM_WF_LEVEL8(NOP, CTRL)                                                                                   \
  NOP "\n\t" SSM_WF_PAIR("%0", "%8", CTRL) SSM_WF_PAIR("%1", "%9", CTRL) SSM_WF_PAIR("%2", "%10", CTRL)           \
      SSM_WF_PAIR("%3", "%11", CTRL) SSM_WF_PAIR("%4", "%12", CTRL) SSM_WF_PAIR("%5", "%13", CTRL)                  \
          SSM_WF_PAIR("%6", "%14", CTRL) SSM_WF_PAIR("%7", "%15", CTRL)

// LEVEL 6 is level 0 as the chunk's first block (the longer wait).
template <int LEVEL>
__device__ __forceinline__ void scan_level8(float* a, float* b) {
#define SSM_WF_OPERANDS                                                                                             \
  : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7]), "+v"(b[0]),    \
    "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(b[4]), "+v"(b[5]), "+v"(b[6]), "+v"(b[7])
  if constexpr (LEVEL == 6) asm volatile(SSM_WF_LEVEL8("s_nop 4", "row_shr:1 row_mask:0xf bank_mask:0xf") SSM_WF_OPERANDS);
  if constexpr (LEVEL == 0) asm volatile(SSM_WF_LEVEL8("s_nop 1", "row_shr:1 row_mask:0xf bank_mask:0xf") SSM_WF_OPERANDS);
  if constexpr (LEVEL == 1) asm volatile(SSM_WF_LEVEL8("s_nop 1", "row_shr:2 row_mask:0xf bank_mask:0xf") SSM_WF_OPERANDS);
  if constexpr (LEVEL == 2) asm volatile(SSM_WF_LEVEL8("s_nop 1", "row_shr:4 row_mask:0xf bank_mask:0xf") SSM_WF_OPERANDS);
  if constexpr (LEVEL == 3) asm volatile(SSM_WF_LEVEL8("s_nop 1", "row_shr:8 row_mask:0xf bank_mask:0xf") SSM_WF_OPERANDS);
  if constexpr (LEVEL == 4) asm volatile(SSM_WF_LEVEL8("s_nop 1", "row_bcast:15 row_mask:0xa bank_mask:0xf") SSM_WF_OPERANDS);
  if constexpr (LEVEL == 5) asm volatile(SSM_WF_LEVEL8("s_nop 1", "row_bcast:31 row_mask:0xc bank_mask:0xf") SSM_WF_OPERANDS);
#undef SSM_WF_OPERANDS
}

// The 16 values of one step's B or C row, as loaded (bf16: 8 words; f32: 16).
template <typename InT>
struct Row;

template <>
struct Row<bf16_t> {
  uint4 w[2];
  __device__ __forceinline__ void load(const void* base, int64_t i) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(base) + i * kN);
    w[0] = p[0];
    w[1] = p[1];
  }
  __device__ __forceinline__ void zero() { w[0] = w[1] = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ float get(int n) const {
    const uint4& q = w[n >> 3];
    const uint32_t v = (n & 7) < 2 ? q.x : (n & 7) < 4 ? q.y : (n & 7) < 6 ? q.z : q.w;
    return __uint_as_float((n & 1) ? (v & 0xFFFF0000u) : (v << 16));
  }
};

template <>
struct Row<float> {
  float4 w[4];
  __device__ __forceinline__ void load(const void* base, int64_t i) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + i * kN);
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = p[q];
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __device__ __forceinline__ float get(int n) const {
    const float4& q = w[n >> 2];
    return (n & 3) == 0 ? q.x : (n & 3) == 1 ? q.y : (n & 3) == 2 ? q.z : q.w;
  }
};

template <typename InT, bool HAS_RESET>
__global__ __launch_bounds__(kWaves * 64) void scan_wavefront_kernel(const WaveArgs a) {
  // Workgroup -> channels, renumbered so that a batch row's workgroups (which
  // read the same B and C) run on one XCD.
  int idx = blockIdx.x;
  if ((a.nblocks & 7) == 0) idx = (idx & 7) * (a.nblocks >> 3) + (idx >> 3);
  const int64_t row = __builtin_amdgcn_readfirstlane(idx * kWaves + static_cast<int>(threadIdx.x >> 6));
  if (row >= a.B * a.D) return;  // whole waves; the kernel has no barrier
  const int lane = threadIdx.x & 63;
  const int64_t b = row / a.D, d = row - b * a.D;
  const int64_t L = a.L;

  float A2[kN], carry[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n) {
    A2[n] = a.A[d * kN + n] * kLog2e;
    carry[n] = a.h0 ? a.h0[row * kN + n] : 0.0f;
  }
  const float bias = a.dt_bias ? a.dt_bias[d] : 0.0f;
  const float dskip = a.Dskip ? a.Dskip[d] : 0.0f;
  const InT* u_g = static_cast<const InT*>(a.u) + row * L;
  const InT* dt_g = static_cast<const InT*>(a.dt) + row * L;
  const InT* z_g = a.z ? static_cast<const InT*>(a.z) + row * L : nullptr;
  const int64_t bc0 = b * L;  // step index of (b, 0) in Bm, Cm and reset

  // Inputs of one chunk for this lane's step (zeros past L).
  struct In {
    float u, dt, z;
    Row<InT> B, C;
    bool rs;
  };
  auto load = [&](int64_t t0, In& x) {
    const int64_t t = t0 + lane;
    if (t < L) {
      x.u = load_elem(u_g, t);
      x.dt = load_elem(dt_g, t);
      x.z = z_g ? load_elem(z_g, t) : 0.0f;
      x.B.load(a.Bm, bc0 + t);
      x.C.load(a.Cm, bc0 + t);
      x.rs = HAS_RESET && a.reset[bc0 + t] != 0;
    } else {
      x.u = x.dt = x.z = 0.0f;
      x.B.zero();
      x.C.zero();
      x.rs = false;
    }
  };

  In cur, nxt;
  load(0, cur);
  for (int64_t t0 = 0; t0 < L; t0 += kT) {
    if (t0 + kT < L) load(t0 + kT, nxt);
    const bool valid = t0 + lane < L;
    // steps past L are identity pairs: delta = 0 gives a = 1 and b = 0
    const float delta = valid ? softplus_f32(cur.dt + bias) : 0.0f;
    const float du = delta * cur.u;
    float av[kN], bv[kN];
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      const float e = fast_exp2(delta * A2[n]);
      av[n] = HAS_RESET && cur.rs ? 0.0f : e;
      bv[n] = cur.B.get(n) * du;
    }
    // inclusive scan of the pairs over the chunk's 64 lanes: row_shr:1, 2, 4,
    // 8 inside rows of 16 lanes, then row_bcast:15 into rows 1 and 3 and
    // row_bcast:31 into rows 2 and 3
    scan_level8<6>(av, bv);
    scan_level8<0>(av + 8, bv + 8);
    scan_level8<1>(av, bv);
    scan_level8<1>(av + 8, bv + 8);
    scan_level8<2>(av, bv);
    scan_level8<2>(av + 8, bv + 8);
    scan_level8<3>(av, bv);
    scan_level8<3>(av + 8, bv + 8);
    scan_level8<4>(av, bv);
    scan_level8<4>(av + 8, bv + 8);
    scan_level8<5>(av, bv);
    scan_level8<5>(av + 8, bv + 8);
    // carry in, read-out, and the carry out of the chunk (lane 63's state)
    float y = 0.0f;
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      const float h = __builtin_fmaf(av[n], carry[n], bv[n]);
      y = __builtin_fmaf(cur.C.get(n), h, y);
      carry[n] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h), 63));
    }
    if (valid) {
      const float g = z_g ? silu_f32(cur.z) : 1.0f;
      const float o = __builtin_fmaf(dskip, cur.u, y) * g;
      if (a.out_bf16)
        store_elem(static_cast<bf16_t*>(a.out), row * L + t0 + lane, o);
      else
        store_elem(static_cast<float*>(a.out), row * L + t0 + lane, o);
    }
    cur = nxt;
  }
  if (a.h_last && lane < kN) {
    float v = carry[0];
#pragma unroll
    for (int n = 1; n < kN; ++n) v = lane == n ? carry[n] : v;
    a.h_last[row * kN + lane] = v;
  }
}

}  // namespace

hipError_t launch_scan_wavefront(const ScanPlan& pl, hipStream_t stream) {
  WaveArgs a{};
  a.B = pl.B;
  a.D = pl.D;
  a.L = pl.L;
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
  const int64_t blocks = (pl.B * pl.D + kWaves - 1) / kWaves;
  a.nblocks = static_cast<int>(blocks);
  SSM_LOG("launch scan_wavefront_kernel: %s in, reset %d; grid %d x %d threads (one wave per channel, 64-step "
          "chunks)",
          pl.in_bf16 ? "bf16" : "f32", pl.reset != nullptr, a.nblocks, kWaves * 64);
  const bool reset = pl.reset != nullptr;
  const dim3 grid(a.nblocks), block(kWaves * 64);
  if (pl.in_bf16) {
    if (reset)
      hipLaunchKernelGGL((scan_wavefront_kernel<bf16_t, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((scan_wavefront_kernel<bf16_t, false>), grid, block, 0, stream, a);
  } else {
    if (reset)
      hipLaunchKernelGGL((scan_wavefront_kernel<float, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((scan_wavefront_kernel<float, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace ssm
