// Single-token decode step of the selective SSM for gfx950 (MI355X).
//
// One application of the recurrence to a stored state, in place
// ("Reproducing Mamba's SSM core in Python", section 3: recurrent inference;
// "Mamba SSM core theory and Keras/TensorFlow implementation", the scan step
// state = A_t*state + B_t*u_t, y_t = sum(C_t*state) + D*u_t):
//
//   delta = softplus(dt_raw + dt_bias)
//   h[n]  = exp(delta A[d,n]) h[n] + delta B[n] u,   y = sum_n C[n] h[n] + D u
//   out   = y * silu(z)
//
// The step reads and rewrites the whole (B, D, N) float32 state, which is
// nearly all of its HBM traffic. Per row it also needs A[d, :] (as many bytes
// as the row's state) and B[b, :], C[b, :]; read per row, those cached reads
// doubled the load instructions and cost about a tenth of the step. So a
// thread owns one group of four consecutive states (one 16-byte load and
// store; LR = N / 4 consecutive lanes cover a row) for a tile of RD
// consecutive channels by RB batch rows: its A values serve RB rows, its B
// and C values RD rows, and u, dt_raw, z, dt_bias and D come as runs of RD
// elements. Every load of the tile is issued before any arithmetic; states
// larger than the L2 are read with nontemporal loads (streamed). The step
// size and gate (a few transcendentals per row) are recomputed by each lane
// of the row, which is cheaper than broadcasting them; the dot product over n
// is a chain of DPP adds that completes in the row's last lane. Shapes whose
// N is not a multiple of four take a scalar variant (one state per lane per
// pass).
//
// With a conv stage the step input is silu(conv_b + sum_k conv_w[k] * window[k])
// over the window (conv_state[0 .. K-2], u): the conv state holds the previous
// K-1 inputs, oldest first, and is shifted in place (by the row's last lane,
// after every lane of the row has read it).
#include "device_math.h"
#include "kernels.h"

namespace ssm {
namespace {

constexpr int kThreads = 256;

struct UpdateArgs {
  int64_t B, D, N, rows;
  int in_bf16, out_bf16;
  float* h;
  const void* u;
  const void* dt;
  const void* z;
  const float* dt_bias;
  const float* A;
  const float* Dskip;
  const void* Bm;
  const void* Cm;
  void* out;
  float* conv_state;     // (B, D, conv_k - 1) or null
  const float* conv_w;   // (D, conv_k) or null (no conv stage)
  const float* conv_b;   // (D) or null
  int conv_k;
  int zoh;               // exact zero-order-hold input coefficient
  int dtiles;            // channel tiles per batch-row tile (tiled variant)
};

// One state's update: h <- e^{delta A} h + coef * B * u, coef = delta or the
// exact zero-order hold (e^{delta A} - 1) / A.
__device__ __forceinline__ float update_state(const UpdateArgs& a, float delta, float A, float h, float B, float u) {
  const float abar = fast_exp2(delta * (A * kLog2e));
  if (!a.zoh) return __builtin_fmaf(abar, h, B * (delta * u));
  const float coef = zoh_coef(delta, delta * A, abar, A != 0.0f ? 1.0f / A : 0.0f);
  return __builtin_fmaf(abar, h, B * (u * coef));
}

// The step input of row `row` (channel d) from its raw input x: x itself, or
// the conv + SiLU over (conv state, x).
__device__ __forceinline__ float step_input(const UpdateArgs& a, int64_t row, int64_t d, float x) {
  if (!a.conv_w) return x;
  const int K = a.conv_k;
  const float* st = a.conv_state + row * (K - 1);
  float pre = __builtin_fmaf(a.conv_w[d * K + K - 1], x, a.conv_b ? a.conv_b[d] : 0.0f);
  for (int k = 0; k < K - 1; ++k) pre = __builtin_fmaf(a.conv_w[d * K + k], st[k], pre);
  return silu_f32(pre);
}

// Shift the row's conv state by one input (called by one lane per row, after
// the row's lanes have read the state).
__device__ __forceinline__ void shift_conv_state(const UpdateArgs& a, int64_t row, float x) {
  if (!a.conv_w || a.conv_k < 2) return;
  const int K = a.conv_k;
  float* st = a.conv_state + row * (K - 1);
  for (int k = 0; k < K - 2; ++k) st[k] = st[k + 1];
  st[K - 2] = x;
}

template <int LR>
__device__ __forceinline__ float row_sum(float y) {
#pragma unroll
  for (int off = LR / 2; off >= 1; off >>= 1) y += __shfl_xor(y, off, LR);
  return y;
}

__device__ __forceinline__ void store_out(const UpdateArgs& a, int64_t row, float v) {
  if (a.out_bf16)
    store_elem(static_cast<bf16_t*>(a.out), row, v);
  else
    store_elem(static_cast<float*>(a.out), row, v);
}

// One 16-byte group of states. STREAM: a nontemporal load (the state is
// read once per step and, when larger than the caches, comes from HBM).
template <bool STREAM>
__device__ __forceinline__ float4 load_state4(const float* p) {
  if constexpr (STREAM) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    const v4f t = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
    return make_float4(t.x, t.y, t.z, t.w);
  } else {
    return *reinterpret_cast<const float4*>(p);
  }
}

// Tiled vector variant: N % 4 == 0, LR = N / 4 lanes per row (a power of two
// <= 64), D % RD == 0 and the (B, D) tensors aligned to runs of RD. A
// workgroup covers RB batch rows by kThreads / LR * RD channels; its threads
// are `slots` of LR lanes, slot s holding channels d0 .. d0 + RD - 1. Batch
// rows past the end (a ragged last tile) repeat the last row's loads and skip
// every store, so the loads stay unconditional.
template <typename InT, int LR, int RD, int RB, bool STREAM>
__global__ __launch_bounds__(kThreads) void state_update_tile(const UpdateArgs a) {
  constexpr int SLOTS = kThreads / LR;
  const int li = threadIdx.x % LR;
  const int bt = blockIdx.x / a.dtiles;
  const int d0 = ((blockIdx.x - bt * a.dtiles) * SLOTS + static_cast<int>(threadIdx.x) / LR) * RD;
  // Whole slots only (LR divides 64, so a slot never straddles a wave): an
  // inactive slot takes no part in the other slots' cross-lane adds.
  if (d0 >= a.D) return;
  const int D = static_cast<int>(a.D), N = static_cast<int>(a.N);
  const int b0 = bt * RB;
  const int nb = min(RB, static_cast<int>(a.B) - b0);
  const int n0 = li * 4;
  using RunIn = Run<InT, RD>;
  using Run4 = Run<InT, 4>;
  using RunF = Run<float, RD>;
  const InT* u_in = static_cast<const InT*>(a.u);
  const InT* dt_in = static_cast<const InT*>(a.dt);
  const InT* z_in = static_cast<const InT*>(a.z);

  // Issue every load of the tile first, the state (from HBM) ahead of the rest.
  int bj[RB];        // batch row j of the tile (the last row repeated past the end)
  int64_t rowj[RB];  // its (b, d0) row index
  float4 hv[RB][RD];
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    bj[j] = min(b0 + j, static_cast<int>(a.B) - 1);
    rowj[j] = static_cast<int64_t>(bj[j]) * D + d0;
#pragma unroll
    for (int i = 0; i < RD; ++i) hv[j][i] = load_state4<STREAM>(a.h + (rowj[j] + i) * N + n0);
  }
  float4 Av[RD];
#pragma unroll
  for (int i = 0; i < RD; ++i) Av[i] = *reinterpret_cast<const float4*>(a.A + static_cast<int64_t>(d0 + i) * N + n0);
  typename Run4::raw Bv[RB], Cv[RB];
  typename RunIn::raw uv[RB], xv[RB], zv[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int64_t bn = static_cast<int64_t>(bj[j]) * N + n0;
    Bv[j] = Run4::load(static_cast<const InT*>(a.Bm) + bn);
    Cv[j] = Run4::load(static_cast<const InT*>(a.Cm) + bn);
    uv[j] = RunIn::load(u_in + rowj[j]);
    xv[j] = RunIn::load(dt_in + rowj[j]);
    zv[j] = z_in ? RunIn::load(z_in + rowj[j]) : typename RunIn::raw{};
  }
  const typename RunF::raw biasv = a.dt_bias ? RunF::load(a.dt_bias + d0) : typename RunF::raw{};
  const typename RunF::raw dskv = a.Dskip ? RunF::load(a.Dskip + d0) : typename RunF::raw{};

#pragma unroll
  for (int j = 0; j < RB; ++j) {
    float Bf[4], Cf[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      Bf[k] = Run4::at(Bv[j], k);
      Cf[k] = Run4::at(Cv[j], k);
    }
    float o[RD];
#pragma unroll
    for (int i = 0; i < RD; ++i) {
      const int64_t row = rowj[j] + i;
      const float delta = softplus_f32(RunIn::at(xv[j], i) + RunF::at(biasv, i));
      const float ui = step_input(a, row, d0 + i, RunIn::at(uv[j], i));
      float4 hn;
      hn.x = update_state(a, delta, Av[i].x, hv[j][i].x, Bf[0], ui);
      hn.y = update_state(a, delta, Av[i].y, hv[j][i].y, Bf[1], ui);
      hn.z = update_state(a, delta, Av[i].z, hv[j][i].z, Bf[2], ui);
      hn.w = update_state(a, delta, Av[i].w, hv[j][i].w, Bf[3], ui);
      if (j < nb) *reinterpret_cast<float4*>(a.h + row * N + n0) = hn;
      float y = Cf[0] * hn.x;
      y = __builtin_fmaf(Cf[1], hn.y, y);
      y = __builtin_fmaf(Cf[2], hn.z, y);
      y = __builtin_fmaf(Cf[3], hn.w, y);
      y = group_sum_last<LR>(y);
      if (a.Dskip) y += RunF::at(dskv, i) * ui;
      o[i] = z_in ? y * silu_f32(RunIn::at(zv[j], i)) : y;
    }
    if (li == LR - 1 && j < nb) {
      if (a.out_bf16)
        store_run<RD>(static_cast<bf16_t*>(a.out) + rowj[j], o);
      else
        store_run<RD>(static_cast<float*>(a.out) + rowj[j], o);
#pragma unroll
      for (int i = 0; i < RD; ++i) shift_conv_state(a, rowj[j] + i, RunIn::at(uv[j], i));
    }
  }
}

// Scalar variant for any N: LR lanes per row, states n = li, li + LR, ...
template <typename InT, int LR>
__global__ __launch_bounds__(kThreads) void state_update_scalar(const UpdateArgs a) {
  const int li = threadIdx.x % LR;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kThreads / LR) + threadIdx.x / LR;
  if (row >= a.rows) return;  // whole rows only (LR divides 64)
  const InT* B_in = static_cast<const InT*>(a.Bm);
  const InT* C_in = static_cast<const InT*>(a.Cm);
  const int64_t b = row / a.D, d = row % a.D;
  const float ux = load_elem(static_cast<const InT*>(a.u), row);
  const float uu = step_input(a, row, d, ux);
  const float delta =
      softplus_f32(load_elem(static_cast<const InT*>(a.dt), row) + (a.dt_bias ? a.dt_bias[d] : 0.0f));
  float y = 0.0f;
  float* hrow = a.h + row * a.N;
  for (int64_t n = li; n < a.N; n += LR) {
    const float hn = update_state(a, delta, a.A[d * a.N + n], hrow[n], load_elem(B_in, b * a.N + n), uu);
    hrow[n] = hn;
    y = __builtin_fmaf(load_elem(C_in, b * a.N + n), hn, y);
  }
  y = row_sum<LR>(y);
  if (li == 0) {
    float o = y + (a.Dskip ? a.Dskip[d] * uu : 0.0f);
    if (a.z) o *= silu_f32(load_elem(static_cast<const InT*>(a.z), row));
    store_out(a, row, o);
    shift_conv_state(a, row, ux);
  }
}

// States larger than this are streamed (nontemporal loads): measured at
// 64 x 2048 x 128 (67 MB), a step whose state comes from HBM takes 33.8 us
// streamed against 38 us cached, while a step repeated on a state that stays
// in the last-level cache takes 32.5 us against 28.6 us. A state larger than
// the L2 (4 MB per XCD) does not stay in it across the layers of a model.
constexpr int64_t kStreamStateBytes = int64_t{32} << 20;

template <typename InT, int LR, int RD, int RB>
hipError_t launch_tile(UpdateArgs a, hipStream_t stream) {
  constexpr int kChannels = kThreads / LR * RD;  // channels per workgroup
  a.dtiles = static_cast<int>((a.D + kChannels - 1) / kChannels);
  const int64_t blocks = a.dtiles * ((a.B + RB - 1) / RB);
  const bool stream_state = a.rows * a.N * static_cast<int64_t>(sizeof(float)) > kStreamStateBytes;
  SSM_LOG("launch state_update_tile<%d lanes per row, %d channels x %d batch rows per thread>: %s in, streamed "
          "state %d; grid %lld x %d threads",
          LR, RD, RB, sizeof(InT) == 2 ? "bf16" : "f32", stream_state, static_cast<long long>(blocks), kThreads);
  if (stream_state)
    hipLaunchKernelGGL((state_update_tile<InT, LR, RD, RB, true>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((state_update_tile<InT, LR, RD, RB, false>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

// Tile of a thread (channels x batch rows). Measured cold (state from HBM)
// at 64 x 2048 x 128, bf16 inputs, against 31.0 us for two rows per thread
// without reuse and 25.5 us for torch's in-place add on a float32 tensor of
// the state's size: 2 x 2 26.9 us, 2 x 1 27.3, 4 x 1 27.7, 2 x 3 28.2,
// 4 x 2 27.9, 4 x 4 32.4 (197 registers, two waves per SIMD), 1 x 2 34.8,
// 1 x 1 40.8. Channel runs matter more than batch rows: with RD = 1, u,
// dt_raw and z are three 2-byte loads per row. `runs2`: the shape allows
// channel runs of two.
template <typename InT, int LR>
hipError_t launch_lr(const UpdateArgs& a, bool runs2, hipStream_t stream) {
  if (runs2) return a.B >= 2 ? launch_tile<InT, LR, 2, 2>(a, stream) : launch_tile<InT, LR, 2, 1>(a, stream);
  return launch_tile<InT, LR, 1, 2>(a, stream);
}

template <typename InT, int LR>
hipError_t launch_scalar(const UpdateArgs& a, hipStream_t stream) {
  const int64_t rows_per_block = kThreads / LR;
  const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  SSM_LOG("launch state_update_scalar<%d lanes per row>: %s in; grid %lld x %d threads", LR,
          sizeof(InT) == 2 ? "bf16" : "f32", static_cast<long long>(blocks), kThreads);
  hipLaunchKernelGGL((state_update_scalar<InT, LR>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

bool aligned_to(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

template <typename InT>
hipError_t launch_dtype(const UpdateArgs& a, hipStream_t stream) {
  // 16-byte state rows need N % 4 == 0, a power-of-two lane count N / 4,
  // base pointers aligned to a 4-state group and fewer than 2^31 rows.
  const bool vec_ok = aligned_to(a.h, 16) && aligned_to(a.A, 16) && aligned_to(a.Bm, 4 * sizeof(InT)) &&
                      aligned_to(a.Cm, 4 * sizeof(InT)) && a.rows < (int64_t{1} << 31);
  // Channel runs of rd elements need D % rd == 0 and the (B, D) and (D)
  // tensors aligned to a run.
  const auto runs_ok = [&](int rd) {
    return a.D % rd == 0 && aligned_to(a.u, rd * sizeof(InT)) && aligned_to(a.dt, rd * sizeof(InT)) &&
           (!a.z || aligned_to(a.z, rd * sizeof(InT))) && aligned_to(a.out, rd * (a.out_bf16 ? 2 : 4)) &&
           (!a.dt_bias || aligned_to(a.dt_bias, rd * 4)) && (!a.Dskip || aligned_to(a.Dskip, rd * 4));
  };
  const bool runs2 = runs_ok(2);
  if (vec_ok) switch (a.N) {
    case 16: return launch_lr<InT, 4>(a, runs2, stream);
    case 32: return launch_lr<InT, 8>(a, runs2, stream);
    case 64: return launch_lr<InT, 16>(a, runs2, stream);
    case 128: return launch_lr<InT, 32>(a, runs2, stream);
    case 256: return launch_lr<InT, 64>(a, runs2, stream);
    default: break;
  }
  if (a.N <= 16) return launch_scalar<InT, 16>(a, stream);
  if (a.N <= 32) return launch_scalar<InT, 32>(a, stream);
  return launch_scalar<InT, 64>(a, stream);
}

}  // namespace

hipError_t launch_state_update(const UpdatePlan& pl, hipStream_t stream) {
  UpdateArgs a{};
  a.B = pl.B;
  a.D = pl.D;
  a.N = pl.N;
  a.rows = pl.B * pl.D;
  a.in_bf16 = pl.in_bf16;
  a.out_bf16 = pl.out_bf16;
  a.h = pl.h;
  a.u = pl.u;
  a.dt = pl.dt;
  a.z = pl.z;
  a.dt_bias = pl.dt_bias;
  a.A = pl.A;
  a.Dskip = pl.Dskip;
  a.Bm = pl.Bm;
  a.Cm = pl.Cm;
  a.out = pl.out;
  a.conv_state = pl.conv_state;
  a.conv_w = pl.conv_w;
  a.conv_b = pl.conv_b;
  a.conv_k = pl.conv_k;
  a.zoh = pl.zoh;
  return pl.in_bf16 ? launch_dtype<bf16_t>(a, stream) : launch_dtype<float>(a, stream);
}

}  // namespace ssm
