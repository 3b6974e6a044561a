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
// nearly all of its HBM traffic, so the kernel is built to keep many bytes of
// state in flight: LR consecutive lanes own one (b, d) row, each lane holding
// four consecutive states (one 16-byte load and store), and every thread
// handles RPT rows whose loads are all issued before any arithmetic; states
// larger than the L2 are read with nontemporal loads (streamed). The
// step size and gate (a few transcendentals per row) are recomputed by each
// lane of the row, which is cheaper than broadcasting them; the dot product
// over n is a chain of DPP adds that completes in the row's last lane, and row
// indices are split into (b, d) in 32-bit arithmetic (fewer than 2^31 rows).
// Shapes whose N is not a multiple of four take a scalar variant (one state
// per lane per pass).
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

template <typename InT>
__device__ __forceinline__ float4 load4(const InT* p, int64_t i);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p, int64_t i) {
  return *reinterpret_cast<const float4*>(p + i);
}
template <>
__device__ __forceinline__ float4 load4<bf16_t>(const bf16_t* p, int64_t i) {
  const uint2 v = *reinterpret_cast<const uint2*>(p + i);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
}

template <int LR>
__device__ __forceinline__ float row_sum(float y) {
#pragma unroll
  for (int off = LR / 2; off >= 1; off >>= 1) y += __shfl_xor(y, off, LR);
  return y;
}

// Sum over each group of LR consecutive lanes, complete in the group's last
// lane only (DPP adds: row_shr inside 16-lane rows, then row_bcast across
// rows). Other lanes end with partial sums; each add's sources lie inside the
// last lane's own group. Measured on the 64 x 2048 x 128 step with the state
// from HBM: 32.2 -> 31.3 us against the all-lane butterfly of shuffles.
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

// Vector variant: N % 4 == 0, LR = N / 4 lanes per row (a power of two <= 64).
template <typename InT, int LR, int RPT, bool STREAM>
__global__ __launch_bounds__(kThreads) void state_update_vec4(const UpdateArgs a) {
  constexpr int ROWS_PER_PASS = kThreads / LR;
  const int li = threadIdx.x % LR;
  const int64_t first = (static_cast<int64_t>(blockIdx.x) * RPT) * ROWS_PER_PASS + threadIdx.x / LR;
  const InT* u_in = static_cast<const InT*>(a.u);
  const InT* dt_in = static_cast<const InT*>(a.dt);
  const InT* z_in = static_cast<const InT*>(a.z);
  const InT* B_in = static_cast<const InT*>(a.Bm);
  const InT* C_in = static_cast<const InT*>(a.Cm);
  const int n0 = li * 4;

  // Issue every load of this thread's rows first.
  float4 hv[RPT], Av[RPT], Bv[RPT], Cv[RPT];
  float uu[RPT], xx[RPT], zz[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int64_t row = first + static_cast<int64_t>(r) * ROWS_PER_PASS;
    if (row < a.rows) {
      const uint32_t row32 = static_cast<uint32_t>(row), D32 = static_cast<uint32_t>(a.D);
      const int64_t b = row32 / D32, d = row32 - static_cast<uint32_t>(b) * D32;
      hv[r] = load_state4<STREAM>(a.h + row * a.N + n0);
      Av[r] = *reinterpret_cast<const float4*>(a.A + d * a.N + n0);
      Bv[r] = load4(B_in, b * a.N + n0);
      Cv[r] = load4(C_in, b * a.N + n0);
      uu[r] = load_elem(u_in, row);
      xx[r] = load_elem(dt_in, row) + (a.dt_bias ? a.dt_bias[d] : 0.0f);
      zz[r] = z_in ? load_elem(z_in, row) : 0.0f;
    }
  }
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int64_t row = first + static_cast<int64_t>(r) * ROWS_PER_PASS;
    // Rows never straddle a wave (LR divides 64), so a row past the end is
    // inactive as a whole and its lanes take no part in the cross-lane adds.
    if (row >= a.rows) continue;
    const int64_t d = static_cast<uint32_t>(row) % static_cast<uint32_t>(a.D);
    const float delta = softplus_f32(xx[r]);
    const float ui = step_input(a, row, d, uu[r]);
    float4 hn;
    hn.x = update_state(a, delta, Av[r].x, hv[r].x, Bv[r].x, ui);
    hn.y = update_state(a, delta, Av[r].y, hv[r].y, Bv[r].y, ui);
    hn.z = update_state(a, delta, Av[r].z, hv[r].z, Bv[r].z, ui);
    hn.w = update_state(a, delta, Av[r].w, hv[r].w, Bv[r].w, ui);
    *reinterpret_cast<float4*>(a.h + row * a.N + n0) = hn;
    float y = Cv[r].x * hn.x;
    y = __builtin_fmaf(Cv[r].y, hn.y, y);
    y = __builtin_fmaf(Cv[r].z, hn.z, y);
    y = __builtin_fmaf(Cv[r].w, hn.w, y);
    y = group_sum_last<LR>(y);
    if (li == LR - 1) {
      float o = y + (a.Dskip ? a.Dskip[d] * ui : 0.0f);
      if (z_in) o *= silu_f32(zz[r]);
      store_out(a, row, o);
      shift_conv_state(a, row, uu[r]);
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

template <typename InT, int LR>
hipError_t launch_vec(const UpdateArgs& a, hipStream_t stream) {
  constexpr int RPT = 2;
  const int64_t rows_per_block = static_cast<int64_t>(kThreads / LR) * RPT;
  const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  SSM_LOG("launch state_update_vec4<%d lanes per row, %d rows per thread>: %s in, streamed state %d; grid %lld x "
          "%d threads",
          LR, RPT, sizeof(InT) == 2 ? "bf16" : "f32", a.rows * a.N * static_cast<int64_t>(sizeof(float)) > kStreamStateBytes,
          static_cast<long long>(blocks), kThreads);
  if (a.rows * a.N * static_cast<int64_t>(sizeof(float)) > kStreamStateBytes)
    hipLaunchKernelGGL((state_update_vec4<InT, LR, RPT, true>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                       0, stream, a);
  else
    hipLaunchKernelGGL((state_update_vec4<InT, LR, RPT, false>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                       0, stream, a);
  return hipGetLastError();
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
  if (vec_ok) switch (a.N) {
    case 16: return launch_vec<InT, 4>(a, stream);
    case 32: return launch_vec<InT, 8>(a, stream);
    case 64: return launch_vec<InT, 16>(a, stream);
    case 128: return launch_vec<InT, 32>(a, stream);
    case 256: return launch_vec<InT, 64>(a, stream);
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
