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
// nearly all of its HBM traffic, so it is laid out for streaming: LR
// consecutive lanes own one (b, d) row and walk its N contiguous states,
// each wave instruction touching 64 consecutive floats. The step-size and gate
// (a handful of transcendentals per row) are recomputed by every lane of the
// row, which is cheaper than broadcasting them; the dot product over n is a
// butterfly of cross-lane adds.
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
};

__device__ __forceinline__ float load_in(const void* p, int64_t i, int bf16) {
  return bf16 ? load_elem(static_cast<const bf16_t*>(p), i) : load_elem(static_cast<const float*>(p), i);
}

template <int LR>
__global__ __launch_bounds__(kThreads) void state_update_kernel(const UpdateArgs a) {
  const int li = threadIdx.x % LR;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kThreads / LR) + threadIdx.x / LR;
  // Rows never straddle a wave (LR divides 64), so a row past the end is
  // inactive as a whole and its lanes take no part in the cross-lane adds.
  if (row >= a.rows) return;
  const int64_t b = row / a.D, d = row % a.D;
  const float uu = load_in(a.u, row, a.in_bf16);
  const float delta = softplus_f32(load_in(a.dt, row, a.in_bf16) + (a.dt_bias ? a.dt_bias[d] : 0.0f));
  const float du = delta * uu;
  float y = 0.0f;
  float* hrow = a.h + row * a.N;
  for (int64_t n = li; n < a.N; n += LR) {
    const float abar = fast_exp2(delta * (a.A[d * a.N + n] * kLog2e));
    const float hn = __builtin_fmaf(abar, hrow[n], load_in(a.Bm, b * a.N + n, a.in_bf16) * du);
    hrow[n] = hn;
    y = __builtin_fmaf(load_in(a.Cm, b * a.N + n, a.in_bf16), hn, y);
  }
#pragma unroll
  for (int off = LR / 2; off >= 1; off >>= 1) y += __shfl_xor(y, off, LR);
  if (li == 0) {
    float o = y + (a.Dskip ? a.Dskip[d] * uu : 0.0f);
    if (a.z) o *= silu_f32(load_in(a.z, row, a.in_bf16));
    if (a.out_bf16)
      store_elem(static_cast<bf16_t*>(a.out), row, o);
    else
      store_elem(static_cast<float*>(a.out), row, o);
  }
}

template <int LR>
hipError_t launch_lr(const UpdateArgs& a, hipStream_t stream) {
  const int64_t rows_per_block = kThreads / LR;
  const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(state_update_kernel<LR>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
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
  if (pl.N <= 16) return launch_lr<16>(a, stream);
  if (pl.N <= 32) return launch_lr<32>(a, stream);
  return launch_lr<64>(a, stream);
}

}  // namespace ssm
