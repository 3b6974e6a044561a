// Host side of the selective-scan forward: sequence splitting, workspace
// sizes and the launch of the kernels in scan_fwd_kernel.h (instantiated in
// scan_fwd_{f32,bf16}_{plain,reset}.hip).
#include "scan_fwd_kernel.h"

namespace ssm {
using fwd::channels_per_block;
using fwd::resident_blocks;

void plan_segments(int64_t B, int64_t D, int64_t L, int64_t N, int requested, int* nseg,
                   int64_t* seg_len, bool plain, int64_t min_steps) {
  int64_t want;
  if (requested > 0) {
    want = requested;
  } else {
    // Split the sequence only when the channels alone fill less than half of
    // one resident round of workgroups (the aggregate pass costs about half a
    // full pass over the data it covers); then aim for exactly one round, with
    // pieces long enough (>= min_steps) that per-piece overheads stay small:
    // 256 steps for a scan (with 512, short sequences on few channels stayed
    // below a round: 1 x 256 x 16384 took 59.8 us in 32 pieces, 51.3 us in
    // 64), 512 for the aggregate entry point, whose passes do less work per
    // step (the same shape: 32 us in 32 pieces, 37 us in 64).
    const int cpw = channels_per_block(N);
    const int64_t blocks = B * ((D + cpw - 1) / cpw);
    const int64_t round = resident_blocks(N, plain);
    want = 2 * blocks >= round ? 1 : round / blocks;
    want = std::min<int64_t>(want, std::max<int64_t>(1, L / min_steps));
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

int64_t scan_grid_blocks(int64_t B, int64_t D, int64_t N, int nseg) {
  const int cpw = channels_per_block(N);
  return static_cast<int64_t>(nseg) * B * ((D + cpw - 1) / cpw);
}

namespace {

fwd::ScanArgs scan_args(const ScanPlan& pl) {
  fwd::ScanArgs a{};
  a.B = pl.B;
  a.D = pl.D;
  a.L = pl.L;
  a.N = pl.N;
  a.seg_len = pl.seg_len;
  a.nseg = pl.nseg;
  const int cpw = channels_per_block(pl.N);
  a.n_dgroups = static_cast<int>((pl.D + cpw - 1) / cpw);
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
  a.dout = pl.dout;
  a.ckpt = pl.ckpt;
  a.seg_P = pl.seg_P;
  a.seg_G = pl.seg_G;
  a.seg_steps = pl.seg_steps;
  a.n_ck = pl.n_ck;
  a.nsegb = pl.nsegb;
  a.conv_w = pl.conv_w;
  a.conv_b = pl.conv_b;
  a.conv_state_in = pl.conv_state_in;
  a.conv_state_out = pl.conv_state_out;
  a.conv_k = pl.conv_k;
  a.uconv_out = pl.uconv_out;
  a.zoh = pl.zoh;
  return a;
}

hipError_t launch(const ScanPlan& pl, const fwd::ScanArgs& a, int nf, int na, bool ck, hipStream_t stream) {
  const bool reset = pl.reset != nullptr;
  if (pl.in_bf16)
    return reset ? fwd::launch_variant<bf16_t, true>(a, nf, na, ck, stream)
                 : fwd::launch_variant<bf16_t, false>(a, nf, na, ck, stream);
  return reset ? fwd::launch_variant<float, true>(a, nf, na, ck, stream)
               : fwd::launch_variant<float, false>(a, nf, na, ck, stream);
}

// Folds the pieces' aggregates in order: P = prod_s P_s, H <- P_s H + H_s.
__global__ __launch_bounds__(256) void aggregate_fold_kernel(const float* wsP, const float* wsH, int nseg,
                                                             int64_t count, float* P, float* H) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= count) return;
  float p = 1.0f, h = 0.0f;
  for (int s = 0; s < nseg; ++s) {
    const float ps = wsP[s * count + i];
    h = __builtin_fmaf(ps, h, wsH[s * count + i]);
    p *= ps;
  }
  P[i] = p;
  H[i] = h;
}

}  // namespace

hipError_t launch_scan(const ScanPlan& pl, hipStream_t stream) {
  fwd::ScanArgs a = scan_args(pl);
  const size_t per = static_cast<size_t>(pl.nseg > 1 ? pl.nseg - 1 : 0) * pl.B * pl.D * pl.N;
  a.ws_P = pl.ws;
  a.ws_H = pl.ws ? pl.ws + per : nullptr;
  const int per_piece = static_cast<int>(pl.B) * a.n_dgroups;
  if (fwd::n16_eligible(a, pl.checkpoint != 0)) return fwd::launch_n16(a, per_piece * pl.nseg, per_piece * (pl.nseg - 1), stream);
  return launch(pl, a, per_piece * pl.nseg, per_piece * (pl.nseg - 1), pl.checkpoint != 0, stream);
}

hipError_t launch_aggregate(const ScanPlan& pl, float* P, float* H, hipStream_t stream) {
  fwd::ScanArgs a = scan_args(pl);
  const int64_t count = pl.B * pl.D * pl.N;
  a.ws_P = pl.nseg > 1 ? pl.ws : P;
  a.ws_H = pl.nseg > 1 ? pl.ws + static_cast<size_t>(pl.nseg) * count : H;
  const int per_piece = static_cast<int>(pl.B) * a.n_dgroups;
  hipError_t e = launch(pl, a, 0, per_piece * pl.nseg, false, stream);
  if (e != hipSuccess || pl.nseg == 1) return e;
  SSM_LOG("launch aggregate_fold_kernel: %lld states, %d pieces; grid %lld x 256 threads",
          static_cast<long long>(count), pl.nseg, static_cast<long long>((count + 255) / 256));
  hipLaunchKernelGGL(aggregate_fold_kernel, dim3(static_cast<unsigned>((count + 255) / 256)), dim3(256), 0, stream,
                     a.ws_P, a.ws_H, pl.nseg, count, P, H);
  return hipGetLastError();
}

}  // namespace ssm
