// Host-side interface between the C-ABI front end (api.cpp) and the HIP
// kernels (scan_fwd.hip, scan_bwd.hip, scan_cplx.hip, scan_cplx_bwd.hip, state_update.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "log.h"

namespace ssm {

// One scan launch after validation. Pointers are device pointers; optional
// ones are nullptr. `ws` holds the per-segment aggregates when nseg > 1.
struct ScanPlan {
  int64_t B, D, L, N;
  int in_bf16, out_bf16;
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
  float* ws;
  int nseg;         // pieces L is split into (1 = no split)
  int64_t seg_len;  // steps per piece (the last may be shorter)
  // Backward forward-sweep (checkpoint != 0): instead of `out`, write the state
  // entering every 16-step chunk to ckpt (B, n_ck, D, N) and each backward
  // segment's adjoint aggregate to seg_P / seg_G (B, nsegb, D, N). seg_len is
  // then a multiple of seg_steps.
  int checkpoint;
  const void* dout;
  float* ckpt;
  float* seg_P;
  float* seg_G;
  int64_t seg_steps;
  int64_t n_ck;
  int nsegb;
  // Causal depthwise conv1d + SiLU applied to u before the scan (conv_w null: none).
  const float* conv_w;         // (D, conv_k)
  const float* conv_b;         // (D) or null
  const float* conv_state_in;  // (B, D, conv_k - 1) or null
  float* conv_state_out;       // (B, D, conv_k - 1) or null
  int conv_k;
  float* uconv_out;            // checkpoint sweep with conv: writes the scan input u' (B, D, L)
  int zoh;                     // 1: exact zero-order-hold Bbar; 0: delta * B
};

struct UpdatePlan {
  int64_t B, D, N;
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
  float* conv_state;    // (B, D, conv_k - 1), updated in place; null without conv
  const float* conv_w;  // (D, conv_k) or null
  const float* conv_b;  // (D) or null
  int conv_k;
  int zoh;              // 1: exact zero-order-hold Bbar; 0: delta * B
};

// Largest supported state size.
constexpr int kMaxState = 256;

// How many pieces the sequence is split into (requested = 0: automatic) and
// the resulting piece length. `plain`: the pass that follows is the plain
// full pass (no conv stage, delta B coefficient) or the aggregate pass, which
// keep more waves resident than the other variants. `min_steps`: the shortest
// automatic piece. Pure host arithmetic.
void plan_segments(int64_t B, int64_t D, int64_t L, int64_t N, int requested, int* nseg,
                   int64_t* seg_len, bool plain = false, int64_t min_steps = 256);

// Workspace bytes for `nseg` pieces: the affine aggregate (decay product and
// end state) of every piece but the last, per (b, d, n), in float32.
size_t scan_workspace_bytes(int64_t B, int64_t D, int64_t N, int nseg);

// Number of workgroups the scan launches use (for grid-limit checks).
int64_t scan_grid_blocks(int64_t B, int64_t D, int64_t N, int nseg);

hipError_t launch_scan(const ScanPlan& plan, hipStream_t stream);
// The forward as a chunked associative scan (scan_fwd_wavefront.hip): N = 16,
// real states, delta B, no conv stage, one piece.
hipError_t launch_scan_wavefront(const ScanPlan& plan, hipStream_t stream);
// Affine aggregate of the whole sequence into P and H (B, D, N): the pieces'
// aggregates (in `ws`, nseg of each when nseg > 1) folded in order.
hipError_t launch_aggregate(const ScanPlan& plan, float* P, float* H, hipStream_t stream);
hipError_t launch_state_update(const UpdatePlan& plan, hipStream_t stream);

// Complex diagonal state (scan_cplx.hip): A, B, C and the states hold
// interleaved (re, im) pairs; `ws` holds the complex per-piece aggregates when
// nseg > 1 (P then H, each (nseg - 1, B, D, N, 2)); the conv, zero-order-hold
// and checkpoint fields are unused.
void plan_cplx_segments(int64_t B, int64_t D, int64_t L, int64_t N, int requested, int* nseg, int64_t* seg_len);
size_t cplx_workspace_bytes(int64_t B, int64_t D, int64_t N, int nseg);
int64_t cplx_scan_grid_blocks(int64_t B, int64_t D, int nseg);
// aggregates_only: just the piece aggregates of a split scan (nothing when nseg == 1).
hipError_t launch_scan_cplx(const ScanPlan& plan, hipStream_t stream, bool aggregates_only = false);
hipError_t launch_state_update_cplx(const UpdatePlan& plan, hipStream_t stream);
hipError_t launch_aggregate_cplx(const ScanPlan& plan, float* P, float* H, hipStream_t stream);

// Backward pass (scan_bwd.hip). The checkpoint sweep runs through launch_scan
// with ScanPlan::checkpoint set; BwdPlan describes the reverse sweep and the
// final reduction.
struct BwdPlan {
  int64_t B, D, L, N;
  int in_bf16, grad_bf16;
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
  const float* ckpt;   // from the checkpoint sweep
  const float* seg_P;
  const float* seg_G;
  void* du;
  void* ddt;
  void* dz;
  float* dA;
  float* dB;
  float* dC;
  float* dD;
  float* dbias;
  float* dh0;
  float* part;  // partial sums, bwd_partial_floats() floats
  int64_t seg_steps;
  int64_t n_ck;
  int nsegb;
  // Conv stage (conv_w null: none). The reverse sweep then reads the scan
  // input u' from uconv and writes its gradient to du_conv; a conv backward
  // turns that into du (the conv input's gradient), dconv_w, dconv_b and
  // dconv_state.
  const float* conv_w;
  const float* conv_b;
  const float* conv_state_in;
  int conv_k;
  const float* uconv;
  float* du_conv;
  float* conv_part;  // bwd_conv_partial_floats() floats
  float* dconv_w;
  float* dconv_b;
  float* dconv_state;
  int zoh;  // 1: exact zero-order-hold Bbar; 0: delta * B
};

// Backward segments: how many pieces the reverse sweep splits L into and
// their length (a multiple of 16). Pure host arithmetic.
void plan_bwd_segments(int64_t B, int64_t D, int64_t L, int64_t N, bool zoh, int* nsegb, int64_t* seg_steps);
// Channels one reverse-sweep workgroup covers.
int bwd_channels_per_block(int64_t N);
// Floats of partial sums the reverse sweep writes and the reduction reads.
size_t bwd_partial_floats(int64_t B, int64_t D, int64_t L, int64_t N, int nsegb);
// Workgroups of the reverse sweep.
int64_t bwd_grid_blocks(int64_t B, int64_t D, int64_t N, int nsegb);
// Floats of partial sums of the conv backward (per row tile: 4 taps + bias).
size_t bwd_conv_partial_floats(int64_t B, int64_t D, int64_t L);
hipError_t launch_scan_bwd(const BwdPlan& plan, hipStream_t stream);
// The conv stage's backward: du_conv (the gradient of the scan input u') to
// du, dconv_w, dconv_b and dconv_state (launched by launch_scan_bwd itself).
hipError_t launch_conv_bwd(const BwdPlan& plan, hipStream_t stream);
// Sums of the backward's partials in a fixed order: dB and dC (bln floats
// each) over `groups` channel groups, dA (dn floats), dD and d dt_bias (D
// floats, null: skipped) over `bs` batch-row segments.
hipError_t launch_bwd_reduce(const float* partB, const float* partC, const float* partA, const float* partD,
                             const float* partBias, float* dB, float* dC, float* dA, float* dD, float* dbias,
                             int64_t bln, int64_t dn, int64_t D, int64_t groups, int64_t bs, hipStream_t stream);

// Backward of the complex-state scan (scan_cplx_bwd.hip): the checkpoint
// sweep writes the state entering every 16 / NPL steps (NPL = states per lane,
// 1 for N <= 16 up to 16 for N = 256) to ckpt (B, n_ck, D, N, 2) and the
// segments' adjoint aggregates to seg_P / seg_G (B, nsegb, D, N, 2); the
// forward pieces come from `sp` (nseg, seg_len, ws), the reverse sweep and
// reduction from `bp` (part: cplx_bwd_partial_floats floats).
void plan_cplx_bwd(int64_t B, int64_t D, int64_t L, int64_t N, int* nsegb, int64_t* seg_steps, int* nseg,
                   int64_t* seg_len, int64_t* n_ck);
size_t cplx_bwd_partial_floats(int64_t B, int64_t D, int64_t L, int64_t N, int nsegb);
int64_t cplx_bwd_grid_blocks(int64_t B, int64_t D, int nsegb);
hipError_t launch_scan_cplx_bwd(const ScanPlan& sp, const BwdPlan& bp, hipStream_t stream);

// Scratch of the allocation-free forward (scan_noalloc.hip): its size, and its
// address on the current device (looked up on the first call per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** ptr);

// Outputs of empty problems: dst[i] = src[i] (src given) or v0 / v1 at even /
// odd i, for n floats (nothing for dst = null or n = 0).
hipError_t launch_fill(float* dst, const float* src, float v0, float v1, int64_t n, hipStream_t stream);

}  // namespace ssm
