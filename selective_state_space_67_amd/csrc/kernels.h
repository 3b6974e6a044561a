// Host-side interface between the C-ABI front end (api.cpp) and the HIP
// kernels (scan_fwd.hip, state_update.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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
};

// Largest supported state size.
constexpr int kMaxState = 256;

// How many pieces the sequence is split into (requested = 0: automatic) and
// the resulting piece length. Pure host arithmetic.
void plan_segments(int64_t B, int64_t D, int64_t L, int64_t N, int requested, int* nseg,
                   int64_t* seg_len);

// Workspace bytes for `nseg` pieces: the affine aggregate (decay product and
// end state) of every piece but the last, per (b, d, n), in float32.
size_t scan_workspace_bytes(int64_t B, int64_t D, int64_t N, int nseg);

// Number of workgroups the scan launches use (for grid-limit checks).
int64_t scan_grid_blocks(int64_t B, int64_t D, int64_t N, int nseg);

hipError_t launch_scan(const ScanPlan& plan, hipStream_t stream);
hipError_t launch_state_update(const UpdatePlan& plan, hipStream_t stream);

}  // namespace ssm
