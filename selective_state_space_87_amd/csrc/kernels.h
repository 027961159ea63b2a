// Internal interface between the C-ABI front end (api.cpp) and the kernel
// launchers (*.hip). Host-only types; nothing here crosses the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace ssm {

struct ScanArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* delta_bias;
  const float* h0;
  void* y;
  float* h_final;
  void* workspace;
  int64_t batch, seqlen, dim, dstate;
  int in_bf16, out_bf16, delta_softplus;
};

struct UpdateArgs {
  float* state;
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* delta_bias;
  void* y;
  int64_t batch, dim, dstate;
  int in_bf16, out_bf16, delta_softplus;
};

// Workspace bytes the scan needs for this shape (0: single pass).
size_t scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

// Enqueue the scan / decode kernels on `stream`. Arguments are already
// validated. Return 0 or the HIP error code of the failing launch.
int launch_scan(const ScanArgs& a, void* stream);
int launch_state_update(const UpdateArgs& a, void* stream);

}  // namespace ssm
