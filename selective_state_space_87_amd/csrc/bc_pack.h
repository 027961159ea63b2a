// B/C pre-pass shared by the scan's forward and backward kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_math.h"

namespace ssm {

// B, C [Bt, L, N] -> one 32-bit word per (b, n, t), time-contiguous, zero
// beyond N and L:
//  * bfloat16 inputs: word = (B bits << 16) | C bits (exact);
//  * float32 inputs: two words (B, C) per step, i.e. a float2 per step.
// A wave owning state n then fetches a whole tile of its B and C with one or
// two scalar loads.
template <bool BF16_IN>
static __global__ __launch_bounds__(256) void bc_pack_kernel(const void* __restrict__ Bin,
                                                      const void* __restrict__ Cin,
                                                      uint32_t* __restrict__ out, int64_t L,
                                                      int64_t Lp, int N, int NS) {
  __shared__ uint32_t sb[64][65];
  __shared__ uint32_t sc[64][65];
  const int64_t b = blockIdx.y;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 64;
  for (int i = threadIdx.x; i < 64 * NS; i += 256) {
    const int tt = i / NS, n = i % NS;
    const int64_t t = t0 + tt;
    const bool ok = t < L && n < N;
    sb[tt][n] = ok ? load_bits<BF16_IN>(Bin, (b * L + t) * N + n) : 0u;
    sc[tt][n] = ok ? load_bits<BF16_IN>(Cin, (b * L + t) * N + n) : 0u;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * NS; i += 256) {
    const int n = i / 64, tt = i % 64;
    const int64_t t = t0 + tt;
    if (t < Lp) {
      const int64_t o = (b * NS + n) * Lp + t;
      if constexpr (BF16_IN) {
        out[o] = (sb[tt][n] << 16) | sc[tt][n];
      } else {
        out[2 * o] = sb[tt][n];
        out[2 * o + 1] = sc[tt][n];
      }
    }
  }
}

// Enqueue the pre-pass for batch rows of length L (padded to Lp) into out.
static inline int launch_bc_pack(const void* B, const void* C, uint32_t* out, int64_t batch, int64_t L,
                                 int64_t Lp, int N, int NS, bool in_bf16, hipStream_t st) {
  if (Lp <= 0) return 0;
  const int64_t chunks = (Lp + 63) / 64;
  if (chunks > 0x7fffffff || batch > 65535) return hipErrorInvalidConfiguration;
  void* kargs[] = {&B, &C, &out, &L, &Lp, &N, &NS};
  const void* fn = in_bf16 ? reinterpret_cast<const void*>(&bc_pack_kernel<true>)
                           : reinterpret_cast<const void*>(&bc_pack_kernel<false>);
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(chunks), static_cast<unsigned>(batch)), dim3(256),
                         kargs, 0, st);
}

}  // namespace ssm
