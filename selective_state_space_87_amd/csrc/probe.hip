// Rate probes behind the benchmark's VALU roofline (declared in ssm_probe.h).
//
// The scan's recurrence costs, per state update, two multiplies, one
// v_exp_f32 and two FMAs (the e^(dt A) transition, the dt B u input term, the
// state update and the C h readout of "从 Transformer 到 Mamba", ybb.press,
// section 3.1). Whether the exponential issues at the FMA rate, at half of it,
// or co-issues beside FMAs decides the roofline; these kernels measure it on
// the device, with registers only.
#include <hip/hip_runtime.h>

#include "ssm_probe.h"

namespace {

constexpr int kChains = 8;

// Keeps a value opaque to the optimiser (no instruction is emitted), so that
// loop-invariant work stays inside the loop.
__device__ __forceinline__ void opaque(float& v) { asm volatile("" : "+v"(v)); }

__global__ __launch_bounds__(256) void exp_kernel(float* out, float seed, int iters) {
  float x[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) x[i] = seed * (threadIdx.x + i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int i = 0; i < kChains; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void fma_kernel(float* out, float seed, float a, float b, int iters) {
  float x[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) x[i] = seed * (threadIdx.x + i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int i = 0; i < kChains; ++i) x[i] = __builtin_fmaf(x[i], a, b);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The scan's tile: two states per lane, eight steps; the step values (dt, dt
// u) in registers, the per-state constants (A log2 e, B, C) as scalar
// operands, as in the scan kernel.
template <int WG>
__global__ __launch_bounds__(WG) void mix_kernel(float* out, float seed, float a0, float a1, float b0, float b1,
                                                 float c0, float c1, int iters) {
  extern __shared__ float pad[];  // sized by the launch to fix the blocks per CU
  float dt[8], du[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    dt[j] = seed * (threadIdx.x + j);
    du[j] = seed * (threadIdx.x - j);
  }
  float h0 = seed, h1 = -seed, acc = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      opaque(dt[j]);
      opaque(du[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e0 = __builtin_amdgcn_exp2f(dt[j] * a0);
      const float e1 = __builtin_amdgcn_exp2f(dt[j] * a1);
      h0 = __builtin_fmaf(e0, h0, du[j] * b0);
      h1 = __builtin_fmaf(e1, h1, du[j] * b1);
      acc = __builtin_fmaf(c0, h0, acc);
      acc = __builtin_fmaf(c1, h1, acc);
    }
  }
  if (threadIdx.x == WG + 1) pad[0] = acc;  // never true: keeps the LDS allocation
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc + h0 + h1;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                   long n) {
  const long stride = static_cast<long>(gridDim.x) * blockDim.x;
  for (long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
  }
}

// Median of `reps` timed launches of `launch` (after one untimed launch), in seconds.
template <typename F>
hipError_t time_launches(F launch, int reps, double* seconds) {
  hipEvent_t e0, e1;
  hipError_t err = hipEventCreate(&e0);
  if (err != hipSuccess) return err;
  err = hipEventCreate(&e1);
  if (err != hipSuccess) {
    (void)hipEventDestroy(e0);
    return err;
  }
  float ms[16];
  if (reps > 16) reps = 16;
  launch();
  for (int r = 0; r < reps && err == hipSuccess; ++r) {
    err = hipEventRecord(e0, nullptr);
    launch();
    if (err == hipSuccess) err = hipEventRecord(e1, nullptr);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms[r], e0, e1);
  }
  if (err == hipSuccess) err = hipGetLastError();
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (err != hipSuccess) return err;
  for (int i = 1; i < reps; ++i) {  // insertion sort: a handful of values
    const float v = ms[i];
    int j = i - 1;
    while (j >= 0 && ms[j] > v) {
      ms[j + 1] = ms[j];
      --j;
    }
    ms[j + 1] = v;
  }
  *seconds = ms[reps / 2] * 1e-3;
  return hipSuccess;
}

}  // namespace

extern "C" int ssm_probe_valu(ssm_probe_rates_t* out) {
  if (out == nullptr) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  hipDeviceProp_t prop;
  err = hipGetDeviceProperties(&prop, dev);
  if (err != hipSuccess) return err;
  const int cus = prop.multiProcessorCount;
  out->cus = cus;
  out->clock_khz = prop.clockRate;

  // Eight waves per SIMD: 8 blocks of 4 waves per CU.
  const int blocks = cus * 8, threads = 256;
  const long nthreads = static_cast<long>(blocks) * threads;
  float* buf = nullptr;
  err = hipMalloc(&buf, nthreads * sizeof(float));
  if (err != hipSuccess) return err;
  double t = 0.0;

  const int exp_iters = 3000;
  err = time_launches([&] { hipLaunchKernelGGL(exp_kernel, dim3(blocks), dim3(threads), 0, nullptr, buf, 1e-3f,
                                               exp_iters); }, 5, &t);
  if (err == hipSuccess) out->exp_lanes_per_s = double(nthreads) * exp_iters * 4 * kChains / t;

  const int fma_iters = 6000;
  if (err == hipSuccess)
    err = time_launches([&] { hipLaunchKernelGGL(fma_kernel, dim3(blocks), dim3(threads), 0, nullptr, buf, 1e-3f,
                                                 0.999f, 1e-4f, fma_iters); }, 5, &t);
  if (err == hipSuccess) out->fma_lanes_per_s = double(nthreads) * fma_iters * 4 * kChains / t;

  // 16 updates per iteration, 6 slots each.
  const int mix_iters = 1500;
  if (err == hipSuccess)
    err = time_launches([&] { hipLaunchKernelGGL(mix_kernel<256>, dim3(blocks), dim3(threads), 0, nullptr, buf,
                                                 1e-3f, -1.4f, -2.9f, 0.5f, 0.25f, 0.7f, -0.3f, mix_iters); }, 5, &t);
  if (err == hipSuccess) out->mix_slots_per_s = double(nthreads) * mix_iters * 16 * 6 / t;

  // Two waves per SIMD: one block of eight waves per CU, held there alone by
  // an LDS allocation above half of the CU's.
  const int mix2_iters = 6000;
  size_t lds = prop.maxSharedMemoryPerMultiProcessor / 2 + 4096;
  if (lds > prop.sharedMemPerBlock) lds = prop.sharedMemPerBlock;
  if (err == hipSuccess)
    err = time_launches([&] { hipLaunchKernelGGL(mix_kernel<512>, dim3(cus), dim3(512), lds, nullptr, buf, 1e-3f,
                                                 -1.4f, -2.9f, 0.5f, 0.25f, 0.7f, -0.3f, mix2_iters); }, 5, &t);
  if (err == hipSuccess) out->mix2_slots_per_s = double(cus) * 512 * mix2_iters * 16 * 6 / t;
  (void)hipFree(buf);
  if (err != hipSuccess) return err;

  // Streaming copy of 1 GiB.
  const long n4 = (1L << 30) / 16;
  f32x4 *src = nullptr, *dst = nullptr;
  err = hipMalloc(&src, n4 * 16);
  if (err != hipSuccess) return err;
  err = hipMalloc(&dst, n4 * 16);
  if (err == hipSuccess) err = hipMemset(src, 0, n4 * 16);
  if (err == hipSuccess)
    err = time_launches([&] { hipLaunchKernelGGL(copy_kernel, dim3(cus * 16), dim3(256), 0, nullptr, src, dst,
                                                 n4); }, 5, &t);
  if (err == hipSuccess) out->copy_bytes_per_s = 2.0 * n4 * 16 / t;
  (void)hipFree(src);
  if (dst) (void)hipFree(dst);
  return err;
}
