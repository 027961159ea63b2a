// Decode: one token's selective state update, in place, for gfx950.
//
// Per (b, d, n) ("从 Transformer 到 Mamba", ybb.press, section 6.3: fixed work
// per token, old state and token in, new state out; the step is the scan's
// step of section 5 for a single token):
//   dt = softplus(delta + bias);  s[n] = exp(dt*A[n]) s[n] + k*B[n]*x
//   y  = (sum_n C[n] s[n] + D x) * silu(z)
// with k = dt, or the exact zero-order-hold coefficient (exp(dt*A[n]) - 1) /
// A[n] ("Mamba新突破", ruibaoantu.com, section 二.3) when ZOH is set.
//
// The state [B, d, N] float32 is read once and written once: the kernel is a
// streaming read-modify-write bound by HBM. A row (b, d) is owned by R lanes
// of one wave, each holding V consecutive states (V a multiple of 4 when
// N % V == 0: V/4 16-byte nontemporal loads and stores per lane, all issued
// before any is used, so each lane keeps V*4 bytes in flight); the row's
// readout is summed across those lanes with xor shuffles inside the wave.
#include <hip/hip_runtime.h>

#include "device_math.h"
#include "kernels.h"

namespace ssm {

namespace {

constexpr int kThreads = 256;
constexpr int kWideV = 16;  // states per lane when N allows
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int V, int R, bool BF16_IN, bool BF16_OUT, bool ZOH>
__global__ __launch_bounds__(kThreads) void state_update_kernel(const UpdateArgs a) {
  constexpr int RPB = kThreads / R;  // rows per block
  const int tid = threadIdx.x;
  const int j = tid % R;
  const int64_t rows = a.batch * a.dim, N = a.dstate;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + tid / R;
  const bool ok = row < rows;
  const int64_t b = ok ? row / a.dim : 0;
  const int64_t ch = ok ? row % a.dim : 0;

  const float x = ok ? load_elem<BF16_IN>(a.x, row) : 0.0f;
  const float dr = ok ? load_elem<BF16_IN>(a.delta, row) : 0.0f;
  const float zz = (ok && a.z) ? load_elem<BF16_IN>(a.z, row) : 0.0f;
  const float bias = (ok && a.delta_bias) ? a.delta_bias[ch] : 0.0f;
  float dt = dr + bias;
  if (a.delta_softplus) dt = softplus_f(dt);
  dt = ok ? dt : 0.0f;
  const float du = dt * x;

  float acc = 0.0f;
  if constexpr (V % 4 == 0) {
    // Lane j owns the 4-state chunks j, j + R, ..., j + (Q-1) R of its row:
    // each load instruction of the R lanes covers R consecutive chunks.
    constexpr int Q = V / 4;
    if (ok) {
      f32x4* sp = reinterpret_cast<f32x4*>(a.state + row * N) + j;
      const f32x4* ap = reinterpret_cast<const f32x4*>(a.A + ch * N) + j;
      f32x4 s[Q], av[Q];
#pragma unroll
      for (int q = 0; q < Q; ++q) s[q] = __builtin_nontemporal_load(sp + q * R);
#pragma unroll
      for (int q = 0; q < Q; ++q) av[q] = ap[q * R];
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int64_t n0 = 4 * (static_cast<int64_t>(q) * R + j);
        float bv[4], cv[4];
        if constexpr (BF16_IN) {
          const uint16_t* bp = static_cast<const uint16_t*>(a.B) + b * N + n0;
          const uint16_t* cp = static_cast<const uint16_t*>(a.C) + b * N + n0;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            bv[v] = bf16_bits_to_f32(bp[v]);
            cv[v] = bf16_bits_to_f32(cp[v]);
          }
        } else {
          const f32x4 b4 = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.B) + b * N + n0);
          const f32x4 c4 = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.C) + b * N + n0);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            bv[v] = b4[v];
            cv[v] = c4[v];
          }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float x2 = dt * (av[q][v] * kLog2e);
          const float abar = exp2_hw(x2);
          float bu = du * bv[v];
          if constexpr (ZOH) bu = x * bv[v] * zoh_coef(dt, x2, abar, inv_or_zero(av[q][v]));
          s[q][v] = fmaf(abar, s[q][v], bu);
          acc = fmaf(cv[v], s[q][v], acc);
        }
      }
#pragma unroll
      for (int q = 0; q < Q; ++q) __builtin_nontemporal_store(s[q], sp + q * R);
    }
  } else {
    for (int64_t n0 = j; n0 < N; n0 += R) {
      if (!ok) continue;
      float* sp = a.state + row * N + n0;
      const float an = a.A[ch * N + n0];
      const float x2 = dt * (an * kLog2e);
      const float abar = exp2_hw(x2);
      const float bn = load_elem<BF16_IN>(a.B, b * N + n0);
      const float bu = ZOH ? x * bn * zoh_coef(dt, x2, abar, inv_or_zero(an)) : du * bn;
      const float s = fmaf(abar, *sp, bu);
      *sp = s;
      acc = fmaf(load_elem<BF16_IN>(a.C, b * N + n0), s, acc);
    }
  }
#pragma unroll
  for (int m = R / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, R);
  if (ok && j == 0) {
    float yv = acc;
    if (a.D) yv = fmaf(a.D[ch], x, yv);
    if (a.z) yv *= silu_f(zz);
    store_elem<BF16_OUT>(a.y, row, yv);
  }
}

template <int V, int R, bool BI, bool BO, bool ZH>
int launch_vr(const UpdateArgs& a, hipStream_t st) {
  constexpr int RPB = kThreads / R;
  const int64_t rows = a.batch * a.dim;
  const int64_t blocks = (rows + RPB - 1) / RPB;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  UpdateArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&state_update_kernel<V, R, BI, BO, ZH>),
                         dim3(static_cast<unsigned>(blocks)), dim3(kThreads), kargs, 0, st);
}

// Lanes per row: enough to cover N with V states each, a power of two <= 64
// (the wide paths need N == R * V exactly; the scalar path loops).
template <int V, bool BI, bool BO, bool ZH>
int launch_v(const UpdateArgs& a, hipStream_t st) {
  const int64_t need = (a.dstate + V - 1) / V;
  if (need <= 1) return launch_vr<V, 1, BI, BO, ZH>(a, st);
  if (need <= 2) return launch_vr<V, 2, BI, BO, ZH>(a, st);
  if (need <= 4) return launch_vr<V, 4, BI, BO, ZH>(a, st);
  if (need <= 8) return launch_vr<V, 8, BI, BO, ZH>(a, st);
  if (need <= 16) return launch_vr<V, 16, BI, BO, ZH>(a, st);
  if (need <= 32) return launch_vr<V, 32, BI, BO, ZH>(a, st);
  return launch_vr<V, 64, BI, BO, ZH>(a, st);
}

// 16-byte state/A/B/C accesses need N % V == 0 and 16-byte aligned bases
// (B and C: 16-byte aligned by the ABI; their rows then stay aligned when
// N * element size is a multiple of 16).
template <bool BI, bool BO, bool ZH>
int launch_io(const UpdateArgs& a, hipStream_t st) {
  const bool base16 = reinterpret_cast<uintptr_t>(a.state) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(a.A) % 16 == 0;
  const bool pow2 = (a.dstate & (a.dstate - 1)) == 0;
  if (base16 && pow2 && a.dstate >= kWideV && a.dstate / kWideV <= 64) return launch_v<kWideV, BI, BO, ZH>(a, st);
  if (base16 && pow2 && a.dstate >= 4 && a.dstate / 4 <= 64) return launch_v<4, BI, BO, ZH>(a, st);
  return launch_v<1, BI, BO, ZH>(a, st);
}

}  // namespace

int launch_state_update(const UpdateArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.batch == 0 || a.dim == 0) return 0;
  if (a.zoh) {
    if (a.in_bf16) return a.out_bf16 ? launch_io<true, true, true>(a, st) : launch_io<true, false, true>(a, st);
    return a.out_bf16 ? launch_io<false, true, true>(a, st) : launch_io<false, false, true>(a, st);
  }
  if (a.in_bf16) return a.out_bf16 ? launch_io<true, true, false>(a, st) : launch_io<true, false, false>(a, st);
  return a.out_bf16 ? launch_io<false, true, false>(a, st) : launch_io<false, false, false>(a, st);
}

}  // namespace ssm
