// Causal depthwise conv1d + SiLU before the selective scan, and its decode
// update, for gfx950.
//
// Per batch b, channel d, step l, filter width K ("从 Transformer 到 Mamba",
// ybb.press, section 5: the block's depthwise Conv1d padded by K-1 and cut to
// the first L outputs, then SiLU; the lyirs.cc "Mamba" notes, block structure
// and the fixed-size conv_state kept between tokens):
//   out = bias[d] + sum_k weight[d, k] * x[b, l-(K-1)+k, d];  y = silu(out)
// Inputs before step 0 come from the carried state [B, d, K-1] (oldest first)
// or are zero; the state after the sequence holds its last K-1 inputs.
//
// Both kernels are HBM-bound streams (x read once, y written once). The
// sequence kernel gives each thread VC = 4 adjacent channels (one 8- or
// 16-byte load per step, consecutive across the wave's lanes) and a segment of
// kSeg steps, walked with a circular register window: the input of step t
// sits in slot t mod KM, so after unrolling by KM nothing moves between
// registers. Filters are applied at a compile-time width KM (4 or 8) with the
// weights right-aligned and zero-padded in front.
#include <hip/hip_runtime.h>

#include "device_math.h"
#include "kernels.h"

namespace ssm {

namespace {

// x and y stream through once: their vector accesses are non-temporal.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSeg = 128;     // steps per thread
constexpr int kGroup = 16;    // steps whose loads are issued together
constexpr int kBlock = 256;   // threads per block (channel groups)

template <int VC, bool BF16>
__device__ __forceinline__ void load_vec(const void* base, int64_t i, float (&v)[VC]) {
  if constexpr (VC == 4 && BF16) {
    const u32x2 r = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(base) + i));
    v[0] = __uint_as_float(r.x << 16);
    v[1] = __uint_as_float(r.x & 0xffff0000u);
    v[2] = __uint_as_float(r.y << 16);
    v[3] = __uint_as_float(r.y & 0xffff0000u);
  } else if constexpr (VC == 4) {
    const f32x4 r = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + i));
    v[0] = r.x;
    v[1] = r.y;
    v[2] = r.z;
    v[3] = r.w;
  } else {
#pragma unroll
    for (int c = 0; c < VC; ++c) v[c] = load_elem<BF16>(base, i + c);
  }
}

template <int VC, bool BF16>
__device__ __forceinline__ void store_vec(void* base, int64_t i, const float (&v)[VC]) {
  if constexpr (VC == 4 && BF16) {
    u32x2 r;
    r.x = static_cast<uint32_t>(f32_to_bf16_bits(v[0])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[1])) << 16);
    r.y = static_cast<uint32_t>(f32_to_bf16_bits(v[2])) | (static_cast<uint32_t>(f32_to_bf16_bits(v[3])) << 16);
    __builtin_nontemporal_store(r, reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + i));
  } else if constexpr (VC == 4) {
    const f32x4 r = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(static_cast<float*>(base) + i));
  } else {
#pragma unroll
    for (int c = 0; c < VC; ++c) store_elem<BF16>(base, i + c, v[c]);
  }
}

template <int KM, int VC, bool BI, bool BO, bool SILU>
__global__ __launch_bounds__(kBlock) void conv1d_fwd_kernel(const ConvArgs a) {
  static_assert(kSeg % KM == 0 && kGroup % KM == 0, "segment and group must be multiples of the window");
  const int64_t L = a.seqlen, Dm = a.dim;
  const int K = static_cast<int>(a.width);
  const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) * VC;
  if (c0 >= Dm) return;
  const int64_t b = blockIdx.z;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kSeg;
  const int64_t row0 = b * L;  // first row of this batch in [B, L, d]

  // Right-aligned, zero-padded weights and the bias of this thread's channels.
  float wp[KM][VC], bv[VC];
#pragma unroll
  for (int c = 0; c < VC; ++c) {
    bv[c] = a.bias ? a.bias[c0 + c] : 0.0f;
#pragma unroll
    for (int i = 0; i < KM; ++i) {
      const int k = i - (KM - K);
      wp[i][c] = k >= 0 ? a.weight[(c0 + c) * K + k] : 0.0f;
    }
  }

  // Input at step t (t may be negative: carried state, or zero).
  auto input = [&](int64_t t, float (&v)[VC]) __attribute__((always_inline)) {
    if (t >= 0) {
      load_vec<VC, BI>(a.x, (row0 + t) * Dm + c0, v);
    } else {
      const int64_t j = (K - 1) + t;  // state slot, oldest first
#pragma unroll
      for (int c = 0; c < VC; ++c) {
        v[c] = (a.state_in && j >= 0) ? a.state_in[((b * Dm) + c0 + c) * (K - 1) + j] : 0.0f;
      }
    }
  };

  // Window: slot s holds the input of the step congruent to s modulo KM.
  float win[KM][VC];
#pragma unroll
  for (int j = 0; j < KM - 1; ++j) {
    // steps t0-KM+1 .. t0-1 go to slots 1 .. KM-1
    input(t0 - (KM - 1) + j, win[1 + j]);
  }
  // One step at slot u: the window already holds the step's input.
  auto emit = [&](int64_t t, int u) __attribute__((always_inline)) {
    float out[VC];
#pragma unroll
    for (int c = 0; c < VC; ++c) {
      float acc = bv[c];
#pragma unroll
      for (int i = 0; i < KM; ++i) acc = fmaf(wp[i][c], win[(u + 1 + i) % KM][c], acc);
      out[c] = SILU ? silu_f(acc) : acc;
    }
    store_vec<VC, BO>(a.y, (row0 + t) * Dm + c0, out);
  };
  const int64_t t_end = min(t0 + kSeg, L);
  int64_t tb = t0;
  // Full groups of kGroup steps: every load of the group is issued before the
  // first is used (no per-step bounds test stands in between).
  for (; tb + kGroup <= t_end; tb += kGroup) {
    float in[kGroup][VC];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) load_vec<VC, BI>(a.x, (row0 + tb + g) * Dm + c0, in[g]);
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
#pragma unroll
      for (int c = 0; c < VC; ++c) win[g % KM][c] = in[g][c];
      emit(tb + g, g % KM);
    }
  }
  // Tail: fewer than kGroup steps, each tested.
#pragma unroll
  for (int g = 0; g < kGroup; ++g) {
    if (tb + g < t_end) {
      input(tb + g, win[g % KM]);
      emit(tb + g, g % KM);
    }
  }

  // The thread holding the last step writes the carried-out state: inputs
  // L-(K-1) .. L-1 (some from the carried-in state when L < K-1).
  const int64_t last_seg = L > 0 ? (L - 1) / kSeg : 0;
  if (a.state_out && K > 1 && static_cast<int64_t>(blockIdx.y) == last_seg) {
    for (int j = 0; j < K - 1; ++j) {
      float v[VC];
      input(L - (K - 1) + j, v);
#pragma unroll
      for (int c = 0; c < VC; ++c) a.state_out[((b * Dm) + c0 + c) * (K - 1) + j] = v[c];
    }
  }
}

template <int KM, bool BI, bool BO, bool SILU>
__global__ __launch_bounds__(kBlock) void conv1d_update_kernel(const ConvUpdateArgs a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t rows = a.batch * a.dim;
  if (i >= rows) return;
  const int64_t ch = i % a.dim;
  const int K = static_cast<int>(a.width);
  float* st = a.state + i * (K - 1);
  // Window of KM inputs, newest last: state (oldest first) then x.
  float win[KM], wp[KM];
#pragma unroll
  for (int s = 0; s < KM; ++s) {
    const int k = s - (KM - K);  // filter tap and, below KM-1, state slot
    wp[s] = k >= 0 ? a.weight[ch * K + k] : 0.0f;
    if (s < KM - 1) win[s] = k >= 0 ? st[k] : 0.0f;
  }
  win[KM - 1] = load_elem<BI>(a.x, i);
  float acc = a.bias ? a.bias[ch] : 0.0f;
#pragma unroll
  for (int s = 0; s < KM; ++s) acc = fmaf(wp[s], win[s], acc);
  // New state: the last K-1 inputs, oldest first.
#pragma unroll
  for (int s = 1; s < KM; ++s) {
    const int j = s - (KM - K) - 1;
    if (j >= 0) st[j] = win[s];
  }
  store_elem<BO>(a.y, i, SILU ? silu_f(acc) : acc);
}

// Decode update with four adjacent channels per thread: their K-1 state
// words per channel are 4 (K-1) consecutive floats, and their filters 4 K
// consecutive floats, so every access is a 16-byte vector access (the state
// rows stream through non-temporally); x and y as in the sequence kernel.
// Requires d % 4 == 0 and 16-byte aligned state, weight and bias.
template <int K, bool BI, bool BO, bool SILU>
__global__ __launch_bounds__(kBlock) void conv1d_update4_kernel(const ConvUpdateArgs a) {
  constexpr int SW = 4 * (K - 1);                  // state floats of the thread's channels
  constexpr int SV = SW / 4;                       // 16-byte state vectors
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t groups = a.batch * a.dim / 4;
  if (g >= groups) return;
  const int64_t i = 4 * g;                         // first row (b * d + ch) of the thread
  const int64_t ch = i % a.dim;
  f32x4 sv[SV > 0 ? SV : 1];
  f32x4 wv[K];
  if constexpr (SV > 0) {
    const f32x4* sp = reinterpret_cast<const f32x4*>(a.state + i * (K - 1));
#pragma unroll
    for (int v = 0; v < SV; ++v) sv[v] = __builtin_nontemporal_load(sp + v);
  }
  const f32x4* wp = reinterpret_cast<const f32x4*>(a.weight + ch * K);
#pragma unroll
  for (int v = 0; v < K; ++v) wv[v] = wp[v];
  float xin[4];
  load_vec<4, BI>(a.x, i, xin);
  f32x4 bias4 = a.bias ? *reinterpret_cast<const f32x4*>(a.bias + ch) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float st[SV > 0 ? SW : 1], w[4 * K];
#pragma unroll
  for (int v = 0; v < SV; ++v) {
    st[4 * v] = sv[v].x; st[4 * v + 1] = sv[v].y; st[4 * v + 2] = sv[v].z; st[4 * v + 3] = sv[v].w;
  }
#pragma unroll
  for (int v = 0; v < K; ++v) {
    w[4 * v] = wv[v].x; w[4 * v + 1] = wv[v].y; w[4 * v + 2] = wv[v].z; w[4 * v + 3] = wv[v].w;
  }
  const float bb[4] = {bias4.x, bias4.y, bias4.z, bias4.w};
  float out[4], ns[SV > 0 ? SW : 1];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // window oldest first: state slots 0..K-2, then x; filter tap k meets slot k
    float acc = bb[c];
#pragma unroll
    for (int k = 0; k < K - 1; ++k) acc = fmaf(w[c * K + k], st[c * (K - 1) + k], acc);
    acc = fmaf(w[c * K + K - 1], xin[c], acc);
    out[c] = SILU ? silu_f(acc) : acc;
#pragma unroll
    for (int k = 0; k + 1 < K - 1; ++k) ns[c * (K - 1) + k] = st[c * (K - 1) + k + 1];
    if constexpr (K > 1) ns[c * (K - 1) + K - 2] = xin[c];
  }
  if constexpr (SV > 0) {
    f32x4* so = reinterpret_cast<f32x4*>(a.state + i * (K - 1));
#pragma unroll
    for (int v = 0; v < SV; ++v) {
      __builtin_nontemporal_store(f32x4{ns[4 * v], ns[4 * v + 1], ns[4 * v + 2], ns[4 * v + 3]}, so + v);
    }
  }
  store_vec<4, BO>(a.y, i, out);
}

template <int KM, int VC, bool BI, bool BO>
int launch_fwd_k(const ConvArgs& a, hipStream_t st) {
  const int64_t groups = (a.dim + VC - 1) / VC;
  const int64_t gx = (groups + kBlock - 1) / kBlock;
  const int64_t gy = a.seqlen > 0 ? (a.seqlen + kSeg - 1) / kSeg : 1;
  if (gx > 0x7fffffff || gy > 65535 || a.batch > 65535) return hipErrorInvalidConfiguration;
  ConvArgs args = a;
  void* kargs[] = {&args};
  const void* fn = a.silu ? reinterpret_cast<const void*>(&conv1d_fwd_kernel<KM, VC, BI, BO, true>)
                          : reinterpret_cast<const void*>(&conv1d_fwd_kernel<KM, VC, BI, BO, false>);
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy),
                                  static_cast<unsigned>(a.batch)),
                         dim3(kBlock), kargs, 0, st);
}

template <bool BI, bool BO>
int launch_fwd_io(const ConvArgs& a, hipStream_t st) {
  // Four channels per thread when rows stay aligned for 8/16-byte accesses.
  const bool vec = a.dim % 4 == 0;
  if (a.width <= 4) return vec ? launch_fwd_k<4, 4, BI, BO>(a, st) : launch_fwd_k<4, 1, BI, BO>(a, st);
  return vec ? launch_fwd_k<8, 4, BI, BO>(a, st) : launch_fwd_k<8, 1, BI, BO>(a, st);
}

template <int KM, bool BI, bool BO>
int launch_upd_k(const ConvUpdateArgs& a, hipStream_t st) {
  const int64_t rows = a.batch * a.dim;
  const int64_t blocks = (rows + kBlock - 1) / kBlock;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  ConvUpdateArgs args = a;
  void* kargs[] = {&args};
  const void* fn = a.silu ? reinterpret_cast<const void*>(&conv1d_update_kernel<KM, BI, BO, true>)
                          : reinterpret_cast<const void*>(&conv1d_update_kernel<KM, BI, BO, false>);
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), kargs, 0, st);
}

template <int K, bool BI, bool BO>
int launch_upd4_k(const ConvUpdateArgs& a, hipStream_t st) {
  const int64_t groups = a.batch * a.dim / 4;
  const int64_t blocks = (groups + kBlock - 1) / kBlock;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  ConvUpdateArgs args = a;
  void* kargs[] = {&args};
  const void* fn = a.silu ? reinterpret_cast<const void*>(&conv1d_update4_kernel<K, BI, BO, true>)
                          : reinterpret_cast<const void*>(&conv1d_update4_kernel<K, BI, BO, false>);
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), kargs, 0, st);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <bool BI, bool BO>
int launch_upd_io(const ConvUpdateArgs& a, hipStream_t st) {
  const bool vec = a.dim % 4 == 0 && aligned16(a.weight) && (a.bias == nullptr || aligned16(a.bias)) &&
                   (a.width == 1 || aligned16(a.state));
  if (vec) {
    switch (a.width) {
      case 2: return launch_upd4_k<2, BI, BO>(a, st);
      case 3: return launch_upd4_k<3, BI, BO>(a, st);
      case 4: return launch_upd4_k<4, BI, BO>(a, st);
      default: break;
    }
  }
  return a.width <= 4 ? launch_upd_k<4, BI, BO>(a, st) : launch_upd_k<8, BI, BO>(a, st);
}

}  // namespace

int launch_conv1d_fwd(const ConvArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.batch == 0 || a.dim == 0) return 0;
  if (a.in_bf16) return a.out_bf16 ? launch_fwd_io<true, true>(a, st) : launch_fwd_io<true, false>(a, st);
  return a.out_bf16 ? launch_fwd_io<false, true>(a, st) : launch_fwd_io<false, false>(a, st);
}

int launch_conv1d_update(const ConvUpdateArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.batch == 0 || a.dim == 0) return 0;
  if (a.in_bf16) return a.out_bf16 ? launch_upd_io<true, true>(a, st) : launch_upd_io<true, false>(a, st);
  return a.out_bf16 ? launch_upd_io<false, true>(a, st) : launch_upd_io<false, false>(a, st);
}

}  // namespace ssm
