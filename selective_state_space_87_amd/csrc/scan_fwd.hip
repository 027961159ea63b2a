// Selective scan forward for gfx950.
//
// Recurrence ("从 Transformer 到 Mamba", ybb.press, sections 3.1 and 5):
//   dt = softplus(delta + bias); h[n] = exp(dt*A[n]) h[n] + dt*B[n]*u;
//   y = (sum_n C[n] h[n] + D u) * silu(z)      (gate as in section 5's block)
//
// Mapping. A channel (b, d) is owned by a group of G = min(N, 4) consecutive
// lanes (a DPP quad); lane j of the group keeps states n in [j*S, (j+1)*S),
// S = N_pad / G, in VGPRs for the whole sequence. Time runs sequentially in
// every lane, so each state chain is visited exactly once (no recomputation).
// Per group of G time steps, lane j does the per-(b,l,d) work of step j:
// loads u, delta, z, computes dt = softplus(delta + bias) and dt*u, and after
// the group applies the D skip, the gate and the store. The other lanes of
// the group read that step's dt and dt*u through DPP broadcasts, and the
// readout partials are summed by a DPP transposed reduction that leaves step
// j's total in lane j. B and C, shared by all channels of a batch row, are
// staged in LDS as float32 tiles of TT steps and read as broadcasts.
//
// The transition exp(dt*A) is exp2(dt * A*log2(e)), one v_exp_f32 per state
// update. This is not a dense contraction, so there is no MFMA here; the
// kernel is VALU-bound (exp + 4 FMA-pipe ops per update).
#include <hip/hip_runtime.h>

#include "device_math.h"
#include "kernels.h"

namespace ssm {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;  // time steps per LDS tile of B and C

template <int NS, int G, bool BF16_IN, bool BF16_OUT>
__global__ __launch_bounds__(kThreads) void scan_fwd_kernel(const ScanArgs a) {
  constexpr int S = NS / G;          // states per lane
  constexpr int CPB = kThreads / G;  // channels per block
  static_assert(kTile % G == 0, "tile must hold whole groups");
  __shared__ float sB[kTile][NS];
  __shared__ float sC[kTile][NS];

  const int tid = threadIdx.x;
  const int j = tid % G;
  const int64_t L = a.seqlen, Dm = a.dim, N = a.dstate;
  const int64_t tiles_d = (Dm + CPB - 1) / CPB;
  const int64_t b = blockIdx.x / tiles_d;
  const int64_t ch = (blockIdx.x % tiles_d) * CPB + tid / G;
  const bool ch_ok = ch < Dm;

  float A2[S], h[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int n = j * S + s;
    const bool ok = ch_ok && n < N;
    A2[s] = ok ? a.A[ch * N + n] * kLog2e : 0.0f;
    h[s] = (ok && a.h0) ? a.h0[(b * Dm + ch) * N + n] : 0.0f;
  }
  const float Dv = (ch_ok && a.D) ? a.D[ch] : 0.0f;
  const float bias = (ch_ok && a.delta_bias) ? a.delta_bias[ch] : 0.0f;
  const bool has_z = a.z != nullptr;
  const int64_t row0 = b * L;

  for (int64_t t0 = 0; t0 < L; t0 += kTile) {
    __syncthreads();
    for (int i = tid; i < kTile * NS; i += kThreads) {
      const int tt = i / NS, n = i % NS;
      const int64_t t = t0 + tt;
      const bool ok = t < L && n < N;
      sB[tt][n] = ok ? load_elem<BF16_IN>(a.B, (row0 + t) * N + n) : 0.0f;
      sC[tt][n] = ok ? load_elem<BF16_IN>(a.C, (row0 + t) * N + n) : 0.0f;
    }
    __syncthreads();
    for (int g = 0; g < kTile && t0 + g < L; g += G) {
      const int64_t t_own = t0 + g + j;
      const bool own_ok = ch_ok && t_own < L;
      const int64_t idx = (row0 + t_own) * Dm + ch;
      const float uo = own_ok ? load_elem<BF16_IN>(a.u, idx) : 0.0f;
      const float dr = own_ok ? load_elem<BF16_IN>(a.delta, idx) : 0.0f;
      const float zz = (own_ok && has_z) ? load_elem<BF16_IN>(a.z, idx) : 0.0f;
      float dt = dr + bias;
      if (a.delta_softplus) dt = softplus_f(dt);
      dt = own_ok ? dt : 0.0f;  // padding steps leave h unchanged: exp2(0) = 1, input 0
      const float du = dt * uo;

      float p[G];
      static_for<0, G>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const float dtk = group_bcast<G, k>(dt);
        const float duk = group_bcast<G, k>(du);
        float acc = 0.0f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const float abar = exp2_hw(dtk * A2[s]);
          h[s] = fmaf(abar, h[s], duk * sB[g + k][j * S + s]);
          acc = fmaf(sC[g + k][j * S + s], h[s], acc);
        }
        p[k] = acc;
      });
      const float ysum = group_transpose_sum<G>(p, j);
      if (own_ok) {
        float yv = fmaf(Dv, uo, ysum);
        if (has_z) yv *= silu_f(zz);
        store_elem<BF16_OUT>(a.y, idx, yv);
      }
    }
  }
  if (a.h_final && ch_ok) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int n = j * S + s;
      if (n < N) a.h_final[(b * Dm + ch) * N + n] = h[s];
    }
  }
}

template <int NS, bool BI, bool BO>
int launch_ns(const ScanArgs& a, hipStream_t st) {
  constexpr int G = NS < 4 ? NS : 4;
  constexpr int CPB = kThreads / G;
  const int64_t tiles_d = (a.dim + CPB - 1) / CPB;
  const int64_t blocks = a.batch * tiles_d;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  ScanArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&scan_fwd_kernel<NS, G, BI, BO>),
                         dim3(static_cast<unsigned>(blocks)), dim3(kThreads), kargs, 0, st);
}

template <bool BI, bool BO>
int launch_dt(const ScanArgs& a, hipStream_t st) {
  const int64_t N = a.dstate;
  if (N <= 1) return launch_ns<1, BI, BO>(a, st);
  if (N <= 2) return launch_ns<2, BI, BO>(a, st);
  if (N <= 4) return launch_ns<4, BI, BO>(a, st);
  if (N <= 8) return launch_ns<8, BI, BO>(a, st);
  if (N <= 16) return launch_ns<16, BI, BO>(a, st);
  if (N <= 32) return launch_ns<32, BI, BO>(a, st);
  return launch_ns<64, BI, BO>(a, st);
}

}  // namespace

size_t scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  (void)batch;
  (void)seqlen;
  (void)dim;
  (void)dstate;
  return 0;
}

int launch_scan(const ScanArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.batch == 0 || a.dim == 0) return 0;
  if (a.in_bf16) {
    return a.out_bf16 ? launch_dt<true, true>(a, st) : launch_dt<true, false>(a, st);
  }
  return a.out_bf16 ? launch_dt<false, true>(a, st) : launch_dt<false, false>(a, st);
}

}  // namespace ssm
