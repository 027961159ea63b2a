// Selective scan forward for gfx950.
//
// Recurrence ("从 Transformer 到 Mamba", ybb.press, sections 3.1 and 5):
//   dt = softplus(delta + bias); h[n] = exp(dt*A[n]) h[n] + dt*B[n]*u;
//   y = (sum_n C[n] h[n] + D u) * silu(z)      (gate as in section 5's block)
//
// Work decomposition. A block owns 64 channels (b, d0..d0+63) of one batch row
// and all N states of each: lane l of every wave is channel d0+l, and wave w
// owns states n = w*S .. w*S+S-1 (S = 1 for N <= 16), kept in VGPRs for the
// whole sequence. Every state chain is therefore walked exactly once, in
// order, and the block has N/S waves (16 for N = 16: four waves per SIMD at
// one block per CU, which the VALU needs to issue near its peak).
//
// Time is processed in tiles of T steps with two phases per tile:
//   * recurrence: each wave advances its states through the tile. B[t, n] and
//     C[t, n] are the same for every lane of the wave; they are read as
//     wave-uniform rows of a float32 copy transposed to [b][n][t] by a small
//     pre-pass. The wave's share of the readout, sum_s C h, goes to an
//     LDS ring (one float per lane and step, XOR-swizzled so that both the
//     writes and the later 16-byte reads are free of bank conflicts).
//   * cooperative: the block finishes tile k (sum of the partial readouts in a
//     fixed order, + D u, * silu(z), store) and prepares tile k+1 (softplus
//     step size and dt*u into LDS, D u and the gate kept in registers). The
//     per-(b, l, d) work is thus done once, not once per wave. Global loads
//     of u, delta and z run two tiles ahead.
// There is no MFMA: this is not a dense contraction. The kernel is bound by
// the VALU (one v_exp_f32 per state update plus 4 FMA-pipe ops).
#include <hip/hip_runtime.h>

#include "device_math.h"
#include "kernels.h"

namespace ssm {

namespace {

constexpr int kPad = 16;  // sequences are padded to a multiple of this many steps

typedef const __attribute__((address_space(4))) uint32_t* const_u32p;

// s_waitcnt immediates (gfx9 encoding); counters not named are left at their
// maxima (no wait on them).
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)
constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0)


int ceil_pow2(int64_t n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// ---------------------------------------------------------------- B/C pre-pass
// B, C [Bt, L, N] -> one 32-bit word per (b, n, t), time-contiguous, zero
// beyond N and L:
//  * bfloat16 inputs: word = (B bits << 16) | C bits (exact);
//  * float32 inputs: two words (B, C) per step, i.e. a float2 per step.
// A wave owning state n then fetches a whole tile of its B and C with one or
// two scalar loads.
template <bool BF16_IN>
__global__ __launch_bounds__(256) void bc_pack_kernel(const void* __restrict__ Bin,
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

// ---------------------------------------------------------------- scan

struct Scan {
  const void* u;
  const void* delta;
  const void* z;
  const float* A;
  const float* D;
  const float* bias;
  const float* h0;
  const uint32_t* BC;  // packed B/C (see bc_pack_kernel)
  void* y;
  float* h_final;
  int64_t L, Lp, dim;
  int N, softplus;
};

template <int S, int W, int T, bool BF16_IN, bool BF16_OUT, bool SOFTPLUS>
__global__ __launch_bounds__(W * 64) void scan_fwd_kernel(const Scan p) {
  constexpr int NS = S * W;        // padded state count
  constexpr int IT = T / W;        // cooperative items per thread per tile
  static_assert(T % W == 0, "tile must split evenly over the waves");
  constexpr int LW = __builtin_ctz(W);
  constexpr int NC = W >= 4 ? W / 4 : 1;            // 16-byte chunks per partial row
  constexpr int LNC = __builtin_ctz(NC);
  constexpr int WPS = BF16_IN ? 1 : 2;              // packed B/C words per step
  constexpr uint32_t IN_B = BF16_IN ? 2 : 4, OUT_B = BF16_OUT ? 2 : 4;

  // Step sizes live in a ring of 4 tile slots (tile k in slot k & 3): tiles
  // are prepared two at a time, every other tile. Partial readouts are
  // double-buffered by tile parity. One barrier per tile separates every
  // writer from every reader.
  __shared__ float2 sDD[4][T][64];                  // (dt, dt*u) per step and channel
  __shared__ __attribute__((aligned(16))) float sP[2][T][64 * W];  // partial readouts

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t tiles_d = (p.dim + 63) / 64;
  const int64_t b = blockIdx.x / tiles_d;
  const int ch_local = static_cast<int>((blockIdx.x % tiles_d) * 64);
  const int64_t ch = ch_local + lane;
  const bool ch_ok = ch < p.dim;
  const int N = p.N;
  const int64_t L = p.L, Lp = p.Lp, Dm = p.dim;
  // Slot of this wave's partial in the lane's row, and the order in which the
  // row's 16-byte chunks are read back. Both are XOR swizzles chosen so that
  // the 4-byte writes and the 16-byte reads hit distinct banks with either
  // 32 or 64 LDS banks.
  const int wpos = lane * W + ((w ^ (lane >> (5 - LW)) ^ (lane >> 5)) & (W - 1));
  const int rswz = ((lane >> (3 - LNC)) ^ (lane >> 3)) & (NC - 1);

  // Recurrence state of this lane: states n = w*S + s of channel ch.
  float A2[S], h[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int n = w * S + s;
    const bool ok = ch_ok && n < N;
    A2[s] = ok ? p.A[ch * N + n] * kLog2e : 0.0f;
    // Pass the loaded initial state through an ALU op here (fma(x, 1, 0) is
    // not folded: it maps -0 to +0), so the loop never inherits a pending load
    // on the state registers.
    h[s] = __builtin_fmaf((ok && p.h0) ? p.h0[(b * Dm + ch) * N + n] : 0.0f, 1.0f, 0.0f);
  }
  const float Dv = (ch_ok && p.D) ? p.D[ch] : 0.0f;
  const float bv = (ch_ok && p.bias) ? p.bias[ch] : 0.0f;
  const bool has_z = p.z != nullptr;

  // Buffer descriptors over this batch row's [L, d] planes; the host keeps
  // each plane below the out-of-range offset. Missing z reads as zeros.
  const uint32_t plane = static_cast<uint32_t>(L * Dm);
  const int64_t pb = b * L * Dm;
  const rsrc_t ru_b = raw_buffer(static_cast<const char*>(p.u) + pb * IN_B, plane * IN_B);
  const rsrc_t rd_b = raw_buffer(static_cast<const char*>(p.delta) + pb * IN_B, plane * IN_B);
  const rsrc_t rz_b = raw_buffer(has_z ? static_cast<const char*>(p.z) + pb * IN_B : nullptr,
                                 has_z ? plane * IN_B : 0u);
  const rsrc_t ry_b = raw_buffer(static_cast<const char*>(p.y) + pb * OUT_B, plane * OUT_B);
  // Element offset of this thread's cooperative item i in tile k:
  // (k*T + w + W*i) * d + ch; out of range past L or d.
  auto item_off = [&](int k, int i, uint32_t elem) -> uint32_t {
    const int t = k * T + w + W * i;
    const bool ok = ch_ok && t >= 0 && t < L;
    return ok ? static_cast<uint32_t>(t * Dm + ch) * elem : kOutOfRange;
  };

  // This wave's packed B/C rows: read-only for the whole kernel (written by
  // the pre-pass launch), so the constant address space turns these
  // wave-uniform loads into scalar loads and the values into SGPR operands.
  const_u32p bcw = (const_u32p)(p.BC) + (b * NS + w * S) * Lp * WPS;
  const int nt = static_cast<int>(Lp / T);

  // Cooperative items of this thread: step w + W*i of each tile, channel ch.
  // Raw inputs (storage bits) are fetched two tiles at a time into two
  // register sets (set = tile parity); D*u and the gate of a tile wait until
  // its readout, up to three tiles later (four sets, set = tile & 3).
  storage_t<BF16_IN> ru[2][IT], rd[2][IT], rz[2][IT];
  float eDu[4][IT], eG[4][IT];

  auto load_raw = [&](int k, auto set) {
    constexpr int R = decltype(set)::value;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const uint32_t off = item_off(k, i, IN_B);
      ru[R][i] = buffer_load_bits<BF16_IN>(ru_b, off);
      rd[R][i] = buffer_load_bits<BF16_IN>(rd_b, off);
      rz[R][i] = buffer_load_bits<BF16_IN>(rz_b, off);
    }
  };
  // Step sizes of tile k into its ring slot (and D*u, gate into registers).
  // Branch-free: padding items get dt = 0 (exp2(0) = 1 and no input, so the
  // state is unchanged) and the flags select rather than branch.
  auto prepare = [&](int k, auto slot) {
    constexpr int SL = decltype(slot)::value;
    constexpr int R = SL & 1;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int tt = w + W * i;
      const int t = k * T + tt;
      const bool ok = ch_ok && t < L;
      const float uv = bits_to_f32<BF16_IN>(ru[R][i]);
      const float x = bits_to_f32<BF16_IN>(rd[R][i]) + bv;
      float dt = SOFTPLUS ? softplus_f(x) : x;
      dt = ok ? dt : 0.0f;
      const float g = silu_f(bits_to_f32<BF16_IN>(rz[R][i]));
      eDu[SL][i] = Dv * uv;
      eG[SL][i] = has_z ? g : 1.0f;
      sDD[SL][tt][lane] = make_float2(dt, dt * uv);
    }
  };
  // Readout of one item of the tile in buffer P: the W partials summed as a
  // fixed tree (every lane, every run, the same order).
  auto gather_item = [&](auto par, int i) -> float {
    constexpr int P = decltype(par)::value;
    const int tt = w + W * i;
    if constexpr (W >= 4) {
      float c4[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float4 v = *reinterpret_cast<const float4*>(&sP[P][tt][lane * W + 4 * (c ^ rswz)]);
        c4[c] = (v.x + v.y) + (v.z + v.w);
      }
#pragma unroll
      for (int m = 1; m < NC; m <<= 1) {
#pragma unroll
        for (int c = 0; c < NC; c += 2 * m) c4[c] += c4[c + m];
      }
      return c4[0];
    } else {
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < W; ++c) acc += sP[P][tt][lane * W + c];
      return acc;
    }
  };

  // Packed B/C of the tile being scanned, wave-uniform (SGPRs), one set per
  // tile parity so the next tile's fetch overlaps this tile's recurrence.
  uint32_t bc[2][S][T * WPS];
  auto load_bc = [&](int k, auto par) {
    constexpr int P = decltype(par)::value;
#pragma unroll
    for (int s = 0; s < S; ++s) {
#pragma unroll
      for (int j = 0; j < T * WPS; ++j) bc[P][s][j] = bcw[(s * Lp + static_cast<int64_t>(k) * T) * WPS + j];
    }
  };

  // Outputs of one tile are held in registers until the next odd tile, so
  // no store is in flight between an even tile's input fetch and its use
  // (stores and loads share one wait counter that may then not be relied on
  // to count in order, and every wait would drain the whole queue).
  float yv[2][IT];
  uint32_t yo[2][IT];

  auto read_dd = [&](float2 (&dd)[T], auto slot) {
    constexpr int SL = decltype(slot)::value;
#pragma unroll
    for (int t = 0; t < T; ++t) dd[t] = sDD[SL][t][lane];
  };
  auto steps = [&](const float2 (&dd)[T], auto par, auto lo, auto hi) {
    constexpr int P = decltype(par)::value;
#pragma unroll
    for (int t = decltype(lo)::value; t < decltype(hi)::value; ++t) {
      float acc = 0.0f;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        float bval, cval;
        if constexpr (BF16_IN) {
          bval = __uint_as_float(bc[P][s][t] & 0xffff0000u);
          cval = __uint_as_float(bc[P][s][t] << 16);
        } else {
          bval = __uint_as_float(bc[P][s][2 * t]);
          cval = __uint_as_float(bc[P][s][2 * t + 1]);
        }
        const float abar = exp2_hw(dd[t].x * A2[s]);
        h[s] = fmaf(abar, h[s], dd[t].y * bval);
        acc = fmaf(cval, h[s], acc);
      }
      sP[P][t][wpos] = acc;
    }
  };

  // Tile k with J = k & 3 (P = k & 1). Its step sizes are already in
  // registers (read during tile k-1), so the recurrence starts right after
  // the barrier. Order: scalar fetch of tile k+1's B/C; first half of the
  // recurrence; LDS reads of tile k+1's step sizes and tile k-1's partials
  // (issued here, waited on after the second half, when the scalar fetch is
  // long done); second half; readout of tile k-1 (stored on odd tiles, two
  // tiles at a time); on even tiles, preparation of tiles k+2 and k+3 and
  // the fetch of the raw inputs of tiles k+4 and k+5. One barrier.
  auto iter = [&](int k, auto jj, const float2 (&dd)[T], float2 (&dd_next)[T]) {
    constexpr int J = decltype(jj)::value;
    constexpr int P = J & 1;
    constexpr int Q = 1 - P;
    load_bc(k + 1 < nt ? k + 1 : k, std::integral_constant<int, Q>{});  // clamped: stays in SGPRs
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    steps(dd, std::integral_constant<int, P>{}, std::integral_constant<int, 0>{},
          std::integral_constant<int, T / 2>{});
    __builtin_amdgcn_sched_barrier(0);
    read_dd(dd_next, std::integral_constant<int, (J + 1) & 3>{});
    float part[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) part[i] = gather_item(std::integral_constant<int, Q>{}, i);
    __builtin_amdgcn_sched_barrier(0);
    steps(dd, std::integral_constant<int, P>{}, std::integral_constant<int, T / 2>{},
          std::integral_constant<int, T>{});
    // Readout of tile k-1 (out of range at k = 0: the stores are dropped).
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      yv[P][i] = (part[i] + eDu[(J + 3) & 3][i]) * eG[(J + 3) & 3][i];
      yo[P][i] = item_off(k - 1, i, OUT_B);
    }
    if constexpr (P == 1) {
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        buffer_store_f32<BF16_OUT>(yv[0][i], ry_b, yo[0][i]);
        buffer_store_f32<BF16_OUT>(yv[1][i], ry_b, yo[1][i]);
      }
    }
    if constexpr (P == 0) {
      prepare(k + 2, std::integral_constant<int, (J + 2) & 3>{});
      prepare(k + 3, std::integral_constant<int, (J + 3) & 3>{});
      load_raw(k + 4, std::integral_constant<int, 0>{});
      load_raw(k + 5, std::integral_constant<int, 1>{});
    }
    __syncthreads();
  };

  float2 ddA[T], ddB[T];
  if (nt > 0) {
    load_raw(0, std::integral_constant<int, 0>{});
    load_raw(1, std::integral_constant<int, 1>{});
    load_bc(0, std::integral_constant<int, 0>{});
    prepare(0, std::integral_constant<int, 0>{});
    prepare(1, std::integral_constant<int, 1>{});
    // Retire every load so far (h0, A, D, bias, tiles 0-1): the wait analysis
    // would otherwise carry them into the loop as possibly pending.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    load_raw(2, std::integral_constant<int, 0>{});
    load_raw(3, std::integral_constant<int, 1>{});
    __syncthreads();
    read_dd(ddA, std::integral_constant<int, 0>{});
    // As above for the LDS counter: retire the first step-size read here.
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
    for (int t = 0; t < T; ++t) ddA[t].x = __builtin_fmaf(ddA[t].x, 1.0f, 0.0f);
  }
  int k = 0;
  for (; k + 3 < nt; k += 4) {
    iter(k, std::integral_constant<int, 0>{}, ddA, ddB);
    iter(k + 1, std::integral_constant<int, 1>{}, ddB, ddA);
    iter(k + 2, std::integral_constant<int, 2>{}, ddA, ddB);
    iter(k + 3, std::integral_constant<int, 3>{}, ddB, ddA);
  }
  if (k < nt) iter(k, std::integral_constant<int, 0>{}, ddA, ddB);
  if (k + 1 < nt) iter(k + 1, std::integral_constant<int, 1>{}, ddB, ddA);
  if (k + 2 < nt) iter(k + 2, std::integral_constant<int, 2>{}, ddA, ddB);
  if (nt > 0) {
    // Held readout of tile nt-2 (when the last tile was even), then tile nt-1.
    const int last = nt - 1;
    if ((last & 1) == 0) {
#pragma unroll
      for (int i = 0; i < IT; ++i) buffer_store_f32<BF16_OUT>(yv[0][i], ry_b, yo[0][i]);
    }
    float part[IT];
    if (last & 1) {
#pragma unroll
      for (int i = 0; i < IT; ++i) part[i] = gather_item(std::integral_constant<int, 1>{}, i);
    } else {
#pragma unroll
      for (int i = 0; i < IT; ++i) part[i] = gather_item(std::integral_constant<int, 0>{}, i);
    }
    const int sl = last & 3;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const float du = sl == 0 ? eDu[0][i] : sl == 1 ? eDu[1][i] : sl == 2 ? eDu[2][i] : eDu[3][i];
      const float g = sl == 0 ? eG[0][i] : sl == 1 ? eG[1][i] : sl == 2 ? eG[2][i] : eG[3][i];
      buffer_store_f32<BF16_OUT>((part[i] + du) * g, ry_b, item_off(last, i, OUT_B));
    }
  }

  if (p.h_final && ch_ok) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int n = w * S + s;
      if (n < N) p.h_final[(b * Dm + ch) * N + n] = h[s];
    }
  }
}

int64_t padded_len(int64_t L) { return (L + kPad - 1) / kPad * kPad; }

// Waves per block and states per lane for a padded state count.
void shape_for(int64_t N, int* NS, int* W, int* S) {
  *NS = ceil_pow2(N);
  *W = *NS < 16 ? *NS : (*NS == 16 ? 8 : 16);
  *S = *NS / *W;
}

template <int S, int W, int T, bool BI, bool BO, bool SP>
int launch_sw(const ScanArgs& a, const Scan& s, hipStream_t st) {
  static_assert(kPad % T == 0, "tile must divide the padding");
  const int64_t tiles_d = (a.dim + 63) / 64;
  const int64_t blocks = a.batch * tiles_d;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  Scan args = s;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&scan_fwd_kernel<S, W, T, BI, BO, SP>),
                         dim3(static_cast<unsigned>(blocks)), dim3(W * 64), kargs, 0, st);
}

// Per padded state count: states per lane S, waves per block W (state
// groups), tile length T. N = 16 uses two states per lane: half the LDS
// traffic per state update of one state per lane, which the LDS bandwidth
// (128 bytes per clock per CU) needs more than the extra waves.
template <bool BI, bool BO, bool SP>
int launch_ns(const ScanArgs& a, const Scan& s, hipStream_t st) {
  int NS, W, S;
  shape_for(a.dstate, &NS, &W, &S);
  switch (NS) {
    case 1: return launch_sw<1, 1, 16, BI, BO, SP>(a, s, st);
    case 2: return launch_sw<1, 2, 16, BI, BO, SP>(a, s, st);
    case 4: return launch_sw<1, 4, 16, BI, BO, SP>(a, s, st);
    case 8: return launch_sw<1, 8, 16, BI, BO, SP>(a, s, st);
    case 16: return launch_sw<2, 8, 8, BI, BO, SP>(a, s, st);
    case 32: return launch_sw<2, 16, 16, BI, BO, SP>(a, s, st);
    default: return launch_sw<4, 16, 16, BI, BO, SP>(a, s, st);
  }
}

template <bool BI, bool BO>
int launch_io(const ScanArgs& a, const Scan& s, hipStream_t st) {
  return a.delta_softplus ? launch_ns<BI, BO, true>(a, s, st) : launch_ns<BI, BO, false>(a, s, st);
}

}  // namespace

size_t scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (batch == 0 || dim == 0 || seqlen == 0) return 0;
  int NS, W, S;
  shape_for(dstate, &NS, &W, &S);
  // Packed B/C: one word per (b, n, t) for bfloat16 inputs, two for float32;
  // sized for the larger so the query does not depend on the dtype.
  return static_cast<size_t>(2 * batch * NS * padded_len(seqlen)) * sizeof(uint32_t);
}

int launch_scan(const ScanArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.batch == 0 || a.dim == 0) return 0;
  int NS, W, S;
  shape_for(a.dstate, &NS, &W, &S);
  const int64_t Lp = padded_len(a.seqlen);
  Scan s;
  s.u = a.u;
  s.delta = a.delta;
  s.z = a.z;
  s.A = a.A;
  s.D = a.D;
  s.bias = a.delta_bias;
  s.h0 = a.h0;
  s.BC = static_cast<const uint32_t*>(a.workspace);
  s.y = a.y;
  s.h_final = a.h_final;
  s.L = a.seqlen;
  s.Lp = Lp;
  s.dim = a.dim;
  s.N = static_cast<int>(a.dstate);
  s.softplus = a.delta_softplus;
  if (Lp > 0) {
    const int64_t chunks = (Lp + 63) / 64;
    if (chunks > 0x7fffffff || a.batch > 65535) return hipErrorInvalidConfiguration;
    const void* bin = a.B;
    const void* cin = a.C;
    uint32_t* out = static_cast<uint32_t*>(a.workspace);
    int64_t L = a.seqlen;
    int64_t Lpv = Lp;
    int N = static_cast<int>(a.dstate);
    void* kargs[] = {&bin, &cin, &out, &L, &Lpv, &N, &NS};
    const void* fn = a.in_bf16 ? reinterpret_cast<const void*>(&bc_pack_kernel<true>)
                               : reinterpret_cast<const void*>(&bc_pack_kernel<false>);
    const int err = hipLaunchKernel(fn, dim3(static_cast<unsigned>(chunks), static_cast<unsigned>(a.batch)),
                                    dim3(256), kargs, 0, st);
    if (err != 0) return err;
  }
  if (a.in_bf16) {
    return a.out_bf16 ? launch_io<true, true>(a, s, st) : launch_io<true, false>(a, s, st);
  }
  return a.out_bf16 ? launch_io<false, true>(a, s, st) : launch_io<false, false>(a, s, st);
}

}  // namespace ssm
