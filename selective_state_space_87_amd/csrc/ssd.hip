// Mamba-2 SSD layer (structured state-space duality) for gfx950, on MFMA.
//
// What is computed ("Mamba的隐藏代价", kongchang.com, section on the value and
// limits of the argument: the selective SSM as y = M o (Q K^T) V with a lower
// triangular semiseparable M, Q from C and K from B, run as matrix products;
// "从 Transformer 到 Mamba", ybb.press, section 9.1: a diagonal state matrix).
// With one scalar decay a[h] per head (the reading under which M is one
// matrix for all states), per batch b, head h, channel p of the head, state n:
//   dt_t = softplus(dt_raw[b,t,h] + dt_bias[h])          (or without softplus)
//   H_t[n,p] = exp(dt_t a[h]) H_{t-1}[n,p] + dt_t B[b,t,n] x[b,t,h,p]
//   y[b,t,h,p] = (sum_n C[b,t,n] H_t[n,p] + D[h] x[b,t,h,p]) * silu(z[b,t,h,p])
//
// Chunked form. The sequence is cut into chunks of Q = 64 steps. With cs_t
// the inclusive sum of dt over the chunk's steps up to t, and H the state
// entering the chunk, the chunk's outputs and its exit state are
//   Y   = diag(exp(a cs_t)) C H                                (state readout)
//       + (S X),  S[t,s] = (C_t . B_s) exp(a (cs_t - cs_s)) dt_s for s <= t
//   H'  = exp(a cs_end) H + (B o w)^T X,  w_s = exp(a (cs_end - cs_s)) dt_s
// four dense contractions (over N, Q, N and Q), which run on the matrix
// cores; only the masking and decay factors are elementwise.
//
// Mapping. One block of eight waves per (batch, head) walks its chunks in
// order; the state [N, P] stays in MFMA accumulators for the whole sequence
// (never written to memory between chunks), so x, dt, B, C, z and y cross HBM
// exactly once. Wave w owns the 16 columns p = 16 (w mod 4) + 0..15 of Y and
// of the state, and half of their rows: Y row tiles {0, 3} or {1, 2} (equal
// shares of the triangular S X) and one half of the state's row tiles; the
// 10 lower 16x16 tiles of S are dealt round robin. Two waves share each SIMD,
// so one's LDS waits overlap the other's matrix instructions. Operands are staged in LDS as float32 and fed to
// v_mfma_f32_16x16x4_f32 (float32 products, float32 accumulation: the same
// arithmetic precision as the recurrence). Row strides are padded so that the
// operand reads of a wave (16 rows x 4 columns, or 4 rows x 16 columns) fall
// in distinct banks, or at worst two lanes to a bank.
#include <hip/hip_runtime.h>

#include "device_math.h"
#include "kernels.h"

namespace ssm {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kQ = 64;         // chunk length
constexpr int kP = 64;         // padded head size
constexpr int kWaves = 8;      // two per SIMD
constexpr int kThreads = 64 * kWaves;
// LDS row strides (floats). An operand read of a wave touches 16 rows x 4
// consecutive columns (A-type: row stride = 4 mod 64 banks spreads them) or
// 4 rows x 16 consecutive columns (B-type: 16 mod 64). B and the state are
// read both ways (and the state written in the accumulator layout, 4 rows
// of 16 per v); a stride of 20 mod 64 keeps every one of those within 2-way.
constexpr int kXS = kP + 16;
constexpr int kSS = kQ + 4;
constexpr int kHS = kP + 20;

// Inclusive prefix sum over the 64 lanes of a wave, on DPP: shifts by 1, 2,
// 4 and 8 inside each row of 16 lanes (lanes without a source add 0), then
// the last lane of each row broadcast into the next row (row_bcast:15) and
// lane 31 into the upper two rows (row_bcast:31).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_src(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, true));
}
__device__ __forceinline__ float wave_inclusive_sum(float v) {
  v += dpp_src<0x111, 0xF>(v);  // row_shr:1
  v += dpp_src<0x112, 0xF>(v);  // row_shr:2
  v += dpp_src<0x114, 0xF>(v);  // row_shr:4
  v += dpp_src<0x118, 0xF>(v);  // row_shr:8
  v += dpp_src<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_src<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// D (16x16) += A (16x4) B (4x16). Lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; element v of the result is D[4 (l / 16) + v][l % 16].
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Chunk inputs in flight: the next chunk's x, B, C (and this lane's gate
// values and, on wave 0, its step size) are loaded into registers while the
// current chunk computes, and moved into LDS after the chunk's last barrier.
// VEC: head size 64 and N equal to its padding, so rows are whole 16-byte
// pieces (16-byte loads); otherwise one element per load.
template <int NP, bool BF16_IN, bool VEC>
struct SsdStage {
  static constexpr int EB = BF16_IN ? 2 : 4;                        // element bytes
  static constexpr int VE = VEC ? 16 / EB : 1;                      // elements per load
  static constexpr int NXL = kQ * kP / (kThreads * VE);             // x loads per thread
  static constexpr int NBL = (kQ * NP + kThreads * VE - 1) / (kThreads * VE);  // B (and C) loads per thread
  typedef std::conditional_t<VEC, u32x4, storage_t<BF16_IN>> word_t;
  word_t xr[NXL], br[NBL], cr[NBL];
  storage_t<BF16_IN> zr[8];
  storage_t<BF16_IN> dtr;
};

// (batch row, head) item of this block. Consecutive block indices go to
// the eight XCDs in turn, each with its own L2; when the grid is a multiple
// of eight, block i takes item (i mod 8) * (grid / 8) + i / 8 (a bijection),
// so every XCD holds a contiguous run of items, the heads of one or two batch
// rows, and B and C of a batch row are fetched into few L2s.
__device__ __forceinline__ int block_item() {
  const unsigned g = gridDim.x, i = blockIdx.x;
  return static_cast<int>((g & 7u) ? i : (i & 7u) * (g >> 3) + (i >> 3));
}

template <bool BF16>
__device__ __forceinline__ void unpack_store(float* dst, u32x4 v) {
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dst[2 * j] = __uint_as_float(v[j] << 16);
      dst[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = __uint_as_float(v[j]);
  }
}

template <int NP, bool BF16_IN, bool BF16_OUT, bool SOFTPLUS, bool VEC>
__global__ __launch_bounds__(kThreads) void ssd_fwd_kernel(const SsdArgs p) {
  constexpr int NPS = NP + 20;  // row stride of B and C in LDS (20 mod 64, or 52 for NP = 32)
  constexpr int NT = NP / 32;   // state row tiles per wave (of NP / 16)
  using Stage = SsdStage<NP, BF16_IN, VEC>;
  constexpr int EB = Stage::EB, VE = Stage::VE;
  __shared__ float sC[kQ * NPS];
  __shared__ float sB[kQ * NPS];
  __shared__ float sX[kQ * kXS];
  __shared__ float sS[kQ * kSS];
  __shared__ float sH[NP * kHS];
  __shared__ float sCs[kQ];  // inclusive sum of dt over the chunk
  __shared__ float sDt[kQ];
  __shared__ float sW[kQ];   // exp(a (cs_end - cs_s)) dt_s

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int lr = lane & 15, lk = lane >> 4;
  const int H = static_cast<int>(p.nheads), P = static_cast<int>(p.headdim), N = static_cast<int>(p.dstate);
  const int item = block_item();
  const int b = item / H;
  const int hd = item % H;
  const int64_t L = p.seqlen;
  const float a2 = p.A[hd] * kLog2e;
  const float bias = p.dt_bias ? p.dt_bias[hd] : 0.0f;
  const float Dh = p.D ? p.D[hd] : 0.0f;
  const int64_t HP = static_cast<int64_t>(H) * P;
  const int64_t xb = static_cast<int64_t>(b) * L * HP + static_cast<int64_t>(hd) * P;  // + t*HP + p
  const int64_t bcb = static_cast<int64_t>(b) * L * N;                                 // + t*N + n
  const int64_t dtb = static_cast<int64_t>(b) * L * H + hd;                            // + t*H
  const int64_t hsb = (static_cast<int64_t>(b) * H + hd) * P * N;                      // + p*N + n
  const int hf = w >> 2;                 // which half of the rows
  const int pcol = 16 * (w & 3) + lr;    // this lane's column of Y and of the state
  const bool p_ok = pcol < P;
  const int yt0 = hf, yt1 = 3 - hf;      // Y row tiles: {0, 3} or {1, 2}
  const int r0 = hf * NT;                // first state row tile

  // State rows of this wave: element v of tile j is (n = 16 (r0 + j) + 4lk + v, p = pcol).
  f32x4 hacc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int n = 16 * (r0 + j) + 4 * lk + v;
      const float h = (p.h0 && p_ok && n < N) ? p.h0[hsb + static_cast<int64_t>(pcol) * N + n] : 0.0f;
      hacc[j][v] = h;
      sH[n * kHS + pcol] = h;
    }
  }

  const int64_t nchunks = (L + kQ - 1) / kQ;
  Stage stg;
  // Issue the loads of chunk c (all masked to zero past the sequence: the
  // descriptors end at the chunk's last valid row).
  auto fetch = [&](int64_t c) __attribute__((always_inline)) {
    const int64_t t0 = c * kQ;
    const int len = static_cast<int>(c < nchunks ? (L - t0 < kQ ? L - t0 : kQ) : 0);
    const char* xbase = static_cast<const char*>(p.x) + (xb + t0 * HP) * EB;
    const rsrc_t rx = raw_buffer(xbase, len > 0 ? static_cast<uint32_t>(((len - 1) * HP + P) * EB) : 0u);
    const rsrc_t rz = raw_buffer(p.z ? static_cast<const char*>(p.z) + (xb + t0 * HP) * EB : nullptr,
                                 (p.z && len > 0) ? static_cast<uint32_t>(((len - 1) * HP + P) * EB) : 0u);
    const int64_t bo = (bcb + t0 * N) * EB;
    const uint32_t nbc = static_cast<uint32_t>(len * N * EB);
    const rsrc_t rb = raw_buffer(static_cast<const char*>(p.B) + bo, nbc);
    const rsrc_t rc = raw_buffer(static_cast<const char*>(p.C) + bo, nbc);
#pragma unroll
    for (int i = 0; i < Stage::NXL; ++i) {
      const int e = (i * kThreads + tid) * VE;
      const int t = e / kP, pp = e % kP;
      const uint32_t off = static_cast<uint32_t>((t * HP + pp) * EB);
      if constexpr (VEC) {
        stg.xr[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
      } else {
        stg.xr[i] = buffer_load_bits<BF16_IN>(rx, pp < P ? off : kOutOfRange);
      }
    }
#pragma unroll
    for (int i = 0; i < Stage::NBL; ++i) {
      const int e = (i * kThreads + tid) * VE;
      const int t = e / NP, n = e % NP;
      const bool in = e < kQ * NP;       // (a thread's last load may fall past the tile)
      const uint32_t off = in ? static_cast<uint32_t>((t * N + n) * EB) : kOutOfRange;
      if constexpr (VEC) {
        stg.br[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
        stg.cr[i] = __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0);
      } else {
        stg.br[i] = buffer_load_bits<BF16_IN>(rb, n < N ? off : kOutOfRange);
        stg.cr[i] = buffer_load_bits<BF16_IN>(rc, n < N ? off : kOutOfRange);
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int t = 16 * ((q >> 2) ? yt1 : yt0) + 4 * lk + (q & 3);
      stg.zr[q] = buffer_load_bits<BF16_IN>(rz, p_ok ? static_cast<uint32_t>((t * HP + pcol) * EB) : kOutOfRange);
    }
    if (w == 0) {
      const rsrc_t rd = raw_buffer(static_cast<const char*>(p.dt) + (dtb + t0 * H) * EB,
                                   len > 0 ? static_cast<uint32_t>(((len - 1) * H + 1) * EB) : 0u);
      stg.dtr = buffer_load_bits<BF16_IN>(rd, static_cast<uint32_t>(lane * H * EB));
    }
  };
  // Move the fetched chunk into LDS (zeros past the sequence, the head size
  // and the state size).
  auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < Stage::NXL; ++i) {
      const int e = (i * kThreads + tid) * VE;
      const int t = e / kP, pp = e % kP;
      if constexpr (VEC) {
        unpack_store<BF16_IN>(&sX[t * kXS + pp], stg.xr[i]);
      } else {
        sX[t * kXS + pp] = bits_to_f32<BF16_IN>(stg.xr[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < Stage::NBL; ++i) {
      const int e = (i * kThreads + tid) * VE;
      const int t = e / NP, n = e % NP;
      if (e >= kQ * NP) break;
      if constexpr (VEC) {
        unpack_store<BF16_IN>(&sB[t * NPS + n], stg.br[i]);
        unpack_store<BF16_IN>(&sC[t * NPS + n], stg.cr[i]);
      } else {
        sB[t * NPS + n] = bits_to_f32<BF16_IN>(stg.br[i]);
        sC[t * NPS + n] = bits_to_f32<BF16_IN>(stg.cr[i]);
      }
    }
  };

  fetch(0);
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t t0 = c * kQ;
    const int len = static_cast<int>(L - t0 < kQ ? L - t0 : kQ);

    // (1) The chunk's inputs into LDS, its step sizes and their running sums;
    // then the next chunk's loads are issued.
    stage();
    float zg[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) zg[q] = bits_to_f32<BF16_IN>(stg.zr[q]);
    if (w == 0) {
      float dt = 0.0f;
      if (lane < len) {
        const float xr = bits_to_f32<BF16_IN>(stg.dtr) + bias;
        dt = SOFTPLUS ? softplus_f(xr) : xr;
      }
      const float cs = wave_inclusive_sum(dt);
      const float cend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), 63));
      sDt[lane] = dt;
      sCs[lane] = cs;
      sW[lane] = exp2_hw(a2 * (cend - cs)) * dt;
    }
    __syncthreads();
    fetch(c + 1);
    const float cend = sCs[kQ - 1];

    // Every contraction below runs k outermost over independent accumulators
    // and is unrolled whole, so that a k-step's operand reads are issued well
    // before its matrix instructions (one wave per SIMD: nothing else hides
    // the LDS latency), and a shared operand (a row of the state, of X) is
    // read once for all of the wave's tiles.
    // (2a) Scores S: the 10 lower 16x16 tiles (ti >= si), q = w and w+8
    // (the second only for waves 0 and 1).
    auto scores = [&](auto nq) __attribute__((always_inline)) {
      constexpr int NQ = decltype(nq)::value;
      int ti[NQ], si[NQ];
      f32x4 g[NQ];
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const int q = w + kWaves * j;
        ti[j] = q == 0 ? 0 : (q < 3 ? 1 : (q < 6 ? 2 : 3));
        si[j] = q - ti[j] * (ti[j] + 1) / 2;
        g[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
      for (int k0 = 0; k0 < NP; k0 += 4) {
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
          g[j] = mfma4(sC[(16 * ti[j] + lr) * NPS + k0 + lk], sB[(16 * si[j] + lr) * NPS + k0 + lk], g[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const int s = 16 * si[j] + lr;
        const float css = sCs[s], dts = sDt[s];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = 16 * ti[j] + 4 * lk + v;
          const float val = g[j][v] * exp2_hw(a2 * (sCs[t] - css)) * dts;
          sS[t * kSS + s] = t >= s ? val : 0.0f;
        }
      }
    };
    if (w < 10 - kWaves) {
      scores(std::integral_constant<int, 2>{});
    } else {
      scores(std::integral_constant<int, 1>{});
    }
    // (2b) Readout of the entering state, diag(exp(a cs_t)) C H.
    const int yt[2] = {yt0, yt1};
    f32x4 yacc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) yacc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k0 = 0; k0 < NP; k0 += 4) {
      const float hv = sH[(k0 + lk) * kHS + pcol];
#pragma unroll
      for (int j = 0; j < 2; ++j) yacc[j] = mfma4(sC[(16 * yt[j] + lr) * NPS + k0 + lk], hv, yacc[j]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int v = 0; v < 4; ++v) yacc[j][v] *= exp2_hw(a2 * sCs[16 * yt[j] + 4 * lk + v]);
    }
    // (2c) Exit state: exp(a cs_end) H + (B o w)^T X.
    const float dend = exp2_hw(a2 * cend);
#pragma unroll
    for (int j = 0; j < NT; ++j) hacc[j] *= dend;
#pragma unroll
    for (int k0 = 0; k0 < kQ; k0 += 4) {
      const int s = k0 + lk;
      const float xv = sX[s * kXS + pcol], wv = sW[s];
#pragma unroll
      for (int j = 0; j < NT; ++j) hacc[j] = mfma4(sB[s * NPS + 16 * (r0 + j) + lr] * wv, xv, hacc[j]);
    }
    __syncthreads();  // S complete; every wave is done reading the entering state

    // (3) Y += S X over s <= t (row tile ti takes the k-steps below 16 (ti + 1)).
    auto diag = [&](auto ta, auto tb) __attribute__((always_inline)) {
      constexpr int TA = decltype(ta)::value, TB = decltype(tb)::value;
#pragma unroll
      for (int k0 = 0; k0 < 16 * (TB + 1); k0 += 4) {
        const float xv = sX[(k0 + lk) * kXS + pcol];
        if (k0 < 16 * (TA + 1)) yacc[0] = mfma4(sS[(16 * TA + lr) * kSS + k0 + lk], xv, yacc[0]);
        yacc[1] = mfma4(sS[(16 * TB + lr) * kSS + k0 + lk], xv, yacc[1]);
      }
    };
    if (hf == 0) {
      diag(std::integral_constant<int, 0>{}, std::integral_constant<int, 3>{});
    } else {
      diag(std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{});
    }
    // (4) Outputs, and the exit state for the next chunk's readout.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = 16 * yt[j] + 4 * lk + v;
        if (t < len && p_ok) {
          const int64_t o = xb + (t0 + t) * HP + pcol;
          float yv = yacc[j][v] + Dh * sX[t * kXS + pcol];
          if (p.z) yv *= silu_f(zg[4 * j + v]);
          store_elem<BF16_OUT>(p.y, o, yv);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int v = 0; v < 4; ++v) sH[(16 * (r0 + j) + 4 * lk + v) * kHS + pcol] = hacc[j][v];
    }
    __syncthreads();  // inputs and the state are free for the next chunk
  }

  if (p.h_final && p_ok) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int n = 16 * (r0 + j) + 4 * lk + v;
        if (n < N) p.h_final[hsb + static_cast<int64_t>(pcol) * N + n] = hacc[j][v];
      }
    }
  }
}

// bfloat16 inputs with P = 64 and N a power of two (>= 32): the same chunked
// form on v_mfma_f32_16x16x32_bf16, eight times the float32 instruction's
// work per cycle. x, B and C are exact in bfloat16, and every product has
// one of them as an operand; the other operand (the decayed scores, the
// state, the w-scaled B) is float32 and enters as the sum of two bfloat16
// halves, hi = bf16(v) and lo = bf16(v - hi), so each product is taken to
// about 16 bits (two instructions where the float32 path needs eight).
//   scores   G = C B^T                     C, B exact            1 x
//   readout  C H                           H = Hhi + Hlo          2 x
//   diagonal S X                           S = Shi + Slo          2 x
//   state    (B o w)^T X = B^T (w x)       w x = hi + lo          2 x
// Operands are read as 16-byte runs of 8 consecutive k: every LDS array is
// laid out with the contraction index contiguous (x, w x and B are also
// stored transposed). x^T's rows are padded by 8 elements (16 bytes), which
// keeps its transposing 2-byte stores on distinct banks; the other arrays
// permute their 16-byte chunks per row (swz), which keeps the operand reads
// on distinct banks.
// With N >= 64 the block has sixteen waves (four per SIMD, at most 128
// registers each), so that one wave's LDS and transcendental latencies hide
// behind three others' work; the LDS arrays (up to 157 KiB at N = 128) allow
// one block per compute unit either way. D x enters the diagonal product as D
// added to the diagonal of S.
// D (16x16) += A (16x32) B (32x16) on bfloat16: lane l supplies
// A[l % 16][8 (l / 16) .. +7] and B[8 (l / 16) .. +7][l % 16]; the result is
// laid out as for the float32 instruction.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Element (p, s) of x^T [P][Q + 8]. The 8-element runs of s are permuted per
// 16 rows of p (run index XOR (p / 16) mod 4): a wave's transposing stores,
// 8 rows 8 apart, then fall on distinct banks, while an operand read (16
// consecutive rows, one run each) keeps its conflict-free pattern.
__device__ __forceinline__ int xt_at(int pp, int s) { return pp * (kQ + 8) + (s ^ (8 * ((pp >> 4) & 3))); }

// Element (r, e) of a bfloat16 array of RE elements per row whose 16-byte
// chunks (8 elements) are permuted per row: chunk c of row r is stored at
// c ^ 2 ((r / (32 / C)) mod (C / 2)), C = RE / 8 chunks per row. gfx950 serves
// a 16-byte LDS read 32 lanes at a time over 128 four-byte banks; an MFMA
// operand read (lane l: row l mod 16, chunk 4 j + l / 16) then touches every
// bank once per 32 lanes, where rows padded by 16 bytes hit each bank twice
// (measured with a probe: 116 against 178 bytes per clock per CU).
template <int RE>
__device__ __forceinline__ int swz(int r, int e) {
  constexpr int C = RE / 8, PER = C >= 16 ? 1 : 16 / C;
  static_assert(RE % 8 == 0 && C >= 2 && C <= 16 && (C & (C - 1)) == 0, "rows of 2 to 16 chunks");
  return r * RE + ((((e >> 3) ^ ((r / PER) & (C - 1))) << 3) | (e & 7));
}

__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16_bits(v);
  lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
}

template <int NP, int WV, bool BF16_OUT, bool SOFTPLUS>
__global__ __launch_bounds__(64 * WV) void ssd_bf16_kernel(const SsdArgs p) {
  constexpr int NTH = 64 * WV;   // threads of the block (WV waves: 8, or 16 for NP >= 64)
  constexpr int QS = kQ + 8;     // row stride of x^T [P][Q] (elements)
  // C, B [Q][NP] and H^T [P][NP] in rows of NP; S [Q][Q], B^T [NP][Q] and
  // (w x)^T [P][Q] in rows of Q; both with permuted 16-byte chunks (swz).
  auto cix = [](int r, int e) __attribute__((always_inline)) { return swz<NP>(r, e); };
  auto qix = [](int r, int e) __attribute__((always_inline)) { return swz<kQ>(r, e); };
  // Y (and its readout) is 4 x 4 tiles of 16 x 16 (t by p); a wave takes YW
  // tiles of one column p: t-tiles {w/4, 3 - w/4} with 8 waves (equal
  // shares of the triangular S X), t-tile w/4 with 16.
  constexpr int YW = 16 / WV;
  // The exit state's 16 x 16 tiles (NP / 16 along n, 4 along p) are dealt
  // to the waves in blocks of SN x SPC; a block reads SN + SPC operand runs
  // per k-step for SN x SPC products, so blocks are square where they can be.
  // (a k-step reads one run of B^T per n-tile and two of (w x)^T per p-tile)
  constexpr int SN = ((WV == 8 && NP >= 64) || (WV == 16 && NP == 128)) ? 2 : 1;
  constexpr int SPC = (WV == 8 && NP == 128) ? 2 : 1;
  constexpr int NGRP = NP / 16 / SN;
  static_assert(NGRP * (4 / SPC) == WV, "state tiles must cover the waves");
  constexpr int XE = kQ * kP / NTH;                             // x elements staged per thread
  constexpr int CPL = 4 * YW;                                   // output channels per lane
  constexpr int NBL = (kQ * NP + NTH * 8 - 1) / (NTH * 8);      // B (and C) loads per thread
  constexpr int NBT = (NP * (kQ / 8) + NTH - 1) / NTH;          // B^T runs per thread
  constexpr int XW0 = NTH - kP * (kQ / 8);                      // first thread of the (w x)^T runs
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef std::conditional_t<XE == 8, u32x4, u32x2> xw_t;       // a thread's run of x
  typedef std::conditional_t<CPL == 8, u32x4, u32x2> zw_t;      // a lane's gate values
  __shared__ __attribute__((aligned(16))) uint16_t sC[kQ * NP];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kQ * NP];
  __shared__ __attribute__((aligned(16))) uint16_t sBt[NP * kQ];     // B^T (exact)
  __shared__ __attribute__((aligned(16))) uint16_t sXw[2][kP * kQ];  // (w x)^T, hi and lo
  __shared__ __attribute__((aligned(16))) uint16_t sXt[2][kP * QS];  // x^T, by chunk parity
  __shared__ __attribute__((aligned(16))) uint16_t sS[2][kQ * kQ];   // S, hi and lo
  __shared__ __attribute__((aligned(16))) uint16_t sHt[2][kP * NP];  // H^T, hi and lo
  __shared__ __attribute__((aligned(16))) float sCs[kQ];
  __shared__ __attribute__((aligned(16))) float sDt[kQ];
  __shared__ float sW[kQ];
  __shared__ __attribute__((aligned(16))) float sE[kQ];  // exp(a cs_t)
  __shared__ __attribute__((aligned(16))) float sYw[WV][YW * 256];  // each wave's Y tiles

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int lr = lane & 15, lk = lane >> 4;
  const int H = static_cast<int>(p.nheads), N = static_cast<int>(p.dstate);
  const int item = block_item();
  const int b = item / H;
  const int hd = item % H;
  const int64_t L = p.seqlen;
  const float a2 = p.A[hd] * kLog2e;
  const float bias = p.dt_bias ? p.dt_bias[hd] : 0.0f;
  const float Dh = p.D ? p.D[hd] : 0.0f;
  const int64_t HP = static_cast<int64_t>(H) * kP;
  const int64_t xb = static_cast<int64_t>(b) * L * HP + static_cast<int64_t>(hd) * kP;
  const int64_t bcb = static_cast<int64_t>(b) * L * N;
  const int64_t dtb = static_cast<int64_t>(b) * L * H + hd;
  const int64_t hsb = (static_cast<int64_t>(b) * H + hd) * kP * N;
  const int pcol = 16 * (w & 3) + lr;
  int yt[YW];
  yt[0] = w >> 2;
  if constexpr (YW == 2) yt[1] = 3 - (w >> 2);
  // Output layout: lane -> row orow of the wave's Y tiles (sequence
  // position ot) and CPL consecutive channels from op.
  constexpr int LPR = 16 / CPL;  // lanes per row
  const int orow = lane / LPR;
  const int ot = 16 * yt[YW == 2 ? (orow >> 4) : 0] + (orow & 15);
  const int op = 16 * (w & 3) + CPL * (lane % LPR);
  const int nb = SN * (w % NGRP), pb = SPC * (w / NGRP);  // this wave's state block

  // S above the diagonal blocks is read (k-steps of 32 cover it) but never
  // written: zero it once.
  for (int i = tid; i < 2 * kQ * kQ; i += NTH) (&sS[0][0])[i] = 0;
  f32x4 hacc[SN * SPC];  // tile (jn, jp) at jn * SPC + jp
#pragma unroll
  for (int j = 0; j < SN * SPC; ++j) {
    const int pc = 16 * (pb + j % SPC) + lr;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int n = 16 * (nb + j / SPC) + 4 * lk + v;
      const float h = p.h0 ? p.h0[hsb + static_cast<int64_t>(pc) * N + n] : 0.0f;
      hacc[j][v] = h;
      split_bf16(h, sHt[0][cix(pc, n)], sHt[1][cix(pc, n)]);
    }
  }

  const int64_t nchunks = (L + kQ - 1) / kQ;
  u32x4 br[NBL], cr[NBL];
  xw_t xr;
  zw_t zr;
  uint16_t dtr = 0;
  auto fetch = [&](int64_t c) __attribute__((always_inline)) {
    const int64_t t0 = c * kQ;
    const int len = static_cast<int>(c < nchunks ? (L - t0 < kQ ? L - t0 : kQ) : 0);
    const uint32_t xbytes = len > 0 ? static_cast<uint32_t>(((len - 1) * HP + kP) * 2) : 0u;
    const rsrc_t rx = raw_buffer(static_cast<const char*>(p.x) + (xb + t0 * HP) * 2, xbytes);
    const rsrc_t rz = raw_buffer(p.z ? static_cast<const char*>(p.z) + (xb + t0 * HP) * 2 : nullptr,
                                 p.z ? xbytes : 0u);
    const int64_t bo = (bcb + t0 * N) * 2;
    const uint32_t nbc = static_cast<uint32_t>(len * N * 2);
    const rsrc_t rb = raw_buffer(static_cast<const char*>(p.B) + bo, nbc);
    const rsrc_t rc = raw_buffer(static_cast<const char*>(p.C) + bo, nbc);
    {
      const int e = tid * XE;  // one XE-element run of x per thread
      const int t = e / kP, pp = e % kP;
      const uint32_t off = static_cast<uint32_t>((t * HP + pp) * 2);
      if constexpr (XE == 8) {
        xr = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
      } else {
        xr = __builtin_amdgcn_raw_buffer_load_b64(rx, off, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < NBL; ++i) {
      const int e = (i * NTH + tid) * 8;
      const uint32_t off = e < kQ * NP ? static_cast<uint32_t>(e * 2) : kOutOfRange;  // N == NP here
      br[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
      cr[i] = __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0);
    }
    // the gate values of this lane's outputs: CPL channels of row ot
    const uint32_t zoff = static_cast<uint32_t>((ot * HP + op) * 2);
    if constexpr (CPL == 8) {
      zr = __builtin_amdgcn_raw_buffer_load_b128(rz, zoff, 0, 0);
    } else {
      zr = __builtin_amdgcn_raw_buffer_load_b64(rz, zoff, 0, 0);
    }
    // Every wave loads the step sizes (wave 0 uses them): memory operations
    // outside branches keep the waits before the staging counted exactly,
    // so the output stores of the chunk stay in flight across it.
    const rsrc_t rd = raw_buffer(static_cast<const char*>(p.dt) + (dtb + t0 * H) * 2,
                                 len > 0 ? static_cast<uint32_t>(((len - 1) * H + 1) * 2) : 0u);
    dtr = buffer_load_bits<true>(rd, static_cast<uint32_t>(lane * H * 2));
  };

  // Stage chunk c from the fetched registers: B and C as they come
  // (row-major, exact), x transposed (into the buffer of c's parity), the
  // gate values, and (wave 0) the step sizes, their running sums and the
  // weights w. B, C and the step arrays are dead once a chunk's first half
  // is done, so the next chunk is staged right after the middle barrier,
  // while the current one finishes: two barriers per chunk.
  zw_t zq;
  auto stage = [&](int64_t c) __attribute__((always_inline)) {
    const int64_t t0 = c * kQ;
    const int len = static_cast<int>(L - t0 < kQ ? L - t0 : kQ);
    uint16_t* xt = sXt[c & 1];
    {
      const int e = tid * XE;
      const int t = e / kP, pp = e % kP;
#pragma unroll
      for (int j = 0; j < XE / 2; ++j) {
        xt[xt_at(pp + 2 * j, t)] = static_cast<uint16_t>(xr[j] & 0xffffu);
        xt[xt_at(pp + 2 * j + 1, t)] = static_cast<uint16_t>(xr[j] >> 16);
      }
    }
#pragma unroll
    for (int i = 0; i < NBL; ++i) {
      const int e = (i * NTH + tid) * 8;
      if (e >= kQ * NP) break;
      const int t = e / NP, n = e % NP;
      *reinterpret_cast<u32x4*>(&sB[cix(t, n)]) = br[i];
      *reinterpret_cast<u32x4*>(&sC[cix(t, n)]) = cr[i];
    }
    zq = zr;
    if (w == 0) {
      float dt = 0.0f;
      if (lane < len) {
        const float xv = bf16_bits_to_f32(dtr) + bias;
        dt = SOFTPLUS ? softplus_f(xv) : xv;
      }
      const float cs = wave_inclusive_sum(dt);
      const float ce = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), 63));
      sDt[lane] = dt;
      sCs[lane] = cs;
      sW[lane] = exp2_hw(a2 * (ce - cs)) * dt;
      sE[lane] = exp2_hw(a2 * cs);
    }
  };

  if (nchunks > 0) {
    fetch(0);
    stage(0);
    __syncthreads();
    fetch(1);
  }
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t t0 = c * kQ;
    const int len = static_cast<int>(L - t0 < kQ ? L - t0 : kQ);
    const uint16_t* xt = sXt[c & 1];
    const float cend = sCs[kQ - 1];

    // (2a) The exit state's operands, (B o w)^T X = B^T (w x): B^T as it is
    // (exact; run (n, s0 .. s0+7) per item) and the w-scaled x^T, split
    // (run (p, s0 .. s0+7) per item, on the last kP * Q / 8 threads).
#pragma unroll
    for (int i = 0; i < NBT; ++i) {
      const int item = i * NTH + tid;
      if (item >= NP * (kQ / 8)) break;
      const int n = item % NP, s0 = 8 * (item / NP);
      u32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = static_cast<uint32_t>(sB[cix(s0 + 2 * j, n)]) |
               (static_cast<uint32_t>(sB[cix(s0 + 2 * j + 1, n)]) << 16);
      }
      *reinterpret_cast<u32x4*>(&sBt[qix(n, s0)]) = v;
    }
    if (tid >= XW0) {
      const int item = tid - XW0;
      const int pp = item % kP, s0 = 8 * (item / kP);
      const u32x4 xv = *reinterpret_cast<const u32x4*>(&xt[xt_at(pp, s0)]);
      uint16_t hi[8], lo[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        split_bf16(__uint_as_float(xv[j] << 16) * sW[s0 + 2 * j], hi[2 * j], lo[2 * j]);
        split_bf16(__uint_as_float(xv[j] & 0xffff0000u) * sW[s0 + 2 * j + 1], hi[2 * j + 1], lo[2 * j + 1]);
      }
      u32x4 vh, vl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vh[j] = static_cast<uint32_t>(hi[2 * j]) | (static_cast<uint32_t>(hi[2 * j + 1]) << 16);
        vl[j] = static_cast<uint32_t>(lo[2 * j]) | (static_cast<uint32_t>(lo[2 * j + 1]) << 16);
      }
      *reinterpret_cast<u32x4*>(&sXw[0][qix(pp, s0)]) = vh;
      *reinterpret_cast<u32x4*>(&sXw[1][qix(pp, s0)]) = vl;
    }
    // (2b) Scores: lower tiles q = w, w + WV; S = G decayed and scaled, split.
    // Computed transposed, G^T = B C^T, so that a lane holds 4 consecutive s
    // of one row t of S and writes them as one 8-byte run per half.
    auto scores = [&](auto nq) __attribute__((always_inline)) {
      constexpr int NQ = decltype(nq)::value;
      int ti[NQ], si[NQ];
      f32x4 g[NQ];
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const int q = w + WV * j;
        ti[j] = q == 0 ? 0 : (q < 3 ? 1 : (q < 6 ? 2 : 3));
        si[j] = q - ti[j] * (ti[j] + 1) / 2;
        g[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
      for (int k0 = 0; k0 < NP; k0 += 32) {
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
          g[j] = mfma32(lds8(&sB[cix(16 * si[j] + lr, k0 + 8 * lk)]), lds8(&sC[cix(16 * ti[j] + lr, k0 + 8 * lk)]),
                        g[j]);
        }
      }
      // g[j][v] = C_t . B_s at t = 16 ti + lr, s = 16 si + 4 lk + v
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const int t = 16 * ti[j] + lr, s0 = 16 * si[j] + 4 * lk;
        const float cst = sCs[t];
        const f32x4 css = *reinterpret_cast<const f32x4*>(&sCs[s0]);
        const f32x4 dts = *reinterpret_cast<const f32x4*>(&sDt[s0]);
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float val = g[j][v] * exp2_hw(a2 * (cst - css[v])) * dts[v];
          // D x enters S X as D on the diagonal of S
          split_bf16(t > s0 + v ? val : (t == s0 + v ? val + Dh : 0.0f), hi[v], lo[v]);
        }
        *reinterpret_cast<u32x2*>(&sS[0][qix(t, s0)]) =
            u32x2{static_cast<uint32_t>(hi[0]) | (static_cast<uint32_t>(hi[1]) << 16),
                  static_cast<uint32_t>(hi[2]) | (static_cast<uint32_t>(hi[3]) << 16)};
        *reinterpret_cast<u32x2*>(&sS[1][qix(t, s0)]) =
            u32x2{static_cast<uint32_t>(lo[0]) | (static_cast<uint32_t>(lo[1]) << 16),
                  static_cast<uint32_t>(lo[2]) | (static_cast<uint32_t>(lo[3]) << 16)};
      }
    };
    if constexpr (WV < 10) {
      if (w < 10 - WV) {
        scores(std::integral_constant<int, 2>{});
      } else {
        scores(std::integral_constant<int, 1>{});
      }
    } else if (w < 10) {
      scores(std::integral_constant<int, 1>{});
    }
    // (2c) Readout of the entering state, diag(exp(a cs_t)) C H.
    f32x4 yacc[YW];
#pragma unroll
    for (int j = 0; j < YW; ++j) yacc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k0 = 0; k0 < NP; k0 += 32) {
      const bf16x8 hh = lds8(&sHt[0][cix(pcol, k0 + 8 * lk)]);
      const bf16x8 hl = lds8(&sHt[1][cix(pcol, k0 + 8 * lk)]);
#pragma unroll
      for (int j = 0; j < YW; ++j) {
        const bf16x8 cv = lds8(&sC[cix(16 * yt[j] + lr, k0 + 8 * lk)]);
        yacc[j] = mfma32(cv, hh, yacc[j]);
        yacc[j] = mfma32(cv, hl, yacc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < YW; ++j) yacc[j] *= *reinterpret_cast<const f32x4*>(&sE[16 * yt[j] + 4 * lk]);
    __syncthreads();  // S and (B o w)^T complete; every wave is done reading H^T

    // (3) Y += S X over s <= t, in k-steps of 32 (tiles 0 and 2 also read
    // the zero block above the diagonal).
    auto diag = [&](auto ta, auto tb) __attribute__((always_inline)) {
      constexpr int TA = decltype(ta)::value, TB = decltype(tb)::value;
#pragma unroll
      for (int k0 = 0; k0 < 16 * (TB + 1); k0 += 32) {
        const bf16x8 xv = lds8(&xt[xt_at(pcol, k0 + 8 * lk)]);
        if (k0 < 16 * (TA + 1)) {
          yacc[0] = mfma32(lds8(&sS[0][qix(16 * TA + lr, k0 + 8 * lk)]), xv, yacc[0]);
          yacc[0] = mfma32(lds8(&sS[1][qix(16 * TA + lr, k0 + 8 * lk)]), xv, yacc[0]);
        }
        yacc[YW - 1] = mfma32(lds8(&sS[0][qix(16 * TB + lr, k0 + 8 * lk)]), xv, yacc[YW - 1]);
        yacc[YW - 1] = mfma32(lds8(&sS[1][qix(16 * TB + lr, k0 + 8 * lk)]), xv, yacc[YW - 1]);
      }
    };
    if constexpr (YW == 2) {
      if (yt[0] == 0) {
        diag(std::integral_constant<int, 0>{}, std::integral_constant<int, 3>{});
      } else {
        diag(std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{});
      }
    } else {
      // one tile: TA = TB (the first product pair is the only one)
      if (yt[0] < 2) {
        const bf16x8 xv = lds8(&xt[xt_at(pcol, 8 * lk)]);
        yacc[0] = mfma32(lds8(&sS[0][qix(16 * yt[0] + lr, 8 * lk)]), xv, yacc[0]);
        yacc[0] = mfma32(lds8(&sS[1][qix(16 * yt[0] + lr, 8 * lk)]), xv, yacc[0]);
      } else {
#pragma unroll
        for (int k0 = 0; k0 < kQ; k0 += 32) {
          const bf16x8 xv = lds8(&xt[xt_at(pcol, k0 + 8 * lk)]);
          yacc[0] = mfma32(lds8(&sS[0][qix(16 * yt[0] + lr, k0 + 8 * lk)]), xv, yacc[0]);
          yacc[0] = mfma32(lds8(&sS[1][qix(16 * yt[0] + lr, k0 + 8 * lk)]), xv, yacc[0]);
        }
      }
    }
    // (4) Exit state: exp(a cs_end) H + B^T (w x).
    const float dend = exp2_hw(a2 * cend);
#pragma unroll
    for (int j = 0; j < SN * SPC; ++j) hacc[j] *= dend;
#pragma unroll
    for (int k0 = 0; k0 < kQ; k0 += 32) {
      bf16x8 xh[SPC], xl[SPC];
#pragma unroll
      for (int jp = 0; jp < SPC; ++jp) {
        xh[jp] = lds8(&sXw[0][qix(16 * (pb + jp) + lr, k0 + 8 * lk)]);
        xl[jp] = lds8(&sXw[1][qix(16 * (pb + jp) + lr, k0 + 8 * lk)]);
      }
#pragma unroll
      for (int jn = 0; jn < SN; ++jn) {
        const bf16x8 bv = lds8(&sBt[qix(16 * (nb + jn) + lr, k0 + 8 * lk)]);
#pragma unroll
        for (int jp = 0; jp < SPC; ++jp) {
          hacc[jn * SPC + jp] = mfma32(bv, xh[jp], hacc[jn * SPC + jp]);
          hacc[jn * SPC + jp] = mfma32(bv, xl[jp], hacc[jn * SPC + jp]);
        }
      }
    }
    // (5) Outputs. Each wave passes its Y tiles through its own LDS scratch
    // so that a lane ends with CPL consecutive channels of one row: the gate
    // values come in and y goes out as 8- or 16-byte runs (rows past the
    // sequence masked by the buffer's range, no branch). Then the exit state
    // (split) for the next chunk's readout.
    {
      float* sy = sYw[w];
#pragma unroll
      for (int j = 0; j < YW; ++j) {
#pragma unroll
        for (int v = 0; v < 4; ++v) sy[(16 * j + 4 * lk + v) * 16 + lr] = yacc[j][v];
      }
      // other lanes' writes of this wave: LDS executes a wave's accesses in
      // order; the fences keep the compiler from reordering across lanes
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float yv[CPL];
#pragma unroll
      for (int i = 0; i < CPL / 4; ++i) {
        const f32x4 y4 = *reinterpret_cast<const f32x4*>(&sy[orow * 16 + CPL * (lane % LPR) + 4 * i]);
#pragma unroll
        for (int v = 0; v < 4; ++v) yv[4 * i + v] = y4[v];
      }
      if (p.z) {
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const uint32_t zw = zq[q >> 1];
          yv[q] *= silu_f(__uint_as_float((q & 1) ? (zw & 0xffff0000u) : (zw << 16)));
        }
      }
      constexpr int OB = BF16_OUT ? 2 : 4;
      const rsrc_t ry = raw_buffer(static_cast<char*>(p.y) + (xb + t0 * HP) * OB,
                                   static_cast<uint32_t>(((len - 1) * HP + kP) * OB));
      const bool in = ot < len;
      const uint32_t off = static_cast<uint32_t>((ot * HP + op) * OB);
      if constexpr (BF16_OUT) {
        zw_t pk;
#pragma unroll
        for (int j = 0; j < CPL / 2; ++j) {
          pk[j] = static_cast<uint32_t>(f32_to_bf16_bits(yv[2 * j])) |
                  (static_cast<uint32_t>(f32_to_bf16_bits(yv[2 * j + 1])) << 16);
        }
        if constexpr (CPL == 8) {
          __builtin_amdgcn_raw_buffer_store_b128(pk, ry, in ? off : kOutOfRange, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b64(pk, ry, in ? off : kOutOfRange, 0, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < CPL / 4; ++i) {
          const u32x4 y4 = {__float_as_uint(yv[4 * i]), __float_as_uint(yv[4 * i + 1]), __float_as_uint(yv[4 * i + 2]),
                            __float_as_uint(yv[4 * i + 3])};
          __builtin_amdgcn_raw_buffer_store_b128(y4, ry, in ? off + 16u * i : kOutOfRange, 0, 0);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < SN * SPC; ++j) {
      const int n = 16 * (nb + j / SPC) + 4 * lk, pc = 16 * (pb + j % SPC) + lr;
      uint16_t hi[4], lo[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) split_bf16(hacc[j][v], hi[v], lo[v]);
      *reinterpret_cast<u32x2*>(&sHt[0][cix(pc, n)]) =
          u32x2{static_cast<uint32_t>(hi[0]) | (static_cast<uint32_t>(hi[1]) << 16),
                static_cast<uint32_t>(hi[2]) | (static_cast<uint32_t>(hi[3]) << 16)};
      *reinterpret_cast<u32x2*>(&sHt[1][cix(pc, n)]) =
          u32x2{static_cast<uint32_t>(lo[0]) | (static_cast<uint32_t>(lo[1]) << 16),
                static_cast<uint32_t>(lo[2]) | (static_cast<uint32_t>(lo[3]) << 16)};
    }
    if (c + 1 < nchunks) stage(c + 1);
    __syncthreads();  // the next chunk is staged and the state written
    fetch(c + 2);
  }

  if (p.h_final) {
#pragma unroll
    for (int j = 0; j < SN * SPC; ++j) {
      const int pc = 16 * (pb + j % SPC) + lr;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int n = 16 * (nb + j / SPC) + 4 * lk + v;
        p.h_final[hsb + static_cast<int64_t>(pc) * N + n] = hacc[j][v];
      }
    }
  }
}

template <int NP, bool BI, bool BO, bool SP>
int launch_np(const SsdArgs& a, hipStream_t st) {
  SsdArgs args = a;
  void* kargs[] = {&args};
  const bool vec = a.headdim == kP && a.dstate == NP;
  const void* fn = vec ? reinterpret_cast<const void*>(&ssd_fwd_kernel<NP, BI, BO, SP, true>)
                       : reinterpret_cast<const void*>(&ssd_fwd_kernel<NP, BI, BO, SP, false>);
  unsigned threads = kThreads;
  if constexpr (BI) {
    constexpr int WV = NP >= 64 ? 16 : 8;
    if (vec) {
      fn = reinterpret_cast<const void*>(&ssd_bf16_kernel<NP, WV, BO, SP>);
      threads = 64 * WV;
    }
  }
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(a.batch * a.nheads)), dim3(threads), kargs, 0, st);
}

template <bool BI, bool BO, bool SP>
int launch_n(const SsdArgs& a, hipStream_t st) {
  if (a.dstate <= 32) return launch_np<32, BI, BO, SP>(a, st);
  if (a.dstate <= 64) return launch_np<64, BI, BO, SP>(a, st);
  return launch_np<128, BI, BO, SP>(a, st);
}

template <bool BI, bool BO>
int launch_io(const SsdArgs& a, hipStream_t st) {
  return a.dt_softplus ? launch_n<BI, BO, true>(a, st) : launch_n<BI, BO, false>(a, st);
}

}  // namespace

int launch_ssd(const SsdArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.batch == 0 || a.nheads == 0) return 0;
  if (a.batch * a.nheads > 0x7fffffff || a.headdim > kSsdMaxHeadDim || a.dstate > kSsdMaxState) {
    return hipErrorInvalidValue;
  }
  if (a.in_bf16) return a.out_bf16 ? launch_io<true, true>(a, st) : launch_io<true, false>(a, st);
  return a.out_bf16 ? launch_io<false, true>(a, st) : launch_io<false, false>(a, st);
}

}  // namespace ssm
