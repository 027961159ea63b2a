// Selective scan forward for gfx950: kernel templates and their launchers,
// shared by the per-dtype translation units (scan_fwd_{bb,bf,fb,ff}.hip).
//
// Recurrence ("从 Transformer 到 Mamba", ybb.press, sections 3.1 and 5):
//   dt = softplus(delta + bias); h[n] = exp(dt*A[n]) h[n] + dt*B[n]*u;
//   y = (sum_n C[n] h[n] + D u) * silu(z)      (gate as in section 5's block)
// With ZOH the input term is k*B[n]*u, k = (exp(dt*A[n]) - 1) / A[n] (the
// zero-order hold of "Mamba新突破", ruibaoantu.com, section 二.3).
//
// Work decomposition. A block owns 64 channels (b, d0..d0+63) of one batch
// row (and one sequence chunk) and all N states of each: lane l of every wave
// is channel d0+l, and wave w owns states n = w*S .. w*S+S-1, kept in VGPRs
// for the whole chunk; every state chain is walked once, in order. Padded N
// up to 8 runs one state per wave; 16 two states per lane on eight waves; 32
// two on sixteen; 64 and 128 run N/8 per lane on eight waves. Where a plan
// splits a channel's states over two blocks (blockIdx.z), each runs half of
// them (32 states: four per lane, B/C through LDS) and writes its partial
// readout, without the gate (the first block's with the skip D u), to a
// plane of its own.
//
// Time is processed in tiles of T steps (8 at N = 16). Per tile:
//   * recurrence: each wave advances its states through the tile. B[t, n] and
//     C[t, n] are the same for every lane of the wave: a pre-pass packs them
//     per state, time-major, and the wave reads a tile of them with scalar
//     loads into SGPRs (from 64 padded states on, where they no longer fit,
//     the block stages them through LDS instead and every lane reads the
//     same entry). The wave's share of the readout, sum_s C h, goes to an
//     LDS ring (XOR-swizzled: conflict-free writes and 16-byte reads).
//   * cooperative: the block finishes an earlier tile (sum of the partial
//     readouts in a fixed order, + D u, * silu(z), store) and prepares later
//     tiles (softplus step size and dt*u into an LDS ring; D u and the gate in
//     registers). Per-(b, l, d) work is done once, not once per wave. Global
//     loads of u, delta and z run two tiles ahead of the preparation.
// At eight waves with scalar B/C (N = 16) the block synchronises once every
// two tiles ("pair barriers"): step sizes are prepared four tiles ahead and a
// tile is read out two tiles after its recurrence, so that everything read
// between two barriers was written before the first of them. Elsewhere there
// is one barrier per tile, with a preparation two tiles ahead and a readout
// one tile behind.
// The two waves sharing a SIMD take the two phases in opposite orders (see
// iter). There is no MFMA: this is not a dense contraction. The kernel is
// bound by the VALU (one v_exp_f32 per state update plus 4 FMA-pipe ops).
#pragma once

#include <hip/hip_runtime.h>

#include "bc_pack.h"
#include "device_math.h"
#include "kernels.h"

namespace ssm {

struct Scan {
  const void* u;
  const void* delta;
  const void* z;
  const float* A;
  const float* D;
  const float* bias;
  const float* h0;     // initial state [B, d, N] of a single-pass scan, or null (zeros)
  const float* carry;  // chunked: chunk c starts from carry[c] ([chunks][B][d][N])
  const uint32_t* BC;  // packed B/C (see bc_pack_kernel); null when staged through LDS
  const void* Bm;      // B and C as given, [B, L, N] (read directly when staged through LDS)
  const void* Cm;
  void* y;             // output; with states split over blocks, the partial-readout planes
  float* h_final;
  float* hsum;         // summary pass: chunk c's final state from zero into slot c + 1;
                       // checkpoint pass: states at every tile start, [B][tiles][NS][d]
  float* ssum;         // summary pass: chunk c's sum of step sizes, [chunks-1][B][d]
  int L, Lp, dim, N, chunk, batch;
  int64_t y_split;     // states split over blocks: elements between partial planes (else 0)
  float* ckpt;         // full scan with checkpoints: states at every tile start, [B][ckpt_tiles][NS][d]
  int ckpt_tiles;
};

// Per (input, output) dtype: launch the scan (and, for float32 output, the
// checkpoint pass) of a planned shape. Defined in scan_fwd_<in><out>.hip.
int launch_scan_bb(const ScanArgs& a, const ScanPlan& pl, const Scan& s, hipStream_t st);
int launch_scan_bf(const ScanArgs& a, const ScanPlan& pl, const Scan& s, hipStream_t st);
int launch_scan_fb(const ScanArgs& a, const ScanPlan& pl, const Scan& s, hipStream_t st);
int launch_scan_ff(const ScanArgs& a, const ScanPlan& pl, const Scan& s, hipStream_t st);
int launch_ckpt_b(const ScanArgs& a, const ScanPlan& pl, const Scan& s, int64_t blocks, hipStream_t st);
int launch_ckpt_f(const ScanArgs& a, const ScanPlan& pl, const Scan& s, int64_t blocks, hipStream_t st);

namespace {

typedef const __attribute__((address_space(4))) uint32_t* const_u32p;

// s_waitcnt immediates (gfx9 encoding); counters not named are left at their
// maxima (no wait on them).
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)
constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0)


// ---------------------------------------------------------------- scan


// Out-of-range markers of the two parts of a buffer offset: the lane part
// (channel beyond d) and the wave-uniform step part (step outside the chunk).
// A chunk's plane is at most 2^30 bytes, so an offset with either marker,
// or both, is beyond every descriptor's size and the access is masked.
constexpr uint32_t kLaneOut = 0x80000000u;
constexpr uint32_t kStepOut = 0x40000000u;

// Waves whose index has this bit set take the "late" tile order (see iter).
constexpr int kLateWaveMask = 4;

// From 64 padded states on, a wave's B/C words for two tiles no longer fit
// in scalar registers: such shapes stage B and C through LDS instead (and
// need no packing pre-pass).
constexpr bool bc_in_lds(int NS) { return NS >= 64; }

// MODE kFull: the scan of one chunk (or of the whole sequence), with readout,
// gate and store. kSummary: the chunk's recurrence from a zero state only,
// exporting its final state and the sum of its step sizes. kCheckpoint: the
// recurrence from h0 only, storing every wave's states at each tile start
// (for the backward pass, which recomputes each tile from them).
// kFullCkpt: kFull that also stores those checkpoints (single pass, N <= 16),
// so that a training step's backward need not recompute them.
constexpr int kFull = 0, kSummary = 1, kCheckpoint = 2, kFullCkpt = 3;

template <int S, int W, int T, bool BF16_IN, bool BF16_OUT, bool SOFTPLUS, bool ZOH, int MODE, bool PAIR = true,
          bool FORCE_BCL = false>
__global__ __launch_bounds__(W * 64) void scan_fwd_kernel(const Scan p) {
  constexpr int NS = S * W;        // padded state count
  // Cooperative items per thread per tile: step w + W*i of the tile. With
  // fewer steps than waves (the backward's checkpoint pass at N = 32, 64, the
  // summary pass from N = 64 on) waves w >= T have none.
  constexpr int IT = T >= W ? T / W : 1;
  static_assert(T % W == 0 || (MODE != kFull && MODE != kFullCkpt && W % T == 0),
                "tile must split evenly over the waves (or the waves over the tile, without readout)");
  const bool has_item = T >= W || threadIdx.x < 64 * T;  // (wave-uniform: w < T)
  constexpr int LW = __builtin_ctz(W);
  constexpr int NC = W >= 4 ? W / 4 : 1;            // 16-byte chunks per partial row
  constexpr int LNC = __builtin_ctz(NC);
  constexpr int WPS = BF16_IN ? 1 : 2;              // packed B/C words per step
  constexpr uint32_t IN_B = BF16_IN ? 2 : 4, OUT_B = BF16_OUT ? 2 : 4;
  constexpr bool READOUT = MODE == kFull || MODE == kFullCkpt;
  constexpr bool SUMMARY = MODE == kSummary;
  constexpr bool BCL = FORCE_BCL || bc_in_lds(NS);  // forced for the 32-state halves of a split 64
  constexpr int NT = W * 64;                        // threads
  constexpr int EB = BCL ? (T * NS + NT - 1) / NT : 1;  // B/C elements per thread per tile
  // Pair barriers (eight waves of 8-step tiles, scalar B/C): one barrier
  // every two tiles. Step sizes are then prepared four tiles ahead (a ring of
  // 8 tile slots), and each tile is read out two tiles after its recurrence
  // (4 partial buffers); D*u and the gate wait in 8 register sets. Otherwise
  // one barrier per tile, a ring of 4 slots, 2 partial buffers and 4 sets.
  // (Measured at (4, 8192, 4096, 16) bf16: 608 -> 584 us.) Its 96 KB of LDS
  // leave room for one block per CU: chunked plans, whose many short blocks
  // gain from two per CU, take PAIR = false (one barrier per tile, 48 KB).
  constexpr bool PB = PAIR && W == 8 && T == 8 && !BCL;
  constexpr int RING = PB ? 8 : 4;
  constexpr int NPB = PB ? 4 : 2;
  constexpr int LAG = PB ? 2 : 1;
  constexpr int UNR = PB ? 8 : 4;
  static_assert(UNR % RING == 0 && RING % NPB == 0, "tile slots must repeat with the unrolled loop");

  // Step sizes live in a ring of RING tile slots (tile k in slot k % RING):
  // tiles are prepared two at a time, every other tile. Partial readouts
  // rotate over NPB buffers (tile k in k % NPB). A barrier after every tile,
  // or after every odd tile with pair barriers, separates every writer from
  // every reader.
  __shared__ float2 sDD[RING][T][64];               // (dt, dt*u), or (dt, u) with ZOH
  __shared__ __attribute__((aligned(16))) float sP[READOUT ? NPB : 1][T][READOUT ? 64 * W : 1];
  // LDS-staged B/C: (B, C) per step and state, a ring of 4 tile slots like
  // the step sizes. Every lane of a wave reads the same entry (a broadcast).
  __shared__ __attribute__((aligned(16))) float2 sBC[BCL ? 4 : 1][BCL ? T : 1][BCL ? NS : 1];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Dm = p.dim, N = p.N;
  const int tiles_d = (Dm + 63) / 64;
  const int b = blockIdx.x / tiles_d;
  const int ch = static_cast<int>(blockIdx.x % tiles_d) * 64 + lane;
  const bool ch_ok = ch < Dm;
  const int c = blockIdx.y;                         // sequence chunk
  // States split over blocks: block z runs states n0 .. n0 + NS - 1 of its
  // channels and writes the partial readout of those states to plane z.
  const int n0 = static_cast<int>(blockIdx.z) * NS;
  const int t0 = c * p.chunk;
  const int len = min(p.L - t0, p.chunk);           // valid steps of this chunk
  const int nt = min(p.Lp - t0, p.chunk) / T;       // tiles (padded steps / T)
  // Slot of this wave's partial in the lane's row, and the order in which the
  // row's 16-byte chunks are read back. Both are XOR swizzles chosen so that
  // the 4-byte writes and the 16-byte reads hit distinct banks with either
  // 32 or 64 LDS banks.
  const int wpos = lane * W + ((w ^ (lane >> (5 - LW)) ^ (lane >> 5)) & (W - 1));
  const int rswz = ((lane >> (3 - LNC)) ^ (lane >> 3)) & (NC - 1);

  // Recurrence state of this lane: states n = w*S + s of channel ch. A
  // single pass starts from h0 (or zeros); a chunked scan starts chunk c from
  // its carried-in state (for chunk 0 a copy of h0, so that h_final may
  // overwrite h0 while other chunks run); the summary pass from zeros.
  const int64_t bdn = (static_cast<int64_t>(b) * Dm + ch) * N;
  const float* hinit = MODE == kSummary ? nullptr
                               : (p.carry ? p.carry + static_cast<int64_t>(c) * p.batch * Dm * N : p.h0);
  float A2[S], h[S];
  float iA[ZOH ? S : 1];                            // 1/A (0 where A = 0), ZOH only
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int n = n0 + w * S + s;
    const bool ok = ch_ok && n < N;
    const float av = ok ? p.A[static_cast<int64_t>(ch) * N + n] : 0.0f;
    A2[s] = av * kLog2e;
    if constexpr (ZOH) iA[s] = inv_or_zero(av);
    // Pass the loaded initial state through an ALU op here (fma(x, 1, 0) is
    // not folded: it maps -0 to +0), so the loop never inherits a pending load
    // on the state registers.
    h[s] = __builtin_fmaf((ok && hinit) ? hinit[bdn + n] : 0.0f, 1.0f, 0.0f);
  }
  // Same ALU pass-through for the per-channel constants.
  // (with states split over blocks, the skip D u enters the first block's
  // partial readout only)
  const float Dv = __builtin_fmaf((ch_ok && p.D && blockIdx.z == 0) ? p.D[ch] : 0.0f, 1.0f, 0.0f);
  const float bv = __builtin_fmaf((ch_ok && p.bias) ? p.bias[ch] : 0.0f, 1.0f, 0.0f);
  const bool has_z = READOUT && p.z != nullptr;
  // Without z the gate is 1: the gate is formed as fma(z, sigmoid(z), g_off)
  // with g_off = 1 and z read as 0 (its descriptor is empty), else g_off = 0.
  const float g_off = has_z ? 0.0f : 1.0f;
  float dt_sum = 0.0f;

  // LDS-staged B/C: thread element j of a tile is entry e = tid + j*NT of
  // the tile's T x NS (B, C) pairs, step e / NS, state n0 + e % NS, read
  // from row e / NS of the [L, N] input (states at or beyond N read as 0).
  int bc_dst[EB];
  uint32_t bc_src[EB];
  if constexpr (BCL) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      const int e = tid + j * NT;
      const int n = n0 + e % NS;
      bc_dst[j] = e < T * NS ? e : -1;
      bc_src[j] = (e < T * NS && n < N) ? static_cast<uint32_t>((e / NS) * N + n) * IN_B : kLaneOut;
    }
  }

  // Buffer descriptors over this chunk of this batch row's [L, d] planes
  // (at most 2^30 bytes each). Missing z reads as zeros.
  const int64_t pb = (static_cast<int64_t>(b) * p.L + t0) * Dm;
  const uint32_t elems = static_cast<uint32_t>(len) * static_cast<uint32_t>(Dm);
  const rsrc_t ru_b = raw_buffer(static_cast<const char*>(p.u) + pb * IN_B, elems * IN_B);
  const rsrc_t rd_b = raw_buffer(static_cast<const char*>(p.delta) + pb * IN_B, elems * IN_B);
  const rsrc_t rz_b = raw_buffer(has_z ? static_cast<const char*>(p.z) + pb * IN_B : nullptr,
                                 has_z ? elems * IN_B : 0u);
  const rsrc_t ry_b = raw_buffer(READOUT ? static_cast<char*>(p.y) + (pb + blockIdx.z * p.y_split) * OUT_B : nullptr,
                                 READOUT ? elems * OUT_B : 0u);
  const uint32_t lane_in = ch_ok ? static_cast<uint32_t>(ch) * IN_B : kLaneOut;
  const uint32_t lane_out = ch_ok ? static_cast<uint32_t>(ch) * OUT_B : kLaneOut;
  // Wave-uniform part of the offset of cooperative item i of tile k: step
  // k*T + w + W*i of the chunk, times the row pitch; out of range outside it.
  auto step_off = [&](int k, int i, uint32_t elem) __attribute__((always_inline)) -> uint32_t {
    const int t = k * T + w + W * i;
    return (has_item && static_cast<unsigned>(t) < static_cast<unsigned>(len))
               ? static_cast<uint32_t>(t) * static_cast<uint32_t>(Dm) * elem
               : kStepOut;
  };

  // This wave's packed B/C rows: read-only for the whole kernel (written by
  // the pre-pass launch), so the constant address space turns these
  // wave-uniform loads into scalar loads and the values into SGPR operands.
  const_u32p bcw = BCL ? nullptr : (const_u32p)(p.BC) + ((static_cast<int64_t>(b) * NS + w * S) * p.Lp + t0) * WPS;
  const int64_t Lp = p.Lp;

  // Cooperative items of this thread: step w + W*i of each tile, channel ch.
  // Raw inputs (storage bits) are fetched two tiles at a time into two
  // register sets (set = tile parity); D*u and the gate of a tile wait until
  // its readout, up to RING - 1 tiles later (RING sets, set = tile % RING).
  storage_t<BF16_IN> ru[2][IT], rd[2][IT], rz[2][IT];
  storage_t<BF16_IN> rbB[BCL ? 2 : 1][EB], rbC[BCL ? 2 : 1][EB];
  float eDu[RING][IT], eG[RING][IT];

  auto load_raw = [&](int k, auto set) __attribute__((always_inline)) {
    constexpr int R = decltype(set)::value;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const uint32_t off = lane_in + step_off(k, i, IN_B);
      ru[R][i] = buffer_load_bits<BF16_IN, kNonTemporal>(ru_b, off);
      rd[R][i] = buffer_load_bits<BF16_IN, kNonTemporal>(rd_b, off);
      if constexpr (READOUT) rz[R][i] = buffer_load_bits<BF16_IN, kNonTemporal>(rz_b, off);
    }
    if constexpr (BCL) {
      // Tile k's rows of B and C: T*N contiguous elements from step t0 + k*T,
      // fewer (down to none) past the chunk's end, where the reads give 0.
      // (the row count is wave-uniform; readfirstlane keeps it, and so the
      // descriptors, in scalar registers, which buffer loads require)
      const int first = k * T;
      const int rows = __builtin_amdgcn_readfirstlane(max(0, min(T, len - first)));
      const int64_t eo = ((static_cast<int64_t>(b) * p.L + t0 + first) * N) * IN_B;
      const uint32_t nb = static_cast<uint32_t>(rows * N) * IN_B;
      const rsrc_t rbb = raw_buffer(static_cast<const char*>(p.Bm) + eo, nb);
      const rsrc_t rcb = raw_buffer(static_cast<const char*>(p.Cm) + eo, nb);
#pragma unroll
      for (int j = 0; j < EB; ++j) {
        rbB[R][j] = buffer_load_bits<BF16_IN>(rbb, bc_src[j]);
        rbC[R][j] = buffer_load_bits<BF16_IN>(rcb, bc_src[j]);
      }
    }
  };
  // Step sizes of tile k into its ring slot (and D*u, gate into registers).
  // Branch-free: padding steps get dt = 0 (exp2(0) = 1 and no input, so the
  // state is unchanged).
  auto prepare = [&](int k, auto slot) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;
    constexpr int R = SL & 1;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int tt = w + W * i;
      const bool t_ok = k * T + tt < len;          // wave-uniform
      const float uv = bits_to_f32<BF16_IN>(ru[R][i]);
      const float x = bits_to_f32<BF16_IN>(rd[R][i]) + bv;
      float dt = SOFTPLUS ? softplus_f(x) : x;
      dt = t_ok ? dt : 0.0f;
      if constexpr (READOUT) {
        const float zv = bits_to_f32<BF16_IN>(rz[R][i]);
        eDu[SL][i] = Dv * uv;
        eG[SL][i] = fmaf(zv, rcp_hw(1.0f + exp2_hw(-zv * kLog2e)), g_off);  // silu(z), or 1
      }
      if (has_item) sDD[SL][tt < T ? tt : 0][lane] = make_float2(dt, ZOH ? uv : dt * uv);
    }
    if constexpr (BCL) {
#pragma unroll
      for (int j = 0; j < EB; ++j) {
        if (bc_dst[j] >= 0) {
          (&sBC[SL][0][0])[bc_dst[j]] =
              make_float2(bits_to_f32<BF16_IN>(rbB[R][j]), bits_to_f32<BF16_IN>(rbC[R][j]));
        }
      }
    }
  };
  // Readout of one item of the tile in buffer P: the W partials, fetched
  // (gather_load) well before they are summed as a fixed tree (gather_sum;
  // every lane, every run, the same order).
  constexpr int GN = W >= 4 ? NC : 1;               // 16-byte reads per item
  constexpr int GW = W >= 4 ? 4 : W;                // floats per read
  auto gather_load = [&](auto par, int i, float (&g)[GN][GW]) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    const int tt = w + W * i;
    if constexpr (W >= 4) {
#pragma unroll
      for (int q = 0; q < NC; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(&sP[P][tt][lane * W + 4 * (q ^ rswz)]);
        g[q][0] = v.x;
        g[q][1] = v.y;
        g[q][2] = v.z;
        g[q][3] = v.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < W; ++q) g[0][q] = sP[P][tt][lane * W + q];
    }
  };
  auto gather_sum = [&](const float (&g)[GN][GW]) __attribute__((always_inline)) -> float {
    if constexpr (W >= 4) {
      float c4[NC];
#pragma unroll
      for (int q = 0; q < NC; ++q) c4[q] = (g[q][0] + g[q][1]) + (g[q][2] + g[q][3]);
#pragma unroll
      for (int m = 1; m < NC; m <<= 1) {
#pragma unroll
        for (int q = 0; q < NC; q += 2 * m) c4[q] += c4[q + m];
      }
      return c4[0];
    } else {
      float acc = 0.0f;
#pragma unroll
      for (int q = 0; q < W; ++q) acc += g[0][q];
      return acc;
    }
  };
  auto gather_item = [&](auto par, int i) __attribute__((always_inline)) -> float {
    float g[GN][GW];
    gather_load(par, i, g);
    return gather_sum(g);
  };

  // Packed B/C of the tile being scanned, wave-uniform (SGPRs), one set per
  // tile parity so the next tile's fetch overlaps this tile's recurrence.
  uint32_t bc[BCL ? 1 : 2][BCL ? 1 : S][BCL ? 1 : T * WPS];
  auto load_bc = [&](int k, auto par) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    if constexpr (!BCL) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int j = 0; j < T * WPS; ++j) bc[P][s][j] = bcw[(s * Lp + static_cast<int64_t>(k) * T) * WPS + j];
      }
    }
  };

  // Outputs of one tile are held in registers until the next odd tile, so
  // no store is in flight between an even tile's input fetch and its use
  // (stores and loads share one wait counter that may then not be relied on
  // to count in order, and every wait would drain the whole queue).
  float yv[2][IT];
  uint32_t yo[2][IT];

  auto read_dd = [&](float2 (&dd)[T], auto slot) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;
#pragma unroll
    for (int t = 0; t < T; ++t) dd[t] = sDD[SL][t][lane];
  };
  auto steps = [&](const float2 (&dd)[T], auto jj, auto lo, auto hi) __attribute__((always_inline)) {
    constexpr int J = decltype(jj)::value;
    constexpr int P = J & 1;
#pragma unroll
    for (int t = decltype(lo)::value; t < decltype(hi)::value; ++t) {
      float acc = 0.0f;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        float bval, cval;
        if constexpr (BCL) {
          // two states' (B, C) per 16-byte broadcast read
          const float4 v = *reinterpret_cast<const float4*>(&sBC[J][t][w * S + (s & ~1)]);
          bval = (s & 1) ? v.z : v.x;
          cval = (s & 1) ? v.w : v.y;
        } else if constexpr (BF16_IN) {
          bval = __uint_as_float(bc[P][s][t] & 0xffff0000u);
          cval = __uint_as_float(bc[P][s][t] << 16);
        } else {
          bval = __uint_as_float(bc[P][s][2 * t]);
          cval = __uint_as_float(bc[P][s][2 * t + 1]);
        }
        const float x2 = dd[t].x * A2[s];
        const float abar = exp2_hw(x2);
        float bu = dd[t].y * bval;                  // dt*u*B, or u*B with ZOH
        if constexpr (ZOH) bu *= zoh_coef(dd[t].x, x2, abar, iA[s]);
        h[s] = fmaf(abar, h[s], bu);
        if constexpr (READOUT) acc = fmaf(cval, h[s], acc);
      }
      if constexpr (READOUT) sP[J % NPB][t][wpos] = acc;
      if constexpr (SUMMARY) dt_sum += dd[t].x;
    }
  };

  // Tile k with J = k % UNR (P = k & 1). Its step sizes are already in
  // registers (read during tile k-1) and its B/C in SGPR set P (fetched
  // during tile k-1). The work of a tile, in the order of the "early" waves:
  //   (1) scalar fetch of tile k+1's B/C; first half of the recurrence;
  //   (2) LDS reads of tile k+1's step sizes and tile k-1's partials
  //       (waited on after the second half, when the scalar fetch is long
  //       done);
  //   (3) second half of the recurrence;
  //   (4) readout of tile k-LAG (stored on odd tiles, two tiles at a time);
  //       on even tiles, preparation of two tiles (k+2 and k+3, or k+4 and
  //       k+5 with pair barriers) and the fetch of the raw inputs of the two
  //       after them.
  // "Late" waves run (2), (4), (1), (3): the readout and the preparation
  // first, then the whole recurrence. A wave raises its issue priority while
  // it runs the recurrence, so the SIMD's arbiter prefers it over the other
  // wave's cooperative work (which mostly waits on memory and LDS). The two waves that share a SIMD take
  // different orders, so while one runs the recurrence the other runs the
  // cooperative work, instead of both waiting on the same phase. Every
  // dependency is on data written before the previous barrier, so both
  // orders are valid.
  auto lds_reads = [&](auto jj, float2 (&dd_next)[T], float (&gp)[IT][GN][GW]) __attribute__((always_inline)) {
    constexpr int J = decltype(jj)::value;
    constexpr int Q = (J + NPB - LAG) % NPB;        // partials of tile k - LAG
    read_dd(dd_next, std::integral_constant<int, (J + 1) % RING>{});
    if constexpr (READOUT) {
#pragma unroll
      for (int i = 0; i < IT; ++i) gather_load(std::integral_constant<int, Q>{}, i, gp[i]);
    }
  };
  auto coop = [&](int k, auto jj, float (&gp)[IT][GN][GW]) __attribute__((always_inline)) {
    constexpr int J = decltype(jj)::value;
    constexpr int P = J & 1;
    if constexpr (READOUT) {
      // Readout of tile k - LAG (out of range for k < LAG: the stores are dropped).
      constexpr int E = (J + RING - LAG) % RING;
#pragma unroll
      for (int i = 0; i < IT; ++i) {
        yv[P][i] = (gather_sum(gp[i]) + eDu[E][i]) * eG[E][i];
        yo[P][i] = lane_out + step_off(k - LAG, i, OUT_B);
      }
      if constexpr (P == 1) {
#pragma unroll
        for (int i = 0; i < IT; ++i) {
          buffer_store_f32<BF16_OUT, kNonTemporal>(yv[0][i], ry_b, yo[0][i]);
          buffer_store_f32<BF16_OUT, kNonTemporal>(yv[1][i], ry_b, yo[1][i]);
        }
      }
    }
    if constexpr (PB) {
      if constexpr (P == 0) {
        prepare(k + 4, std::integral_constant<int, (J + 4) % RING>{});
        prepare(k + 5, std::integral_constant<int, (J + 5) % RING>{});
        load_raw(k + 6, std::integral_constant<int, 0>{});
        load_raw(k + 7, std::integral_constant<int, 1>{});
      }
    } else if constexpr (P == 0) {
      prepare(k + 2, std::integral_constant<int, (J + 2) & 3>{});
      prepare(k + 3, std::integral_constant<int, (J + 3) & 3>{});
      load_raw(k + 4, std::integral_constant<int, 0>{});
      load_raw(k + 5, std::integral_constant<int, 1>{});
    }
  };
  auto iter = [&](int k, auto jj, auto late, const float2 (&dd)[T], float2 (&dd_next)[T]) __attribute__((always_inline)) {
    constexpr int J = decltype(jj)::value;
    constexpr int P = J & 1;
    constexpr int Q = 1 - P;
    float gp[IT][GN][GW];
    if constexpr (MODE == kFullCkpt) {
      // as the checkpoint pass below, into the caller's checkpoint array,
      // non-temporal (the backward reads them back long after)
      const rsrc_t rck = raw_buffer(p.ckpt + ((static_cast<int64_t>(b) * p.ckpt_tiles + k) * NS + w * S) * Dm,
                                    static_cast<uint32_t>(S * Dm * 4));
#pragma unroll
      for (int s = 0; s < S; ++s) {
        buffer_store_f32<false, kNonTemporal>(h[s], rck, ch_ok ? static_cast<uint32_t>((s * Dm + ch) * 4) : kLaneOut);
      }
    }
    if constexpr (MODE == kCheckpoint) {
      // Branch-free through a descriptor over this wave's rows of tile k
      // (lanes beyond d are dropped by the buffer unit): a branch here would
      // leave the wait analysis unable to count the memory queue in order.
      const rsrc_t rck = raw_buffer(p.hsum + ((static_cast<int64_t>(b) * nt + k) * NS + w * S) * Dm,
                                    static_cast<uint32_t>(S * Dm * 4));
#pragma unroll
      for (int s = 0; s < S; ++s) {
        buffer_store_f32<false, kNonTemporal>(h[s], rck, ch_ok ? static_cast<uint32_t>((s * Dm + ch) * 4) : kLaneOut);
      }
    }
    if constexpr (decltype(late)::value) {
      lds_reads(jj, dd_next, gp);
      __builtin_amdgcn_sched_barrier(0);
      coop(k, jj, gp);
      __builtin_amdgcn_sched_barrier(0);
      load_bc(k + 1 < nt ? k + 1 : k, std::integral_constant<int, Q>{});  // clamped: stays in SGPRs
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(2);
      steps(dd, jj, std::integral_constant<int, 0>{},
            std::integral_constant<int, T / 2>{});
      steps(dd, jj, std::integral_constant<int, T / 2>{},
            std::integral_constant<int, T>{});
      __builtin_amdgcn_s_setprio(0);
    } else {
      load_bc(k + 1 < nt ? k + 1 : k, std::integral_constant<int, Q>{});  // clamped: stays in SGPRs
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(2);
      steps(dd, jj, std::integral_constant<int, 0>{},
            std::integral_constant<int, T / 2>{});
      __builtin_amdgcn_sched_barrier(0);
      lds_reads(jj, dd_next, gp);
      __builtin_amdgcn_sched_barrier(0);
      steps(dd, jj, std::integral_constant<int, T / 2>{},
            std::integral_constant<int, T>{});
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      coop(k, jj, gp);
    }
    if constexpr (!PB || (J & 1) == 1) __syncthreads();
  };

  float2 ddA[T], ddB[T];
  if (nt > 0) {
    load_raw(0, std::integral_constant<int, 0>{});
    load_raw(1, std::integral_constant<int, 1>{});
    load_bc(0, std::integral_constant<int, 0>{});
    prepare(0, std::integral_constant<int, 0>{});
    prepare(1, std::integral_constant<int, 1>{});
    // Retire every load so far (state, A, D, bias, tiles 0-1): the wait
    // analysis would otherwise carry them into the loop as possibly pending.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    load_raw(2, std::integral_constant<int, 0>{});
    load_raw(3, std::integral_constant<int, 1>{});
    if constexpr (PB) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      prepare(2, std::integral_constant<int, 2>{});
      prepare(3, std::integral_constant<int, 3>{});
      load_raw(4, std::integral_constant<int, 0>{});
      load_raw(5, std::integral_constant<int, 1>{});
    }
    if constexpr (READOUT) {
      // Out-of-range stores (dropped by the buffer unit) in the places of an
      // odd tile's output stores: loop entry then sees the same queue of
      // memory operations as the back edge, and the waits of the first tile
      // need not cover stores.
#pragma unroll
      for (int i = 0; i < 2 * IT; ++i) buffer_store_f32<BF16_OUT>(0.0f, ry_b, kLaneOut + 64u * i);
    }
    __syncthreads();
    read_dd(ddA, std::integral_constant<int, 0>{});
    // As above for the LDS counter: retire the first step-size read here.
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
    for (int t = 0; t < T; ++t) ddA[t].x = __builtin_fmaf(ddA[t].x, 1.0f, 0.0f);
  }
  auto run = [&](auto late) __attribute__((always_inline)) {
    int k = 0;
    for (; k + UNR - 1 < nt; k += UNR) {
      static_for<0, UNR>([&](auto jj) __attribute__((always_inline)) {
        constexpr int J = decltype(jj)::value;
        if constexpr ((J & 1) == 0) iter(k + J, jj, late, ddA, ddB);
        else iter(k + J, jj, late, ddB, ddA);
      });
    }
    static_for<0, UNR - 1>([&](auto jj) __attribute__((always_inline)) {
      constexpr int J = decltype(jj)::value;
      if (k + J < nt) {
        if constexpr ((J & 1) == 0) iter(k + J, jj, late, ddA, ddB);
        else iter(k + J, jj, late, ddB, ddA);
      }
    });
  };
  // Two orders only where two waves of the block share each SIMD (eight
  // waves); elsewhere the second copy of the loop would cost registers.
  if constexpr (W == 8) {
    if ((w & kLateWaveMask) != 0) {
      run(std::true_type{});
    } else {
      run(std::false_type{});
    }
  } else {
    run(std::false_type{});
  }

  if constexpr (READOUT) {
    if (nt > 0) {
      const int last = nt - 1;
      // Held readout of an even last iteration (tile last - LAG), still unstored.
      if ((last & 1) == 0) {
#pragma unroll
        for (int i = 0; i < IT; ++i) buffer_store_f32<BF16_OUT>(yv[0][i], ry_b, yo[0][i]);
      }
      // The last LAG tiles are read out here, after a barrier over their
      // partials (the loop ends with one only after an odd tile, or after
      // every tile without pair barriers).
      if (PB && (last & 1) == 0) __syncthreads();
      // Tile tl = nt - LAG + D sits in ring slot tl % RING and partial buffer
      // tl % NPB. The loop runs tiles in groups of UNR (a multiple of RING)
      // from tile 0, so both follow at compile time from (nt - 1) % UNR: one
      // branch per value, with constant register-set indexes (an index
      // computed at run time would put the ring in scratch memory).
      static_for<0, UNR>([&](auto jl) __attribute__((always_inline)) {
        constexpr int JL = decltype(jl)::value;
        if ((nt - 1) % UNR == JL) {
          static_for<0, LAG>([&](auto dl) __attribute__((always_inline)) {
            constexpr int D = decltype(dl)::value;
            constexpr int R = ((JL - (LAG - 1) + D) % RING + RING) % RING;
            const int tl = nt - LAG + D;
            if (tl >= 0) {
#pragma unroll
              for (int i = 0; i < IT; ++i) {
                const float part = gather_item(std::integral_constant<int, R % NPB>{}, i);
                buffer_store_f32<BF16_OUT>((part + eDu[R][i]) * eG[R][i], ry_b,
                                           lane_out + step_off(tl, i, OUT_B));
              }
            }
          });
        }
      });
    }
    if (p.h_final && ch_ok && c == static_cast<int>(gridDim.y) - 1) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int n = n0 + w * S + s;
        if (n < N) p.h_final[bdn + n] = h[s];
      }
    }
  } else if constexpr (MODE == kSummary) {
    if (ch_ok) {
      const int64_t cb = static_cast<int64_t>(c) * p.batch + b;
      const int64_t cb1 = cb + p.batch;              // slot c + 1
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int n = n0 + w * S + s;
        if (n < N) p.hsum[(cb1 * Dm + ch) * N + n] = h[s];
      }
      if (w == 0) p.ssum[cb * Dm + ch] = dt_sum;
    }
  }
}

// In-order fold of the chunk summaries with the recurrence's combine rule:
// the state entering chunk c+1 is exp(A * sum of chunk c's step sizes) times
// the state entering chunk c, plus chunk c's final state from zero. One
// thread per (b, d, n). Slot 0 receives the initial state (h0 or zeros);
// slot c+1, which holds chunk c's summary state, is overwritten in place with
// the state entering chunk c+1.
__global__ __launch_bounds__(256) void carry_fold_kernel(const float* __restrict__ A,
                                                         const float* __restrict__ h0,
                                                         float* __restrict__ hsum,
                                                         const float* __restrict__ ssum,
                                                         int64_t bdn_total, int dim, int N,
                                                         int folds) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= bdn_total) return;
  const int n = static_cast<int>(i % N);
  const int64_t bd = i / N;
  const int ch = static_cast<int>(bd % dim);
  const int64_t bd_total = bdn_total / N;
  const float a2 = A[static_cast<int64_t>(ch) * N + n] * kLog2e;
  float h = h0 ? h0[i] : 0.0f;
  hsum[i] = h;
  for (int c = 0; c < folds; ++c) {
    const float decay = exp2_hw(a2 * ssum[c * bd_total + bd]);
    float* slot = hsum + (c + 1) * bdn_total + i;
    h = fmaf(decay, h, *slot);
    *slot = h;
  }
}

template <int S, int W, int T, bool BI, bool BO, bool SP, bool ZH, bool FBCL = false>
int launch_sw(const ScanArgs& a, const ScanPlan& pl, const Scan& s, hipStream_t st) {
  static_assert(kPadSteps % T == 0, "tile must divide the padding");
  const int64_t blocks = a.batch * pl.dim_blocks;
  if (blocks > 0x7fffffff || pl.chunks > 65535) return hipErrorInvalidConfiguration;
  Scan args = s;
  void* kargs[] = {&args};
  if (pl.chunks > 1) {
    // The summary's result (a chunk's final state and step-size sum) does
    // not depend on its tiling. With B/C staged through LDS it takes shorter
    // tiles (4 steps at 8 states per lane, 2 at 16): with no readout between
    // steps, 8-step tiles ran out of registers (spilled to scratch).
    constexpr int TS = bc_in_lds(S * W) ? 32 / S : T;
    int err = hipLaunchKernel(reinterpret_cast<const void*>(&scan_fwd_kernel<S, W, TS, BI, BO, SP, ZH, kSummary, false>),
                              dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(pl.chunks - 1)),
                              dim3(W * 64), kargs, 0, st);
    if (err != 0) return err;
    const int64_t bdn = a.batch * a.dim * a.dstate;
    const float* A = a.A;
    const float* h0 = a.h0;
    float* hsum = args.hsum;
    const float* ssum = args.ssum;
    int dim = static_cast<int>(a.dim), N = static_cast<int>(a.dstate);
    int folds = static_cast<int>(pl.chunks - 1);
    void* fargs[] = {&A, &h0, &hsum, &ssum, const_cast<int64_t*>(&bdn), &dim, &N, &folds};
    err = hipLaunchKernel(reinterpret_cast<const void*>(&carry_fold_kernel),
                          dim3(static_cast<unsigned>((bdn + 255) / 256)), dim3(256), fargs, 0, st);
    if (err != 0) return err;
  }
  const void* full = pl.chunks > 1
                         ? reinterpret_cast<const void*>(&scan_fwd_kernel<S, W, T, BI, BO, SP, ZH, kFull, false, FBCL>)
                         : reinterpret_cast<const void*>(&scan_fwd_kernel<S, W, T, BI, BO, SP, ZH, kFull, true, FBCL>);
  if (s.ckpt != nullptr) {
    // checkpoints from the scan itself: single pass, N <= 16 (the backward's tiles)
    if constexpr (S * W <= 16 && !FBCL) {
      if (pl.chunks != 1 || pl.splits != 1) return hipErrorInvalidValue;
      full = reinterpret_cast<const void*>(&scan_fwd_kernel<S, W, T, BI, BO, SP, ZH, kFullCkpt, true>);
    } else {
      return hipErrorInvalidValue;
    }
  }
  return hipLaunchKernel(full, dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(pl.chunks),
                                    static_cast<unsigned>(pl.splits)),
                         dim3(W * 64), kargs, 0, st);
}

// Per padded state count: states per lane S, waves per block W (state
// groups), tile length T. N = 16 uses two states per lane on eight waves:
// half the LDS traffic per state update of one state per lane, which the LDS
// bandwidth (128 bytes per clock per CU) needs more than the extra waves.
template <bool BI, bool BO, bool SP, bool ZH>
int launch_ns(const ScanArgs& a, const ScanPlan& pl, const Scan& s, hipStream_t st) {
  switch (pl.NS) {
    case 1: return launch_sw<1, 1, 16, BI, BO, SP, ZH>(a, pl, s, st);
    case 2: return launch_sw<1, 2, 16, BI, BO, SP, ZH>(a, pl, s, st);
    case 4: return launch_sw<1, 4, 16, BI, BO, SP, ZH>(a, pl, s, st);
    case 8: return launch_sw<1, 8, 16, BI, BO, SP, ZH>(a, pl, s, st);
    case 16: return launch_sw<2, 8, 8, BI, BO, SP, ZH>(a, pl, s, st);
    case 32:
      // the 32-state halves of a split 64-state plan (float32 partials): four
      // states per lane on eight waves, B/C through LDS like the whole
      if constexpr (!BO) {
        if (pl.splits > 1) return launch_sw<4, 8, 8, BI, BO, SP, ZH, true>(a, pl, s, st);
      }
      if (pl.splits > 1) return hipErrorInvalidValue;
      return launch_sw<2, 16, 16, BI, BO, SP, ZH>(a, pl, s, st);
    case 64: return launch_sw<8, 8, 8, BI, BO, SP, ZH>(a, pl, s, st);   // B/C through LDS
    case 128: return launch_sw<16, 8, 8, BI, BO, SP, ZH>(a, pl, s, st);  // B/C through LDS
    default: return hipErrorInvalidValue;
  }
}

template <bool BI, bool BO>
int launch_io(const ScanArgs& a, const ScanPlan& pl, const Scan& s, hipStream_t st) {
  if (a.zoh) return a.delta_softplus ? launch_ns<BI, BO, true, true>(a, pl, s, st)
                                     : launch_ns<BI, BO, false, true>(a, pl, s, st);
  return a.delta_softplus ? launch_ns<BI, BO, true, false>(a, pl, s, st)
                          : launch_ns<BI, BO, false, false>(a, pl, s, st);
}

// Checkpoint pass of the backward: the recurrence only, storing every wave's
// states at each tile start, in tiles of scan_tile_steps(NS) steps (the
// backward kernel's). The layout of the checkpoints does not depend on the
// mapping, so the pass may use its own: at N = 16, one state per lane over
// sixteen waves (four per SIMD) hides the latency of a recurrence that has
// no readout to interleave (660 -> 609 us at (4, 8192, 4096, 16) bf16);
// otherwise the backward kernel's (states per lane S, waves W, tile T).
template <int S, int W, int T, bool BI, bool SP, bool ZH>
int launch_ckpt_sw(const Scan& s, int64_t blocks, hipStream_t st) {
  Scan args = s;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&scan_fwd_kernel<S, W, T, BI, false, SP, ZH, kCheckpoint>),
                         dim3(static_cast<unsigned>(blocks)), dim3(W * 64), kargs, 0, st);
}

template <bool BI, bool SP, bool ZH>
int launch_ckpt_ns(const ScanPlan& pl, const Scan& s, int64_t blocks, hipStream_t st) {
  switch (pl.NS) {
    case 1: return launch_ckpt_sw<1, 1, 16, BI, SP, ZH>(s, blocks, st);
    case 2: return launch_ckpt_sw<1, 2, 16, BI, SP, ZH>(s, blocks, st);
    case 4: return launch_ckpt_sw<1, 4, 16, BI, SP, ZH>(s, blocks, st);
    case 8: return launch_ckpt_sw<1, 8, 16, BI, SP, ZH>(s, blocks, st);
    case 16: return launch_ckpt_sw<1, 16, 8, BI, SP, ZH>(s, blocks, st);
    case 32: return launch_ckpt_sw<4, 8, 4, BI, SP, ZH>(s, blocks, st);
    case 64: return launch_ckpt_sw<8, 8, 2, BI, SP, ZH>(s, blocks, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool BI>
int launch_ckpt_io(const ScanArgs& a, const ScanPlan& pl, const Scan& s, int64_t blocks, hipStream_t st) {
  if (a.zoh) return a.delta_softplus ? launch_ckpt_ns<BI, true, true>(pl, s, blocks, st)
                                     : launch_ckpt_ns<BI, false, true>(pl, s, blocks, st);
  return a.delta_softplus ? launch_ckpt_ns<BI, true, false>(pl, s, blocks, st)
                          : launch_ckpt_ns<BI, false, false>(pl, s, blocks, st);
}

}  // namespace

}  // namespace ssm
