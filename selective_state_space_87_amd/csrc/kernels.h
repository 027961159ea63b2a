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
  int in_bf16, out_bf16, delta_softplus, zoh;
  int allow_split;  // the plan may split a channel's states over blocks (see ScanPlan)
  float* ckpt;      // or null: also write the backward's state checkpoints (N <= 16)
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
  int in_bf16, out_bf16, delta_softplus, zoh;
};

struct ScanBwdArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* delta_bias;
  const float* h0;
  const float* dy;
  const float* dh_final;
  float* du;
  float* ddelta;
  float* dA;
  float* dB;
  float* dC;
  float* dD;
  float* dz;
  float* ddelta_bias;
  float* dh0;
  void* workspace;
  int64_t batch, seqlen, dim, dstate;
  int in_bf16, delta_softplus, zoh;
  const float* ckpt_in;  // or null: state checkpoints written by the forward (else recomputed)
};

struct ConvArgs {
  const void* x;
  const float* weight;
  const float* bias;
  const float* state_in;
  void* y;
  float* state_out;
  int64_t batch, seqlen, dim, width;
  int in_bf16, out_bf16, silu;
};

struct ConvUpdateArgs {
  float* state;
  const void* x;
  const float* weight;
  const float* bias;
  void* y;
  int64_t batch, dim, width;
  int in_bf16, out_bf16, silu;
};

struct SsdArgs {
  const void* x;         // [B, L, H, P]
  const void* dt;        // [B, L, H]
  const float* A;        // [H]
  const void* B;         // [B, L, N]
  const void* C;         // [B, L, N]
  const float* D;        // [H] or null
  const void* z;         // [B, L, H, P] or null
  const float* dt_bias;  // [H] or null
  const float* h0;       // [B, H, P, N] or null
  void* y;               // [B, L, H, P]
  float* h_final;        // [B, H, P, N] or null
  int64_t batch, seqlen, nheads, headdim, dstate;
  int in_bf16, out_bf16, dt_softplus;
};
// Largest head size and state size of the SSD kernel.
constexpr int64_t kSsdMaxHeadDim = 64;
constexpr int64_t kSsdMaxState = 128;

// How a scan of a given shape is run. The sequence is split into `chunks`
// pieces of `chunk` steps (the last may be shorter) when there are too few
// channel blocks to fill the device, or when one batch row's [L, d] plane is
// too large for 32-bit buffer offsets. A chunked scan is three launches after
// the B/C pre-pass: per-chunk summaries (local final state from zero, and the
// sum of the step sizes), an in-order fold of the summaries into each chunk's
// incoming state, and the full scan of every chunk from that state.
// With 64 or 128 padded states and too few channel blocks for the device but
// too many for time chunks to pay, a single-pass scan instead splits every
// channel's states over `splits` = 2 blocks of half the states each: each writes
// the float32 partial readout of its states, sum_n C h (the first block's
// plus D u), to a plane of the workspace (`part_plane` elements apart), and
// a combine pass forms y = (part_0 + part_1) silu(z).
// Pure function of the sizes (not of the device or the dtypes).
struct ScanPlan {
  bool ok;                 // false: sizes beyond what the kernels address
  int NS, W, S;            // padded state count, waves per block, states per lane
  int64_t Lp;              // sequence length padded to a multiple of kPadSteps
  int64_t chunk, chunks;   // steps per chunk (multiple of kPadSteps), chunk count
  int64_t dim_blocks;      // blocks of 64 channels per batch row
  int splits;              // blocks per channel (state groups of NS / splits)
  int64_t part_plane;      // elements per partial-readout plane (multiple of 64)
  size_t off_bc, off_hsum, off_ssum, off_part, bytes;  // workspace layout
};

constexpr int64_t kPadSteps = 16;        // tiles never straddle this boundary
constexpr int64_t kPlaneBytesMax = int64_t(1) << 30;   // per chunk and batch row
constexpr int64_t kChunkMinSteps = 1024;
// Blocks a chunked scan aims for: many per CU (about 12 for 256 CUs), so
// that each block's sequential walk is short and the last blocks to finish
// leave little of the device idle. Measured on the long-sequence shape
// (1, 262144, 2560, 16): 512 -> 6.0 ms, 1024 -> 5.5 ms, 2048 -> 5.0 ms,
// 3072 -> 4.75 ms, 4096 -> 4.78 ms.
constexpr int64_t kBlockSlots = 3072;
constexpr int64_t kChunkWhenBlocksAtMost = 128;
// From 64 padded states on (a block holds 8x the work of the N = 16 shape,
// and the summary pass adds about 0.8 of a pass over the split steps), a
// scan is split only when at most a quarter of the CUs would have a block,
// into about one block per CU. Measured (bf16, gate): (1, 8192, 4096, 128)
// 3317 -> 1752 us, (1, 8192, 2048, 64) 1719 -> 480 us; at 128 blocks,
// (2, 8192, 4096, 128), splitting lost (3356 -> 3500 us at 512 slots).
constexpr int64_t kBlockSlotsLarge = 256;
constexpr int64_t kChunkLargeWhenBlocksAtMost = 64;
// 64 or 128 padded states at 65 to 128 channel blocks: two blocks per channel.
constexpr int64_t kSplitWhenBlocksAtMost = 128;

// allow_split = false keeps every channel in one block (no partial planes in
// the workspace).
ScanPlan plan_scan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, bool allow_split = true);

// Backward: same state mapping (N <= 16), the forward's tiles; workspace
// = packed B/C, per-tile state checkpoints [B][tiles][NS][d], per-block
// partials of dB and dC [blocks_d][B][Lp][NS], per-batch partials of dA
// [B][d][N], dD and the bias gradient [B][d].
constexpr int64_t kBwdMaxState = 64;
// Backward (and its checkpoint pass) per padded state count NS: states per
// lane S, waves W and tile length T, with S * T = 16 from N = 16 on, so the
// per-tile register arrays stay the same size (eight waves of at most 256
// registers): NS <= 8: (1, NS, 16); 16: (2, 8, 8); 32: (4, 8, 4); 64: (8, 8, 2).
constexpr int bwd_tile_steps(int NS) { return NS <= 8 ? 16 : 128 / NS; }
constexpr int bwd_waves(int NS) { return NS <= 8 ? NS : 8; }
// Largest state size of the scan (padded to a power of two: 128).
constexpr int64_t kMaxScanStates = 128;
struct ScanBwdPlan {
  bool ok;
  int NS, W, S;
  int64_t Lp, dim_blocks;
  size_t off_bc, off_ckpt, off_dbp, off_dcp, off_dap, off_ddp, off_dbiasp, bytes;
};
ScanBwdPlan plan_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);
// Bytes of the backward's state checkpoints [B][Lp / T][NS][d] float32 (T =
// bwd_tile_steps(NS)), as the forward with checkpoints writes them; 0 where
// the backward does not run (its plan) or N > 16.
size_t scan_checkpoint_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

// Workspace bytes the scan needs for this shape.
size_t scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

// Enqueue the scan / decode kernels on `stream`. Arguments are already
// validated. Return 0 or the HIP error code of the failing launch.
int launch_scan(const ScanArgs& a, void* stream);
// The same, with the workspace in the library's fixed per-device scratch array
// (a.workspace is ignored); scan_scratch_bytes() is that array's size.
int launch_scan_noalloc(const ScanArgs& a, void* stream);
size_t scan_scratch_bytes();
int launch_state_update(const UpdateArgs& a, void* stream);
int launch_scan_bwd(const ScanBwdArgs& a, void* stream);
// Forward recurrence only (N <= 16, one pass over each batch row), storing the
// states at every tile start into ckpt [B][tiles][NS][d]; B/C already packed
// at bc. Tiles are scan_tile_steps(NS) steps long.
int launch_scan_checkpoints(const ScanArgs& a, const uint32_t* bc, float* ckpt, void* stream);
int scan_tile_steps(int NS);
int launch_conv1d_fwd(const ConvArgs& a, void* stream);
int launch_conv1d_update(const ConvUpdateArgs& a, void* stream);
int launch_ssd(const SsdArgs& a, void* stream);

}  // namespace ssm
