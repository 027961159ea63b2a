// Execution plan of the selective scan (host only, no HIP): state mapping,
// sequence chunking and workspace layout, as a pure function of the sizes.
#include "kernels.h"

namespace ssm {

namespace {

int ceil_pow2(int64_t n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t m) { return ceil_div(a, m) * m; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

ScanPlan plan_scan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, bool allow_split) {
  ScanPlan p{};
  p.ok = batch >= 0 && seqlen >= 0 && dim >= 0 && dstate >= 1 && dstate <= kMaxScanStates &&
         seqlen < (int64_t(1) << 30) && dim < (int64_t(1) << 24);
  if (!p.ok) return p;
  // States: N padded to a power of two; one wave per state up to N = 8;
  // N = 16 two states per lane on eight waves, N = 32 two on sixteen, and
  // from 64 on NS / 8 states per lane on eight waves (B/C staged in LDS).
  p.NS = ceil_pow2(dstate);
  p.W = p.NS < 16 ? p.NS : (p.NS == 16 || p.NS >= 64 ? 8 : 16);
  p.S = p.NS / p.W;
  p.Lp = round_up(seqlen, kPadSteps);
  p.dim_blocks = ceil_div(dim, 64);
  p.chunks = 1;
  p.chunk = p.Lp;
  p.splits = 1;
  p.part_plane = 0;
  if (batch > 0 && dim > 0 && p.Lp > 0) {
    const int64_t blocks = batch * p.dim_blocks;
    int64_t k = 1;
    // From 64 padded states on a block holds 8x the work of the N = 16
    // shape: such scans are split only when most of the device would
    // otherwise idle, and into fewer chunks.
    const bool large = p.NS >= 64;
    if (blocks <= (large ? kChunkLargeWhenBlocksAtMost : kChunkWhenBlocksAtMost) &&
        p.Lp >= 2 * kChunkMinSteps) {
      k = (large ? kBlockSlotsLarge : kBlockSlots) / blocks;
      if (p.Lp / kChunkMinSteps < k) k = p.Lp / kChunkMinSteps;
      if (k < 1) k = 1;
    }
    // Every chunk's plane (counted at 4 bytes per element, whatever the
    // dtype) must stay within 32-bit buffer offsets with room for the
    // out-of-range markers.
    const int64_t steps_max = kPlaneBytesMax / (dim * 4) / kPadSteps * kPadSteps;
    if (steps_max < kPadSteps) {
      p.ok = false;
      return p;
    }
    if (ceil_div(p.Lp, steps_max) > k) k = ceil_div(p.Lp, steps_max);
    p.chunk = round_up(ceil_div(p.Lp, k), kPadSteps);
    if (p.chunk > steps_max) p.chunk = steps_max;
    p.chunks = ceil_div(p.Lp, p.chunk);
    // Two blocks of half the padded states per channel where one block per
    // channel would leave at least half of the device idle and the sequence
    // is not split in time. The partial readouts cross HBM once in float32
    // (written, then read by the combine pass), small beside 64 or 128 state
    // updates per element.
    if (allow_split && p.NS >= 64 && p.chunks == 1 && blocks > kChunkLargeWhenBlocksAtMost &&
        blocks <= kSplitWhenBlocksAtMost) {
      p.splits = 2;
      p.part_plane = round_up(batch * seqlen * dim, 64);
    }
  }
  // Workspace: packed B/C (one word per (b, n, step) for bfloat16 inputs,
  // two for float32; sized for float32; none from 64 padded states on, where
  // the kernel reads B and C as given), then the chunk summaries, then the
  // partial-readout planes of a split plan ([splits][B, L, d] float32).
  size_t off = 0;
  p.off_bc = off;
  if (batch > 0 && dim > 0 && p.Lp > 0 && p.NS < 64) off += align256(size_t(2 * batch * p.NS * p.Lp) * 4);
  p.off_hsum = off;
  if (p.chunks > 1) off += align256(size_t(p.chunks * batch * dim * dstate) * 4);
  p.off_ssum = off;
  if (p.chunks > 1) off += align256(size_t((p.chunks - 1) * batch * dim) * 4);
  p.off_part = off;
  if (p.splits > 1) off += align256(size_t(p.splits * p.part_plane) * 4);
  p.bytes = off;
  return p;
}

ScanBwdPlan plan_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  ScanBwdPlan p{};
  p.ok = batch >= 0 && seqlen >= 0 && dim >= 0 && dstate >= 1 && dstate <= kBwdMaxState &&
         seqlen < (int64_t(1) << 30) && dim < (int64_t(1) << 24) && batch < (int64_t(1) << 24) &&
         seqlen * dim * 4 <= kPlaneBytesMax;  // one pass per batch row: 32-bit buffer offsets
  if (!p.ok) return p;
  p.NS = ceil_pow2(dstate);
  p.W = bwd_waves(p.NS);
  p.S = p.NS / p.W;
  p.Lp = round_up(seqlen, kPadSteps);
  p.dim_blocks = ceil_div(dim, 64);
  // The kernel also addresses one batch row's packed B/C words (up to two per
  // step and state, float32 inputs) and one row of the per-block dB / dC
  // partials ([Lp][NS] floats) through 32-bit buffer offsets.
  if (int64_t(p.NS) * p.Lp * 8 > kPlaneBytesMax || int64_t(p.NS) * p.Lp * 4 > kPlaneBytesMax) {
    p.ok = false;
    return p;
  }
  const int64_t tiles = p.Lp / bwd_tile_steps(p.NS);  // checkpoint spacing
  size_t off = 0;
  p.off_bc = off;
  off += align256(size_t(2 * batch * p.NS * p.Lp) * 4);
  p.off_ckpt = off;
  off += align256(size_t(batch * tiles * p.NS * dim) * 4);
  p.off_dbp = off;
  off += align256(size_t(p.dim_blocks * batch * p.Lp * p.NS) * 4);
  p.off_dcp = off;
  off += align256(size_t(p.dim_blocks * batch * p.Lp * p.NS) * 4);
  p.off_dap = off;
  off += align256(size_t(batch * dim * dstate) * 4);
  p.off_ddp = off;
  off += align256(size_t(batch * dim) * 4);
  p.off_dbiasp = off;
  off += align256(size_t(batch * dim) * 4);
  p.bytes = off;
  return p;
}

size_t scan_checkpoint_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  const ScanBwdPlan p = plan_scan_bwd(batch, seqlen, dim, dstate);
  if (!p.ok || p.NS > 16) return 0;
  return size_t(batch) * size_t(p.Lp / bwd_tile_steps(p.NS)) * size_t(p.NS) * size_t(dim) * 4;
}

size_t scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  const ScanPlan p = plan_scan(batch, seqlen, dim, dstate);
  return p.ok ? p.bytes : 0;
}

}  // namespace ssm
