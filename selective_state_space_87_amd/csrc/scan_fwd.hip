// Selective scan forward for gfx950: host-side launch of a planned scan.
// The kernels are in scan_fwd_impl.h, instantiated per dtype pair in
// scan_fwd_{bb,bf,fb,ff}.hip.
#include <hip/hip_runtime.h>

#include "scan_fwd_impl.h"

namespace ssm {

int scan_tile_steps(int NS) { return bwd_tile_steps(NS); }

namespace {

// Combine pass of a scan whose channels' states are split over two blocks:
// y = (part_0 + part_1) * silu(z) (part_0 holds the skip D u), over the
// flattened [B, L, d] elements, four consecutive elements per thread
// (16-byte partial loads; z and y move as 8- or 16-byte runs). HBM-bound.
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

template <bool BI, bool BO>
__global__ __launch_bounds__(256) void scan_split_combine_kernel(const float* __restrict__ part, int64_t plane,
                                                                 const void* __restrict__ z, void* __restrict__ y,
                                                                 int64_t total) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * 4;
  for (int64_t i0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4; i0 < total; i0 += stride) {
    if (i0 + 4 <= total) {
      const f32x4v p0 = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(part + i0));
      const f32x4v p1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(part + plane + i0));
      float v[4] = {p0.x + p1.x, p0.y + p1.y, p0.z + p1.z, p0.w + p1.w};
      if (z) {
        float zv[4];
        if constexpr (BI) {
          const u32x2v zb = __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(static_cast<const uint16_t*>(z) + i0));
          zv[0] = __uint_as_float(zb.x << 16);
          zv[1] = __uint_as_float(zb.x & 0xffff0000u);
          zv[2] = __uint_as_float(zb.y << 16);
          zv[3] = __uint_as_float(zb.y & 0xffff0000u);
        } else {
          const f32x4v zf = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(static_cast<const float*>(z) + i0));
          zv[0] = zf.x, zv[1] = zf.y, zv[2] = zf.z, zv[3] = zf.w;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] *= silu_f(zv[j]);
      }
      if constexpr (BO) {
        const u32x2v o = {static_cast<uint32_t>(f32_to_bf16_bits(v[0])) |
                              (static_cast<uint32_t>(f32_to_bf16_bits(v[1])) << 16),
                          static_cast<uint32_t>(f32_to_bf16_bits(v[2])) |
                              (static_cast<uint32_t>(f32_to_bf16_bits(v[3])) << 16)};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x2v*>(static_cast<uint16_t*>(y) + i0));
      } else {
        const f32x4v o = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4v*>(static_cast<float*>(y) + i0));
      }
    } else {
      for (int64_t i = i0; i < total; ++i) {
        const float out = (part[i] + part[plane + i]) * (z ? silu_f(load_elem<BI>(z, i)) : 1.0f);
        store_elem<BO>(y, i, out);
      }
    }
  }
}

template <bool BI, bool BO>
int launch_split_combine(const ScanArgs& a, const ScanPlan& pl, const float* part, hipStream_t st) {
  const int64_t total = a.batch * a.seqlen * a.dim;
  if (total == 0) return 0;
  const int64_t groups = (total + 3) / 4;
  const int64_t grid = groups < 256 * 2048 ? (groups + 255) / 256 : 2048;
  const int64_t plane = pl.part_plane;
  const void* z = a.z;
  void* y = a.y;
  void* kargs[] = {const_cast<float**>(&part), const_cast<int64_t*>(&plane), &z, &y, const_cast<int64_t*>(&total)};
  return hipLaunchKernel(reinterpret_cast<const void*>(&scan_split_combine_kernel<BI, BO>),
                         dim3(static_cast<unsigned>(grid)), dim3(256), kargs, 0, st);
}

}  // namespace

int launch_scan_checkpoints(const ScanArgs& a, const uint32_t* bc, float* ckpt, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const ScanPlan pl = plan_scan(a.batch, a.seqlen, a.dim, a.dstate);
  if (!pl.ok || pl.NS > kBwdMaxState || a.batch == 0 || a.dim == 0) return hipErrorInvalidValue;
  // one pass over the whole sequence: each batch row's plane must fit the
  // 32-bit buffer offsets
  if (a.seqlen * a.dim * 4 > kPlaneBytesMax) return hipErrorInvalidValue;
  Scan s{};
  s.u = a.u;
  s.delta = a.delta;
  s.A = a.A;
  s.bias = a.delta_bias;
  s.h0 = a.h0;
  s.BC = bc;
  s.Bm = a.B;   // read directly where B/C are staged through LDS (N = 64)
  s.Cm = a.C;
  s.hsum = ckpt;
  s.L = static_cast<int>(a.seqlen);
  s.Lp = static_cast<int>(pl.Lp);
  s.dim = static_cast<int>(a.dim);
  s.N = static_cast<int>(a.dstate);
  s.chunk = static_cast<int>(pl.Lp);
  s.batch = static_cast<int>(a.batch);
  const int64_t blocks = a.batch * pl.dim_blocks;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  return a.in_bf16 ? launch_ckpt_b(a, pl, s, blocks, st) : launch_ckpt_f(a, pl, s, blocks, st);
}

int launch_scan(const ScanArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.batch == 0 || a.dim == 0) return 0;
  const ScanPlan pl = plan_scan(a.batch, a.seqlen, a.dim, a.dstate, a.allow_split != 0);
  if (!pl.ok) return hipErrorInvalidValue;
  char* ws = static_cast<char*>(a.workspace);
  Scan s;
  s.u = a.u;
  s.delta = a.delta;
  s.z = a.z;
  s.A = a.A;
  s.D = a.D;
  s.bias = a.delta_bias;
  s.h0 = a.h0;
  s.carry = pl.chunks > 1 ? reinterpret_cast<const float*>(ws + pl.off_hsum) : nullptr;
  const bool bcl = bc_in_lds(pl.NS);
  s.BC = bcl ? nullptr : reinterpret_cast<const uint32_t*>(ws + pl.off_bc);
  s.Bm = a.B;
  s.Cm = a.C;
  s.y = a.y;
  s.h_final = a.h_final;
  s.hsum = pl.chunks > 1 ? reinterpret_cast<float*>(ws + pl.off_hsum) : nullptr;
  s.ssum = pl.chunks > 1 ? reinterpret_cast<float*>(ws + pl.off_ssum) : nullptr;
  s.L = static_cast<int>(a.seqlen);
  s.Lp = static_cast<int>(pl.Lp);
  s.dim = static_cast<int>(a.dim);
  s.N = static_cast<int>(a.dstate);
  s.chunk = static_cast<int>(pl.chunk);
  s.batch = static_cast<int>(a.batch);
  s.y_split = 0;
  s.ckpt = nullptr;
  s.ckpt_tiles = 0;
  // Checkpoints for the backward (N <= 16): a single-pass scan writes them
  // itself; a chunked one is preceded by the checkpoint pass.
  const bool ckpt_in_scan = a.ckpt != nullptr && pl.chunks == 1;
  if (ckpt_in_scan) {
    s.ckpt = a.ckpt;
    s.ckpt_tiles = static_cast<int>(pl.Lp / bwd_tile_steps(pl.NS));
  }
  if (a.ckpt != nullptr && (pl.NS > 16 || pl.splits > 1)) return hipErrorInvalidValue;
  if (pl.splits > 1) {
    // Each block runs half of the padded states of its channels (64 of 128,
    // or 32 of 64) and writes their partial readout (float32, without the
    // gate; the first block's with the skip D u) to its plane; the combine
    // pass then forms y.
    float* part = reinterpret_cast<float*>(ws + pl.off_part);
    Scan sh = s;
    sh.y = part;
    sh.y_split = pl.part_plane;
    sh.z = nullptr;
    ScanPlan ph = pl;
    ph.NS = pl.NS / pl.splits;
    ph.S = ph.NS / ph.W;
    int err = a.in_bf16 ? launch_scan_bf(a, ph, sh, st) : launch_scan_ff(a, ph, sh, st);
    if (err != 0) return err;
    if (a.in_bf16) return a.out_bf16 ? launch_split_combine<true, true>(a, pl, part, st)
                                     : launch_split_combine<true, false>(a, pl, part, st);
    return a.out_bf16 ? launch_split_combine<false, true>(a, pl, part, st)
                      : launch_split_combine<false, false>(a, pl, part, st);
  }
  if (!bcl) {
    const int err = launch_bc_pack(a.B, a.C, reinterpret_cast<uint32_t*>(ws + pl.off_bc), a.batch, a.seqlen,
                                   pl.Lp, static_cast<int>(a.dstate), pl.NS, a.in_bf16 != 0, st);
    if (err != 0) return err;
  }
  if (a.ckpt != nullptr && !ckpt_in_scan && pl.Lp > 0) {
    // before the scan, which may overwrite h0 with h_final
    const int err = launch_scan_checkpoints(a, reinterpret_cast<const uint32_t*>(ws + pl.off_bc), a.ckpt, st);
    if (err != 0) return err;
  }
  if (a.in_bf16) return a.out_bf16 ? launch_scan_bb(a, pl, s, st) : launch_scan_bf(a, pl, s, st);
  return a.out_bf16 ? launch_scan_fb(a, pl, s, st) : launch_scan_ff(a, pl, s, st);
}

}  // namespace ssm
