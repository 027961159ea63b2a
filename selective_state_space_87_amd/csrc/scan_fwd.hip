// Selective scan forward for gfx950: host-side launch of a planned scan.
// The kernels are in scan_fwd_impl.h, instantiated per dtype pair in
// scan_fwd_{bb,bf,fb,ff}.hip.
#include <hip/hip_runtime.h>

#include "scan_fwd_impl.h"

namespace ssm {

int scan_tile_steps(int NS) { return bwd_tile_steps(NS); }

namespace {

// Combine pass of a scan whose channels' states are split over two blocks:
// y = (part_0 + part_1 + D u) * silu(z), in that order, over the flattened
// [B, L, d] elements, four consecutive elements per thread (16-byte partial
// loads; u, z and y move as 8- or 16-byte runs). HBM-bound.
template <bool BI, bool BO>
__global__ __launch_bounds__(256) void scan_split_combine_kernel(const float* __restrict__ part, int64_t plane,
                                                                 const void* __restrict__ u,
                                                                 const void* __restrict__ z,
                                                                 const float* __restrict__ D, void* __restrict__ y,
                                                                 int64_t total, int dim) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * 4;
  for (int64_t i0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4; i0 < total; i0 += stride) {
    int ch = static_cast<int>(i0 % dim);
    float v[4];
    if (i0 + 4 <= total) {
      const float4 p0 = *reinterpret_cast<const float4*>(part + i0);
      const float4 p1 = *reinterpret_cast<const float4*>(part + plane + i0);
      float uv[4], zv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (BI) {
        const uint2 ub = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(u) + i0);
        uv[0] = __uint_as_float(ub.x << 16);
        uv[1] = __uint_as_float(ub.x & 0xffff0000u);
        uv[2] = __uint_as_float(ub.y << 16);
        uv[3] = __uint_as_float(ub.y & 0xffff0000u);
        if (z) {
          const uint2 zb = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(z) + i0);
          zv[0] = __uint_as_float(zb.x << 16);
          zv[1] = __uint_as_float(zb.x & 0xffff0000u);
          zv[2] = __uint_as_float(zb.y << 16);
          zv[3] = __uint_as_float(zb.y & 0xffff0000u);
        }
      } else {
        const float4 uf = *reinterpret_cast<const float4*>(static_cast<const float*>(u) + i0);
        uv[0] = uf.x, uv[1] = uf.y, uv[2] = uf.z, uv[3] = uf.w;
        if (z) {
          const float4 zf = *reinterpret_cast<const float4*>(static_cast<const float*>(z) + i0);
          zv[0] = zf.x, zv[1] = zf.y, zv[2] = zf.z, zv[3] = zf.w;
        }
      }
      const float pa[4] = {p0.x, p0.y, p0.z, p0.w}, pc[4] = {p1.x, p1.y, p1.z, p1.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float dv = D ? D[ch] : 0.0f;
        v[j] = ((pa[j] + pc[j]) + dv * uv[j]) * (z ? silu_f(zv[j]) : 1.0f);
        ch = ch + 1 == dim ? 0 : ch + 1;
      }
      if constexpr (BO) {
        const uint2 o = {static_cast<uint32_t>(f32_to_bf16_bits(v[0])) |
                             (static_cast<uint32_t>(f32_to_bf16_bits(v[1])) << 16),
                         static_cast<uint32_t>(f32_to_bf16_bits(v[2])) |
                             (static_cast<uint32_t>(f32_to_bf16_bits(v[3])) << 16)};
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + i0) = o;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(y) + i0) = make_float4(v[0], v[1], v[2], v[3]);
      }
    } else {
      for (int64_t i = i0; i < total; ++i) {
        const float uv = load_elem<BI>(u, i);
        const float dv = D ? D[ch] : 0.0f;
        const float out = ((part[i] + part[plane + i]) + dv * uv) * (z ? silu_f(load_elem<BI>(z, i)) : 1.0f);
        store_elem<BO>(y, i, out);
        ch = ch + 1 == dim ? 0 : ch + 1;
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
  const void* u = a.u;
  const void* z = a.z;
  const float* D = a.D;
  void* y = a.y;
  int dim = static_cast<int>(a.dim);
  void* kargs[] = {const_cast<float**>(&part), const_cast<int64_t*>(&plane), &u, &z, &D, &y,
                   const_cast<int64_t*>(&total), &dim};
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
  if (pl.splits > 1) {
    // Each block runs half of the padded states of its channels (64 of 128,
    // or 32 of 64) and writes their partial readout (float32, no skip, no
    // gate) to its plane; the combine pass then forms y.
    float* part = reinterpret_cast<float*>(ws + pl.off_part);
    Scan sh = s;
    sh.y = part;
    sh.y_split = pl.part_plane;
    sh.D = nullptr;
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
  if (a.in_bf16) return a.out_bf16 ? launch_scan_bb(a, pl, s, st) : launch_scan_bf(a, pl, s, st);
  return a.out_bf16 ? launch_scan_fb(a, pl, s, st) : launch_scan_ff(a, pl, s, st);
}

}  // namespace ssm
