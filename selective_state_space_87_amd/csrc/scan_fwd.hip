// Selective scan forward for gfx950: host-side launch of a planned scan.
// The kernels are in scan_fwd_impl.h, instantiated per dtype pair in
// scan_fwd_{bb,bf,fb,ff}.hip.
#include <hip/hip_runtime.h>

#include "scan_fwd_impl.h"

namespace ssm {

int scan_tile_steps(int NS) { return bwd_tile_steps(NS); }

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
  const ScanPlan pl = plan_scan(a.batch, a.seqlen, a.dim, a.dstate);
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
  if (!bcl) {
    const int err = launch_bc_pack(a.B, a.C, reinterpret_cast<uint32_t*>(ws + pl.off_bc), a.batch, a.seqlen,
                                   pl.Lp, static_cast<int>(a.dstate), pl.NS, a.in_bf16 != 0, st);
    if (err != 0) return err;
  }
  if (a.in_bf16) return a.out_bf16 ? launch_scan_bb(a, pl, s, st) : launch_scan_bf(a, pl, s, st);
  return a.out_bf16 ? launch_scan_fb(a, pl, s, st) : launch_scan_ff(a, pl, s, st);
}

}  // namespace ssm
