// C-ABI front end of libssm_scan.so: host-side validation, then dispatch to
// the kernel launchers. Plain C++ (no HIP headers): every check runs before
// anything touches the device, so an invalid call returns a status without
// side effects (and without a HIP device being present at all).
#include <cstdint>

#include "kernels.h"
#include "ssm_scan.h"

namespace {

constexpr int64_t kMaxScanState = ssm::kMaxScanStates;
constexpr int64_t kMaxDecodeState = 256;
constexpr int64_t kMaxCkptState = 16;  // forward checkpoints: the backward's tiles match the scan's
constexpr int64_t kMaxElems = int64_t(1) << 52;
constexpr int64_t kMaxConvWidth = 8;
constexpr int64_t kMaxConvSeq = int64_t(65535) * 64;  // 65535 segments of 64 steps

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};

Range span(const void* p, int64_t elems, int64_t elem_bytes) {
  Range r;
  if (p == nullptr || elems <= 0) return r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + static_cast<uintptr_t>(elems * elem_bytes);
  return r;
}

bool overlaps(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool safe_mul(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > kMaxElems / a) return false;
  *out = a * b;
  return *out <= kMaxElems;
}

int map_hip(int err) { return err == 0 ? SSM_OK : SSM_E_HIP; }

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_status_string(int status) {
  switch (status) {
    case SSM_OK: return "ok";
    case SSM_E_NULLPTR: return "a required pointer is NULL";
    case SSM_E_SHAPE: return "negative, overflowing or inconsistent size";
    case SSM_E_DTYPE: return "dtype code must be 0 (float32) or 1 (bfloat16)";
    case SSM_E_ALIGN: return "pointer not aligned as documented";
    case SSM_E_WORKSPACE: return "workspace missing or smaller than ssm_scan_workspace_bytes()";
    case SSM_E_ALIAS: return "an output overlaps an input it may not overlap";
    case SSM_E_UNSUPPORTED: return "size or option outside the supported range";
    case SSM_E_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

size_t ssm_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1 || dstate > kMaxScanState) return 0;
  int64_t t;
  if (!safe_mul(batch, seqlen, &t) || !safe_mul(t, dim, &t)) return 0;
  return ssm::scan_workspace_bytes(batch, seqlen, dim, dstate);
}

int64_t ssm_scan_chunks(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1 || dstate > kMaxScanState) return 0;
  int64_t t;
  if (!safe_mul(batch, seqlen, &t) || !safe_mul(t, dim, &t)) return 0;
  const ssm::ScanPlan p = ssm::plan_scan(batch, seqlen, dim, dstate);
  return p.ok ? p.chunks : 0;
}

}  // extern "C"

namespace {

// Validation and dispatch of the scan forward; with `noalloc` the workspace
// is the library's scratch array (workspace and workspace_bytes unused).
int scan_fwd_entry(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int in_dtype, int out_dtype,
                   int flags, const void* u, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, const float* h0, void* y,
                   float* h_final, void* workspace, size_t workspace_bytes, void* stream, bool noalloc,
                   bool want_ckpt = false, float* ckpt = nullptr) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1) return SSM_E_SHAPE;
  if (dstate > kMaxScanState) return SSM_E_UNSUPPORTED;
  // checkpoints for the backward: its sizes and N <= 16
  if (want_ckpt && (dstate > kMaxCkptState || !ssm::plan_scan_bwd(batch, seqlen, dim, dstate).ok)) {
    return SSM_E_UNSUPPORTED;
  }
  if ((in_dtype != 0 && in_dtype != 1) || (out_dtype != 0 && out_dtype != 1)) return SSM_E_DTYPE;
  if ((flags & ~(SSM_FLAG_SOFTPLUS | SSM_FLAG_ZOH)) != 0) return SSM_E_UNSUPPORTED;
  int64_t bl, bld, bln, bdn, dn;
  if (!safe_mul(batch, seqlen, &bl) || !safe_mul(bl, dim, &bld) || !safe_mul(bl, dstate, &bln) ||
      !safe_mul(batch, dim, &bdn) || !safe_mul(bdn, dstate, &bdn) || !safe_mul(dim, dstate, &dn)) {
    return SSM_E_SHAPE;
  }
  ssm::ScanPlan plan = ssm::plan_scan(batch, seqlen, dim, dstate);
  if (!plan.ok) return SSM_E_UNSUPPORTED;
  // The allocation-free entry runs a plan that splits states over blocks only
  // when its partial-readout planes fit the library's scratch array.
  bool allow_split = true;
  if (noalloc && plan.splits > 1 && plan.bytes > ssm::scan_scratch_bytes()) {
    allow_split = false;
    plan = ssm::plan_scan(batch, seqlen, dim, dstate, false);
  }
  if (batch == 0 || dim == 0) return SSM_OK;  // no channel: nothing to compute or write
  const int64_t isz = in_dtype == 1 ? 2 : 4, osz = out_dtype == 1 ? 2 : 4;
  if (A == nullptr) return SSM_E_NULLPTR;
  if (seqlen > 0 && (u == nullptr || delta == nullptr || B == nullptr || C == nullptr || y == nullptr)) {
    return SSM_E_NULLPTR;
  }
  const void* vec_ptrs[] = {u, delta, B, C, z, y};
  for (const void* p : vec_ptrs) {
    if (p && !aligned(p, 16)) return SSM_E_ALIGN;
  }
  const void* f32_ptrs[] = {A, D, delta_bias, h0, h_final};
  for (const void* p : f32_ptrs) {
    if (p && !aligned(p, 4)) return SSM_E_ALIGN;
  }
  const size_t need = plan.bytes;
  if (!noalloc && need > 0 && workspace != nullptr && !aligned(workspace, 16)) return SSM_E_ALIGN;
  if (noalloc) {
    if (need > ssm::scan_scratch_bytes()) return SSM_E_WORKSPACE;
    workspace = nullptr;  // a separate device allocation: overlaps nothing of the caller's
  } else if (need > 0 && (workspace == nullptr || workspace_bytes < need)) {
    return SSM_E_WORKSPACE;
  }

  const Range ry = span(y, seqlen > 0 ? bld : 0, osz);
  const Range rhf = span(h_final, bdn, 4);
  const Range rh0 = span(h0, bdn, 4);
  const Range inputs[] = {span(u, bld, isz), span(delta, bld, isz), span(z, bld, isz),
                          span(B, bln, isz), span(C, bln, isz), span(A, dn, 4),
                          span(D, dim, 4), span(delta_bias, dim, 4), rh0};
  for (const Range& r : inputs) {
    if (overlaps(ry, r)) return SSM_E_ALIAS;
  }
  if (overlaps(ry, rhf)) return SSM_E_ALIAS;
  for (int i = 0; i < 8; ++i) {  // h_final may equal h0 exactly, nothing else
    if (overlaps(rhf, inputs[i])) return SSM_E_ALIAS;
  }
  if (overlaps(rhf, rh0) && !(rhf.lo == rh0.lo && rhf.hi == rh0.hi)) return SSM_E_ALIAS;
  const Range rws = span(workspace, (need > 0 && !noalloc) ? static_cast<int64_t>(need) : 0, 1);
  for (const Range& r : inputs) {
    if (overlaps(rws, r)) return SSM_E_ALIAS;
  }
  if (overlaps(rws, ry) || overlaps(rws, rhf)) return SSM_E_ALIAS;
  if (want_ckpt && seqlen > 0) {
    if (ckpt == nullptr) return SSM_E_NULLPTR;
    if (!aligned(ckpt, 4)) return SSM_E_ALIGN;
    const Range rck = span(ckpt, static_cast<int64_t>(ssm::scan_checkpoint_bytes(batch, seqlen, dim, dstate)), 1);
    for (const Range& r : inputs) {
      if (overlaps(rck, r)) return SSM_E_ALIAS;
    }
    if (overlaps(rck, ry) || overlaps(rck, rhf) || overlaps(rck, rws)) return SSM_E_ALIAS;
  }

  ssm::ScanArgs a;
  a.u = u;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = D;
  a.z = z;
  a.delta_bias = delta_bias;
  a.h0 = h0;
  a.y = y;
  a.h_final = h_final;
  a.workspace = workspace;
  a.batch = batch;
  a.seqlen = seqlen;
  a.dim = dim;
  a.dstate = dstate;
  a.in_bf16 = in_dtype;
  a.out_bf16 = out_dtype;
  a.delta_softplus = (flags & SSM_FLAG_SOFTPLUS) != 0;
  a.zoh = (flags & SSM_FLAG_ZOH) != 0;
  a.allow_split = allow_split ? 1 : 0;
  a.ckpt = (want_ckpt && seqlen > 0) ? ckpt : nullptr;
  return map_hip(noalloc ? ssm::launch_scan_noalloc(a, stream) : ssm::launch_scan(a, stream));
}

}  // namespace

extern "C" {

int ssm_selective_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                           int in_dtype, int out_dtype, int flags,
                           const void* u, const void* delta, const float* A,
                           const void* B, const void* C, const float* D, const void* z,
                           const float* delta_bias, const float* h0,
                           void* y, float* h_final,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return scan_fwd_entry(batch, seqlen, dim, dstate, in_dtype, out_dtype, flags, u, delta, A, B, C, D, z,
                        delta_bias, h0, y, h_final, workspace, workspace_bytes, stream, false);
}

int ssm_selective_scan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                   int in_dtype, int out_dtype, int flags,
                                   const void* u, const void* delta, const float* A,
                                   const void* B, const void* C, const float* D, const void* z,
                                   const float* delta_bias, const float* h0,
                                   void* y, float* h_final, void* stream) {
  return scan_fwd_entry(batch, seqlen, dim, dstate, in_dtype, out_dtype, flags, u, delta, A, B, C, D, z,
                        delta_bias, h0, y, h_final, nullptr, 0, stream, true);
}

size_t ssm_scan_checkpoint_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1 || dstate > kMaxCkptState) return 0;
  int64_t t;
  if (!safe_mul(batch, seqlen, &t) || !safe_mul(t, dim, &t) || !safe_mul(t, dstate, &t)) return 0;
  return ssm::scan_checkpoint_bytes(batch, seqlen, dim, dstate);
}

int ssm_selective_scan_fwd_ckpt(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                int in_dtype, int out_dtype, int flags,
                                const void* u, const void* delta, const float* A,
                                const void* B, const void* C, const float* D, const void* z,
                                const float* delta_bias, const float* h0,
                                void* y, float* h_final, float* checkpoints,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return scan_fwd_entry(batch, seqlen, dim, dstate, in_dtype, out_dtype, flags, u, delta, A, B, C, D, z,
                        delta_bias, h0, y, h_final, workspace, workspace_bytes, stream, false, true, checkpoints);
}

int ssm_selective_state_update(int64_t batch, int64_t dim, int64_t dstate,
                               int in_dtype, int out_dtype, int flags,
                               float* state, const void* x, const void* delta,
                               const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias,
                               void* y, void* stream) {
  if (batch < 0 || dim < 0 || dstate < 1) return SSM_E_SHAPE;
  if (dstate > kMaxDecodeState) return SSM_E_UNSUPPORTED;
  if ((in_dtype != 0 && in_dtype != 1) || (out_dtype != 0 && out_dtype != 1)) return SSM_E_DTYPE;
  if ((flags & ~(SSM_FLAG_SOFTPLUS | SSM_FLAG_ZOH)) != 0) return SSM_E_UNSUPPORTED;
  int64_t bd, bdn, bn, dn;
  if (!safe_mul(batch, dim, &bd) || !safe_mul(bd, dstate, &bdn) || !safe_mul(batch, dstate, &bn) ||
      !safe_mul(dim, dstate, &dn)) {
    return SSM_E_SHAPE;
  }
  if (bd == 0) return SSM_OK;
  if (state == nullptr || x == nullptr || delta == nullptr || A == nullptr || B == nullptr ||
      C == nullptr || y == nullptr) {
    return SSM_E_NULLPTR;
  }
  const void* vec_ptrs[] = {x, delta, B, C, z, y};
  for (const void* p : vec_ptrs) {
    if (p && !aligned(p, 16)) return SSM_E_ALIGN;
  }
  const void* f32_ptrs[] = {state, A, D, delta_bias};
  for (const void* p : f32_ptrs) {
    if (p && !aligned(p, 4)) return SSM_E_ALIGN;
  }
  const int64_t isz = in_dtype == 1 ? 2 : 4, osz = out_dtype == 1 ? 2 : 4;
  const Range rs = span(state, bdn, 4);
  const Range ry = span(y, bd, osz);
  const Range inputs[] = {span(x, bd, isz), span(delta, bd, isz), span(z, bd, isz),
                          span(B, bn, isz), span(C, bn, isz), span(A, dn, 4),
                          span(D, dim, 4), span(delta_bias, dim, 4)};
  for (const Range& r : inputs) {
    if (overlaps(ry, r) || overlaps(rs, r)) return SSM_E_ALIAS;
  }
  if (overlaps(ry, rs)) return SSM_E_ALIAS;

  ssm::UpdateArgs a;
  a.state = state;
  a.x = x;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = D;
  a.z = z;
  a.delta_bias = delta_bias;
  a.y = y;
  a.batch = batch;
  a.dim = dim;
  a.dstate = dstate;
  a.in_bf16 = in_dtype;
  a.out_bf16 = out_dtype;
  a.delta_softplus = (flags & SSM_FLAG_SOFTPLUS) != 0;
  a.zoh = (flags & SSM_FLAG_ZOH) != 0;
  return map_hip(ssm::launch_state_update(a, stream));
}

size_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1) return 0;
  int64_t t;
  if (!safe_mul(batch, seqlen, &t) || !safe_mul(t, dim, &t) || !safe_mul(t, dstate, &t)) return 0;
  const ssm::ScanBwdPlan p = ssm::plan_scan_bwd(batch, seqlen, dim, dstate);
  return p.ok ? p.bytes : 0;
}

}  // extern "C"

namespace {

// Validation and dispatch of the scan backward; with `want_ckpt` the states
// at the tile starts come from `ckpt` (written by the forward with
// checkpoints) instead of the checkpoint pass.
int scan_bwd_entry(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int in_dtype, int flags,
                   const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                   const void* z, const float* delta_bias, const float* h0, const float* dy,
                   const float* dh_final, float* du, float* ddelta, float* dA, float* dB, float* dC, float* dD,
                   float* dz, float* ddelta_bias, float* dh0, void* workspace, size_t workspace_bytes,
                   void* stream, bool want_ckpt, const float* ckpt) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1) return SSM_E_SHAPE;
  if (want_ckpt && dstate > kMaxCkptState) return SSM_E_UNSUPPORTED;
  if (in_dtype != 0 && in_dtype != 1) return SSM_E_DTYPE;
  if ((flags & ~(SSM_FLAG_SOFTPLUS | SSM_FLAG_ZOH)) != 0) return SSM_E_UNSUPPORTED;
  int64_t bl, bld, bln, bdn, dn, bldn;
  if (!safe_mul(batch, seqlen, &bl) || !safe_mul(bl, dim, &bld) || !safe_mul(bl, dstate, &bln) ||
      !safe_mul(batch, dim, &bdn) || !safe_mul(bdn, dstate, &bdn) || !safe_mul(dim, dstate, &dn) ||
      !safe_mul(bld, dstate, &bldn)) {
    return SSM_E_SHAPE;
  }
  const ssm::ScanBwdPlan plan = ssm::plan_scan_bwd(batch, seqlen, dim, dstate);
  if (!plan.ok) return SSM_E_UNSUPPORTED;
  if (dim == 0) return SSM_OK;
  if (A == nullptr || dA == nullptr) return SSM_E_NULLPTR;
  if (bl > 0 && (u == nullptr || delta == nullptr || B == nullptr || C == nullptr || dy == nullptr ||
                 du == nullptr || ddelta == nullptr || dB == nullptr || dC == nullptr)) {
    return SSM_E_NULLPTR;
  }
  const void* vec_ptrs[] = {u, delta, B, C, z};
  for (const void* p : vec_ptrs) {
    if (p && !aligned(p, 16)) return SSM_E_ALIGN;
  }
  const void* f32_ptrs[] = {A, D, delta_bias, h0, dy, dh_final, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0};
  for (const void* p : f32_ptrs) {
    if (p && !aligned(p, 4)) return SSM_E_ALIGN;
  }
  const size_t need = plan.bytes;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return SSM_E_WORKSPACE;
  const bool use_ckpt = want_ckpt && bl > 0;
  if (use_ckpt && ckpt == nullptr) return SSM_E_NULLPTR;
  if (use_ckpt && !aligned(ckpt, 4)) return SSM_E_ALIGN;
  const int64_t ck_bytes = use_ckpt ? static_cast<int64_t>(ssm::scan_checkpoint_bytes(batch, seqlen, dim, dstate)) : 0;
  const int64_t isz = in_dtype == 1 ? 2 : 4;
  const Range inputs[] = {span(u, bld, isz), span(delta, bld, isz), span(z, bld, isz), span(B, bln, isz),
                          span(C, bln, isz), span(A, dn, 4), span(D, dim, 4), span(delta_bias, dim, 4),
                          span(h0, bdn, 4), span(dy, bld, 4), span(dh_final, bdn, 4),
                          span(use_ckpt ? ckpt : nullptr, ck_bytes, 1)};
  const Range outputs[] = {span(du, bld, 4), span(ddelta, bld, 4), span(dA, dn, 4), span(dB, bln, 4),
                           span(dC, bln, 4), span(D ? dD : nullptr, dim, 4), span(z ? dz : nullptr, bld, 4),
                           span(delta_bias ? ddelta_bias : nullptr, dim, 4), span(dh0, bdn, 4),
                           span(workspace, static_cast<int64_t>(need), 1)};
  constexpr int kOut = sizeof(outputs) / sizeof(outputs[0]);
  for (int i = 0; i < kOut; ++i) {
    for (const Range& r : inputs) {
      if (overlaps(outputs[i], r)) return SSM_E_ALIAS;
    }
    for (int j = i + 1; j < kOut; ++j) {
      if (overlaps(outputs[i], outputs[j])) return SSM_E_ALIAS;
    }
  }

  ssm::ScanBwdArgs a;
  a.u = u;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = D;
  a.z = z;
  a.delta_bias = delta_bias;
  a.h0 = h0;
  a.dy = dy;
  a.dh_final = dh_final;
  a.du = du;
  a.ddelta = ddelta;
  a.dA = dA;
  a.dB = dB;
  a.dC = dC;
  a.dD = D ? dD : nullptr;
  a.dz = z ? dz : nullptr;
  a.ddelta_bias = delta_bias ? ddelta_bias : nullptr;
  a.dh0 = dh0;
  a.workspace = workspace;
  a.batch = batch;
  a.seqlen = seqlen;
  a.dim = dim;
  a.dstate = dstate;
  a.in_bf16 = in_dtype;
  a.delta_softplus = (flags & SSM_FLAG_SOFTPLUS) != 0;
  a.zoh = (flags & SSM_FLAG_ZOH) != 0;
  a.ckpt_in = use_ckpt ? ckpt : nullptr;
  return map_hip(ssm::launch_scan_bwd(a, stream));
}

}  // namespace

extern "C" {

int ssm_selective_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                           int in_dtype, int flags,
                           const void* u, const void* delta, const float* A,
                           const void* B, const void* C, const float* D, const void* z,
                           const float* delta_bias, const float* h0,
                           const float* dy, const float* dh_final,
                           float* du, float* ddelta, float* dA, float* dB, float* dC,
                           float* dD, float* dz, float* ddelta_bias, float* dh0,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return scan_bwd_entry(batch, seqlen, dim, dstate, in_dtype, flags, u, delta, A, B, C, D, z, delta_bias, h0, dy,
                        dh_final, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, workspace, workspace_bytes,
                        stream, false, nullptr);
}

int ssm_selective_scan_bwd_ckpt(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                int in_dtype, int flags,
                                const void* u, const void* delta, const float* A,
                                const void* B, const void* C, const float* D, const void* z,
                                const float* delta_bias, const float* h0,
                                const float* dy, const float* dh_final,
                                float* du, float* ddelta, float* dA, float* dB, float* dC,
                                float* dD, float* dz, float* ddelta_bias, float* dh0,
                                const float* checkpoints,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return scan_bwd_entry(batch, seqlen, dim, dstate, in_dtype, flags, u, delta, A, B, C, D, z, delta_bias, h0, dy,
                        dh_final, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, workspace, workspace_bytes,
                        stream, true, checkpoints);
}

int ssm_causal_conv1d_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                          int in_dtype, int out_dtype, int silu_activation,
                          const void* x, const float* weight, const float* bias,
                          const float* state_in, void* y, float* state_out, void* stream) {
  if (batch < 0 || seqlen < 0 || dim < 0 || width < 1) return SSM_E_SHAPE;
  if (width > kMaxConvWidth || batch > 65535 || seqlen > kMaxConvSeq) return SSM_E_UNSUPPORTED;
  if ((in_dtype != 0 && in_dtype != 1) || (out_dtype != 0 && out_dtype != 1)) return SSM_E_DTYPE;
  int64_t bl, bld, bd, bds, dk;
  if (!safe_mul(batch, seqlen, &bl) || !safe_mul(bl, dim, &bld) || !safe_mul(batch, dim, &bd) ||
      !safe_mul(bd, width - 1, &bds) || !safe_mul(dim, width, &dk)) {
    return SSM_E_SHAPE;
  }
  if (batch == 0 || dim == 0) return SSM_OK;
  if (weight == nullptr) return SSM_E_NULLPTR;
  if (seqlen > 0 && (x == nullptr || y == nullptr)) return SSM_E_NULLPTR;
  if ((x && !aligned(x, 16)) || (y && !aligned(y, 16))) return SSM_E_ALIGN;
  const void* f32_ptrs[] = {weight, bias, state_in, state_out};
  for (const void* p : f32_ptrs) {
    if (p && !aligned(p, 4)) return SSM_E_ALIGN;
  }
  const int64_t isz = in_dtype == 1 ? 2 : 4, osz = out_dtype == 1 ? 2 : 4;
  const Range ry = span(y, seqlen > 0 ? bld : 0, osz);
  const Range rso = span(state_out, bds, 4);
  const Range inputs[] = {span(x, bld, isz), span(weight, dk, 4), span(bias, dim, 4), span(state_in, bds, 4)};
  for (const Range& r : inputs) {
    if (overlaps(ry, r) || overlaps(rso, r)) return SSM_E_ALIAS;
  }
  if (overlaps(ry, rso)) return SSM_E_ALIAS;

  ssm::ConvArgs a;
  a.x = x;
  a.weight = weight;
  a.bias = bias;
  a.state_in = state_in;
  a.y = y;
  a.state_out = state_out;
  a.batch = batch;
  a.seqlen = seqlen;
  a.dim = dim;
  a.width = width;
  a.in_bf16 = in_dtype;
  a.out_bf16 = out_dtype;
  a.silu = silu_activation ? 1 : 0;
  return map_hip(ssm::launch_conv1d_fwd(a, stream));
}

int ssm_causal_conv1d_update(int64_t batch, int64_t dim, int64_t width,
                             int in_dtype, int out_dtype, int silu_activation,
                             float* state, const void* x, const float* weight, const float* bias,
                             void* y, void* stream) {
  if (batch < 0 || dim < 0 || width < 1) return SSM_E_SHAPE;
  if (width > kMaxConvWidth) return SSM_E_UNSUPPORTED;
  if ((in_dtype != 0 && in_dtype != 1) || (out_dtype != 0 && out_dtype != 1)) return SSM_E_DTYPE;
  int64_t bd, bds, dk;
  if (!safe_mul(batch, dim, &bd) || !safe_mul(bd, width - 1, &bds) || !safe_mul(dim, width, &dk)) {
    return SSM_E_SHAPE;
  }
  if (bd == 0) return SSM_OK;
  if (x == nullptr || weight == nullptr || y == nullptr || (width > 1 && state == nullptr)) {
    return SSM_E_NULLPTR;
  }
  if (!aligned(x, 16) || !aligned(y, 16)) return SSM_E_ALIGN;
  const void* f32_ptrs[] = {state, weight, bias};
  for (const void* p : f32_ptrs) {
    if (p && !aligned(p, 4)) return SSM_E_ALIGN;
  }
  const int64_t isz = in_dtype == 1 ? 2 : 4, osz = out_dtype == 1 ? 2 : 4;
  const Range ry = span(y, bd, osz);
  const Range rs = span(state, bds, 4);
  const Range inputs[] = {span(x, bd, isz), span(weight, dk, 4), span(bias, dim, 4)};
  for (const Range& r : inputs) {
    if (overlaps(ry, r) || overlaps(rs, r)) return SSM_E_ALIAS;
  }
  if (overlaps(ry, rs)) return SSM_E_ALIAS;

  ssm::ConvUpdateArgs a;
  a.state = state;
  a.x = x;
  a.weight = weight;
  a.bias = bias;
  a.y = y;
  a.batch = batch;
  a.dim = dim;
  a.width = width;
  a.in_bf16 = in_dtype;
  a.out_bf16 = out_dtype;
  a.silu = silu_activation ? 1 : 0;
  return map_hip(ssm::launch_conv1d_update(a, stream));
}

int ssm_ssd_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                int in_dtype, int out_dtype, int flags,
                const void* x, const void* dt, const float* A, const void* B, const void* C,
                const float* D, const void* z, const float* dt_bias, const float* h0,
                void* y, float* h_final, void* stream) {
  if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 1 || dstate < 1) return SSM_E_SHAPE;
  if (headdim > ssm::kSsdMaxHeadDim || dstate > ssm::kSsdMaxState) return SSM_E_UNSUPPORTED;
  if ((in_dtype != 0 && in_dtype != 1) || (out_dtype != 0 && out_dtype != 1)) return SSM_E_DTYPE;
  if ((flags & ~SSM_FLAG_SOFTPLUS) != 0) return SSM_E_UNSUPPORTED;  // no zero-order-hold option here
  int64_t bl, blh, blhp, bln, bh, bhpn;
  if (!safe_mul(batch, seqlen, &bl) || !safe_mul(bl, nheads, &blh) || !safe_mul(blh, headdim, &blhp) ||
      !safe_mul(bl, dstate, &bln) || !safe_mul(batch, nheads, &bh) || !safe_mul(bh, headdim, &bhpn) ||
      !safe_mul(bhpn, dstate, &bhpn)) {
    return SSM_E_SHAPE;
  }
  if (bh > 0x7fffffff) return SSM_E_UNSUPPORTED;
  // a chunk's rows of x, z and y are addressed with 32-bit offsets
  if (nheads * headdim >= (int64_t(1) << 23)) return SSM_E_UNSUPPORTED;
  if (bh == 0) return SSM_OK;  // no head: nothing to compute or write
  if (A == nullptr) return SSM_E_NULLPTR;
  if (seqlen > 0 && (x == nullptr || dt == nullptr || B == nullptr || C == nullptr || y == nullptr)) {
    return SSM_E_NULLPTR;
  }
  const void* vec_ptrs[] = {x, dt, B, C, z, y};
  for (const void* q : vec_ptrs) {
    if (q && !aligned(q, 16)) return SSM_E_ALIGN;
  }
  const void* f32_ptrs[] = {A, D, dt_bias, h0, h_final};
  for (const void* q : f32_ptrs) {
    if (q && !aligned(q, 4)) return SSM_E_ALIGN;
  }
  const int64_t isz = in_dtype == 1 ? 2 : 4, osz = out_dtype == 1 ? 2 : 4;
  const Range ry = span(y, seqlen > 0 ? blhp : 0, osz);
  const Range rhf = span(h_final, bhpn, 4);
  const Range rh0 = span(h0, bhpn, 4);
  const Range inputs[] = {span(x, blhp, isz), span(dt, blh, isz), span(z, blhp, isz), span(B, bln, isz),
                          span(C, bln, isz), span(A, nheads, 4), span(D, nheads, 4), span(dt_bias, nheads, 4),
                          rh0};
  for (const Range& r : inputs) {
    if (overlaps(ry, r)) return SSM_E_ALIAS;
  }
  if (overlaps(ry, rhf)) return SSM_E_ALIAS;
  for (int i = 0; i < 8; ++i) {  // h_final may equal h0 exactly, nothing else
    if (overlaps(rhf, inputs[i])) return SSM_E_ALIAS;
  }
  if (overlaps(rhf, rh0) && !(rhf.lo == rh0.lo && rhf.hi == rh0.hi)) return SSM_E_ALIAS;

  ssm::SsdArgs a;
  a.x = x;
  a.dt = dt;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = D;
  a.z = z;
  a.dt_bias = dt_bias;
  a.h0 = h0;
  a.y = y;
  a.h_final = h_final;
  a.batch = batch;
  a.seqlen = seqlen;
  a.nheads = nheads;
  a.headdim = headdim;
  a.dstate = dstate;
  a.in_bf16 = in_dtype;
  a.out_bf16 = out_dtype;
  a.dt_softplus = (flags & SSM_FLAG_SOFTPLUS) != 0;
  return map_hip(ssm::launch_ssd(a, stream));
}

}  // extern "C"
