// Launch stand-ins for the sanitizer build of the C-ABI front end (api.cpp
// and plan.cpp compiled with AddressSanitizer and UndefinedBehaviorSanitizer,
// no HIP). Validation runs exactly as in the real library; a call that passes
// it reaches these functions, which report a launch failure (SSM_E_HIP at the
// ABI), so nothing here can compute a result.
#include <cstddef>
#include <cstdint>

#include "kernels.h"

namespace ssm {

namespace {
constexpr int kNoDevice = 100;  // any non-zero HIP error code
}

int launch_scan(const ScanArgs&, void*) { return kNoDevice; }
int launch_scan_noalloc(const ScanArgs&, void*) { return kNoDevice; }
size_t scan_scratch_bytes() { return size_t(64) << 20; }
int launch_state_update(const UpdateArgs&, void*) { return kNoDevice; }
int launch_scan_bwd(const ScanBwdArgs&, void*) { return kNoDevice; }
int launch_scan_checkpoints(const ScanArgs&, const uint32_t*, float*, void*) { return kNoDevice; }
int scan_tile_steps(int NS) { return bwd_tile_steps(NS); }
int launch_conv1d_fwd(const ConvArgs&, void*) { return kNoDevice; }
int launch_conv1d_update(const ConvUpdateArgs&, void*) { return kNoDevice; }
int launch_ssd(const SsdArgs&, void*) { return kNoDevice; }

}  // namespace ssm
