// Selective scan forward: instances for float32 inputs and float32 outputs.
#include "scan_fwd_impl.h"

namespace ssm {

int launch_scan_ff(const ScanArgs& a, const ScanPlan& pl, const Scan& s, hipStream_t st) {
  return launch_io<false, false>(a, pl, s, st);
}

}  // namespace ssm
