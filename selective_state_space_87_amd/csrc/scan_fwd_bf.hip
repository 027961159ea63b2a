// Selective scan forward: instances for bfloat16 inputs and float32 outputs.
#include "scan_fwd_impl.h"

namespace ssm {

int launch_scan_bf(const ScanArgs& a, const ScanPlan& pl, const Scan& s, hipStream_t st) {
  return launch_io<true, false>(a, pl, s, st);
}

}  // namespace ssm
