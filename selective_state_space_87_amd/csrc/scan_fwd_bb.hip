// Selective scan forward: instances for bfloat16 inputs and bfloat16 outputs.
#include "scan_fwd_impl.h"

namespace ssm {

int launch_scan_bb(const ScanArgs& a, const ScanPlan& pl, const Scan& s, hipStream_t st) {
  return launch_io<true, true>(a, pl, s, st);
}

}  // namespace ssm
