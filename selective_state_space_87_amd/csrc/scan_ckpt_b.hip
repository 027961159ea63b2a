// Checkpoint pass of the scan backward (the forward recurrence only, states
// stored at every tile start): instances for bfloat16 inputs.
#include "scan_fwd_impl.h"

namespace ssm {

int launch_ckpt_b(const ScanArgs& a, const ScanPlan& pl, const Scan& s, int64_t blocks, hipStream_t st) {
  return launch_ckpt_io<true>(a, pl, s, blocks, st);
}

}  // namespace ssm
