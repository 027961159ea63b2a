// Allocation-free variant of the selective scan forward: the workspace of
// ssm_selective_scan_fwd (packed B/C rows and, for a chunked plan, the chunk
// summaries) lives in a device array of fixed size that the library owns,
// one copy per GPU, instead of a buffer the caller passes. For callers that
// cannot allocate device memory at the time of the call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace ssm {

namespace {

// Largest workspace the allocation-free entry point serves (64 MiB: the
// long-sequence shape (1, 262144, 2560, 16) needs about 45 MB). Every GPU the
// library runs on holds one copy from the first use of this file's code until
// the process ends.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

}  // namespace

size_t scan_scratch_bytes() { return kScratchBytes; }

int launch_scan_noalloc(const ScanArgs& args, void* stream) {
  // The array's name is a host-side stand-in in this code: its device
  // address is looked up once per device, with that device current, and
  // only that address is handed to the kernels.
  static std::mutex mu;
  static void* dev_ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (dev_ptr[dev] == nullptr) {
      void* p = nullptr;
      err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (err != hipSuccess) return err;
      if (p == nullptr) return hipErrorInvalidSymbol;
      dev_ptr[dev] = p;
    }
    ws = dev_ptr[dev];
  }
  ScanArgs a = args;
  a.workspace = ws;
  return launch_scan(a, stream);
}

}  // namespace ssm
