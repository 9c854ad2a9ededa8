// scan_inst_bf16_apply.hip -- the scan kernels of one element type (bfloat16 I/O) and one
// pass (apply), instantiated in a unit of their own so that the passes compile in parallel.
#include "scan_kernels.h"

namespace selscan {

hipError_t launch_scan_bf16_apply(bool ti, int S, int K, const ScanParams& p, hipStream_t stream) {
  return ti ? dispatch_sk<uint16_t, true, MODE_APPLY>(S, K, p, stream) : dispatch_sk<uint16_t, false, MODE_APPLY>(S, K, p, stream);
}

}  // namespace selscan
