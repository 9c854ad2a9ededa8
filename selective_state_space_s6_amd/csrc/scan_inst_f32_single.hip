// scan_inst_f32_single.hip -- the scan kernels of one element type (fp32 I/O) and one
// pass (single), instantiated in a unit of their own so that the passes compile in parallel.
#include "scan_kernels.h"

namespace selscan {

hipError_t launch_scan_f32_single(bool ti, int S, int K, const ScanParams& p, hipStream_t stream) {
  return ti ? dispatch_sk<float, true, MODE_SINGLE>(S, K, p, stream) : dispatch_sk<float, false, MODE_SINGLE>(S, K, p, stream);
}

}  // namespace selscan
