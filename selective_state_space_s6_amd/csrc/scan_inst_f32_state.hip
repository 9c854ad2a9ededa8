// scan_inst_f32_state.hip -- the scan kernels of one element type (fp32 I/O) and one
// pass (state), instantiated in a unit of their own so that the passes compile in parallel.
#include "scan_kernels.h"

namespace selscan {

hipError_t launch_scan_f32_state(bool ti, int S, int K, const ScanParams& p, hipStream_t stream) {
  return ti ? dispatch_sk<float, true, MODE_STATE>(S, K, p, stream) : dispatch_sk<float, false, MODE_STATE>(S, K, p, stream);
}

}  // namespace selscan
