// Launchers of the state-scan kernels for fp16 inputs, 64-row chunks,
// general kernels (both rules; any slab width).
#include "gdr_scan_launch.hpp"

namespace gdr {
gdr_status launch_scan_h16(const Prob& r, ScanArgs& a, hipStream_t s) {
  return launch_scan_policy<PolicyH16, false>(r, a, s);
}
}  // namespace gdr
