// Launchers of the linear rule's own state-scan kernels for fp16 inputs
// (64-column slabs, 64-row chunks).
#include "gdr_scan_launch.hpp"

namespace gdr {
gdr_status launch_scan_h16_linear(const Prob& r, ScanArgs& a, hipStream_t s) {
  return launch_scan_policy<PolicyH16, true>(r, a, s);
}
}  // namespace gdr
