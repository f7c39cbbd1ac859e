// Launchers of the state-scan kernels for fp16 inputs, 32-row chunks.
#include "gdr_scan_launch.hpp"

namespace gdr {
gdr_status launch_scan32_h16(const Prob& r, ScanArgs& a, hipStream_t s) {
  return launch_scan_policy<PolicyH16, false, 32>(r, a, s);
}
}  // namespace gdr
