// Launchers of the state-scan kernels for 32-row chunks with fp32 inputs,
// both rules.
#include "gdr_scan_launch.hpp"

namespace gdr {
gdr_status launch_scan32_f32(const Prob& r, ScanArgs& a, hipStream_t s) {
  return launch_scan_policy<PolicyF32, false, 32>(r, a, s);
}
}  // namespace gdr
