// Launchers of the state-scan kernels for 128-row chunks with fp32 inputs
// and operands, both rules.
#include "gdr_scan_launch.hpp"

namespace gdr {
gdr_status launch_scan128_f32(const Prob& r, ScanArgs& a, hipStream_t s) {
  return launch_scan_policy<PolicyF32, false, 128>(r, a, s);
}
}  // namespace gdr
