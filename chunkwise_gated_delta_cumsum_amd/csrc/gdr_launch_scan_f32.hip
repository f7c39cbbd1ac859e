// Launchers of the state-scan kernels with fp32 inputs and operands, both
// rules (the linear rule's own instantiation with 64-column slabs).
#include "gdr_scan_launch.hpp"

namespace gdr {
gdr_status launch_scan_f32(const Prob& r, ScanArgs& a, hipStream_t s) {
  if (r.linear && r.bv == 64) return launch_scan_policy<PolicyF32, true>(r, a, s);
  return launch_scan_policy<PolicyF32, false>(r, a, s);
}
}  // namespace gdr
