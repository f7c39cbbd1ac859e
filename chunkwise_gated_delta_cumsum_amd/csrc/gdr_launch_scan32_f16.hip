// Launchers of the state-scan kernels for 32-row chunks with 16-bit
// operands (bf16 inputs), both rules.
#include "gdr_scan_launch.hpp"

namespace gdr {
gdr_status launch_scan32_f16(const Prob& r, ScanArgs& a, hipStream_t s) {
  return launch_scan_policy<PolicyF16, false, 32>(r, a, s);
}
}  // namespace gdr
