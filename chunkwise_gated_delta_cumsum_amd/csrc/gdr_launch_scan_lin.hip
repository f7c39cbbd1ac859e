// Launchers of the linear rule's own state-scan instantiation with 16-bit
// operands (bf16 inputs, 64-column slabs).
#include "gdr_scan_launch.hpp"

namespace gdr {
gdr_status launch_scan_f16_linear(const Prob& r, ScanArgs& a, hipStream_t s) {
  return launch_scan_policy<PolicyF16, true>(r, a, s);
}
}  // namespace gdr
