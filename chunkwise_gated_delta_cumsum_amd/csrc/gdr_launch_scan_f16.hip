// Launchers of the state-scan kernels with 16-bit operands (bf16 inputs),
// general kernels (both rules; any slab width).
#include "gdr_scan_launch.hpp"

namespace gdr {
gdr_status launch_scan_f16(const Prob& r, ScanArgs& a, hipStream_t s) {
  return launch_scan_policy<PolicyF16, false>(r, a, s);
}
}  // namespace gdr
