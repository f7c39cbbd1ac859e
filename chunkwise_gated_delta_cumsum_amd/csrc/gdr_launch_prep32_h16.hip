// Launchers of the chunk-prep kernels for fp16 inputs, 32-row chunks.
#include "gdr_prep_launch.hpp"

namespace gdr {
gdr_status launch_prep32_h16(const Prob& r, PrepArgs& a, bool dump, hipStream_t s) {
  return launch_prep_cp<32, PolicyH16>(r, a, dump, s);
}
}  // namespace gdr
