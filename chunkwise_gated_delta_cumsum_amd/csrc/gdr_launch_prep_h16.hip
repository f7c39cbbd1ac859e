// Launchers of the chunk-prep kernels for fp16 inputs, 64-row chunks.
#include "gdr_prep_launch.hpp"

namespace gdr {
gdr_status launch_prep_h16(const Prob& r, PrepArgs& a, bool dump, hipStream_t s) {
  return launch_prep_cp<64, PolicyH16>(r, a, dump, s);
}
}  // namespace gdr
