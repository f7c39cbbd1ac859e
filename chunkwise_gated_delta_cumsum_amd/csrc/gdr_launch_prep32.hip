// Launchers of the chunk-prep kernels for 32-row chunks.
#include "gdr_prep_launch.hpp"

namespace gdr {
gdr_status launch_prep32(const Prob& r, PrepArgs& a, bool dump, hipStream_t s) {
  return launch_prep_c<32>(r, a, dump, s);
}
}  // namespace gdr
