// Launchers of the chunk-prep kernels (one decay per row, one per key
// channel), for both precision policies; C is the chunk length (this unit
// instantiates C = 64, gdr_launch_prep128.hip C = 128 and
// gdr_launch_prep32.hip C = 32).
#include "gdr_prep_launch.hpp"

namespace gdr {
gdr_status launch_prep(const Prob& r, PrepArgs& a, bool dump, hipStream_t s) {
  if (r.h16) {
    if (r.C == 128) return launch_prep128_h16(r, a, dump, s);
    if (r.C == 32) return launch_prep32_h16(r, a, dump, s);
    return launch_prep_h16(r, a, dump, s);
  }
  if (r.C == 128) return launch_prep128(r, a, dump, s);
  if (r.C == 32) return launch_prep32(r, a, dump, s);
  return launch_prep_c<64>(r, a, dump, s);
}
}  // namespace gdr
