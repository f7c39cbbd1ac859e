// Launchers of the chunk-prep kernels (one decay per row, one per key
// channel), for both precision policies.
#include "gdr_launch.hpp"

namespace gdr {
namespace {

template <int K, bool PERCH, class P>
gdr_status launch_prep_k(const Prob& r, PrepArgs& a, bool dump, hipStream_t s) {
  // (batch, q/k head, chunk) units rounded up to the 8 XCDs, times the
  // value heads of each q/k head; surplus workgroups exit
  const size_t units8 = ((size_t)r.B * r.H * r.N + 7) / 8 * 8;
  const unsigned grid = (unsigned)(units8 * (r.HV / r.H));
  if constexpr (PERCH) {
    if (dump) return launch(chunk_prep_kda_kernel<K, P, true>, grid, 256, a, s);
    return launch(chunk_prep_kda_kernel<K, P, false>, grid, 256, a, s);
  } else {
    if (dump) return launch(chunk_prep_kernel<K, P, true>, grid, 256, a, s);
    return launch(chunk_prep_kernel<K, P, false>, grid, 256, a, s);
  }
}

template <bool PERCH, class P>
gdr_status launch_prep_p(const Prob& r, PrepArgs& a, bool dump, hipStream_t s) {
  return r.K == 64 ? launch_prep_k<64, PERCH, P>(r, a, dump, s)
                   : launch_prep_k<128, PERCH, P>(r, a, dump, s);
}

}  // namespace

gdr_status launch_prep(const Prob& r, PrepArgs& a, bool dump, hipStream_t s) {
  if (r.f32)
    return r.perch ? launch_prep_p<true, PolicyF32>(r, a, dump, s)
                   : launch_prep_p<false, PolicyF32>(r, a, dump, s);
  return r.perch ? launch_prep_p<true, PolicyF16>(r, a, dump, s)
                 : launch_prep_p<false, PolicyF16>(r, a, dump, s);
}


}  // namespace gdr
