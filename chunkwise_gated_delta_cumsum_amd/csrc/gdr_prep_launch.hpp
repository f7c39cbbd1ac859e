// Launch templates of the chunk-prep kernels, instantiated by the prep
// launcher translation units.
#pragma once
#include "gdr_launch.hpp"

namespace gdr {

template <int K, int C, bool PERCH, class P>
gdr_status launch_prep_k(const Prob& r, PrepArgs& a, bool dump, hipStream_t s) {
  // (batch, chunk) units rounded up to the 8 XCDs, times the value heads;
  // surplus workgroups exit (see prep_block)
  const size_t units8 = ((size_t)r.B * r.N + 7) / 8 * 8;
  const unsigned grid = (unsigned)(units8 * r.HV);
  constexpr unsigned block = C * 4;   // one wave per 16-row block
  if constexpr (PERCH) {
    if (r.l2norm)
      return dump ? launch(chunk_prep_kda_kernel<K, C, P, true, true>, grid, block, a, s)
                  : launch(chunk_prep_kda_kernel<K, C, P, false, true>, grid, block, a, s);
    return dump ? launch(chunk_prep_kda_kernel<K, C, P, true, false>, grid, block, a, s)
                : launch(chunk_prep_kda_kernel<K, C, P, false, false>, grid, block, a, s);
  } else {
    if (dump) return launch(chunk_prep_kernel<K, C, P, true>, grid, block, a, s);
    return launch(chunk_prep_kernel<K, C, P, false>, grid, block, a, s);
  }
}

template <int C, bool PERCH, class P>
gdr_status launch_prep_p(const Prob& r, PrepArgs& a, bool dump, hipStream_t s) {
  return r.K == 64 ? launch_prep_k<64, C, PERCH, P>(r, a, dump, s)
                   : launch_prep_k<128, C, PERCH, P>(r, a, dump, s);
}

template <int C, class P>
gdr_status launch_prep_cp(const Prob& r, PrepArgs& a, bool dump, hipStream_t s) {
  return r.perch ? launch_prep_p<C, true, P>(r, a, dump, s)
                 : launch_prep_p<C, false, P>(r, a, dump, s);
}

// fp32 and bf16 inputs; fp16 inputs have launcher units of their own
// (gdr_launch_prep*_h16.hip)
template <int C>
gdr_status launch_prep_c(const Prob& r, PrepArgs& a, bool dump, hipStream_t s) {
  if (r.f32) return launch_prep_cp<C, PolicyF32>(r, a, dump, s);
  return launch_prep_cp<C, PolicyF16>(r, a, dump, s);
}

}  // namespace gdr
