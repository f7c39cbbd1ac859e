// Launch templates of the state-scan kernels, instantiated by the scan
// launcher translation units.
#pragma once
#include "gdr_launch.hpp"

namespace gdr {

// The full pass reads the chain pass's copy of the initial state when there
// is one (the state is then updated in place, see ScanArgs::s0_copy).
inline ScanArgs full_pass_args(const ScanArgs& a) {
  ScanArgs f = a;
  if (a.s0_copy) f.s0 = a.s0_copy;
  f.s0_copy = nullptr;
  return f;
}

template <int K, int V, bool PERCH, class P, int BV>
gdr_status launch_scan_kvb(const Prob& r, ScanArgs& a, hipStream_t s) {
  const size_t BH = (size_t)r.B * r.HV;
  auto grid_for = [](size_t units, int nslab) {
    // units rounded up to a multiple of the 8 XCDs; surplus workgroups exit
    return (unsigned)((units + 7) / 8 * 8 * nslab);
  };
  gdr_status st;
  if (r.nseg > 1) {
    st = launch(chunk_scan_kernel<K, V, PERCH, P, kScanChain, BV>,
                grid_for(BH * (r.nseg - 1), (K + V) / BV), kScanWaves * 64, a, s);
    if (st != GDR_OK) return st;
  }
  ScanArgs f = full_pass_args(a);
  return launch(chunk_scan_kernel<K, V, PERCH, P, kScanFull, BV>,
                grid_for(BH * r.nseg, V / BV), kScanWaves * 64, f, s);
}

// The linear rule with 64-column slabs runs its own instantiation (no Y, one
// barrier per chunk step); with 32-column slabs it takes the general kernels,
// which drop the prediction term at run time.
template <int K, int V, bool PERCH, class P>
gdr_status launch_scan_lin(const Prob& r, ScanArgs& a, hipStream_t s) {
  const size_t BH = (size_t)r.B * r.HV;
  auto grid_for = [](size_t units, int nslab) {
    return (unsigned)((units + 7) / 8 * 8 * nslab);
  };
  gdr_status st;
  if (r.nseg > 1) {
    st = launch(chunk_scan_kernel<K, V, PERCH, P, kScanChain, 64, true>,
                grid_for(BH * (r.nseg - 1), (K + V) / 64), kScanWaves * 64, a, s);
    if (st != GDR_OK) return st;
  }
  ScanArgs f = full_pass_args(a);
  return launch(chunk_scan_kernel<K, V, PERCH, P, kScanFull, 64, true>,
                grid_for(BH * r.nseg, V / 64), kScanWaves * 64, f, s);
}

// LINEAR selects the linear rule's instantiation (64-column slabs);
// otherwise the general kernels at the problem's slab width.
template <int K, int V, bool PERCH, class P, bool LINEAR>
gdr_status launch_scan_kv(const Prob& r, ScanArgs& a, hipStream_t s) {
  if constexpr (LINEAR) {
    return launch_scan_lin<K, V, PERCH, P>(r, a, s);
  } else {
    return r.bv == 32 ? launch_scan_kvb<K, V, PERCH, P, 32>(r, a, s)
                      : launch_scan_kvb<K, V, PERCH, P, 64>(r, a, s);
  }
}

template <bool PERCH, class P, bool LINEAR>
gdr_status launch_scan_p(const Prob& r, ScanArgs& a, hipStream_t s) {
  if (r.K == 64)
    return r.V == 64 ? launch_scan_kv<64, 64, PERCH, P, LINEAR>(r, a, s)
                     : launch_scan_kv<64, 128, PERCH, P, LINEAR>(r, a, s);
  return r.V == 64 ? launch_scan_kv<128, 64, PERCH, P, LINEAR>(r, a, s)
                   : launch_scan_kv<128, 128, PERCH, P, LINEAR>(r, a, s);
}

template <class P, bool LINEAR>
gdr_status launch_scan_policy(const Prob& r, ScanArgs& a, hipStream_t s) {
  return r.perch ? launch_scan_p<true, P, LINEAR>(r, a, s)
                 : launch_scan_p<false, P, LINEAR>(r, a, s);
}

}  // namespace gdr
