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

// The chain pass (with sequence segments), then the full pass.  LIN selects
// the linear rule's own instantiation (64-column slabs, 64-row chunks: no Y,
// one barrier per chunk step); the general kernels drop the prediction term
// at run time.
template <int K, int V, bool PERCH, class P, int BV, int C, bool LIN = false>
gdr_status launch_scan_kvb(const Prob& r, ScanArgs& a, hipStream_t s) {
  constexpr int NW = scan_waves<K, C>();
  const size_t BHQ = (size_t)r.B * r.H;
  const int G = r.HV / r.H;
  auto grid_for = [&](int nsegu, int nslab) {
    // (batch, q/k head, segment) groups rounded up to a multiple of the 8
    // XCDs, times the value heads of a group and the slabs; surplus
    // workgroups exit (see unit_block)
    return (unsigned)((BHQ * nsegu + 7) / 8 * 8 * G * nslab);
  };
  gdr_status st;
  if (r.nseg > 1) {
    st = launch(chunk_scan_kernel<K, V, PERCH, P, kScanChain, BV, C, LIN>,
                grid_for(r.nseg - 1, (K + V) / BV), NW * 64, a, s);
    if (st != GDR_OK) return st;
  }
  ScanArgs f = full_pass_args(a);
  return launch(chunk_scan_kernel<K, V, PERCH, P, kScanFull, BV, C, LIN>,
                grid_for(r.nseg, V / BV), NW * 64, f, s);
}

// State columns per scan workgroup for 128-row chunks: 32 with K = 128 (8
// waves of one state row tile each; wider slabs would not fit the registers
// of two waves per SIMD), 64 with K = 64 (4 waves).
template <int K>
constexpr int slab_c128() { return K == 128 ? 32 : 64; }

// LINEAR selects the linear rule's instantiation (64-column slabs, 64-row
// chunks); otherwise the general kernels at the problem's slab width.
// 32-row chunks take the general kernels (2 waves) at 32 or 64 columns.
template <int K, int V, bool PERCH, class P, bool LINEAR, int C>
gdr_status launch_scan_kv(const Prob& r, ScanArgs& a, hipStream_t s) {
  if constexpr (C == 128) {
    return launch_scan_kvb<K, V, PERCH, P, slab_c128<K>(), 128>(r, a, s);
  } else if constexpr (C == 32) {
    return r.bv == 32 ? launch_scan_kvb<K, V, PERCH, P, 32, 32>(r, a, s)
                      : launch_scan_kvb<K, V, PERCH, P, 64, 32>(r, a, s);
  } else if constexpr (LINEAR) {
    return launch_scan_kvb<K, V, PERCH, P, 64, 64, true>(r, a, s);
  } else {
    return r.bv == 32 ? launch_scan_kvb<K, V, PERCH, P, 32, 64>(r, a, s)
                      : launch_scan_kvb<K, V, PERCH, P, 64, 64>(r, a, s);
  }
}

template <bool PERCH, class P, bool LINEAR, int C>
gdr_status launch_scan_p(const Prob& r, ScanArgs& a, hipStream_t s) {
  if (r.K == 64)
    return r.V == 64 ? launch_scan_kv<64, 64, PERCH, P, LINEAR, C>(r, a, s)
                     : launch_scan_kv<64, 128, PERCH, P, LINEAR, C>(r, a, s);
  return r.V == 64 ? launch_scan_kv<128, 64, PERCH, P, LINEAR, C>(r, a, s)
                   : launch_scan_kv<128, 128, PERCH, P, LINEAR, C>(r, a, s);
}

template <class P, bool LINEAR, int C = 64>
gdr_status launch_scan_policy(const Prob& r, ScanArgs& a, hipStream_t s) {
  return r.perch ? launch_scan_p<true, P, LINEAR, C>(r, a, s)
                 : launch_scan_p<false, P, LINEAR, C>(r, a, s);
}

}  // namespace gdr
