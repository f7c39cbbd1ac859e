// Launchers of the decode-step kernel.
#include "gdr_launch.hpp"

namespace gdr {
namespace {

template <int K, int V, int VB, bool PERCH>
gdr_status launch_decode_kvb(int in_fmt, DecodeArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)((size_t)a.B * a.HV * (V / VB));
  if (in_fmt == 0) return launch(decode_step_kernel<K, V, VB, PERCH, float>, grid, 256, a, s);
  if (in_fmt == 2) return launch(decode_step_kernel<K, V, VB, PERCH, _Float16>, grid, 256, a, s);
  return launch(decode_step_kernel<K, V, VB, PERCH, uint16_t>, grid, 256, a, s);
}

template <int K, int V, bool PERCH>
gdr_status launch_decode_kv(int vb, int in_fmt, DecodeArgs& a, hipStream_t s) {
  if (vb == 32) return launch_decode_kvb<K, V, 32, PERCH>(in_fmt, a, s);
  if constexpr (V == 128)
    if (vb == 128) return launch_decode_kvb<K, V, 128, PERCH>(in_fmt, a, s);
  return launch_decode_kvb<K, V, 64, PERCH>(in_fmt, a, s);
}

template <bool PERCH>
gdr_status launch_decode_p(int K, int V, int vb, int in_fmt, DecodeArgs& a, hipStream_t s) {
  if (K == 64)
    return V == 64 ? launch_decode_kv<64, 64, PERCH>(vb, in_fmt, a, s)
                   : launch_decode_kv<64, 128, PERCH>(vb, in_fmt, a, s);
  return V == 64 ? launch_decode_kv<128, 64, PERCH>(vb, in_fmt, a, s)
                 : launch_decode_kv<128, 128, PERCH>(vb, in_fmt, a, s);
}

}  // namespace

gdr_status launch_decode(int K, int V, int vb, bool perch, int in_fmt, DecodeArgs& a,
                         hipStream_t s) {
  return perch ? launch_decode_p<true>(K, V, vb, in_fmt, a, s)
               : launch_decode_p<false>(K, V, vb, in_fmt, a, s);
}

}  // namespace gdr
