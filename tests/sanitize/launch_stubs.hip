// Kernel launchers of the C ABI replaced by stubs that fail, for the
// host-side sanitizer build of gdr_api.hip (tests/test_sanitizers.py): that
// build runs only calls that return before any launch (validation, size and
// choice queries, and calls made without a GPU), so no kernel code is needed.
#include "gdr_launch.hpp"

namespace gdr {
gdr_status launch_prep(const Prob&, PrepArgs&, bool, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_prep128(const Prob&, PrepArgs&, bool, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_prep32(const Prob&, PrepArgs&, bool, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_scan_f16(const Prob&, ScanArgs&, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_scan_f16_linear(const Prob&, ScanArgs&, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_scan_f32(const Prob&, ScanArgs&, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_scan128_f16(const Prob&, ScanArgs&, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_scan128_f32(const Prob&, ScanArgs&, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_scan32_f16(const Prob&, ScanArgs&, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_scan32_f32(const Prob&, ScanArgs&, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_prep_h16(const Prob&, PrepArgs&, bool, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_prep128_h16(const Prob&, PrepArgs&, bool, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_prep32_h16(const Prob&, PrepArgs&, bool, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_scan_h16(const Prob&, ScanArgs&, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_scan_h16_linear(const Prob&, ScanArgs&, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_scan128_h16(const Prob&, ScanArgs&, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_scan32_h16(const Prob&, ScanArgs&, hipStream_t) { return GDR_ERR_HIP; }
gdr_status launch_decode(int, int, int, bool, int, DecodeArgs&, hipStream_t) {
  return GDR_ERR_HIP;
}
gdr_status launch_check(const Prob&, CheckArgs&, hipStream_t) { return GDR_ERR_HIP; }
}  // namespace gdr
