// Kernel launchers of the library, shared by gdr_api.hip (the host logic of
// the C ABI) and the launcher translation units, one per kernel family
// (gdr_launch_prep.hip, gdr_launch_prep128.hip, gdr_launch_scan_f16.hip,
// gdr_launch_scan_lin.hip, gdr_launch_scan_f32.hip, gdr_launch_scan128_f16.hip,
// gdr_launch_scan128_f32.hip, gdr_launch_scan32_f16.hip, gdr_launch_scan32_f32.hip,
// gdr_launch_prep32.hip, gdr_launch_decode.hip, gdr_launch_check.hip, and the
// fp16-input units gdr_launch_prep_h16.hip, gdr_launch_prep128_h16.hip,
// gdr_launch_prep32_h16.hip, gdr_launch_scan_h16.hip, gdr_launch_scan_lin_h16.hip,
// gdr_launch_scan128_h16.hip, gdr_launch_scan32_h16.hip), which instantiate the
// kernels and compile in parallel.
#pragma once
#include <hip/hip_runtime.h>

#include "gdr.h"
#include "gdr_check.hpp"
#include "gdr_decode.hpp"
#include "gdr_prep_kda.hpp"
#include "gdr_scan.hpp"

namespace gdr {

// A validated problem (see validate in gdr_api.hip).
struct Prob {
  int B, T, H, HV, K, V, N;
  int C;             // chunk length, 32, 64 or 128
  bool perch, f32;
  bool h16;          // fp16 q, k, v (else bf16 when !f32)
  float scale;
  size_t es;        // bytes per q/k/v element and per workspace fragment element
  int nseg, seg_len; // sequence segments of the state scan
  int bv;            // state columns per scan workgroup (32 or 64)
  bool l2norm;       // L2-normalise the q and k rows in the prep kernels
  bool linear;       // decayed linear attention (no erase term)
  int ofmt;          // o storage: kOutF32, kOutBF16 or kOutF16 (rounded once from fp32)
};

template <class Kern, class Args>
inline gdr_status launch(Kern kern, unsigned grid, unsigned block, Args& args, hipStream_t s) {
  void* kargs[] = {&args};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kern), dim3(grid),
                                       dim3(block), kargs, 0, s);
  return e == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

// Both stages and the decode step, on the caller's stream.
gdr_status launch_prep(const Prob& r, PrepArgs& a, bool dump, hipStream_t s);
gdr_status launch_prep128(const Prob& r, PrepArgs& a, bool dump, hipStream_t s);
gdr_status launch_prep32(const Prob& r, PrepArgs& a, bool dump, hipStream_t s);
gdr_status launch_scan_f16(const Prob& r, ScanArgs& a, hipStream_t s);
gdr_status launch_scan_f16_linear(const Prob& r, ScanArgs& a, hipStream_t s);
gdr_status launch_scan_f32(const Prob& r, ScanArgs& a, hipStream_t s);
gdr_status launch_scan128_f16(const Prob& r, ScanArgs& a, hipStream_t s);
gdr_status launch_scan128_f32(const Prob& r, ScanArgs& a, hipStream_t s);
gdr_status launch_scan32_f16(const Prob& r, ScanArgs& a, hipStream_t s);
gdr_status launch_scan32_f32(const Prob& r, ScanArgs& a, hipStream_t s);
// fp16 inputs (PolicyH16)
gdr_status launch_prep_h16(const Prob& r, PrepArgs& a, bool dump, hipStream_t s);
gdr_status launch_prep128_h16(const Prob& r, PrepArgs& a, bool dump, hipStream_t s);
gdr_status launch_prep32_h16(const Prob& r, PrepArgs& a, bool dump, hipStream_t s);
gdr_status launch_scan_h16(const Prob& r, ScanArgs& a, hipStream_t s);
gdr_status launch_scan_h16_linear(const Prob& r, ScanArgs& a, hipStream_t s);
gdr_status launch_scan128_h16(const Prob& r, ScanArgs& a, hipStream_t s);
gdr_status launch_scan32_h16(const Prob& r, ScanArgs& a, hipStream_t s);
// in_fmt: 0 fp32, 1 bf16, 2 fp16 inputs
gdr_status launch_decode(int K, int V, int vb, bool perch, int in_fmt, DecodeArgs& a,
                         hipStream_t s);
// The input range check (clears a.flags, then one pass over the inputs).
gdr_status launch_check(const Prob& r, CheckArgs& a, hipStream_t s);

}  // namespace gdr
