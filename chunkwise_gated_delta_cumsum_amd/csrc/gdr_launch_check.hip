// The input range check kernels (see gdr_check.hpp) and their launcher.
#include "gdr_launch.hpp"

namespace gdr {

namespace {

__device__ __forceinline__ void flag_or(uint32_t* flags, uint32_t f) {
  // OR across the wave, then one vector atomic from lane 0
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) f |= (uint32_t)__shfl_xor((int)f, m);
  if ((threadIdx.x & 63) == 0 && f) atomicOr(flags, f);
}

__global__ void check_clear_kernel(uint32_t* flags) {
  if (threadIdx.x == 0) *flags = 0u;
}

// Bits of one 16-bit value (magnitude bits u): bf16 (inf/NaN from 0x7f80, fp16
// overflow from 0x4780) or fp16 (inf/NaN from 0x7c00, never out of range).
__device__ __forceinline__ uint32_t h16_bits(uint32_t u, int fmt, bool range) {
  if (u >= (fmt == 2 ? 0x7c00u : 0x7f80u)) return GDR_CHECK_NONFINITE;
  return (fmt == 1 && range && u >= 0x4780u) ? (uint32_t)GDR_CHECK_FP16_RANGE : 0u;
}

// bits of 8 16-bit values packed in 16 bytes
__device__ __forceinline__ uint32_t h16x8_bits(chk_u32x4 w, int fmt, bool range) {
  uint32_t f = 0;
  const uint32_t part[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f |= h16_bits((part[i] >> (16 * h)) & 0x7fffu, fmt, range);
    }
  }
  return f;
}

__device__ __forceinline__ uint32_t f32_bits(uint32_t u) {
  return (u & 0x7f800000u) == 0x7f800000u ? (uint32_t)GDR_CHECK_NONFINITE : 0u;
}

// One pass over a tensor of n elements (16-bit or fp32): 16-byte pieces
// grid-strided, then the tail one element at a time (n need not be a
// multiple of the piece).
__device__ __forceinline__ uint32_t scan_tensor(const void* x, size_t n, int fmt,
                                                bool range, size_t tid, size_t nthreads) {
  uint32_t f = 0;
  const bool h16 = fmt != 0;
  const size_t per = h16 ? 8 : 4;
  const size_t npieces = n / per;
  const chk_u32x4* p = reinterpret_cast<const chk_u32x4*>(x);
  for (size_t i = tid; i < npieces; i += nthreads) {
    const chk_u32x4 w = __builtin_nontemporal_load(p + i);
    if (h16) {
      f |= h16x8_bits(w, fmt, range);
    } else {
      f |= f32_bits(w[0]) | f32_bits(w[1]) | f32_bits(w[2]) | f32_bits(w[3]);
    }
  }
  for (size_t i = npieces * per + tid; i < n; i += nthreads) {
    if (h16) {
      f |= h16_bits(reinterpret_cast<const uint16_t*>(x)[i] & 0x7fffu, fmt, range);
    } else {
      f |= f32_bits(reinterpret_cast<const uint32_t*>(x)[i]);
    }
  }
  return f;
}

// q, k, v and beta, grid-strided.
__global__ void __launch_bounds__(256) check_tensors_kernel(CheckArgs a) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nth = (size_t)gridDim.x * blockDim.x;
  uint32_t f = scan_tensor(a.q, a.nqk, a.fmt, a.qk_range, tid, nth);
  f |= scan_tensor(a.k, a.nqk, a.fmt, a.qk_range, tid, nth);
  f |= scan_tensor(a.v, a.nv, a.fmt, true, tid, nth);
  f |= scan_tensor(a.beta, a.nbeta, 0, false, tid, nth);
  flag_or(a.flags, f);
}

// g: finiteness, and per (batch, chunk, value head, channel) the sum of the
// positive g over the chunk's rows.  One thread per (b, chunk, hv) and
// group of 4 channels (per-channel g) or per (b, chunk, hv) (one decay per
// row); consecutive threads take consecutive channels, then heads.
__global__ void __launch_bounds__(256) check_decay_kernel(CheckArgs a) {
  const int W = a.perch ? a.K / 4 : 1;
  const size_t total = (size_t)a.B * a.N * a.HV * W;
  const size_t nth = (size_t)gridDim.x * blockDim.x;
  uint32_t f = 0;
  for (size_t u = (size_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += nth) {
    const int w = (int)(u % W);
    const size_t bnh = u / W;
    const int hv = (int)(bnh % a.HV);
    const size_t bn = bnh / a.HV;
    const int n = (int)(bn % a.N), b = (int)(bn / a.N);
    const int t0 = n * a.C, t1 = min(a.T, t0 + a.C);
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    for (int t = t0; t < t1; ++t) {
      const size_t row = ((size_t)b * a.T + t) * a.HV + hv;
      if (a.perch) {
        const chk_f32x4 x = __builtin_nontemporal_load(
            reinterpret_cast<const chk_f32x4*>(a.g + row * a.K) + w);
        f |= f32_bits(__float_as_uint(x[0])) | f32_bits(__float_as_uint(x[1])) |
             f32_bits(__float_as_uint(x[2])) | f32_bits(__float_as_uint(x[3]));
        s0 += fmaxf(x[0], 0.f); s1 += fmaxf(x[1], 0.f);
        s2 += fmaxf(x[2], 0.f); s3 += fmaxf(x[3], 0.f);
      } else {
        const float x = __builtin_nontemporal_load(a.g + row);
        f |= f32_bits(__float_as_uint(x));
        s0 += fmaxf(x, 0.f);
      }
    }
    if (a.decay && fmaxf(fmaxf(s0, s1), fmaxf(s2, s3)) > kDecayLimit)
      f |= GDR_CHECK_DECAY_RANGE;
  }
  flag_or(a.flags, f);
}

// Workgroups of 256 lanes for `units` grid-strided units: enough to cover
// them, at most 8 rounds of the 256 compute units, at least one.
unsigned check_grid(size_t units) {
  const size_t want = (units + 255) / 256;
  return (unsigned)(want < 1 ? 1 : (want > 2048 ? 2048 : want));
}
}  // namespace

gdr_status launch_check(const Prob& r, CheckArgs& a, hipStream_t s) {
  uint32_t* flags = a.flags;
  gdr_status st = launch(check_clear_kernel, 1, 64, flags, s);
  if (st != GDR_OK) return st;
  const size_t per = a.fmt != 0 ? 8 : 4;
  size_t most = a.nqk > a.nv ? a.nqk : a.nv;
  if (a.nbeta > most) most = a.nbeta;
  st = launch(check_tensors_kernel, check_grid((most + per - 1) / per), 256, a, s);
  if (st != GDR_OK) return st;
  const size_t decay_units = (size_t)r.B * r.N * r.HV * (r.perch ? r.K / 4 : 1);
  return launch(check_decay_kernel, check_grid(decay_units), 256, a, s);
}

}  // namespace gdr
