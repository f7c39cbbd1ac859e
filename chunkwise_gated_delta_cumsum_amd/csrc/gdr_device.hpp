// Device-side building blocks shared by the gfx950 kernels.
//
// MFMA fragment convention used everywhere in this library (wave64):
//   lane l, r = l % 16, grp = l / 16.
//   * A operand of a 16 x 32 tile: lane holds row r, 8 values at logical
//     k = kslot(grp, i), i = 0..7.
//   * B operand of a 32 x 16 tile: lane holds column r at the same k slots.
//   * C/D accumulator of a 16 x 16 tile: lane holds column r, rows 4*grp + j.
// kslot(grp, i) = 4*grp + (i & 3) + 16*(i >> 2) is chosen so that two
// vertically stacked accumulator tiles (rows 0-15 and 16-31) ARE a B operand
// with k = row, and the accumulator of X is the A operand of X^T.  Products
// therefore chain through registers without a transpose.  Both operands of
// every product use the same k slots, so the hardware's own k order inside
// an instruction does not matter.
#pragma once
#include <type_traits>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

#ifdef GDR_WG_TIMES
// Start and end of every workgroup on the chip-wide constant-rate clock
// (profiling builds only): [kernel kind][block][2], kind 0 prep, 1 chain
// pass, 3 full pass.
__device__ long long gdr_wg_times[4][32768][2];
#define GDR_WGT(kind, which)                                                      \
  do {                                                                            \
    if (threadIdx.x == 0 && blockIdx.x < 32768)                                   \
      gdr_wg_times[kind][blockIdx.x][which] = wall_clock64();                     \
  } while (0)
#else
#define GDR_WGT(kind, which) do {} while (0)
#endif

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Chunk lengths the kernels are built for.  Every tiling works on 16-row
// blocks of the chunk, one block per prep wave.
constexpr int kChunkMin = 32, kChunkMax = 128;

// Barrier for LDS traffic only: wait for this wave's LDS operations, then
// the workgroup barrier.  No kernel here reads global memory that another
// wave of its workgroup wrote, so outstanding global loads (a prefetch) and
// stores (outputs draining to memory) stay in flight; __syncthreads would
// wait for both.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int kslot(int grp, int i) {
  return 4 * grp + (i & 3) + 16 * (i >> 2);
}

// Key-channel order of the state.  Products over key channels do not care
// which channel sits in which k slot, so the state keeps its rows in an order
// where fragment slot i of lane group g (state row kslot(g, i) of a 32-row
// block) holds key channel 8g + i: every k or q fragment is then 8
// consecutive channels of one input row, a single 16-byte load.  Row x of
// the state is key channel chan_of_row(x); the inverse is row_of_chan.
__host__ __device__ __forceinline__ int chan_of_row(int x) {
  return (x & ~31) + 8 * ((x & 15) >> 2) + 4 * ((x & 31) >> 4) + (x & 3);
}
__host__ __device__ __forceinline__ int row_of_chan(int c) {
  return (c & ~31) + 4 * ((c & 31) >> 3) + 16 * ((c & 7) >> 2) + (c & 3);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Optional L2 normalisation of query and key rows inside the kernels, with
// the normaliser of the scalar-g kernel page: x * rsqrt(sum(x^2) + 1e-6).
// The sums run in fp32, and the factor multiplies the raw row in fp32
// wherever its values enter a product or an fp16 operand.
constexpr float kL2NormEps = 1e-6f;

// Sum of squares of the input elements in 16 bytes (8 fp16, 8 bf16 or 4 fp32).
template <class IN>
__device__ __forceinline__ float sumsq16(u32x4 v) {
  float s = 0.f;
  if constexpr (std::is_same_v<IN, _Float16>) {
    // each half through a scalar bit cast (a bit cast of v[i] to a vector of
    // two halves inside this unrolled loop compiled to four copies of v[0])
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = v[i];
      const float lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
      const float hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
      s += lo * lo + hi * hi;
    }
  } else if constexpr (sizeof(IN) == 2) {   // bf16 bits
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(v[i] << 16), hi = __uint_as_float(v[i] & 0xffff0000u);
      s += lo * lo + hi * hi;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) s += __uint_as_float(v[i]) * __uint_as_float(v[i]);
  }
  return s;
}


__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Four fp32 values rounded to bf16 (nearest even), as the bits of 8 bytes.
__device__ __forceinline__ u16x4 bf16x4_rne(f32x4 x) {
  u16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_bit_cast(uint16_t, (__bf16)x[i]);
  return r;
}

// Four fp32 values rounded to fp16 (nearest even), as the bits of 8 bytes.
__device__ __forceinline__ u16x4 f16x4_rne(f32x4 x) {
  u16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_bit_cast(uint16_t, (_Float16)x[i]);
  return r;
}

// Storage formats of o (gdr_problem::o_dtype).
constexpr int kOutF32 = 0, kOutBF16 = 1, kOutF16 = 2;

// Stores 4 consecutive o values at element offset e of o (fp32, or rounded
// once to bf16 or fp16 by fmt), streamed: o is not read again on the device.
__device__ __forceinline__ void store_o4(void* o, size_t e, f32x4 x, int fmt) {
  if (fmt == kOutBF16)
    __builtin_nontemporal_store(bf16x4_rne(x), reinterpret_cast<u16x4*>(
                                                   static_cast<uint16_t*>(o) + e));
  else if (fmt == kOutF16)
    __builtin_nontemporal_store(f16x4_rne(x), reinterpret_cast<u16x4*>(
                                                  static_cast<uint16_t*>(o) + e));
  else
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(static_cast<float*>(o) + e));
}

// Index of this wave in its workgroup, as a scalar.  Branches on it are then
// uniform scalar branches: an MFMA inside one is skipped as a whole instead of
// running under a partial EXEC mask, which MFMA does not honour.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// ---- products -------------------------------------------------------------
// 16x16 tile += (16 x 32) * (32 x 16)
__device__ __forceinline__ f32x4 mma32(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
  return c;
}
// 16x16 tile += (16 x 16) * (16 x 16) in fp32; lane holds k = 4*grp + i.
__device__ __forceinline__ f32x4 mma16_f32(f32x4 a, f32x4 b, f32x4 c) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
  return c;
}

// ---- precision policies ---------------------------------------------------
// F16: bf16 inputs, fp16 MFMA operands, fp16 workspace fragments.
// H16: fp16 inputs, used as they are as fp16 MFMA operands; fp16 workspace.
// F32: fp32 inputs, fp32 MFMA, fp32 workspace fragments.
// gfrag_t: the operand type of the decayed-dot Gram products, which take
// the raw input values (products of two 16-bit inputs are exact in fp32).
struct PolicyF16 {
  using in_t = uint16_t;   // bf16 bits
  using frag_t = half8;
  using ws_t = _Float16;
  using raw_t = u16x8;     // 8 input elements as loaded, before conversion
  using gfrag_t = bf16x8;
  static constexpr bool kF32 = false;
  __device__ static __forceinline__ raw_t load_raw(const in_t* row, int grp) {
    const u16x4 lo = *reinterpret_cast<const u16x4*>(row + 4 * grp);
    const u16x4 hi = *reinterpret_cast<const u16x4*>(row + 16 + 4 * grp);
    return raw_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  // 8 consecutive input elements (16 bytes), in slot order
  __device__ static __forceinline__ raw_t load_raw8(const in_t* p) {
    return *reinterpret_cast<const raw_t*>(p);
  }
  // convert raw input elements to a fragment; zero when !valid
  __device__ static __forceinline__ frag_t from_raw(raw_t x, bool valid) {
    frag_t f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = valid ? (_Float16)bf16_to_f32(x[i]) : (_Float16)0.f;
    return f;
  }
  // exact for every bf16 value inside the fp16 range (8 < 11 mantissa bits),
  // so the rounding mode of the packed conversion never matters there
  __device__ static __forceinline__ frag_t frag_from_raw(raw_t x) {
    const u32x4 d = __builtin_bit_cast(u32x4, x);
    frag_t f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto h2 = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(d[i] << 16),
                                                 __uint_as_float(d[i] & 0xffff0000u));
      f[2 * i] = h2[0];
      f[2 * i + 1] = h2[1];
    }
    return f;
  }
  __device__ static __forceinline__ float in_to_f32(in_t x) { return bf16_to_f32(x); }
  __device__ static __forceinline__ float raw_f32(raw_t x, int i) { return bf16_to_f32(x[i]); }
  // raw elements times f (fp32), rounded once to the fragment type
  __device__ static __forceinline__ frag_t frag_scaled(raw_t x, float f) {
    frag_t r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (_Float16)(bf16_to_f32(x[i]) * f);
    return r;
  }
  // 16x16 tile += (16 x 16) * (16 x 16), lane holds k = 4*grp + i; fp16
  // operands (the inverse is consumed as fp16 anyway), fp32 accumulation
  __device__ static __forceinline__ f32x4 mma16(f32x4 a, f32x4 b, f32x4 c) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    const h4 ah = {(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3]};
    const h4 bh = {(_Float16)b[0], (_Float16)b[1], (_Float16)b[2], (_Float16)b[3]};
    return __builtin_amdgcn_mfma_f32_16x16x16f16(ah, bh, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag_t make(const float* v) {
    frag_t f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (_Float16)v[i];
    return f;
  }
  __device__ static __forceinline__ frag_t make2(f32x4 lo, f32x4 hi) {
    frag_t f;
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = (_Float16)lo[i]; f[4 + i] = (_Float16)hi[i]; }
    return f;
  }
};

struct PolicyH16 {
  using in_t = _Float16;
  using frag_t = half8;
  using ws_t = _Float16;
  using raw_t = u16x8;     // fp16 bits as loaded
  using gfrag_t = half8;
  static constexpr bool kF32 = false;
  __device__ static __forceinline__ float h(uint16_t x) {
    return (float)__builtin_bit_cast(_Float16, x);
  }
  __device__ static __forceinline__ raw_t load_raw(const in_t* row, int grp) {
    const u16x4 lo = *reinterpret_cast<const u16x4*>(row + 4 * grp);
    const u16x4 hi = *reinterpret_cast<const u16x4*>(row + 16 + 4 * grp);
    return raw_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ static __forceinline__ raw_t load_raw8(const in_t* p) {
    return *reinterpret_cast<const raw_t*>(p);
  }
  __device__ static __forceinline__ frag_t from_raw(raw_t x, bool valid) {
    const frag_t f = __builtin_bit_cast(frag_t, x);
    return valid ? f : frag_t{};
  }
  __device__ static __forceinline__ frag_t frag_from_raw(raw_t x) {
    return __builtin_bit_cast(frag_t, x);
  }
  __device__ static __forceinline__ float in_to_f32(in_t x) { return (float)x; }
  __device__ static __forceinline__ float raw_f32(raw_t x, int i) { return h(x[i]); }
  __device__ static __forceinline__ frag_t frag_scaled(raw_t x, float f) {
    frag_t r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (_Float16)(h(x[i]) * f);
    return r;
  }
  __device__ static __forceinline__ f32x4 mma16(f32x4 a, f32x4 b, f32x4 c) {
    return PolicyF16::mma16(a, b, c);
  }
  __device__ static __forceinline__ frag_t make(const float* v) { return PolicyF16::make(v); }
  __device__ static __forceinline__ frag_t make2(f32x4 lo, f32x4 hi) {
    return PolicyF16::make2(lo, hi);
  }
};

struct PolicyF32 {
  using in_t = float;
  using frag_t = f32x8;
  using ws_t = float;
  using raw_t = f32x8;
  using gfrag_t = f32x8;
  static constexpr bool kF32 = true;
  __device__ static __forceinline__ raw_t load_raw(const in_t* row, int grp) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(row + 4 * grp);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(row + 16 + 4 * grp);
    return raw_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ static __forceinline__ raw_t load_raw8(const in_t* p) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
    return raw_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ static __forceinline__ frag_t from_raw(raw_t x, bool valid) {
    frag_t f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = valid ? x[i] : 0.f;
    return f;
  }
  __device__ static __forceinline__ frag_t frag_from_raw(raw_t x) { return x; }
  __device__ static __forceinline__ frag_t frag_scaled(raw_t x, float f) { return x * f; }
  __device__ static __forceinline__ float in_to_f32(in_t x) { return x; }
  __device__ static __forceinline__ float raw_f32(raw_t x, int i) { return x[i]; }
  __device__ static __forceinline__ f32x4 mma16(f32x4 a, f32x4 b, f32x4 c) {
    return mma16_f32(a, b, c);
  }
  __device__ static __forceinline__ frag_t make(const float* v) {
    frag_t f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = v[i];
    return f;
  }
  __device__ static __forceinline__ frag_t make2(f32x4 lo, f32x4 hi) {
    frag_t f;
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = lo[i]; f[4 + i] = hi[i]; }
    return f;
  }
};

// ---- fragment loads -------------------------------------------------------
// A/B fragment of a row-contiguous source (row pointer already offset to the
// first k of the 32-block): elements row[kslot(grp, i)].
template <class P>
__device__ __forceinline__ typename P::frag_t frag_row_f32(const float* row, int grp) {
  f32x4 lo = *reinterpret_cast<const f32x4*>(row + 4 * grp);
  f32x4 hi = *reinterpret_cast<const f32x4*>(row + 16 + 4 * grp);
  return P::make2(lo, hi);
}

// Same, from the input element type (bf16 bits or fp32), converted to the
// policy's fragment type.
__device__ __forceinline__ half8 frag_row_in(const uint16_t* row, int grp, PolicyF16) {
  u16x4 lo = *reinterpret_cast<const u16x4*>(row + 4 * grp);
  u16x4 hi = *reinterpret_cast<const u16x4*>(row + 16 + 4 * grp);
  half8 f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = (_Float16)bf16_to_f32(lo[i]);
    f[4 + i] = (_Float16)bf16_to_f32(hi[i]);
  }
  return f;
}
__device__ __forceinline__ half8 frag_row_in(const _Float16* row, int grp, PolicyH16) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  const h4 lo = *reinterpret_cast<const h4*>(row + 4 * grp);
  const h4 hi = *reinterpret_cast<const h4*>(row + 16 + 4 * grp);
  return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ f32x8 frag_row_in(const float* row, int grp, PolicyF32) {
  f32x4 lo = *reinterpret_cast<const f32x4*>(row + 4 * grp);
  f32x4 hi = *reinterpret_cast<const f32x4*>(row + 16 + 4 * grp);
  f32x8 f;
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[i] = lo[i]; f[4 + i] = hi[i]; }
  return f;
}

// Raw bf16 fragment (no conversion) for exact bf16 x bf16 Gram products.
__device__ __forceinline__ bf16x8 frag_row_bf16(const uint16_t* row, int grp) {
  u16x4 lo = *reinterpret_cast<const u16x4*>(row + 4 * grp);
  u16x4 hi = *reinterpret_cast<const u16x4*>(row + 16 + 4 * grp);
  u16x8 u;
#pragma unroll
  for (int i = 0; i < 4; ++i) { u[i] = lo[i]; u[4 + i] = hi[i]; }
  return __builtin_bit_cast(bf16x8, u);
}

// A/B fragment of a row-contiguous workspace-type source: row[kslot(grp, i)].
__device__ __forceinline__ half8 frag_row_ws(const _Float16* row, int grp) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  const h4 lo = *reinterpret_cast<const h4*>(row + 4 * grp);
  const h4 hi = *reinterpret_cast<const h4*>(row + 16 + 4 * grp);
  return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ f32x8 frag_row_ws(const float* row, int grp) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(row + 4 * grp);
  const f32x4 hi = *reinterpret_cast<const f32x4*>(row + 16 + 4 * grp);
  return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Workspace fragment: 8 consecutive ws_t per lane.
__device__ __forceinline__ half8 frag_ws(const _Float16* p) {
  return *reinterpret_cast<const half8*>(p);
}
__device__ __forceinline__ f32x8 frag_ws(const float* p) {
  f32x4 lo = *reinterpret_cast<const f32x4*>(p);
  f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
  f32x8 f;
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[i] = lo[i]; f[4 + i] = hi[i]; }
  return f;
}
// Workspace writes are streamed (non-temporal): the next kernel reads them
// from another XCD's L2 or from memory anyway, and lines that stay dirty in
// this L2 only lengthen the write-back at the kernel boundary.
__device__ __forceinline__ void store_ws(_Float16* p, f32x4 lo, f32x4 hi) {
  half8 f;
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[i] = (_Float16)lo[i]; f[4 + i] = (_Float16)hi[i]; }
  __builtin_nontemporal_store(f, reinterpret_cast<half8*>(p));
}
__device__ __forceinline__ void store_ws(float* p, f32x4 lo, f32x4 hi) {
  __builtin_nontemporal_store(lo, reinterpret_cast<f32x4*>(p));
  __builtin_nontemporal_store(hi, reinterpret_cast<f32x4*>(p + 4));
}
__device__ __forceinline__ void store_ws8(_Float16* p, const float* v) {
  half8 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (_Float16)v[i];
  __builtin_nontemporal_store(f, reinterpret_cast<half8*>(p));
}
__device__ __forceinline__ void store_ws8(float* p, const float* v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

__device__ __forceinline__ void store_ws4(_Float16* p, const float* v) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<h4*>(p) = h4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
}
__device__ __forceinline__ void store_ws4(float* p, const float* v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
}

// A fragment's 8 elements to 8 consecutive workspace-type elements whose
// address is 16-byte aligned (LDS or global)
__device__ __forceinline__ void store_frag16(_Float16* p, half8 f) {
  *reinterpret_cast<half8*>(p) = f;
}
__device__ __forceinline__ void store_frag16(float* p, f32x8 f) {
  *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
}

// ---- workspace layout -----------------------------------------------------
// Per chunk (one value head, C = 64 or 128 rows), in fragment order so every
// lane reads or writes 8 consecutive elements:
//   wt : W^ = M^-T diag(beta exp(gamma_last - gamma)) k   as the A operand of
//        W^T (rows d, k = c): [K/16 row tiles][C/32 k-blocks][64 lanes][8]
//   ah : A^ = A_qk M^-1 as an A operand (rows i, k = c), lower triangular:
//        only the k-blocks kb <= I/2 of row tile I are stored, in order
//        (ah_frag below), [C/16 (C/32 + 1) / 4 ... ][64][8]
//   rs : 256 fp32: [0..C) exp(gamma_c) (one decay per row; 1 per channel),
//        [C..C+K) exp(gamma_last) per key channel in the state's row order
//        (C + K <= 256); with one decay per row only [C] is written
//   qh, kh : the scan's q and k operands as A fragments (rows c, k = d):
//        [C/16][K/32][64][8] per chunk; lane (r, g) of fragment (ct, kb) holds
//        key channels 32 kb + 8 g .. +7 of row 16 ct + r.  Per channel they
//        are q exp(gamma) scale and k exp(gamma), one per value-head chunk;
//        with one decay per row they are q and k themselves, converted to
//        the workspace type, one per query-head chunk.
//   phi, eend : sequence segments (when more than one): transitions
//        [B*HV][nseg-1][K][K] in the workspace type (A-fragment order) and
//        zero-start end states [B*HV][nseg-1][K*V] fp32 (tile order).
//   s0c : with sequence segments, room for a copy of the initial state
//        [B*HV][K][V] fp32, used when the state is updated in place.
struct WsLayout {
  size_t wt, ah, rs, qh, kh, phi, eend, s0c, total;
};

__host__ __device__ inline size_t ws_align(size_t x) { return (x + 255) & ~(size_t)255; }

// Fragments of A^ per chunk (the lower-triangular k-blocks), and the index of
// fragment (row tile I, k-block kb <= I / 2) among them.
__host__ __device__ constexpr int ah_frags(int C) {
  return (C / 16) * (C / 16 + 2) / 4;   // sum over I of (I / 2 + 1)
}
__host__ __device__ constexpr int ah_frag(int I, int kb) {
  return (I / 2) * (I / 2 + 1) + (I & 1) * (I / 2 + 1) + kb;
}

// nchunks = B * HV * N value-head chunks; qkchunks = chunks that carry their
// own q/k fragments (B * H * N with one decay per row, nchunks per channel).
__host__ __device__ inline WsLayout ws_layout(size_t nchunks, size_t qkchunks, int C, int K,
                                              int V, size_t elem, size_t nheads, int nseg) {
  WsLayout L;
  size_t off = 0;
  L.wt = off; off = ws_align(off + nchunks * (size_t)K * C * elem);
  L.ah = off; off = ws_align(off + nchunks * (size_t)ah_frags(C) * 512 * elem);
  L.rs = off; off = ws_align(off + nchunks * 256 * sizeof(float));
  L.qh = off; off = ws_align(off + qkchunks * (size_t)C * K * elem);
  L.kh = off; off = ws_align(off + qkchunks * (size_t)C * K * elem);
  L.phi = L.eend = L.s0c = off;
  if (nseg > 1) {
    L.phi = off; off = ws_align(off + nheads * (nseg - 1) * (size_t)K * K * elem);
    L.eend = off; off = ws_align(off + nheads * (nseg - 1) * (size_t)K * V * sizeof(float));
    L.s0c = off; off = ws_align(off + nheads * (size_t)K * V * sizeof(float));
  }
  L.total = off;
  return L;
}

}  // namespace gdr
