// Decode: one token of the gated delta rule per (batch, value head), the
// recurrent form the chunkwise algorithm reproduces (sec-03 notes, the naive
// recurrence the chunk form equals; "Chunkwise parallel algorithms" page,
// section 2.1, the delta rule; decode as the per-token half of serving in
// its inference discussion):
//
//   S' = diag(d) S + beta k u^T,  d = exp(g) (one value, or one per key channel)
//   u  = v - (diag(d) S)^T k
//   o  = scale S'^T q = scale ((diag(d) S)^T q + beta u (q . k))
//
// optionally with q and k L2-normalised first (x rsqrt(sum x^2 + 1e-6)),
// which the kernel applies as factors on the raw rows' sums, in fp32; or,
// for the decayed linear attention (the page's Mamba2 SSD section), with
// u = v: no erase term.
//
// The step reads and writes the K x V fp32 state once; every other operand is
// a vector, so the kernel is bound by HBM bandwidth on the state.  The
// columns of one state are independent (each column's sums run over the K
// rows only), so one workgroup of four waves takes VB columns of one
// (batch, value head): a lane owns four consecutive columns of K/4/RPI rows
// (RPI rows per wave instruction, VB/4 lanes per row), loads them all up
// front as 16-byte pieces of rows (coalesced), forms its partial column sums
// of k^T (dS) and q^T (dS), and keeps the values in registers for the
// update, which it writes back in place of the loads (so the state may be
// updated in place).  Narrow slabs give more workgroups per state, which
// keeps more of them in flight when the batch is small.
#pragma once
#include "gdr_device.hpp"

namespace gdr {

struct DecodeArgs {
  const void* q;         // [B, H, K]
  const void* k;         // [B, H, K]
  const void* v;         // [B, HV, V]
  const float* g;        // [B, HV] or [B, HV, K]
  const float* beta;     // [B, HV]
  const float* s_in;     // [B, HV, K, V] or null (zero state)
  float* s_out;          // [B, HV, K, V]; may equal s_in
  void* o;               // [B, HV, V] in the format o_fmt
  int o_fmt;             // kOutF32, kOutBF16 or kOutF16
  int B, H, HV;
  float scale;
  int l2norm;            // 1: L2-normalise q and k first
  int linear;            // 1: decayed linear attention: u = v (no erase term)
};

template <class T>
__device__ __forceinline__ float decode_in(const void* p, size_t i);
template <>
__device__ __forceinline__ float decode_in<float>(const void* p, size_t i) {
  return static_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float decode_in<uint16_t>(const void* p, size_t i) {
  return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16);   // bf16 bits
}
template <>
__device__ __forceinline__ float decode_in<_Float16>(const void* p, size_t i) {
  return (float)static_cast<const _Float16*>(p)[i];
}

template <int K, int V, int VB, bool PERCH, class IN>
__global__ __launch_bounds__(256) void decode_step_kernel(DecodeArgs a) {
  constexpr int LPR = VB / 4;       // lanes per state row
  constexpr int RPI = 64 / LPR;     // rows per wave instruction
  constexpr int RW = K / 4;         // rows per wave
  constexpr int IT = RW / RPI;      // float4 pieces per lane
  static_assert(RW % RPI == 0, "decode tile shape");
  __shared__ __attribute__((aligned(16))) float sq[K], sk[K], sd[K], sv[VB];
  __shared__ f32x4 sA[4][LPR], sB[4][LPR];
  __shared__ float sqk, srq, srk;   // q . k and the row normalisers of q and k

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int bh = blockIdx.x / (V / VB);
  const int v0 = (blockIdx.x % (V / VB)) * VB;   // first column of this slab
  const int b = bh / a.HV, hv = bh % a.HV;
  const int h = hv / (a.HV / a.H);
  const int c4 = lane % LPR;                 // columns 4 c4 .. 4 c4 + 3
  const int r0 = RW * wave + lane / LPR;     // first row; then every RPI rows

  // the state strip first: its loads are the long ones
  f32x4 s[IT];
  const size_t sbase = (size_t)bh * K * V;
  if (a.s_in) {
#pragma unroll
    for (int it = 0; it < IT; ++it)
      s[it] = *reinterpret_cast<const f32x4*>(a.s_in + sbase + (size_t)(r0 + RPI * it) * V + v0 +
                                              4 * c4);
  } else {
#pragma unroll
    for (int it = 0; it < IT; ++it) s[it] = zero4();
  }

  // the token's vectors into LDS
  const size_t qk0 = ((size_t)b * a.H + h) * K;
  if (tid < K) {
    sq[tid] = decode_in<IN>(a.q, qk0 + tid);
    sk[tid] = decode_in<IN>(a.k, qk0 + tid);
    sd[tid] = __expf(PERCH ? a.g[(size_t)bh * K + tid] : a.g[bh]);
  }
  if (tid >= 128 && tid - 128 < VB)
    sv[tid - 128] = decode_in<IN>(a.v, (size_t)bh * V + v0 + tid - 128);
  __syncthreads();
  if (wave == 0) {
    float x = 0.f, nq = 0.f, nk = 0.f;
    for (int i = lane; i < K; i += 64) {
      x += sq[i] * sk[i];
      nq += sq[i] * sq[i];
      nk += sk[i] * sk[i];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      x += __shfl_xor(x, off, 64);
      nq += __shfl_xor(nq, off, 64);
      nk += __shfl_xor(nk, off, 64);
    }
    if (lane == 0) {
      // with in-kernel normalisation, q^ = rq q and k^ = rk k: the sums
      // below use the raw rows and take the factors afterwards
      const float rq = a.l2norm ? rsqrtf(nq + kL2NormEps) : 1.f;
      const float rk = a.l2norm ? rsqrtf(nk + kL2NormEps) : 1.f;
      srq = rq;
      srk = rk;
      sqk = x * rq * rk;
    }
  }

  // decay, then the partial column sums k^T (dS) and q^T (dS) of this lane
  f32x4 A = zero4(), Bq = zero4();
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int row = r0 + RPI * it;
    s[it] *= sd[row];
    A += sk[row] * s[it];
    Bq += sq[row] * s[it];
  }
  // lanes holding the same columns in one wave: lane ^ LPR, ^ 2 LPR, ...
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      A[j] += __shfl_xor(A[j], off, 64);
      Bq[j] += __shfl_xor(Bq[j], off, 64);
    }
  if (lane < LPR) {
    sA[wave][c4] = A;
    sB[wave][c4] = Bq;
  }
  __syncthreads();
  A = srk * (sA[0][c4] + sA[1][c4] + sA[2][c4] + sA[3][c4]);
  Bq = srq * (sB[0][c4] + sB[1][c4] + sB[2][c4] + sB[3][c4]);
  const float bt = a.beta[bh];
  const f32x4 vv = *reinterpret_cast<const f32x4*>(sv + 4 * c4);
  const f32x4 u = a.linear ? vv : vv - A;
  if (wave == 0 && lane < LPR)
    store_o4(a.o, (size_t)bh * V + v0 + 4 * c4, a.scale * (Bq + (bt * sqk) * u), a.o_fmt);
  const f32x4 bu = (bt * srk) * u;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int row = r0 + RPI * it;
    __builtin_nontemporal_store(s[it] + sk[row] * bu, reinterpret_cast<f32x4*>(
                                    a.s_out + sbase + (size_t)row * V + v0 + 4 * c4));
  }
}

}  // namespace gdr
