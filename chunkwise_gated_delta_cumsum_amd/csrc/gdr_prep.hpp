// Chunk preparation: everything that is parallel across chunks.
//
// One workgroup (4 waves) per (batch, value head, chunk of C = 64 rows).
// Steps, following the sec-03 notes ("in-chunk cumsum and lower-triangular
// solve", "decayed dot function") and the UT transform of the "Chunkwise
// parallel algorithms" page (section 2.3):
//   1. gamma = inclusive cumsum of g over the chunk.
//   2. Gram tiles of k k^T and k q^T on MFMA (lower 16x16 tiles only), the
//      decay exp(gamma_i - gamma_j), beta on columns and the masks: strict
//      lower for A_kk, lower with diagonal for A_qk (scale folded in).  A_qk
//      is formed transposed, so its accumulator tiles are directly the B
//      operands of step 4b and stay in registers.
//   3. M = I + A_kk; M^-1 by blocks: each wave inverts one 16x16 unit-lower
//      diagonal block by forward substitution, then wave J forms block column
//      J: X_IJ = -D_I sum_m L_Im X_mJ for I > J.
//   4. Fold the UT transform into the operands of the serial scan:
//        W^ = M^-T diag(beta exp(gamma_last - gamma)) k   (so W^T Z = K~^T diag(beta) r)
//        A^ = A_qk M^-1                                   (so A^ Z = A_qk r)
//      with r = U - W S = M^-1 (v - exp(gamma) k S) = M^-1 Z.  Both are written
//      in MFMA fragment order, fp16 (bf16 inputs) or fp32 (fp32 inputs).
// This file holds the kernel for one decay per row (scalar g) and the steps
// 3-4 both kernels share; the per-key-channel (KDA) kernel is in
// gdr_prep_kda.hpp.
#pragma once
#include "gdr_device.hpp"

namespace gdr {

struct PrepArgs {
  const void* q;
  const void* k;
  const float* g;
  const float* beta;
  int B, T, H, HV, N;
  float scale;
  void* wt;
  void* ah;
  float* rs;
  void* qh;
  void* kh;
  float* d_gamma;  // optional inspection outputs (fp32)
  float* d_akk;
  float* d_aqk;
  float* d_minv;
};

#ifdef GDR_PREP_PROFILE
__device__ long long gdr_prep_prof[16 * 4];
#define GDR_PPROF(ph)                                                         \
  do {                                                                        \
    if (cid == 7 && lane == 0) gdr_prep_prof[(ph) * 4 + wave] = clock64();    \
  } while (0)
#else
#define GDR_PPROF(ph) do {} while (0)
#endif

// XCD-aware placement of chunks: the value heads that share one q/k head get
// the same (id % 8), so their q/k rows meet in one L2.
__device__ __forceinline__ bool prep_block(int B, int H, int G, int N, int& b, int& hv, int& n) {
  const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
  const long unit = (long)(slot / G) * 8 + xcd;      // (b, h, n)
  const int gi = slot % G;
  if (unit >= (long)B * H * N) return false;
  n = (int)(unit % N);
  const long bhq = unit / N;
  b = (int)(bhq / H);
  hv = (int)(bhq % H) * G + gi;
  return true;
}

constexpr int kLP = kChunk + 4;   // row stride of the C x C fp32 LDS tiles

// ---- step 3: M^-1 by 16-row blocks ----------------------------------------
// In: sL = strictly lower A_kk diag(beta) (= M - I), row-major, stride kLP;
// the caller has synchronised after writing it.  Out: sMT = M^-T (row j holds
// column j of M^-1), and the diagonal blocks of sL hold D_I = M_II^-1.
// Ends with a workgroup barrier.
template <class P>
__device__ __forceinline__ void unit_lower_inverse(float* sL, float* sMT, int tid, int wave,
                                                   int r, int grp) {
  constexpr int C = kChunk, LP = kLP;
  for (int i = tid * 4; i < C * LP; i += 256 * 4) *reinterpret_cast<f32x4*>(sMT + i) = zero4();
  __syncthreads();
  // 3a. wave `blk` inverts its diagonal block by forward substitution
  {
    const int blk = wave, j = r;
    float* Lb = sL + (16 * blk) * LP + 16 * blk;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == j) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s -= Lb[i * LP + m] * x[m];
      x[i] = s;
    }
    if (grp == 0) {
      float* mt = sMT + (16 * blk + j) * LP + 16 * blk;  // row j of D^T
#pragma unroll
      for (int i = 0; i < 16; i += 4)
        *reinterpret_cast<f32x4*>(mt + i) = f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]};
    }
    // D row-major into the (now unused) diagonal block of L, after every lane
    // of the wave has finished reading it
    __builtin_amdgcn_wave_barrier();
    if (grp == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) Lb[i * LP + j] = x[i];
    }
  }
  __syncthreads();
  // 3b. wave J forms block column J of M^-1
  {
    const int J = wave;
    for (int I = J + 1; I < 4; ++I) {
      f32x4 tacc = zero4();
      for (int m = J; m < I; ++m) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(sL + (16 * I + r) * LP + 16 * m + 4 * grp);
        const f32x4 bv2 = *reinterpret_cast<const f32x4*>(sMT + (16 * J + r) * LP + 16 * m + 4 * grp);
        tacc = P::mma16(av, bv2, tacc);
      }
      const f32x4 dv = *reinterpret_cast<const f32x4*>(sL + (16 * I + r) * LP + 16 * I + 4 * grp);
      const f32x4 x = P::mma16(dv, tacc, zero4());
      // row j = 16J + r of M^-T holds column j of M^-1; this wave is its only
      // writer and reader, so no barrier is needed until the next phase
      *reinterpret_cast<f32x4*>(sMT + (16 * J + r) * LP + 16 * I + 4 * grp) = -x;
    }
  }
  __syncthreads();
}

// ---- step 4a: W^ = M^-T diag(s) k -> A fragments of W^T --------------------
// W^T tile row x is key channel chan_of_row(x), the state's row order.
// kval(c, d) returns the B element diag(s) k at row c, channel d when
// kRowScale is false; with kRowScale, kval returns raw k and rscale(c) = s_c
// multiplies the M^-T entries instead.
template <int K, class P, bool kRowScale, class KVal, class RScale>
__device__ __forceinline__ void fold_w(const float* sMT, typename P::ws_t* wt_chunk, int wave,
                                       int lane, int r, int grp, KVal kval, RScale rscale) {
  constexpr int LP = kLP;
  using ws_t = typename P::ws_t;
  for (int jd = wave; jd < K / 16; jd += 4) {
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
    const int d = chan_of_row(16 * jd + r);   // W^T rows follow the state's row order
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float vb[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) vb[s] = kval(32 * kb + kslot(grp, s), d);
      const typename P::frag_t fb = P::make(vb);
#pragma unroll
      for (int Ic = 0; Ic < 4; ++Ic) {
        if (32 * kb + 31 < 16 * Ic) continue;
        const float* row = sMT + (16 * Ic + r) * LP + 32 * kb;
        float va[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          va[s] = row[kslot(grp, s)];
          if constexpr (kRowScale) va[s] *= rscale(32 * kb + kslot(grp, s));
        }
        acc[Ic] = mma32(P::make(va), fb, acc[Ic]);
      }
    }
    ws_t* wt = wt_chunk + (size_t)jd * 2 * 512;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) store_ws(wt + kb * 512 + lane * 8, acc[2 * kb], acc[2 * kb + 1]);
  }
}

// ---- step 4b: A^ = A_qk M^-1, as A^T = M^-T A_qk^T (column tile = wave) ----
// aqT[J] holds the A_qk^T tile (J, wave) in accumulator layout (zero for J >
// wave).
template <class P>
__device__ __forceinline__ void fold_aqk(const f32x4 (&aqT)[4], const float* sMT,
                                         typename P::ws_t* ah_chunk, int wave, int lane, int r,
                                         int grp) {
  constexpr int LP = kLP;
  const int Ii = wave;
  f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if (32 * kb > 16 * Ii + 15) continue;
    const typename P::frag_t fb = P::make2(aqT[2 * kb], aqT[2 * kb + 1]);
#pragma unroll
    for (int Ic = 0; Ic < 4; ++Ic) {
      if (Ic > Ii || 32 * kb + 31 < 16 * Ic) continue;
      const typename P::frag_t fa = frag_row_f32<P>(sMT + (16 * Ic + r) * LP + 32 * kb, grp);
      acc[Ic] = mma32(fa, fb, acc[Ic]);
    }
  }
  typename P::ws_t* ah = ah_chunk + (size_t)Ii * 2 * 512;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) store_ws(ah + kb * 512 + lane * 8, acc[2 * kb], acc[2 * kb + 1]);
}

// ---- inspection dumps shared by both kernels ---------------------------------
__device__ __forceinline__ void dump_akk(float* out, const float* sL, int tid) {
  constexpr int C = kChunk;
  for (int e = tid; e < C * C; e += 256) {
    const int i = e / C, j = e % C;
    out[e] = (j < i && (i >> 4) >= (j >> 4)) ? sL[i * kLP + j] : 0.f;
  }
}
__device__ __forceinline__ void dump_aqk(float* out, const f32x4 (&aqT)[4], int wave, int r,
                                         int grp) {
  // tile (J, wave) of A_qk^T: rows c' = 16J + 4grp + j4, column i = 16 wave + r
  for (int J = 0; J < 4; ++J)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int cp = 16 * J + 4 * grp + j4, i = 16 * wave + r;
      out[i * kChunk + cp] = J <= wave ? aqT[J][j4] : 0.f;
    }
}
__device__ __forceinline__ void dump_minv(float* out, const float* sMT, int tid) {
  constexpr int C = kChunk;
  for (int e = tid; e < C * C; e += 256) out[e] = sMT[(e % C) * kLP + e / C];
}

// ---- the kernel for one decay per row --------------------------------------
template <int K, class P, bool DUMP>
__global__ __launch_bounds__(256) void chunk_prep_kernel(PrepArgs a) {
  using in_t = typename P::in_t;
  using ws_t = typename P::ws_t;
  constexpr int C = kChunk;
  constexpr int KP = K + 16 / (int)sizeof(in_t);  // q/k tile row, +16 bytes
  constexpr int LP = kLP;
  constexpr int KB = K / 32;
  constexpr int VEC = 16 / (int)sizeof(in_t);      // elements per 16-byte load
  constexpr int VPR = K / VEC;                     // 16-byte vectors per row
  constexpr int LPT = C * VPR / 256;               // row vectors per thread

  constexpr size_t QBYTES = (size_t)C * KP * sizeof(in_t);
  constexpr size_t MBYTES = (size_t)C * LP * sizeof(float);
  __shared__ __attribute__((aligned(16))) in_t sK[C * KP];
  // the q tile, then (once the Gram tiles are done) M^-T in fp32
  __shared__ __attribute__((aligned(16))) char sQbuf[QBYTES > MBYTES ? QBYTES : MBYTES];
  in_t* sQ = reinterpret_cast<in_t*>(sQbuf);
  __shared__ __attribute__((aligned(16))) float sL[C * LP];    // A_kk beta (strict); D_I later
  __shared__ float sGam[C];
  __shared__ float sBeta[C];
  __shared__ float sKs[C];     // beta_c exp(gamma_last - gamma_c)
  float* sMT = reinterpret_cast<float*>(sQbuf);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r = lane & 15, grp = lane >> 4;
  int b, hv, n;
  if (!prep_block(a.B, a.H, a.HV / a.H, a.N, b, hv, n)) return;
  const int h = hv / (a.HV / a.H);
  const int cid = (b * a.HV + hv) * a.N + n;
  const int T = a.T;
  const int t0 = n * C;
  GDR_PPROF(0);

  // ---- issue every global load of the chunk up front ----------------------
  const in_t* qg = static_cast<const in_t*>(a.q);
  const in_t* kg = static_cast<const in_t*>(a.k);
  uint4 kv[LPT], qv[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int e = tid + 256 * i, c = e / VPR, cv = (e % VPR) * VEC;
    const int t = min(t0 + c, T - 1);
    const size_t off = (((size_t)b * T + t) * a.H + h) * K + cv;
    kv[i] = *reinterpret_cast<const uint4*>(kg + off);
    qv[i] = *reinterpret_cast<const uint4*>(qg + off);
  }
  float gv = 0.f, bv = 0.f;
  if (wave == 0) {
    const int t = t0 + lane;
    if (t < T) {
      const size_t idx = ((size_t)b * T + t) * a.HV + hv;
      gv = a.g[idx];
      bv = a.beta[idx];
    }
  }

  // ---- q/k rows into LDS (tail rows zeroed) --------------------------------
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int e = tid + 256 * i, c = e / VPR, cv = (e % VPR) * VEC;
    const bool ok = t0 + c < T;
    *reinterpret_cast<uint4*>(sK + c * KP + cv) = ok ? kv[i] : uint4{0u, 0u, 0u, 0u};
    *reinterpret_cast<uint4*>(sQ + c * KP + cv) = ok ? qv[i] : uint4{0u, 0u, 0u, 0u};
  }

  // ---- 1. gamma ------------------------------------------------------------
  if (wave == 0) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(gv, off, 64);
      if (lane >= off) gv += o;
    }
    sGam[lane] = gv;
    sBeta[lane] = bv;
    const float glast = __shfl(gv, 63, 64);
    sKs[lane] = bv * __expf(glast - gv);
  }
  __syncthreads();
  GDR_PPROF(1);

  // ---- 2. decayed dots ----------------------------------------------------
  // A_qk^T tiles (rows c' in block J, columns i in block w) for J <= w stay
  // in this wave's registers; A_kk tiles go to LDS.  Work per wave: w+1 A_qk
  // tiles and 4-w A_kk tiles.  The Gram products are exact bf16 x bf16 (or
  // fp32) products; the decay exp(gamma_i - gamma_j) is applied in fp32 per
  // entry, and only where j <= i.
  f32x4 aqT[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) aqT[j] = zero4();
  {
    auto gram = [&](const in_t* xs, int I, const in_t* ys, int J) -> f32x4 {
      f32x4 acc = zero4();
      const in_t* ra = xs + (16 * I + r) * KP;
      const in_t* rb = ys + (16 * J + r) * KP;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if constexpr (P::kF32)
          acc = mma32(frag_row_in(ra + 32 * kb, grp, P{}), frag_row_in(rb + 32 * kb, grp, P{}), acc);
        else
          acc = mma32(frag_row_bf16(ra + 32 * kb, grp), frag_row_bf16(rb + 32 * kb, grp), acc);
      }
      return acc;
    };

    // A_qk^T = k q^T: tiles (J, w), rows c' (k), columns i (q)
    for (int J = 0; J <= wave; ++J) {
      const f32x4 acc = gram(sK, J, sQ, wave);
      f32x4 val;
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int cp = 16 * J + 4 * grp + j4, i = 16 * wave + r;
        val[j4] = (cp <= i) ? acc[j4] * sBeta[cp] * a.scale * __expf(sGam[i] - sGam[cp]) : 0.f;
      }
      aqT[J] = val;
    }
    // A_kk lower tiles, wave w takes 4-w of them
    constexpr int TI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
    constexpr int TJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
    const int first = (wave == 0) ? 0 : (wave == 1) ? 4 : (wave == 2) ? 7 : 9;
    const int count = 4 - wave;
    for (int tj = first; tj < first + count; ++tj) {
      const int I = TI[tj], J = TJ[tj];
      const f32x4 acc = gram(sK, I, sK, J);
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int i = 16 * I + 4 * grp + j4, j = 16 * J + r;
        sL[i * LP + j] = (i > j) ? acc[j4] * sBeta[j] * __expf(sGam[i] - sGam[j]) : 0.f;
      }
    }
  }

  __syncthreads();   // sL complete
  GDR_PPROF(2);

  if constexpr (DUMP) {
    if (a.d_gamma)
      for (int e = tid; e < C; e += 256) a.d_gamma[(size_t)cid * C + e] = sGam[e];
    if (a.d_akk) dump_akk(a.d_akk + (size_t)cid * C * C, sL, tid);
    if (a.d_aqk) dump_aqk(a.d_aqk + (size_t)cid * C * C, aqT, wave, r, grp);
  }

  // ---- 3. M^-1 (sQ is dead: sMT takes its place) ---------------------------
  unit_lower_inverse<P>(sL, sMT, tid, wave, r, grp);
  GDR_PPROF(4);

  if constexpr (DUMP) {
    if (a.d_minv) dump_minv(a.d_minv + (size_t)cid * C * C, sMT, tid);
  }

  // ---- 4a. W^ (beta exp(gamma_last - gamma) scales the rows of M^-T) -------
  fold_w<K, P, true>(sMT, static_cast<ws_t*>(a.wt) + (size_t)cid * K * C, wave, lane, r, grp,
                     [&](int c, int d) { return P::in_to_f32(sK[c * KP + d]); },
                     [&](int c) { return sKs[c]; });
  GDR_PPROF(5);

  // ---- 4b. A^ ----------------------------------------------------------------
  fold_aqk<P>(aqT, sMT, static_cast<ws_t*>(a.ah) + (size_t)cid * C * C, wave, lane, r, grp);
  GDR_PPROF(6);

  // ---- row scalars --------------------------------------------------------
  {
    float* rs = a.rs + (size_t)cid * 256;
    if (tid < C) rs[tid] = __expf(sGam[tid]);
    if (tid < K) rs[64 + tid] = __expf(sGam[C - 1]);
  }
  GDR_PPROF(7);
}

}  // namespace gdr
