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
#include <type_traits>
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
  int l2norm;      // 1: L2-normalise every q and k row first
  int linear;      // 1: decayed linear attention (no erase term): A_kk = 0, M = I
  float* d_gamma;  // optional inspection outputs (fp32)
  float* d_akk;
  float* d_aqk;
  float* d_minv;
};

#ifdef GDR_PREP_PROFILE
// phase timestamps of one chunk, kept in registers and written at the end so
// that the marks themselves add no memory traffic to the phases
__device__ long long gdr_prep_prof[16 * 4];
#define GDR_PPROF_DECL long long gdr_pt_[8] = {0, 0, 0, 0, 0, 0, 0, 0}
#define GDR_PPROF(ph) gdr_pt_[ph] = clock64()
#define GDR_PPROF_FLUSH                                                        \
  do {                                                                         \
    if (cid == 7 && lane == 0)                                                 \
      for (int ph_ = 0; ph_ < 8; ++ph_) gdr_prep_prof[ph_ * 4 + wave] = gdr_pt_[ph_]; \
  } while (0)
#else
#define GDR_PPROF_DECL do {} while (0)
#define GDR_PPROF(ph) do {} while (0)
#define GDR_PPROF_FLUSH do {} while (0)
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

// Calls f(std::integral_constant<int, I>{}) for I = B .. E-1.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---- step 3: M^-1 by 16-row blocks ----------------------------------------
// In: sL = strictly lower A_kk diag(beta) (= M - I), row-major, stride kLP;
// the caller has synchronised after writing it.  Out: sMT = M^-T (row j holds
// column j of M^-1, upper blocks zero), and the diagonal blocks of sL hold
// D_I = M_II^-1.  Ends with a workgroup barrier.
//   3a. wave I inverts its diagonal block by forward substitution (lane r
//       computes column r of D_I);
//   3b. wave J forms block column J of M^-1, X_IJ = -D_I sum_{m<I} L_Im X_mJ,
//       keeping the X_mJ in registers: an accumulator tile is the B operand
//       of a 16x16x16 product (k = its rows), so no tile goes through LDS
//       until the wave writes its row block of M^-T.
template <class P, int J>
__device__ __forceinline__ void inverse_column(const float* sL, float* sMT, const float (&x)[16],
                                               int r, int grp) {
  constexpr int LP = kLP;
  f32x4 X[4];
#pragma unroll
  for (int I = 0; I < 4; ++I) X[I] = zero4();
  X[J] = f32x4{x[4 * grp], x[4 * grp + 1], x[4 * grp + 2], x[4 * grp + 3]};   // D_J
  static_for<J + 1, 4>([&](auto ic) {
    constexpr int I = decltype(ic)::value;
    f32x4 tacc = zero4();
#pragma unroll
    for (int m = J; m < I; ++m) {
      const f32x4 av = *reinterpret_cast<const f32x4*>(sL + (16 * I + r) * LP + 16 * m + 4 * grp);
      tacc = P::mma16(av, X[m], tacc);
    }
    const f32x4 dv = *reinterpret_cast<const f32x4*>(sL + (16 * I + r) * LP + 16 * I + 4 * grp);
    X[I] = -P::mma16(dv, tacc, zero4());
  });
  // row 16J + r of M^-T = column 16J + r of M^-1: X_IJ[4grp + j4][r] at
  // columns 16I + 4grp + j4 (zero above the diagonal block)
#pragma unroll
  for (int I = 0; I < 4; ++I)
    *reinterpret_cast<f32x4*>(sMT + (16 * J + r) * LP + 16 * I + 4 * grp) = X[I];
}

template <class P>
__device__ __forceinline__ void unit_lower_inverse(float* sL, float* sMT, int tid, int wave,
                                                   int r, int grp) {
  constexpr int LP = kLP;
  // 3a. column r of D = M_II^-1 for the wave's diagonal block I = wave
  float x[16];
  {
    float* Lb = sL + (16 * wave) * LP + 16 * wave;
    const int j = r;
    // column-oriented forward substitution: once x[m] is final it is removed
    // from every later row, so the dependent chain is 16 FMAs long instead of
    // 120; each x[i] still subtracts the terms in the order m = 0, 1, ...
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
    for (int m = 0; m < 15; ++m)
#pragma unroll
      for (int i = m + 1; i < 16; ++i) x[i] -= Lb[i * LP + m] * x[m];
    // D row-major into the (now unused) diagonal block of L, after every lane
    // of the wave has finished reading it
    __builtin_amdgcn_wave_barrier();
    if (grp == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) Lb[i * LP + j] = x[i];
    }
  }
  lds_barrier();   // every D_I is in sL
  switch (wave) {
    case 0: inverse_column<P, 0>(sL, sMT, x, r, grp); break;
    case 1: inverse_column<P, 1>(sL, sMT, x, r, grp); break;
    case 2: inverse_column<P, 2>(sL, sMT, x, r, grp); break;
    default: inverse_column<P, 3>(sL, sMT, x, r, grp); break;
  }
  lds_barrier();
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

// Step 2 for one decay per row, for wave W (a template argument, so every
// tile, mask and table below is known at compile time).  Every wave has five
// 16x16 tile jobs: the A_qk^T tiles (J, W) for J <= W, kept in registers as
// the B operands of step 4b, then 4 - W of the A_kk tiles, written to sL.
// The Gram products are exact bf16 x bf16 (or fp32) products; the decay
// exp(gamma_i - gamma_j), beta and the scale are applied in fp32 per entry,
// with a mask only on diagonal tiles.  The operands of job j+1 are read from
// LDS while the products of job j run.
template <int W, int K, class P>
__device__ __forceinline__ void gram_tiles(const typename P::in_t* sK, const typename P::in_t* sQ,
                                           float* sL, const float* sGam, const float* sBeta,
                                           const float* sRq, const float* sRk, float scale,
                                           bool linear, int r, int grp, f32x4 (&aqT)[4]) {
  using in_t = typename P::in_t;
  using gfrag_t = std::conditional_t<P::kF32, f32x8, bf16x8>;
  constexpr int KB = K / 32;
  constexpr int KP = K + 16 / (int)sizeof(in_t);
  constexpr int LP = kLP;
  constexpr int TI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
  constexpr int TJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
  constexpr int FIRST = W == 0 ? 0 : W == 1 ? 4 : W == 2 ? 7 : 9;
  // job j: (x block, y block, is A_qk^T)
  auto jx = [](int j) { return j <= W ? j : TI[FIRST + j - W - 1]; };
  auto jy = [](int j) { return j <= W ? W : TJ[FIRST + j - W - 1]; };

  // gamma and beta of the rows this lane touches: rows 16X + 4grp + (0..3)
  // of the accumulator and row 16X + r of the columns, for every block X
  // (beta and the row factors of k on the k rows; the q row factor on
  // column i of A_qk^T; all 1 without in-kernel normalisation)
  f32x4 g4[4], b4[4], rk4[4];
  float g1[4], b1[4];
#pragma unroll
  for (int X = 0; X < 4; ++X) {
    g4[X] = *reinterpret_cast<const f32x4*>(sGam + 16 * X + 4 * grp);
    rk4[X] = *reinterpret_cast<const f32x4*>(sRk + 16 * X + 4 * grp);
    b4[X] = *reinterpret_cast<const f32x4*>(sBeta + 16 * X + 4 * grp) * rk4[X];
    g1[X] = sGam[16 * X + r];
    b1[X] = sBeta[16 * X + r] * sRk[16 * X + r];
  }
  const float rq1 = sRq[16 * W + r];

  auto frag = [&](const in_t* row) -> gfrag_t {
    if constexpr (P::kF32)
      return frag_row_in(row, grp, P{});
    else
      return frag_row_bf16(row, grp);
  };
  auto load_job = [&](int j, gfrag_t (&fx)[KB], gfrag_t (&fy)[KB]) {
    const in_t* ra = sK + (16 * jx(j) + r) * KP;
    const in_t* rb = (j <= W ? sQ : sK) + (16 * jy(j) + r) * KP;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      fx[kb] = frag(ra + 32 * kb);
      fy[kb] = frag(rb + 32 * kb);
    }
  };
  gfrag_t cx[KB], cy[KB], nx[KB], ny[KB];
  load_job(0, cx, cy);
  static_for<0, 5>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    constexpr int X = j <= W ? j : TI[FIRST + j - W - 1];
    constexpr int Y = j <= W ? W : TJ[FIRST + j - W - 1];
    if constexpr (j < 4) load_job(j + 1, nx, ny);
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) acc = mma32(cx[kb], cy[kb], acc);
    f32x4 val;
    if constexpr (j <= W) {
      // A_qk^T tile (X, W): rows c' = 16X + 4grp + j4 (k), column i = 16W + r (q)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const float x = acc[j4] * b4[X][j4] * (scale * rq1) * __expf(g1[W] - g4[X][j4]);
        val[j4] = (X < W || 4 * grp + j4 <= r) ? x : 0.f;
      }
      aqT[X] = val;
    } else {
      // A_kk tile (X, Y): rows i = 16X + 4grp + j4, column j = 16Y + r
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const float x = acc[j4] * b1[Y] * rk4[X][j4] * __expf(g4[X][j4] - g1[Y]);
        // (the linear rule has no erase term: M = I)
        sL[(16 * X + 4 * grp + j4) * LP + 16 * Y + r] =
            ((X > Y || 4 * grp + j4 > r) && !linear) ? x : 0.f;
      }
    }
    if constexpr (j < 4) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        cx[kb] = nx[kb];
        cy[kb] = ny[kb];
      }
    }
  });
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
  __shared__ float sRq[C];     // row factors of q and k (L2 normalisation; else 1)
  __shared__ float sRk[C];
  float* sMT = reinterpret_cast<float*>(sQbuf);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r = lane & 15, grp = lane >> 4;
  int b, hv, n;
  if (!prep_block(a.B, a.H, a.HV / a.H, a.N, b, hv, n)) return;
  const int h = hv / (a.HV / a.H);
  const int cid = (b * a.HV + hv) * a.N + n;
  const int T = a.T;
  const int t0 = n * C;
  GDR_PPROF_DECL;
  GDR_PPROF(0);
  GDR_WGT(0, 0);

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

  // ---- optional L2 normalisation of the q and k rows -----------------------
  // The rows stay raw in LDS; each row's factor rsqrt(sum x^2 + 1e-6) (1 when
  // normalisation is off) multiplies it in fp32 wherever its values enter a
  // product or an fp16 operand: the Gram entries, the W^ row scalars and the
  // q/k fragments of the scan.  In each load round the VPR consecutive
  // threads c VPR .. c VPR + VPR-1 hold row c (VPR divides the wave), so a
  // row's sum of squares is a butterfly over VPR lanes.
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    float fq = 1.f, fk = 1.f;
    if (a.l2norm) {
      float sq = sumsq16<in_t>(__builtin_bit_cast(u32x4, qv[i]));
      float sk = sumsq16<in_t>(__builtin_bit_cast(u32x4, kv[i]));
#pragma unroll
      for (int off = 1; off < VPR; off <<= 1) {
        sq += __shfl_xor(sq, off, 64);
        sk += __shfl_xor(sk, off, 64);
      }
      fq = rsqrtf(sq + kL2NormEps);
      fk = rsqrtf(sk + kL2NormEps);
    }
    const int e = tid + 256 * i;
    if (e % VPR == 0) {
      sRq[e / VPR] = fq;
      sRk[e / VPR] = fk;
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
  lds_barrier();
  GDR_PPROF(1);

  // ---- 2. decayed dots (gram_tiles) ----------------------------------------
  f32x4 aqT[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) aqT[j] = zero4();
  switch (wave) {
    case 0: gram_tiles<0, K, P>(sK, sQ, sL, sGam, sBeta, sRq, sRk, a.scale,
                                   a.linear != 0, r, grp, aqT); break;
    case 1: gram_tiles<1, K, P>(sK, sQ, sL, sGam, sBeta, sRq, sRk, a.scale,
                                   a.linear != 0, r, grp, aqT); break;
    case 2: gram_tiles<2, K, P>(sK, sQ, sL, sGam, sBeta, sRq, sRk, a.scale,
                                   a.linear != 0, r, grp, aqT); break;
    default: gram_tiles<3, K, P>(sK, sQ, sL, sGam, sBeta, sRq, sRk, a.scale,
                                   a.linear != 0, r, grp, aqT); break;
  }

  // ---- q and k for the scan, in its fragment order -------------------------
  // (after the Gram products, so that their stores drain while the inverse
  // runs; before the barrier after which M^-T overwrites the q tile)
  // Read straight from the inputs, an MFMA fragment would touch 16 rows per
  // 16 lanes, which the vector memory path serves at a quarter of its
  // contiguous rate; here the rows already sit in LDS, so each query head's
  // q and k are written once (by the first of its value heads) as fragments
  // the scan loads with 16 contiguous bytes per lane.  Piece pc = (ct KB +
  // kb) 64 + lane holds channels 32 kb + 8 (lane / 16) .. +7 of row
  // 16 ct + lane % 16; tail rows are the zero rows of the LDS tile.
  if (hv % (a.HV / a.H) == 0) {
    using frag_t = typename P::frag_t;
    constexpr int KB = K / 32;
    const size_t qcid = ((size_t)b * a.H + h) * a.N + n;
    ws_t* qd = static_cast<ws_t*>(a.qh) + qcid * C * K;
    ws_t* kd = static_cast<ws_t*>(a.kh) + qcid * C * K;
#pragma unroll
    for (int pc = tid; pc < C * K / 8; pc += 256) {
      const int ln = pc & 63, tkb = pc >> 6;
      const int row = 16 * (tkb / KB) + (ln & 15), ch = 32 * (tkb % KB) + 8 * (ln >> 4);
      const auto qraw = P::load_raw8(sQ + row * KP + ch), kraw = P::load_raw8(sK + row * KP + ch);
      // normalised rows: the raw values times the row factor, in fp32, then
      // rounded once to the fragment type
      const frag_t qf = a.l2norm ? P::frag_scaled(qraw, sRq[row]) : P::frag_from_raw(qraw);
      const frag_t kf = a.l2norm ? P::frag_scaled(kraw, sRk[row]) : P::frag_from_raw(kraw);
      __builtin_nontemporal_store(qf, reinterpret_cast<frag_t*>(qd + (size_t)pc * 8));
      __builtin_nontemporal_store(kf, reinterpret_cast<frag_t*>(kd + (size_t)pc * 8));
    }
  }

  lds_barrier();   // sL complete
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
                     [&](int c) { return sKs[c] * sRk[c]; });
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
  GDR_PPROF_FLUSH;
  GDR_WGT(0, 1);
}

}  // namespace gdr
