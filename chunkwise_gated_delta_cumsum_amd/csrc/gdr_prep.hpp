// Chunk preparation: everything that is parallel across chunks.
//
// One workgroup per (batch, value head, chunk of C = 32, 64 or 128 rows), one
// wave per 16-row block of the chunk (NB = C / 16 waves).  Steps, following
// the sec-03 notes ("in-chunk cumsum and lower-triangular solve", "decayed
// dot function") and the UT transform of the "Chunkwise parallel
// algorithms" page (section 2.3):
//   1. gamma = inclusive cumsum of g over the chunk.
//   2. Gram tiles of k k^T and k q^T on MFMA (lower 16x16 tiles only), the
//      decay exp(gamma_i - gamma_j), beta on columns and the masks: strict
//      lower for A_kk, lower with diagonal for A_qk (scale folded in).  A_qk
//      is formed transposed, so its accumulator tiles are directly the B
//      operands of step 4b and stay in registers.  Wave W needs the q rows
//      of its own block only, which it loads straight into registers; k
//      goes through LDS.
//   3. M = I + A_kk; M^-1 by blocks: each wave inverts one 16x16 unit-lower
//      diagonal block by forward substitution, then wave J forms block column
//      J: X_IJ = -D_I sum_m L_Im X_mJ for I > J.  M^-T then overwrites A_kk in
//      LDS.
//   4. Fold the UT transform into the operands of the serial scan:
//        W^ = M^-T diag(beta exp(gamma_last - gamma)) k   (so W^T Z = K~^T diag(beta) r)
//        A^ = A_qk M^-1                                   (so A^ Z = A_qk r)
//      with r = U - W S = M^-1 (v - exp(gamma) k S) = M^-1 Z.  Both are written
//      in MFMA fragment order, fp16 (bf16 inputs) or fp32 (fp32 inputs).
// This file holds the kernel for one decay per row (scalar g) and the steps
// 3-4 both kernels share; the per-key-channel (KDA) kernel is in
// gdr_prep_kda.hpp.
//
// Gram products sum over key channels, so any order of the channels inside
// a fragment gives the same products as long as both operands use it: the
// Gram fragments hold 8 consecutive channels per lane (one 16-byte load),
// the order the scan's q and k fragments use as well.
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
__device__ long long gdr_prep_prof[16 * 8];
#define GDR_PPROF_DECL long long gdr_pt_[8] = {0, 0, 0, 0, 0, 0, 0, 0}
#define GDR_PPROF(ph) gdr_pt_[ph] = clock64()
#define GDR_PPROF_FLUSH                                                        \
  do {                                                                         \
    if (cid == 7 && lane == 0)                                                 \
      for (int ph_ = 0; ph_ < 8; ++ph_) gdr_prep_prof[ph_ * 8 + wave] = gdr_pt_[ph_]; \
  } while (0)
#else
#define GDR_PPROF_DECL do {} while (0)
#define GDR_PPROF(ph) do {} while (0)
#define GDR_PPROF_FLUSH do {} while (0)
#endif

// XCD-aware placement of chunks: workgroups are dealt to the 8 XCDs round
// robin, so the HV value heads of one (batch, chunk) get the same (id % 8)
// and consecutive slots: the value heads that share a q/k head read its rows
// through one L2, and so do all heads reading their g and beta, which share
// the cache lines of one token ([B, T, HV] rows of HV values).
__device__ __forceinline__ bool prep_block(int B, int H, int G, int N, int& b, int& hv, int& n) {
  const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
  const int HV = H * G;
  const long unit = (long)(slot / HV) * 8 + xcd;     // (b, n)
  if (unit >= (long)B * N) return false;
  b = (int)(unit / N);
  n = (int)(unit % N);
  hv = slot % HV;
  return true;
}

// Row stride of the C x C fp32 LDS tiles.
template <int C>
constexpr int lds_ld() { return C + 4; }

// Calls f(std::integral_constant<int, I>{}) for I = B .. E-1.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Calls f(std::integral_constant<int, W>{}) for the wave index w (a scalar),
// so that code specialised per wave is chosen by one uniform branch.
template <int NB, int W = 0, class F>
__device__ __forceinline__ void for_wave(int w, F&& f) {
  if constexpr (W < NB) {
    if (w == W)
      f(std::integral_constant<int, W>{});
    else
      for_wave<NB, W + 1>(w, f);
  }
}

// ---- step 3: M^-1 by 16-row blocks ----------------------------------------
// In: sL = strictly lower A_kk diag(beta) (= M - I), row-major, stride
// lds_ld<C>(); the caller has synchronised after writing it.  Out: sL = M^-T
// (row j holds column j of M^-1, zero left of the diagonal block).  Ends with
// a workgroup barrier.
//   3a. wave I inverts its diagonal block by forward substitution (lane r
//       computes column r of D_I) and writes D_I over the block;
//   3b. wave J forms block column J of M^-1, X_IJ = -D_I sum_{m<I} L_Im X_mJ,
//       keeping the X_mJ in registers: an accumulator tile is the B operand
//       of a 16x16x16 product (k = its rows), so no tile goes through LDS;
//   3c. once every wave has read L, wave J writes its row block of M^-T.
template <int C, class P, int J>
__device__ __forceinline__ void inverse_column(const float* sL, const float (&x)[16], int r,
                                               int grp, f32x4 (&X)[C / 16]) {
  constexpr int LP = lds_ld<C>();
  constexpr int NB = C / 16;
#pragma unroll
  for (int I = 0; I < NB; ++I) X[I] = zero4();
  X[J] = f32x4{x[4 * grp], x[4 * grp + 1], x[4 * grp + 2], x[4 * grp + 3]};   // D_J
  static_for<J + 1, NB>([&](auto ic) {
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
}

template <int C, class P>
__device__ __forceinline__ void unit_lower_inverse(float* sL, int wave, int r, int grp) {
  constexpr int LP = lds_ld<C>();
  constexpr int NB = C / 16;
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
    // D row-major into the diagonal block of L, after every lane of the wave
    // has finished reading it
    __builtin_amdgcn_wave_barrier();
    if (grp == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) Lb[i * LP + j] = x[i];
    }
  }
  lds_barrier();   // every D_I is in sL
  f32x4 X[NB];
  for_wave<NB>(wave, [&](auto jc) {
    inverse_column<C, P, decltype(jc)::value>(sL, x, r, grp, X);
  });
  lds_barrier();   // every wave has read L
  // row 16J + r of M^-T = column 16J + r of M^-1: X_IJ[4grp + j4][r] at
  // columns 16I + 4grp + j4 (zero left of the diagonal block)
#pragma unroll
  for (int I = 0; I < NB; ++I)
    *reinterpret_cast<f32x4*>(sL + (16 * wave + r) * LP + 16 * I + 4 * grp) = X[I];
  lds_barrier();
}

// The linear rule has M = I: M^-T is the identity, no inverse to form.
template <int C>
__device__ __forceinline__ void identity_inverse(float* sL, int tid) {
  constexpr int LP = lds_ld<C>();
  for (int e = tid; e < C * C; e += C * 4) sL[(e / C) * LP + e % C] = (e / C == e % C) ? 1.f : 0.f;
  lds_barrier();
}

// ---- step 4a: W^ = M^-T diag(s) k -> A fragments of W^T --------------------
// W^T tile row x is key channel chan_of_row(x), the state's row order.
// kval(c, d) returns the B element diag(s) k at row c, channel d when
// kRowScale is false; with kRowScale, kval returns raw k and rscale(c) = s_c
// multiplies the M^-T entries instead.
template <int K, int C, class P, bool kRowScale, class KVal, class RScale>
__device__ __forceinline__ void fold_w(const float* sMT, typename P::ws_t* wt_chunk, int wave,
                                       int lane, int r, int grp, KVal kval, RScale rscale) {
  constexpr int LP = lds_ld<C>();
  constexpr int NB = C / 16, CB = C / 32;
  using ws_t = typename P::ws_t;
  for (int jd = wave; jd < K / 16; jd += NB) {
    f32x4 acc[NB];
#pragma unroll
    for (int Ic = 0; Ic < NB; ++Ic) acc[Ic] = zero4();
    const int d = chan_of_row(16 * jd + r);   // W^T rows follow the state's row order
#pragma unroll
    for (int kb = 0; kb < CB; ++kb) {
      float vb[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) vb[s] = kval(32 * kb + kslot(grp, s), d);
      const typename P::frag_t fb = P::make(vb);
#pragma unroll
      for (int Ic = 0; Ic < NB; ++Ic) {
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
    ws_t* wt = wt_chunk + (size_t)jd * CB * 512;
#pragma unroll
    for (int kb = 0; kb < CB; ++kb)
      store_ws(wt + kb * 512 + lane * 8, acc[2 * kb], acc[2 * kb + 1]);
  }
}

// ---- step 4b: A^ = A_qk M^-1, as A^T = M^-T A_qk^T (column tile = wave) ----
// aqT[J] holds the A_qk^T tile (J, wave) in accumulator layout (zero for J >
// wave).  Only the k-blocks that meet the lower triangle are stored (ah_frag).
template <int C, class P>
__device__ __forceinline__ void fold_aqk(const f32x4 (&aqT)[C / 16], const float* sMT,
                                         typename P::ws_t* ah_chunk, int wave, int lane, int r,
                                         int grp) {
  constexpr int LP = lds_ld<C>();
  constexpr int NB = C / 16, CB = C / 32;
  const int Ii = wave;
  f32x4 acc[NB];
#pragma unroll
  for (int Ic = 0; Ic < NB; ++Ic) acc[Ic] = zero4();
#pragma unroll
  for (int kb = 0; kb < CB; ++kb) {
    if (32 * kb > 16 * Ii + 15) continue;
    const typename P::frag_t fb = P::make2(aqT[2 * kb], aqT[2 * kb + 1]);
#pragma unroll
    for (int Ic = 0; Ic < NB; ++Ic) {
      if (Ic > Ii || 32 * kb + 31 < 16 * Ic) continue;
      const typename P::frag_t fa = frag_row_f32<P>(sMT + (16 * Ic + r) * LP + 32 * kb, grp);
      acc[Ic] = mma32(fa, fb, acc[Ic]);
    }
  }
#pragma unroll
  for (int kb = 0; kb < CB; ++kb) {
    if (kb > Ii / 2) continue;
    store_ws(ah_chunk + (size_t)ah_frag(Ii, kb) * 512 + lane * 8, acc[2 * kb], acc[2 * kb + 1]);
  }
}

// ---- the linear rule (M = I): W^ = diag(s) k and A^ = A_qk, no products ------
// fold_w and fold_aqk with M^-T = I, element by element: the same accumulator
// tiles (lane: column r, rows 4 grp + j) and the same stores.  Each W^ entry
// is rounded once from fp32 (the product path rounds s to fp16 first); A^
// equals the product path's bits (I times an fp16 value is exact).
template <int K, int C, class P, bool kRowScale, class KVal, class RScale>
__device__ __forceinline__ void fold_w_identity(typename P::ws_t* wt_chunk, int wave, int lane,
                                                int r, int grp, KVal kval, RScale rscale) {
  constexpr int NB = C / 16, CB = C / 32;
  using ws_t = typename P::ws_t;
  for (int jd = wave; jd < K / 16; jd += NB) {
    const int d = chan_of_row(16 * jd + r);
    f32x4 acc[NB];
#pragma unroll
    for (int Ic = 0; Ic < NB; ++Ic)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 16 * Ic + 4 * grp + j;
        acc[Ic][j] = kRowScale ? kval(c, d) * rscale(c) : kval(c, d);
      }
    ws_t* wt = wt_chunk + (size_t)jd * CB * 512;
#pragma unroll
    for (int kb = 0; kb < CB; ++kb)
      store_ws(wt + kb * 512 + lane * 8, acc[2 * kb], acc[2 * kb + 1]);
  }
}

template <int C, class P>
__device__ __forceinline__ void fold_aqk_identity(const f32x4 (&aqT)[C / 16],
                                                  typename P::ws_t* ah_chunk, int wave,
                                                  int lane) {
  constexpr int CB = C / 32;
  const int Ii = wave;
#pragma unroll
  for (int kb = 0; kb < CB; ++kb) {
    if (kb > Ii / 2) continue;
    store_ws(ah_chunk + (size_t)ah_frag(Ii, kb) * 512 + lane * 8, aqT[2 * kb], aqT[2 * kb + 1]);
  }
}

// ---- inspection dumps shared by both kernels ---------------------------------
template <int C>
__device__ __forceinline__ void dump_akk(float* out, const float* sL, int tid) {
  for (int e = tid; e < C * C; e += C * 4) {
    const int i = e / C, j = e % C;
    out[e] = (j < i && (i >> 4) >= (j >> 4)) ? sL[i * lds_ld<C>() + j] : 0.f;
  }
}
template <int C>
__device__ __forceinline__ void dump_aqk(float* out, const f32x4 (&aqT)[C / 16], int wave, int r,
                                         int grp) {
  // tile (J, wave) of A_qk^T: rows c' = 16J + 4grp + j4, column i = 16 wave + r
  for (int J = 0; J < C / 16; ++J)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int cp = 16 * J + 4 * grp + j4, i = 16 * wave + r;
      out[i * C + cp] = J <= wave ? aqT[J][j4] : 0.f;
    }
}
template <int C>
__device__ __forceinline__ void dump_minv(float* out, const float* sMT, int tid) {
  for (int e = tid; e < C * C; e += C * 4) out[e] = sMT[(e % C) * lds_ld<C>() + e / C];
}

// The jobs of step 2 for one decay per row: every wave W has NB + 1 tile
// jobs, the A_qk^T tiles (J, W) for J <= W (kept in registers as the B
// operands of step 4b), then NB - W of the lower A_kk tiles (X, Y), X >= Y,
// taken in row order (tile t = X (X + 1) / 2 + Y) from the wave's first one.
template <int NB>
struct GramJobs {
  static constexpr int first(int W) { return W * NB - W * (W - 1) / 2; }
  static constexpr int tile_x(int t) {
    int X = 0;
    while ((X + 1) * (X + 2) / 2 <= t) ++X;
    return X;
  }
  static constexpr int tile_y(int t) { return t - tile_x(t) * (tile_x(t) + 1) / 2; }
  // job j of wave W: x block (k rows), y block (q rows of W, or k rows)
  static constexpr int x(int W, int j) { return j <= W ? j : tile_x(first(W) + j - W - 1); }
  static constexpr int y(int W, int j) { return j <= W ? W : tile_y(first(W) + j - W - 1); }
};

// Step 2 for one decay per row, for wave W (a template argument, so every
// tile, mask and table below is known at compile time).  The Gram products
// are exact bf16 x bf16 (or fp32) products; the decay exp(gamma_i -
// gamma_j), beta and the scale are applied in fp32 per entry, with a mask
// only on diagonal tiles.  The k operands of job j+1 are read from LDS while
// the products of job j run; the q operand is the wave's own register
// fragments qW.
template <int W, int K, int C, class P, class GF>
__device__ __forceinline__ void gram_tiles(const typename P::in_t* sK, const GF (&qW)[K / 32],
                                           float* sL, const float* sGam, const float* sBeta,
                                           const float* sRk, float rq1, float scale,
                                           bool linear, int r, int grp, f32x4 (&aqT)[C / 16]) {
  using in_t = typename P::in_t;
  constexpr int KB = K / 32;
  constexpr int NB = C / 16;
  constexpr int KP = K + 16 / (int)sizeof(in_t);
  constexpr int LP = lds_ld<C>();
  using J_ = GramJobs<NB>;

  // gamma and beta of the rows this lane touches: rows 16X + 4grp + (0..3)
  // of the accumulator and row 16X + r of the columns, for every block X
  // (beta and the row factors of k on the k rows; all 1 without in-kernel
  // normalisation)
  f32x4 g4[NB], b4[NB], rk4[NB];
  float g1[NB], b1[NB];
#pragma unroll
  for (int X = 0; X < NB; ++X) {
    g4[X] = *reinterpret_cast<const f32x4*>(sGam + 16 * X + 4 * grp);
    rk4[X] = *reinterpret_cast<const f32x4*>(sRk + 16 * X + 4 * grp);
    b4[X] = *reinterpret_cast<const f32x4*>(sBeta + 16 * X + 4 * grp) * rk4[X];
    g1[X] = sGam[16 * X + r];
    b1[X] = sBeta[16 * X + r] * sRk[16 * X + r];
  }

  auto frag = [&](const in_t* row) -> GF {
    return __builtin_bit_cast(GF, P::load_raw8(row));
  };
  auto load_job = [&](int j, GF (&fx)[KB], GF (&fy)[KB]) {
    const in_t* ra = sK + (16 * J_::x(W, j) + r) * KP + 8 * grp;
    const in_t* rb = sK + (16 * J_::y(W, j) + r) * KP + 8 * grp;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      fx[kb] = frag(ra + 32 * kb);
      if (j > W) fy[kb] = frag(rb + 32 * kb);
    }
  };
  GF cx[KB], cy[KB], nx[KB], ny[KB];
  load_job(0, cx, cy);
  static_for<0, NB + 1>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    constexpr int X = J_::x(W, j);
    constexpr int Y = J_::y(W, j);
    if constexpr (j < NB) load_job(j + 1, nx, ny);
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) acc = mma32(cx[kb], j <= W ? qW[kb] : cy[kb], acc);
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
    if constexpr (j < NB) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        cx[kb] = nx[kb];
        cy[kb] = ny[kb];
      }
    }
  });
}

// ---- the kernel for one decay per row --------------------------------------
template <int K, int C, class P, bool DUMP>
__global__ __launch_bounds__(C * 4) void chunk_prep_kernel(PrepArgs a) {
  using in_t = typename P::in_t;
  using ws_t = typename P::ws_t;
  using frag_t = typename P::frag_t;
  using raw_t = typename P::raw_t;
  // Gram fragments: the raw 16-bit inputs (exact products) or fp32
  using gfrag_t = typename P::gfrag_t;
  constexpr int NB = C / 16;                        // waves, one 16-row block each
  constexpr int NT = NB * 64;
  constexpr int KP = K + 16 / (int)sizeof(in_t);    // k tile row, +16 bytes
  constexpr int LP = lds_ld<C>();
  constexpr int KB = K / 32;
  constexpr int VEC = 16 / (int)sizeof(in_t);       // elements per 16-byte load
  constexpr int VPR = K / VEC;                      // 16-byte vectors per row
  constexpr int LPT = C * VPR / NT;                 // row vectors per thread
  static_assert(LPT * NT == C * VPR, "k rows per thread");

  __shared__ __attribute__((aligned(16))) in_t sK[C * KP];
  // A_kk beta (strict); D_I on the diagonal blocks; M^-T after the inverse
  __shared__ __attribute__((aligned(16))) float sL[C * LP];
  __shared__ __attribute__((aligned(16))) float sGam[C];
  __shared__ __attribute__((aligned(16))) float sBeta[C];
  __shared__ float sKs[C];     // beta_c exp(gamma_last - gamma_c)
  __shared__ __attribute__((aligned(16))) float sRk[C];   // row factors of k (L2 norm; else 1)

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
  // k rows whole (coalesced) into LDS; this wave's q rows 16 wave + r as
  // fragments, 8 consecutive channels per lane; g and beta per row.  Rows
  // past T read row T-1 and are zeroed below.
  const in_t* qg = static_cast<const in_t*>(a.q);
  const in_t* kg = static_cast<const in_t*>(a.k);
  uint4 kv[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int e = tid + NT * i, c = e / VPR, cv = (e % VPR) * VEC;
    const int t = min(t0 + c, T - 1);
    kv[i] = *reinterpret_cast<const uint4*>(kg + (((size_t)b * T + t) * a.H + h) * K + cv);
  }
  const int qrow = 16 * wave + r;
  const bool qvalid = t0 + qrow < T;
  raw_t qr[KB];
  {
    const in_t* qp = qg + (((size_t)b * T + min(t0 + qrow, T - 1)) * a.H + h) * K + 8 * grp;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qr[kb] = P::load_raw8(qp + 32 * kb);
  }
  // g, beta values per lane of wave 0 (lanes past C hold zeros: with 32-row
  // chunks half the wave)
  constexpr int GPL = (C + 63) / 64;
  float gv[GPL], bv[GPL];
  if (wave == 0) {
#pragma unroll
    for (int u = 0; u < GPL; ++u) {
      const int t = t0 + 64 * u + lane;
      gv[u] = bv[u] = 0.f;
      if (64 * u + lane < C && t < T) {
        const size_t idx = ((size_t)b * T + t) * a.HV + hv;
        gv[u] = a.g[idx];
        bv[u] = a.beta[idx];
      }
    }
  }

  // ---- optional L2 normalisation of the q and k rows -----------------------
  // The rows stay raw; each row's factor rsqrt(sum x^2 + 1e-6) (1 when
  // normalisation is off) multiplies it in fp32 wherever its values enter a
  // product or an fp16 operand: the Gram entries, the W^ row scalars and the
  // q/k fragments of the scan.  In each k load round the VPR consecutive
  // threads c VPR .. c VPR + VPR-1 hold row c (VPR divides the wave), so a
  // row's sum of squares is a butterfly over VPR lanes; a q row's channels
  // sit in the four lanes r + 16 grp.
  float rq1 = 1.f;
  if (a.l2norm) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      float sk = sumsq16<in_t>(__builtin_bit_cast(u32x4, kv[i]));
#pragma unroll
      for (int off = 1; off < VPR; off <<= 1) sk += __shfl_xor(sk, off, 64);
      const int e = tid + NT * i;
      if (e % VPR == 0) sRk[e / VPR] = rsqrtf(sk + kL2NormEps);
    }
    float sq = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) sq += P::raw_f32(qr[kb], j) * P::raw_f32(qr[kb], j);
    sq += __shfl_xor(sq, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    rq1 = rsqrtf(sq + kL2NormEps);
  } else {
    for (int c = tid; c < C; c += NT) sRk[c] = 1.f;
  }

  // ---- k rows into LDS (tail rows zeroed); q fragments (tail rows zero) ----
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int e = tid + NT * i, c = e / VPR, cv = (e % VPR) * VEC;
    const bool ok = t0 + c < T;
    *reinterpret_cast<uint4*>(sK + c * KP + cv) = ok ? kv[i] : uint4{0u, 0u, 0u, 0u};
  }
  gfrag_t qW[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    if (!qvalid) qr[kb] = raw_t{};
    qW[kb] = __builtin_bit_cast(gfrag_t, qr[kb]);
  }

  // ---- 1. gamma ------------------------------------------------------------
  if (wave == 0) {
    float base = 0.f;
#pragma unroll
    for (int u = 0; u < GPL; ++u) {
      float x = gv[u];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(x, off, 64);
        if (lane >= off) x += o;
      }
      x += base;
      base = __shfl(x, 63, 64);
      gv[u] = x;
    }
    // base is now gamma_last
#pragma unroll
    for (int u = 0; u < GPL; ++u) {
      if (64 * u + lane < C) {
        sGam[64 * u + lane] = gv[u];
        sBeta[64 * u + lane] = bv[u];
        sKs[64 * u + lane] = bv[u] * __expf(base - gv[u]);
      }
    }
  }
  lds_barrier();
  GDR_PPROF(1);

  // ---- 2. decayed dots (gram_tiles) ----------------------------------------
  f32x4 aqT[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) aqT[j] = zero4();
  for_wave<NB>(wave, [&](auto wc) {
    gram_tiles<decltype(wc)::value, K, C, P>(sK, qW, sL, sGam, sBeta, sRk, rq1, a.scale,
                                             a.linear != 0, r, grp, aqT);
  });

  // ---- q and k for the scan, in its fragment order -------------------------
  // Read straight from the inputs, an MFMA fragment of the scan would touch
  // 16 rows per 16 lanes, which the vector memory path serves at a quarter
  // of its contiguous rate; so each query head's q and k are written once
  // (by the first of its value heads) as fragments the scan loads with 16
  // contiguous bytes per lane.  Fragment (ct, kb), lane (r, g) holds channels
  // 32 kb + 8 g .. +7 of row 16 ct + r: wave W writes row tile W, q from its
  // registers and k from the LDS tile (tail rows are zero in both).  Issued
  // after the Gram products, so that the stores drain while the inverse runs.
  if (hv % (a.HV / a.H) == 0) {
    const size_t qcid = ((size_t)b * a.H + h) * a.N + n;
    ws_t* qd = static_cast<ws_t*>(a.qh) + (qcid * NB + wave) * KB * 512 + lane * 8;
    ws_t* kd = static_cast<ws_t*>(a.kh) + (qcid * NB + wave) * KB * 512 + lane * 8;
    const float rk1 = sRk[qrow];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const raw_t kraw = P::load_raw8(sK + qrow * KP + 32 * kb + 8 * grp);
      // normalised rows: the raw values times the row factor, in fp32, then
      // rounded once to the fragment type
      const frag_t qf = a.l2norm ? P::frag_scaled(qr[kb], rq1) : P::frag_from_raw(qr[kb]);
      const frag_t kf = a.l2norm ? P::frag_scaled(kraw, rk1) : P::frag_from_raw(kraw);
      __builtin_nontemporal_store(qf, reinterpret_cast<frag_t*>(qd + (size_t)kb * 512));
      __builtin_nontemporal_store(kf, reinterpret_cast<frag_t*>(kd + (size_t)kb * 512));
    }
  }

  lds_barrier();   // sL complete
  GDR_PPROF(2);

  if constexpr (DUMP) {
    if (a.d_gamma)
      for (int e = tid; e < C; e += NT) a.d_gamma[(size_t)cid * C + e] = sGam[e];
    if (a.d_akk) dump_akk<C>(a.d_akk + (size_t)cid * C * C, sL, tid);
    if (a.d_aqk) dump_aqk<C>(a.d_aqk + (size_t)cid * C * C, aqT, wave, r, grp);
    lds_barrier();   // sL is read before the inverse overwrites it
  }

  // ---- 3. M^-1 (M^-T replaces A_kk in sL) ------------------------------------
  // (the linear rule has M = I: nothing to invert; the identity is written
  // only for the inspection dump)
  if (a.linear) {
    if constexpr (DUMP) identity_inverse<C>(sL, tid);
  } else {
    unit_lower_inverse<C, P>(sL, wave, r, grp);
  }
  GDR_PPROF(4);

  if constexpr (DUMP) {
    if (a.d_minv) dump_minv<C>(a.d_minv + (size_t)cid * C * C, sL, tid);
  }

  // ---- 4a. W^ (beta exp(gamma_last - gamma) scales the rows of M^-T) -------
  ws_t* const wt_chunk = static_cast<ws_t*>(a.wt) + (size_t)cid * K * C;
  auto k_at = [&](int c, int d) { return P::in_to_f32(sK[c * KP + d]); };
  auto w_scale = [&](int c) { return sKs[c] * sRk[c]; };
  if (a.linear)
    fold_w_identity<K, C, P, true>(wt_chunk, wave, lane, r, grp, k_at, w_scale);
  else
    fold_w<K, C, P, true>(sL, wt_chunk, wave, lane, r, grp, k_at, w_scale);
  GDR_PPROF(5);

  // ---- 4b. A^ ----------------------------------------------------------------
  ws_t* const ah_chunk = static_cast<ws_t*>(a.ah) + (size_t)cid * ah_frags(C) * 512;
  if (a.linear)
    fold_aqk_identity<C, P>(aqT, ah_chunk, wave, lane);
  else
    fold_aqk<C, P>(aqT, sL, ah_chunk, wave, lane, r, grp);
  GDR_PPROF(6);

  // ---- row scalars --------------------------------------------------------
  {
    float* rs = a.rs + (size_t)cid * 256;
    for (int e = tid; e < C; e += NT) rs[e] = __expf(sGam[e]);
    // one decay per row: exp(gamma_last) is one value for every key channel
    if (tid == 0) rs[C] = __expf(sGam[C - 1]);
  }
  GDR_PPROF(7);
  GDR_PPROF_FLUSH;
  GDR_WGT(0, 1);
}

}  // namespace gdr
