// Chunk preparation kernel: everything that is parallel across chunks.
//
// One workgroup (4 waves) per (batch, value head, chunk of C = 64 rows).
// Steps, following the sec-03 notes ("in-chunk cumsum and lower-triangular
// solve", "decayed dot function") and the UT transform of the "Chunkwise
// parallel algorithms" page (section 2.3):
//   1. gamma = inclusive cumsum of g over the chunk (wave-level scan; per key
//      channel for the KDA form).
//   2. Gram tiles of k k^T and q k^T on MFMA, lower 16x16 tiles only, then the
//      decay exp(gamma_i - gamma_j), beta on columns, and the masks: strict
//      lower for A_kk, lower with diagonal for A_qk (scale folded in).  exp is
//      never taken for j > i.  With per-channel decay the off-diagonal tiles
//      use the factorisation exp(gamma_i - gamma_r) * exp(gamma_r - gamma_j)
//      about the last row r of the column tile (both factors <= 1 when g <= 0);
//      diagonal tiles, and every tile when g has enough positive drift to
//      overflow fp16, are summed explicitly in fp32.
//   3. M = I + A_kk; M^-1 by blocks: the four 16x16 unit-lower diagonal blocks
//      by forward substitution (one lane per column), then the off-diagonal
//      blocks X_IJ = -D_I sum_m L_Im X_mJ by increasing distance on fp32 MFMA.
//   4. Fold the UT transform into the operands of the serial scan:
//        W^ = M^-T diag(beta exp(gamma_last - gamma)) k   (so W^T Z = K~^T diag(beta) r)
//        A^ = A_qk M^-1                                   (so A^ Z = A_qk r)
//      with r = U - W S = M^-1 (v - exp(gamma) k S) = M^-1 Z.  Both are written
//      in MFMA fragment order, fp16 (bf16 inputs) or fp32 (fp32 inputs).
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

// Largest per-channel positive drift (sum over the chunk of max(g, 0)) for
// which the factored per-channel Gram stays inside the fp16 range.
constexpr float kPosDriftLimit = 0.5f;

template <int K, bool PERCH, class P, bool DUMP>
__global__ __launch_bounds__(256) void chunk_prep_kernel(PrepArgs a) {
  using in_t = typename P::in_t;
  using frag_t = typename P::frag_t;
  using ws_t = typename P::ws_t;
  constexpr int C = kChunk;
  constexpr int KP = K + 16 / (int)sizeof(in_t);  // q/k tile row, +16 bytes
  constexpr int LP = C + 4;                        // C x C fp32 tile row
  constexpr int GS = PERCH ? K : 1;                // gamma row stride
  constexpr int KB = K / 32;

  __shared__ __attribute__((aligned(16))) float sL[C * LP];   // A_kk*beta (strict); D_I later
  __shared__ __attribute__((aligned(16))) float sA[C * LP];   // A_qk*beta*scale
  __shared__ __attribute__((aligned(16))) float sMT[C * LP];  // M^-T
  __shared__ __attribute__((aligned(16))) in_t sK[C * KP];
  __shared__ __attribute__((aligned(16))) in_t sQ[C * KP];
  __shared__ __attribute__((aligned(16))) float sGam[C * GS];
  __shared__ float sBeta[C];
  __shared__ float sKs[C];      // beta_c exp(gamma_last - gamma_c), one decay per row
  __shared__ float sPos[256];   // per-thread positive drift (per-channel form)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int cid = blockIdx.x;  // (b * HV + hv) * N + n
  const int n = cid % a.N;
  const int bh = cid / a.N;
  const int b = bh / a.HV, hv = bh % a.HV;
  const int h = hv / (a.HV / a.H);
  const int T = a.T;
  const int t0 = n * C;

  for (int i = tid * 4; i < C * LP; i += 256 * 4) {
    *reinterpret_cast<f32x4*>(sL + i) = zero4();
    *reinterpret_cast<f32x4*>(sA + i) = zero4();
    *reinterpret_cast<f32x4*>(sMT + i) = zero4();
  }

  // ---- 1. beta, gamma ------------------------------------------------------
  bool unsafe = false;
  if constexpr (!PERCH) {
    if (wave == 0) {
      const int t = t0 + lane;
      float gv = 0.f, bv = 0.f;
      if (t < T) {
        const size_t idx = ((size_t)b * T + t) * a.HV + hv;
        gv = a.g[idx];
        bv = a.beta[idx];
      }
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
  } else {
    if (tid < C) {
      const int t = t0 + tid;
      sBeta[tid] = (t < T) ? a.beta[((size_t)b * T + t) * a.HV + hv] : 0.f;
    }
    constexpr int PARTS = 256 / K;
    constexpr int RP = C / PARTS;
    const int d = tid % K, part = tid / K;
    float run = 0.f, pos = 0.f;
    for (int i = 0; i < RP; ++i) {
      const int c = part * RP + i, t = t0 + c;
      const float gv = (t < T) ? a.g[(((size_t)b * T + t) * a.HV + hv) * K + d] : 0.f;
      run += gv;
      pos += fmaxf(gv, 0.f);
      sGam[c * K + d] = run;
    }
    sPos[tid] = pos;
    __syncthreads();
    float offv = 0.f, post = 0.f;
    for (int p = 0; p < PARTS; ++p) {
      if (p < part) offv += sGam[((p + 1) * RP - 1) * K + d];
      post += sPos[p * K + d];
    }
    __syncthreads();
    for (int i = 0; i < RP; ++i) sGam[(part * RP + i) * K + d] += offv;
    unsafe = __syncthreads_or(post > kPosDriftLimit) != 0;
  }

  // ---- load the q and k rows of the chunk ---------------------------------
  {
    constexpr int VEC = 16 / (int)sizeof(in_t);
    constexpr int VPR = K / VEC;
    const in_t* qg = static_cast<const in_t*>(a.q);
    const in_t* kg = static_cast<const in_t*>(a.k);
    for (int e = tid; e < C * VPR; e += 256) {
      const int c = e / VPR, cv = (e % VPR) * VEC, t = t0 + c;
      uint4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
      if (t < T) {
        const size_t off = (((size_t)b * T + t) * a.H + h) * K + cv;
        kv = *reinterpret_cast<const uint4*>(kg + off);
        qv = *reinterpret_cast<const uint4*>(qg + off);
      }
      *reinterpret_cast<uint4*>(sK + c * KP + cv) = kv;
      *reinterpret_cast<uint4*>(sQ + c * KP + cv) = qv;
    }
  }
  __syncthreads();

  // ---- 2. decayed dots, lower 16x16 tiles --------------------------------
  {
    constexpr int TI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
    constexpr int TJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
    for (int job = wave; job < 20; job += 4) {
      const bool qk = job >= 10;
      const int I = TI[job % 10], J = TJ[job % 10];
      const in_t* xs = qk ? sQ : sK;
      float* dst = qk ? sA : sL;
      const float cscale = qk ? a.scale : 1.f;
      f32x4 acc = zero4();
      if constexpr (!PERCH) {
        const in_t* ra = xs + (16 * I + r) * KP;
        const in_t* rb = sK + (16 * J + r) * KP;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          if constexpr (P::kF32)
            acc = mma32(frag_row_in(ra + 32 * kb, grp, P{}), frag_row_in(rb + 32 * kb, grp, P{}), acc);
          else
            acc = mma32(frag_row_bf16(ra + 32 * kb, grp), frag_row_bf16(rb + 32 * kb, grp), acc);
        }
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int i = 16 * I + 4 * grp + j4, j = 16 * J + r;
          const bool keep = qk ? (i >= j) : (i > j);
          float val = 0.f;
          if (keep) val = acc[j4] * __expf(sGam[i] - sGam[j]) * sBeta[j] * cscale;
          dst[i * LP + j] = val;
        }
      } else {
        if (I > J && !unsafe) {
          const int ref = 16 * J + 15;
          const int ia = 16 * I + r, jb = 16 * J + r;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            float va[8], vb[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const int d = 32 * kb + kslot(grp, s);
              const float gr = sGam[ref * K + d];
              va[s] = P::in_to_f32(xs[ia * KP + d]) * __expf(sGam[ia * K + d] - gr);
              vb[s] = P::in_to_f32(sK[jb * KP + d]) * __expf(gr - sGam[jb * K + d]);
            }
            acc = mma32(P::make(va), P::make(vb), acc);
          }
        } else {
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            const int i = 16 * I + 4 * grp + j4, j = 16 * J + r;
            const bool keep = qk ? (i >= j) : (i > j);
            float s = 0.f;
            if (keep) {
              for (int d = 0; d < K; ++d)
                s += P::in_to_f32(xs[i * KP + d]) * P::in_to_f32(sK[j * KP + d]) *
                     __expf(sGam[i * K + d] - sGam[j * K + d]);
            }
            acc[j4] = s;
          }
        }
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int i = 16 * I + 4 * grp + j4, j = 16 * J + r;
          const bool keep = qk ? (i >= j) : (i > j);
          dst[i * LP + j] = keep ? acc[j4] * sBeta[j] * cscale : 0.f;
        }
      }
    }
  }
  __syncthreads();

  if constexpr (DUMP) {
    if (a.d_gamma)
      for (int e = tid; e < C * GS; e += 256) a.d_gamma[(size_t)cid * C * GS + e] = sGam[e];
    if (a.d_akk)
      for (int e = tid; e < C * C; e += 256) a.d_akk[(size_t)cid * C * C + e] = sL[(e / C) * LP + e % C];
    if (a.d_aqk)
      for (int e = tid; e < C * C; e += 256) a.d_aqk[(size_t)cid * C * C + e] = sA[(e / C) * LP + e % C];
    __syncthreads();
  }

  // ---- 3a. inverse of the four diagonal 16x16 blocks ---------------------
  if (wave == 0) {
    const int blk = lane >> 4, j = lane & 15;
    float* Lb = sL + (16 * blk) * LP + 16 * blk;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == j) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s -= Lb[i * LP + m] * x[m];
      x[i] = s;
    }
    float* mt = sMT + (16 * blk + j) * LP + 16 * blk;  // row j of D^T
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      *reinterpret_cast<f32x4*>(mt + i) = f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]};
#pragma unroll
    for (int i = 0; i < 16; ++i) Lb[i * LP + j] = x[i];  // D row-major in place
  }
  __syncthreads();

  // ---- 3b. off-diagonal blocks by distance -------------------------------
#pragma unroll
  for (int dist = 1; dist < 4; ++dist) {
    if (wave < 4 - dist) {
      const int J = wave, I = J + dist;
      f32x4 tacc = zero4();
      for (int m = J; m < I; ++m) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(sL + (16 * I + r) * LP + 16 * m + 4 * grp);
        const f32x4 bv = *reinterpret_cast<const f32x4*>(sMT + (16 * J + r) * LP + 16 * m + 4 * grp);
        tacc = mma16_f32(av, bv, tacc);
      }
      const f32x4 dv = *reinterpret_cast<const f32x4*>(sL + (16 * I + r) * LP + 16 * I + 4 * grp);
      f32x4 x = mma16_f32(dv, tacc, zero4());
      *reinterpret_cast<f32x4*>(sMT + (16 * J + r) * LP + 16 * I + 4 * grp) = -x;
    }
    __syncthreads();
  }

  if constexpr (DUMP) {
    if (a.d_minv)
      for (int e = tid; e < C * C; e += 256)
        a.d_minv[(size_t)cid * C * C + e] = sMT[(e % C) * LP + e / C];
  }

  // ---- 4a. W^ = M^-T diag(s) k  -> A fragments of W^T -------------------
  for (int jd = wave; jd < K / 16; jd += 4) {
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
    const int d = 16 * jd + r;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float vb[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int cp = 32 * kb + kslot(grp, s);
        float kv = P::in_to_f32(sK[cp * KP + d]);
        if constexpr (PERCH) kv *= sBeta[cp] * __expf(sGam[(C - 1) * K + d] - sGam[cp * K + d]);
        vb[s] = kv;
      }
      const frag_t fb = P::make(vb);
#pragma unroll
      for (int Ic = 0; Ic < 4; ++Ic) {
        if (32 * kb + 31 < 16 * Ic) continue;
        const float* row = sMT + (16 * Ic + r) * LP + 32 * kb;
        float va[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          va[s] = row[kslot(grp, s)];
          if constexpr (!PERCH) va[s] *= sKs[32 * kb + kslot(grp, s)];
        }
        acc[Ic] = mma32(P::make(va), fb, acc[Ic]);
      }
    }
    ws_t* wt = static_cast<ws_t*>(a.wt) + ((size_t)cid * (K / 16) + jd) * 2 * 512;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) store_ws(wt + kb * 512 + lane * 8, acc[2 * kb], acc[2 * kb + 1]);
  }

  // ---- 4b. A^ = A_qk M^-1, computed as A^T = M^-T A_qk^T ------------------
  {
    const int Ii = wave;
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (32 * kb > 16 * Ii + 15) continue;
      const frag_t fb = frag_row_f32<P>(sA + (16 * Ii + r) * LP + 32 * kb, grp);
#pragma unroll
      for (int Ic = 0; Ic < 4; ++Ic) {
        if (Ic > Ii || 32 * kb + 31 < 16 * Ic) continue;
        const frag_t fa = frag_row_f32<P>(sMT + (16 * Ic + r) * LP + 32 * kb, grp);
        acc[Ic] = mma32(fa, fb, acc[Ic]);
      }
    }
    ws_t* ah = static_cast<ws_t*>(a.ah) + ((size_t)cid * 4 + Ii) * 2 * 512;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) store_ws(ah + kb * 512 + lane * 8, acc[2 * kb], acc[2 * kb + 1]);
  }

  // ---- row scalars --------------------------------------------------------
  {
    float* rs = a.rs + (size_t)cid * 256;
    if (tid < C) rs[tid] = PERCH ? 1.f : __expf(sGam[tid]);
    if (tid < K) rs[64 + tid] = __expf(PERCH ? sGam[(C - 1) * K + tid] : sGam[C - 1]);
  }

  // ---- per-channel decay: q exp(gamma) scale and k exp(gamma) fragments ---
  if constexpr (PERCH) {
    for (int e = tid; e < 4 * KB * 64; e += 256) {
      const int ln = e & 63, f = e >> 6, rt = f / KB, kb = f % KB;
      const int c = 16 * rt + (ln & 15), gg = ln >> 4;
      float qv[8], kv[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int d = 32 * kb + kslot(gg, s);
        const float eg = __expf(sGam[c * K + d]);
        qv[s] = P::in_to_f32(sQ[c * KP + d]) * eg * a.scale;
        kv[s] = P::in_to_f32(sK[c * KP + d]) * eg;
      }
      const size_t off = (((size_t)cid * 4 + rt) * KB + kb) * 512 + ln * 8;
      store_ws8(static_cast<ws_t*>(a.qh) + off, qv);
      store_ws8(static_cast<ws_t*>(a.kh) + off, kv);
    }
  }
}

}  // namespace gdr
