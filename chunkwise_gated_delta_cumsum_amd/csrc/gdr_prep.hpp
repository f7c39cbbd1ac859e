// Chunk preparation kernel: everything that is parallel across chunks.
//
// One workgroup (4 waves) per (batch, value head, chunk of C = 64 rows).
// Steps, following the sec-03 notes ("in-chunk cumsum and lower-triangular
// solve", "decayed dot function") and the UT transform of the "Chunkwise
// parallel algorithms" page (section 2.3):
//   1. gamma = inclusive cumsum of g over the chunk (wave-level scan; per key
//      channel for the KDA form).
//   2. Gram tiles of k k^T and k q^T on MFMA (lower 16x16 tiles only), then
//      the decay exp(gamma_i - gamma_j), beta on columns and the masks:
//      strict lower for A_kk, lower with diagonal for A_qk (scale folded in).
//      exp is never taken for j > i.  A_qk is formed transposed, so its
//      accumulator tiles are directly the B operands of step 4b and stay in
//      registers.  With per-channel decay every tile uses the factorisation
//      exp(gamma_i - gamma_r) exp(gamma_r - gamma_j) about a reference row r
//      (the last row of the column tile off the diagonal, the middle row on
//      it), guarded by a range check; tiles that fail it are summed
//      explicitly in fp32.
//   3. M = I + A_kk; M^-1 by blocks: each wave inverts one 16x16 unit-lower
//      diagonal block by forward substitution, then wave J forms block column
//      J: X_IJ = -D_I sum_m L_Im X_mJ for I > J, on fp32 MFMA.
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

#ifdef GDR_PREP_PROFILE
__device__ long long gdr_prep_prof[16 * 4];
#define GDR_PPROF(ph)                                                         \
  do {                                                                        \
    if (cid == 7 && lane == 0) gdr_prep_prof[(ph) * 4 + wave] = clock64();    \
  } while (0)
#else
#define GDR_PPROF(ph) do {} while (0)
#endif

// Range limits of the factored per-channel decay (fp16 operands): the sum of
// max(g, 0) over a chunk, and the decay across one 16-row diagonal block.
constexpr float kPosDriftLimit = 0.5f;
constexpr float kDiagDecayLimit = 8.f;

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

template <int K, bool PERCH, class P, bool DUMP>
__global__ __launch_bounds__(256) void chunk_prep_kernel(PrepArgs a) {
  using in_t = typename P::in_t;
  using frag_t = typename P::frag_t;
  using ws_t = typename P::ws_t;
  constexpr int C = kChunk;
  constexpr int KP = K + 16 / (int)sizeof(in_t);  // q/k tile row, +16 bytes
  constexpr int LP = C + 4;                        // C x C fp32 tile row
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
  __shared__ __attribute__((aligned(16))) float sGam[PERCH ? C * K : C];
  __shared__ float sBeta[C];
  __shared__ float sKs[C];     // beta_c exp(gamma_last - gamma_c), one decay per row
  __shared__ float sPos[256];
  __shared__ int sFlag[8];     // per-channel: [0] positive drift, [1..4] diagonal blocks
  float* sMT = reinterpret_cast<float*>(sQbuf);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  constexpr int GPT = PERCH ? C * K / 4 / 256 : 1;   // float4 of g per thread
  f32x4 gq[GPT];
  if constexpr (!PERCH) {
    if (wave == 0) {
      const int t = t0 + lane;
      if (t < T) {
        const size_t idx = ((size_t)b * T + t) * a.HV + hv;
        gv = a.g[idx];
        bv = a.beta[idx];
      }
    }
  } else {
    if (tid < C) {
      const int t = t0 + tid;
      bv = (t < T) ? a.beta[((size_t)b * T + t) * a.HV + hv] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int e = tid + 256 * i, c = e / (K / 4), d4 = (e % (K / 4)) * 4;
      const int t = t0 + c;
      gq[i] = zero4();
      if (t < T) gq[i] = *reinterpret_cast<const f32x4*>(a.g + (((size_t)b * T + t) * a.HV + hv) * K + d4);
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
  if constexpr (!PERCH) {
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
  } else {
    if (tid < C) sBeta[tid] = bv;
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int e = tid + 256 * i, c = e / (K / 4), d4 = (e % (K / 4)) * 4;
      *reinterpret_cast<f32x4*>(sGam + c * K + d4) = gq[i];
    }
    __syncthreads();
    // column scans: thread (d, part) scans RP rows, then adds the earlier parts
    constexpr int PARTS = 256 / K;
    constexpr int RP = C / PARTS;
    const int d = tid % K, part = tid / K;
    float run = 0.f, pos = 0.f;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      const float x = sGam[(part * RP + i) * K + d];
      run += x;
      pos += fmaxf(x, 0.f);
      sGam[(part * RP + i) * K + d] = run;
    }
    sPos[tid] = pos;
    __syncthreads();
    float offv = 0.f, post = 0.f;
#pragma unroll
    for (int p = 0; p < PARTS; ++p) {
      if (p < part) offv += sGam[((p + 1) * RP - 1) * K + d];
      post += sPos[p * K + d];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RP; ++i) sGam[(part * RP + i) * K + d] += offv;
    if (tid < 8) sFlag[tid] = 0;
    __syncthreads();
    // range checks of the factored form
    if (post > kPosDriftLimit) sFlag[0] = 1;
    if (part == 0) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        float lo = sGam[(16 * blk) * K + d], hi = lo;
#pragma unroll
        for (int i = 1; i < 16; ++i) {
          const float x = sGam[(16 * blk + i) * K + d];
          lo = fminf(lo, x);
          hi = fmaxf(hi, x);
        }
        if (hi - lo > kDiagDecayLimit) sFlag[1 + blk] = 1;
      }
    }
  }
  __syncthreads();
  GDR_PPROF(1);

  // ---- 2. decayed dots ----------------------------------------------------
  // A_qk^T tiles (rows c' in block J, columns i in block w) for J <= w stay
  // in this wave's registers; A_kk tiles go to LDS.  Work per wave: w+1 A_qk
  // tiles and 4-w A_kk tiles.
  f32x4 aqT[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) aqT[j] = zero4();
  {
    // One tile job: x rows of block I (A operand) against y rows of block J
    // (B operand); x_late says which side holds the later tokens.  The decay
    // exp(gamma_late - gamma_early) is factored about a reference row: the
    // last row of the earlier block off the diagonal, the middle row on it.
    auto gram = [&](const in_t* xs, int I, const in_t* ys, int J, bool x_late, bool diag,
                    int flag) -> f32x4 {
      f32x4 acc = zero4();
      const in_t* ra = xs + (16 * I + r) * KP;
      const in_t* rb = ys + (16 * J + r) * KP;
      if constexpr (!PERCH) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          if constexpr (P::kF32)
            acc = mma32(frag_row_in(ra + 32 * kb, grp, P{}), frag_row_in(rb + 32 * kb, grp, P{}), acc);
          else
            acc = mma32(frag_row_bf16(ra + 32 * kb, grp), frag_row_bf16(rb + 32 * kb, grp), acc);
        }
      } else {
        const int ref = diag ? 16 * J + 7 : 16 * (x_late ? J : I) + 15;
        const float sx = x_late ? 1.f : -1.f;   // sign of (gamma_x - gamma_ref)
        const int ia = 16 * I + r, jb = 16 * J + r;
        if (!flag) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            float va[8], vb[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
              const int d = 32 * kb + kslot(grp, s);
              const float gr = sGam[ref * K + d];
              va[s] = P::in_to_f32(xs[ia * KP + d]) * __expf(sx * (sGam[ia * K + d] - gr));
              vb[s] = P::in_to_f32(ys[jb * KP + d]) * __expf(sx * (gr - sGam[jb * K + d]));
            }
            acc = mma32(P::make(va), P::make(vb), acc);
          }
        } else {
          // explicit sum for the accumulator entries this lane owns (row
          // 16I + 4grp + j4 of x, row 16J + r of y); entries whose later row
          // precedes the earlier one are masked by the caller and left 0
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            const int i = 16 * I + 4 * grp + j4, j = 16 * J + r;
            const int late = x_late ? i : j, early = x_late ? j : i;
            float s = 0.f;
            if (late >= early) {
              for (int d = 0; d < K; ++d)
                s += P::in_to_f32(xs[i * KP + d]) * P::in_to_f32(ys[j * KP + d]) *
                     __expf(sGam[late * K + d] - sGam[early * K + d]);
            }
            acc[j4] = s;
          }
        }
      }
      return acc;
    };

    // A_qk^T = k q^T: tiles (J, w), rows c' (k), columns i (q)
    for (int J = 0; J <= wave; ++J) {
      int flag = 0;
      if constexpr (PERCH) flag = sFlag[0] | (J == wave ? sFlag[1 + J] : 0);
      const f32x4 acc = gram(sK, J, sQ, wave, false, J == wave, flag);
      f32x4 val;
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int cp = 16 * J + 4 * grp + j4, i = 16 * wave + r;
        float x = 0.f;
        if (cp <= i) {
          x = acc[j4] * sBeta[cp] * a.scale;
          if constexpr (!PERCH) x *= __expf(sGam[i] - sGam[cp]);
        }
        val[j4] = x;
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
      int flag = 0;
      if constexpr (PERCH) flag = sFlag[0] | (I == J ? sFlag[1 + I] : 0);
      const f32x4 acc = gram(sK, I, sK, J, true, I == J, flag);
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int i = 16 * I + 4 * grp + j4, j = 16 * J + r;
        float x = 0.f;
        if (i > j) {
          x = acc[j4] * sBeta[j];
          if constexpr (!PERCH) x *= __expf(sGam[i] - sGam[j]);
        }
        sL[i * LP + j] = x;
      }
    }
  }

  // q and k as A fragments for the scan (rows c, k = d).  One decay per row:
  // raw q, k in fp16, written once per (batch, q/k head, chunk) by the first
  // value head of the group.  Per-channel decay: q exp(gamma) scale and
  // k exp(gamma), per value head.
  {
    const bool writer = PERCH || (hv % (a.HV / a.H)) == 0;
    const size_t fid = PERCH ? (size_t)cid : ((size_t)b * a.H + h) * a.N + n;
    if (writer) {
      for (int e = tid; e < 4 * KB * 64; e += 256) {
        const int ln = e & 63, f = e >> 6, rt = f / KB, kb = f % KB;
        const int c = 16 * rt + (ln & 15), gg = ln >> 4;
        const auto qr = P::load_raw(sQ + c * KP + 32 * kb, gg);
        const auto kr = P::load_raw(sK + c * KP + 32 * kb, gg);
        float qx[8], kx[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          qx[s] = P::raw_f32(qr, s);
          kx[s] = P::raw_f32(kr, s);
          if constexpr (PERCH) {
            const float eg = __expf(sGam[c * K + 32 * kb + kslot(gg, s)]);
            qx[s] *= eg * a.scale;
            kx[s] *= eg;
          }
        }
        const size_t off = ((fid * 4 + rt) * KB + kb) * 512 + ln * 8;
        store_ws8(static_cast<ws_t*>(a.qh) + off, qx);
        store_ws8(static_cast<ws_t*>(a.kh) + off, kx);
      }
    }
  }
  __syncthreads();   // sL complete; sQ free for M^-T
  GDR_PPROF(2);

  if constexpr (DUMP) {
    constexpr int GS = PERCH ? K : 1;
    if (a.d_gamma)
      for (int e = tid; e < C * GS; e += 256) a.d_gamma[(size_t)cid * C * GS + e] = sGam[e];
    if (a.d_akk)
      for (int e = tid; e < C * C; e += 256) {
        const int i = e / C, j = e % C;
        a.d_akk[(size_t)cid * C * C + e] = (j < i && (i >> 4) >= (j >> 4)) ? sL[i * LP + j] : 0.f;
      }
    if (a.d_aqk) {
      // tile (J, wave) of A_qk^T: rows c' = 16J + 4grp + j4, column i = 16 wave + r
      for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int cp = 16 * J + 4 * grp + j4, i = 16 * wave + r;
          a.d_aqk[(size_t)cid * C * C + i * C + cp] = J <= wave ? aqT[J][j4] : 0.f;
        }
    }
  }

  // ---- 3a. each wave inverts its diagonal block ---------------------------
  for (int i = tid * 4; i < C * LP; i += 256 * 4) *reinterpret_cast<f32x4*>(sMT + i) = zero4();
  __syncthreads();
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
  GDR_PPROF(3);

  // ---- 3b. wave J forms block column J of M^-1 ----------------------------
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
  GDR_PPROF(4);

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
        float kx = P::in_to_f32(sK[cp * KP + d]);
        if constexpr (PERCH) kx *= sBeta[cp] * __expf(sGam[(C - 1) * K + d] - sGam[cp * K + d]);
        vb[s] = kx;
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
  GDR_PPROF(5);

  // ---- 4b. A^ = A_qk M^-1, as A^T = M^-T A_qk^T (column tile = wave) ------
  {
    const int Ii = wave;
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (32 * kb > 16 * Ii + 15) continue;
      const frag_t fb = P::make2(aqT[2 * kb], aqT[2 * kb + 1]);
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
  GDR_PPROF(6);

  // ---- row scalars --------------------------------------------------------
  {
    float* rs = a.rs + (size_t)cid * 256;
    if (tid < C) rs[tid] = PERCH ? 1.f : __expf(sGam[tid]);
    if (tid < K) rs[64 + tid] = __expf(PERCH ? sGam[(C - 1) * K + tid] : sGam[C - 1]);
  }
  GDR_PPROF(7);
}

}  // namespace gdr
