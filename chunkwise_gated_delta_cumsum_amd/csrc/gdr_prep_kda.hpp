// Chunk preparation with one decay per key channel (the KDA form of the
// "Chunkwise parallel algorithms" page and the sec-03 notes' per-channel
// decay).  Same outputs as chunk_prep_kernel, but gamma is a C x K matrix,
// so the decay cannot be pulled out of the Gram products: it must be folded
// into their operands, exp(gamma_i - gamma_j) = f(i) f'(j) per channel, with
// every factor kept in range.
//
// One wave per 16-row block (NB = C / 16 waves for C = 64 or 128 rows).
// Wave I owns the rows of block I (rows 16I..16I+15); lane (r, grp) holds row
// 16I + r at channels 8grp .. 8grp+7 of every 32-channel group (fragment
// slot i holds channel 8grp + i: the state's key-channel order, see
// chan_of_row), in registers, from the global loads on.  Per chunk:
//   1. s = in-block inclusive cumsum of g (a DPP scan across the 16 lanes of
//      a row), block totals to LDS; gamma_i = pre[I] + s_i with pre[m] the
//      sum of the totals of the blocks before m.
//   2. Off-diagonal tiles (I > J) factor the decay about the block edges:
//        exp(g_i - g_j) = exp(s_i) * exp(pre[I] - pre[J+1]) * exp(s15_J - s_j)
//      (g = gamma here).  With g <= 0 every factor is at most 1, so nothing
//      overflows; underflow only hits entries that are themselves below the
//      fp16 range.  The first factor goes on the later row (register
//      fragments of block I), the other two on the earlier row (block J's
//      fragment, shared through LDS, times a per-channel table).
//   3. Diagonal tiles factor about the block's middle row m,
//      exp(s_i - s_m) exp(s_m - s_j): with fp16 operands while |s - s_m| <= 4
//      on the block (16-bit inputs), else on fp32 MFMA, exact while
//      |s - s_m| <= 80.  Beyond that (decays near e^-80 within 8 rows) the
//      wave sums the 16x16 entries explicitly, exp per channel and entry.
//   4. q exp(gamma) scale and k exp(gamma) (the scan's operands) and
//      beta k exp(gamma_last - gamma) (for W^) from the same factors and the
//      per-block tables exp(pre[I]) and exp(pre[NB] - pre[I+1]).
// Steps 3-4 of the UT transform (inverse and folding) are shared with the
// scalar kernel.  With g > 0 the factors grow as exp(sum of the positive g in
// the chunk); fp16 operands stay finite while that sum is below about 8.
#pragma once
#include "gdr_prep.hpp"

namespace gdr {

// The in-block cumsums are kept in log2 units (g / ln 2), so that every
// factor below is one exp2 (a single v_exp_f32) of a sum or difference of
// them.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Threshold of the fp32 middle-row factorisation of a diagonal block.
constexpr float kDiagExpLimit = 80.f;
// Within e^+-4 of the middle row every factor of a diagonal block's operands
// is in the fp16 normal range for rows of unit scale (|x| e^4 < 65504, and
// the entries of the strictly lower part carry e^(s_i - s_j) <= 1 for
// g <= 0), so the 16-bit path forms the diagonal tiles with fp16 operands.
constexpr float kDiagF16Limit = 4.f;

// Inclusive scan across the 16 lanes of each DPP row (lanes 16g .. 16g+15).
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  // lanes whose source would lie before the row start read 0
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_scan16(float x) {
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  x += row_shr<8>(x);
  return x;
}

// NORM: L2-normalise the q and k rows (qk_l2norm); a template argument so
// that the unnormalised kernel carries no row-factor products.
template <int K, int C, class P, bool DUMP, bool NORM>
__global__ __launch_bounds__(C * 4) void chunk_prep_kda_kernel(PrepArgs a) {
  using in_t = typename P::in_t;
  using frag_t = typename P::frag_t;
  using ws_t = typename P::ws_t;
  using raw_t = typename P::raw_t;
  constexpr int NB = C / 16;                        // waves, one 16-row block each
  constexpr int NT = NB * 64;
  constexpr int KB = K / 32;
  constexpr int LP = lds_ld<C>();
  constexpr int SP = K + 16 / (int)sizeof(ws_t);   // row of the W^ operand tile, +16 bytes
  constexpr int NPAIR = NB * (NB - 1) / 2;          // off-diagonal block pairs J < I

  constexpr size_t KE_BYTES = (size_t)(NB - 1) * KB * 64 * sizeof(frag_t);
  constexpr size_t TAB_BYTES = (size_t)(NB + NB + NPAIR) * K * sizeof(float);
  constexpr size_t SK_BYTES = (size_t)C * SP * sizeof(ws_t);
  // the W^ operand tile takes the bytes of the earlier-row fragments and the
  // tables once they are dead
  constexpr size_t X_BYTES = KE_BYTES + TAB_BYTES > SK_BYTES ? KE_BYTES + TAB_BYTES : SK_BYTES;
  constexpr size_t L_BYTES = (size_t)C * LP * sizeof(float);
  // Loads: each wave's 16 rows of g, q and k arrive as whole rows (16 bytes
  // per lane, a row per 16..32 lanes) and pass through a per-wave staging
  // area into the row-per-lane layout below; read straight into that layout,
  // each 16-lane group would touch 16 rows, which the vector memory path
  // serves at a quarter of its contiguous rate.  Padded staging rows put the
  // 16 rows of one read on distinct banks.
  constexpr int GSR = K * 4 + 16;                           // staged g row (bytes)
  constexpr int QSR = K * (int)sizeof(in_t) + 16;           // staged q / k row
  constexpr int STG = 16 * GSR > 32 * QSR ? 16 * GSR : 32 * QSR;
  constexpr size_t BIG = NB * (size_t)STG > X_BYTES + L_BYTES ? NB * (size_t)STG
                                                               : X_BYTES + L_BYTES;
  static_assert(NB * 512 * sizeof(float) <= L_BYTES, "diagonal scratch fits the A_kk tile");
  // one LDS block, in phases: the load staging first; then sX = earlier-row
  // fragments of blocks 0..NB-2 and the per-channel tables, later sSK =
  // beta k exp(gamma_last - gamma), row-major (c, d), for W^; and sL = A_kk
  // beta (strict; D_I later, M^-T after the inverse)
  __shared__ __attribute__((aligned(16))) char sBig[BIG];
  char* sX = sBig;
  ws_t* sSK = reinterpret_cast<ws_t*>(sBig);
  float* sL = reinterpret_cast<float*>(sBig + X_BYTES);
  __shared__ __attribute__((aligned(16))) float sTot[NB * K];  // s at row 15 of each block
  __shared__ __attribute__((aligned(16))) float sMid[NB * K];  // s at row 7 of each block
  __shared__ float sBeta[C];
  frag_t* sKE = reinterpret_cast<frag_t*>(sX);                  // [NB-1][KB][64]
  float* sPf = reinterpret_cast<float*>(sX + KE_BYTES);         // [NB][K] exp(pre[I])
  float* sSf = sPf + NB * K;                                     // [NB][K] exp(pre[NB] - pre[I+1])
  float* sCf = sSf + NB * K;                                     // [NPAIR][K] exp(pre[I] - pre[J+1])

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int r = lane & 15, grp = lane >> 4;
  int b, hv, n;
  if (!prep_block(a.B, a.H, a.HV / a.H, a.N, b, hv, n)) return;
  const int h = hv / (a.HV / a.H);
  const int cid = (b * a.HV + hv) * a.N + n;
  const int T = a.T;
  const int I = wave;
  const int i = 16 * I + r;                 // this lane's row in the chunk
  const int t = n * C + i;
  const bool valid = t < T;
  GDR_PPROF_DECL;
  GDR_PPROF(0);

  // ---- loads: this lane's row, channels 32kb + 8grp + (0..7) ---------------
  // Rows past T read row T-1; the valid masks below zero their g and beta.
  raw_t qr[KB], kr[KB];
  f32x4 glo[KB], ghi[KB];
  float bv;
  {
    constexpr int GLPR = K * 4 / 16, GRPI = 64 / GLPR, GNI = 16 / GRPI;
    constexpr int QLPR = K * (int)sizeof(in_t) / 16, QRPI = 64 / QLPR, QNI = 16 / QRPI;
    static_assert(GRPI * GNI == 16 && QRPI * QNI == 16, "whole rows per load instruction");
    u32x4 graw[GNI], qraw[QNI], kraw[QNI];
#pragma unroll
    for (int j = 0; j < GNI; ++j) {
      const int tt = min(n * C + 16 * I + GRPI * j + lane / GLPR, T - 1);
      graw[j] = *reinterpret_cast<const u32x4*>(
          a.g + (((size_t)b * T + tt) * a.HV + hv) * K + (lane % GLPR) * 4);
    }
#pragma unroll
    for (int j = 0; j < QNI; ++j) {
      const int tt = min(n * C + 16 * I + QRPI * j + lane / QLPR, T - 1);
      const size_t off = (((size_t)b * T + tt) * a.H + h) * K + (lane % QLPR) * (16 / sizeof(in_t));
      qraw[j] = *reinterpret_cast<const u32x4*>(static_cast<const in_t*>(a.q) + off);
      kraw[j] = *reinterpret_cast<const u32x4*>(static_cast<const in_t*>(a.k) + off);
    }
    bv = a.beta[((size_t)b * T + min(t, T - 1)) * a.HV + hv];
    char* stg = sBig + (size_t)I * STG;
    // g rows in, this lane's row out; then q and k rows over the same bytes
    // (the LDS operations of one wave complete in order)
#pragma unroll
    for (int j = 0; j < GNI; ++j)
      *reinterpret_cast<u32x4*>(stg + (GRPI * j + lane / GLPR) * GSR + (lane % GLPR) * 16) = graw[j];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const char* src = stg + r * GSR + (32 * kb + 8 * grp) * 4;
      glo[kb] = *reinterpret_cast<const f32x4*>(src);
      ghi[kb] = *reinterpret_cast<const f32x4*>(src + 16);
    }
#pragma unroll
    for (int j = 0; j < QNI; ++j) {
      char* dst = stg + (QRPI * j + lane / QLPR) * QSR + (lane % QLPR) * 16;
      *reinterpret_cast<u32x4*>(dst) = qraw[j];
      *reinterpret_cast<u32x4*>(dst + 16 * QSR) = kraw[j];
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      qr[kb] = P::load_raw8(reinterpret_cast<const in_t*>(stg + r * QSR) + 32 * kb + 8 * grp);
      kr[kb] = P::load_raw8(reinterpret_cast<const in_t*>(stg + (16 + r) * QSR) + 32 * kb + 8 * grp);
    }
  }
  // rows past T: zero q and k once, here, rather than at every use
  if (!valid) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      qr[kb] = raw_t{};
      kr[kb] = raw_t{};
    }
  }
  // optional L2 normalisation of this lane's q and k row: its channels are
  // spread over the lanes r, r + 16, r + 32, r + 48 (grp), 8 per k block.
  // The raw values stay in registers; the row factors rsqrt(sum x^2 + 1e-6)
  // multiply them in fp32 where they are converted below.
  float fq = 1.f, fk = 1.f;
  if constexpr (NORM) {
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = P::raw_f32(qr[kb], j), y = P::raw_f32(kr[kb], j);
        sq += x * x;
        sk += y * y;
      }
    sq += __shfl_xor(sq, 16, 64);
    sk += __shfl_xor(sk, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    sk += __shfl_xor(sk, 32, 64);
    fq = rsqrtf(sq + kL2NormEps);
    fk = rsqrtf(sk + kL2NormEps);
  }
  if (!valid) bv = 0.f;

  // ---- 1. in-block cumsum ----------------------------------------------------
  float s[KB][8];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s[kb][j] = row_scan16(valid ? glo[kb][j] * kLog2e : 0.f);
      s[kb][4 + j] = row_scan16(valid ? ghi[kb][j] * kLog2e : 0.f);
    }
  if (r == 15 || r == 7) {
    float* dst = (r == 15 ? sTot : sMid) + I * K;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      *reinterpret_cast<f32x4*>(dst + 32 * kb + 8 * grp) = f32x4{s[kb][0], s[kb][1], s[kb][2], s[kb][3]};
      *reinterpret_cast<f32x4*>(dst + 32 * kb + 8 * grp + 4) = f32x4{s[kb][4], s[kb][5], s[kb][6], s[kb][7]};
    }
  }
  if (grp == 0) sBeta[i] = bv;
  lds_barrier();
  GDR_PPROF(1);

  // ---- per-channel tables (all threads) --------------------------------------
  {
    const int d = tid % K, part = tid / K;
    // pre[m] = sum of the block totals before block m, in the order m = 0, 1, ...
    auto pre = [&](int m) {
      float x = 0.f;
      for (int j = 0; j < m; ++j) x += sTot[j * K + d];
      return x;
    };
    float* rs = a.rs + (size_t)cid * 256;
    for (int it = part; it < 2 * NB + NPAIR + 1; it += NT / K) {
      if (it < NB) {
        sPf[it * K + d] = ex2(pre(it));
      } else if (it < 2 * NB) {
        sSf[(it - NB) * K + d] = ex2(pre(NB) - pre(it - NB + 1));
      } else if (it < 2 * NB + NPAIR) {
        // pair p = I2 (I2 - 1) / 2 + J2 with J2 < I2
        const int p = it - 2 * NB;
        int I2 = 1;
        while ((I2 + 1) * I2 / 2 <= p) ++I2;
        const int J2 = p - I2 * (I2 - 1) / 2;
        sCf[p * K + d] = ex2(pre(I2) - pre(J2 + 1));
      } else {
        rs[C + row_of_chan(d)] = ex2(pre(NB));   // in the state's row order
      }
    }
    for (int e = tid; e < C; e += NT) rs[e] = 1.f;
  }
  lds_barrier();   // the tables are complete

  // ---- 2/3. own-block factors, earlier-row fragments, diagonal tiles ----------
  // kl = k exp(s), ql = q exp(s): the later-row side (reference row 16I - 1),
  // kept as MFMA fragments for the off-diagonal tiles; ke = k exp(s15 - s):
  // the earlier-row side (reference row 16I + 15), shared through LDS.  The
  // same factors give this row's scan operands q exp(gamma) scale and
  // k exp(gamma) (stored here) and its W^ operand row
  // beta k exp(gamma_last - gamma) (kept as a fragment until its LDS tile is
  // free), so no fp32 copy of the row outlives this loop.
  frag_t kLf[KB], qLf[KB], wxf[KB];
  f32x4 dkk = zero4(), dqk = zero4();      // diagonal A_kk and A_qk^T tiles (raw dots)
  bool far = false;
  const size_t off0 = (size_t)cid * NB * KB * 512 + ((size_t)I * KB) * 512 + lane * 8;
  // Per k block in three parts, each of whose fp32 rows die at its end (the
  // empty asm statements pin each fragment's conversion in place, and the
  // scheduling fences keep the parts from overlapping): held together, the
  // rows of every part would need more registers than three workgroups per
  // CU leave.
  auto qv_of = [&](int kb, int j) {
    const float x = P::raw_f32(qr[kb], j);
    return NORM ? x * fq : x;
  };
  auto kv_of = [&](int kb, int j) {
    const float x = P::raw_f32(kr[kb], j);
    return NORM ? x * fk : x;
  };
  auto f4 = [](const float* p) { return *reinterpret_cast<const f32x4*>(p); };
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int d0 = 32 * kb + 8 * grp;
    {  // a. the later-row side and the scan operands
      const f32x4 pa = f4(sPf + I * K + d0), pb = f4(sPf + I * K + d0 + 4);
      float kl[8], ql[8], qx[8], kx[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float el = ex2(s[kb][j]);
        kl[j] = kv_of(kb, j) * el;
        ql[j] = qv_of(kb, j) * el;
        const float pf = j < 4 ? pa[j] : pb[j - 4];   // exp(gamma_i) = exp(s) exp(pre[I])
        qx[j] = ql[j] * pf * a.scale;
        kx[j] = kl[j] * pf;
      }
      kLf[kb] = P::make(kl);
      qLf[kb] = P::make(ql);
      asm volatile("" : "+v"(kLf[kb]), "+v"(qLf[kb]));
      store_ws8(static_cast<ws_t*>(a.qh) + off0 + (size_t)kb * 512, qx);
      store_ws8(static_cast<ws_t*>(a.kh) + off0 + (size_t)kb * 512, kx);
    }
    __builtin_amdgcn_sched_barrier(0);
    {  // b. the earlier-row side and the W^ operand row
      const f32x4 t15a = f4(sTot + I * K + d0), t15b = f4(sTot + I * K + d0 + 4);
      const f32x4 wa = f4(sSf + I * K + d0), wb = f4(sSf + I * K + d0 + 4);
      float ke[8], wx[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float s15 = j < 4 ? t15a[j] : t15b[j - 4];
        ke[j] = kv_of(kb, j) * ex2(s15 - s[kb][j]);
        // exp(gamma_last - gamma_i) = exp(s15 - s) exp(pre[NB] - pre[I+1])
        wx[j] = bv * ke[j] * (j < 4 ? wa[j] : wb[j - 4]);
      }
      if (I < NB - 1) sKE[(I * KB + kb) * 64 + lane] = P::make(ke);
      wxf[kb] = P::make(wx);
      asm volatile("" : "+v"(wxf[kb]));
    }
    __builtin_amdgcn_sched_barrier(0);
    {  // c. the diagonal tile, factored about the block's middle row
      const f32x4 tma = f4(sMid + I * K + d0), tmb = f4(sMid + I * K + d0 + 4);
      float a1[8], b1[8], b2[8];
      bool wide = false;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float dl = s[kb][j] - (j < 4 ? tma[j] : tmb[j - 4]);
        far |= !(fabsf(dl) <= kDiagExpLimit * kLog2e);
        wide |= !(fabsf(dl) <= kDiagF16Limit * kLog2e);
        const float dm = ex2(dl), dmi = ex2(-dl);
        const float kv = kv_of(kb, j);
        a1[j] = kv * dm;
        b1[j] = kv * dmi;
        b2[j] = qv_of(kb, j) * dm;
      }
      if (P::kF32 || __any(wide)) {
        const f32x8 fa1 = {a1[0], a1[1], a1[2], a1[3], a1[4], a1[5], a1[6], a1[7]};
        const f32x8 fb1 = {b1[0], b1[1], b1[2], b1[3], b1[4], b1[5], b1[6], b1[7]};
        const f32x8 fb2 = {b2[0], b2[1], b2[2], b2[3], b2[4], b2[5], b2[6], b2[7]};
        dkk = mma32(fa1, fb1, dkk);   // rows i, columns j of block I
        dqk = mma32(fb1, fb2, dqk);   // rows c' (k), columns i (q) of block I
      } else {
        // every factor within e^+-kDiagF16Limit: fp16 operands, the
        // precision of the off-diagonal tiles, in one MFMA instead of eight
        const frag_t ha1 = P::make(a1), hb1 = P::make(b1), hb2 = P::make(b2);
        dkk = mma32(ha1, hb1, dkk);
        dqk = mma32(hb1, hb2, dqk);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (__any(far)) {
    // Explicit diagonal block: lane (r, grp) sums its channels for the pairs
    // (row r, row (r - m) mod 16), m = 0..15, the four channel groups are
    // added across lanes, and the entries are routed through LDS (the A_kk
    // tile is not written yet) into accumulator layout.  This branch is rare:
    // it loads its rows of g, q and k again (from L2) and redoes their
    // cumsum, so that none of them has to stay live through the loop above.
    raw_t qr2[KB], kr2[KB];
    float s2[KB][8];
    {
      const int tt = min(t, T - 1);
      const float* grow = a.g + (((size_t)b * T + tt) * a.HV + hv) * K;
      const size_t qoff = (((size_t)b * T + tt) * a.H + h) * K;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(grow + 32 * kb + 8 * grp);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(grow + 32 * kb + 8 * grp + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s2[kb][j] = row_scan16(valid ? g0[j] : 0.f);
          s2[kb][4 + j] = row_scan16(valid ? g1[j] : 0.f);
        }
        qr2[kb] = P::load_raw8(static_cast<const in_t*>(a.q) + qoff + 32 * kb + 8 * grp);
        kr2[kb] = P::load_raw8(static_cast<const in_t*>(a.k) + qoff + 32 * kb + 8 * grp);
      }
    }
    float* scr = sL + wave * 512;   // [2][16][16]
    for (int m = 0; m < 16; ++m) {
      const int jr = (r - m) & 15;
      const int src = jr + 16 * grp;
      float pk = 0.f, pq = 0.f;
      // q and k are converted again in every pass from their 16-bit values
      // (the empty asm keeps the fp32 rows from being held across the loop)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) asm volatile("" : "+v"(qr2[kb]), "+v"(kr2[kb]));
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float qv = valid ? (NORM ? P::raw_f32(qr2[kb], j) * fq : P::raw_f32(qr2[kb], j)) : 0.f;
          const float kv = valid ? (NORM ? P::raw_f32(kr2[kb], j) * fk : P::raw_f32(kr2[kb], j)) : 0.f;
          const float kj = __shfl(kv, src, 64);
          const float sj = __shfl(s2[kb][j], src, 64);
          const float e = __expf(s2[kb][j] - sj);
          pk += kv * kj * e;
          pq += qv * kj * e;
          // a few exchanges in flight at a time, not all 64 of a pass
          if ((j & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
      pk += __shfl_xor(pk, 16, 64);
      pk += __shfl_xor(pk, 32, 64);
      pq += __shfl_xor(pq, 16, 64);
      pq += __shfl_xor(pq, 32, 64);
      if (grp == 0 && jr <= r) {
        scr[r * 16 + jr] = pk;          // A_kk (i = r, j = jr)
        scr[256 + jr * 16 + r] = pq;    // A_qk^T (c' = jr, i = r)
      }
    }
    // the wave's own LDS writes are complete before it reads them back
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      const int rr = 4 * grp + j4;
      dkk[j4] = rr > r ? scr[rr * 16 + r] : 0.f;
      dqk[j4] = rr <= r ? scr[256 + rr * 16 + r] : 0.f;
    }
  }
  if constexpr (DUMP) {
    if (a.d_gamma) {
      float* dg = a.d_gamma + ((size_t)cid * C + i) * K;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int d = 32 * kb + 8 * grp + j;
          float pre = 0.f;
          for (int m = 0; m < I; ++m) pre += sTot[m * K + d];
          dg[d] = (pre + s[kb][j]) * kLn2;   // natural units
        }
    }
  }
  lds_barrier();   // sKE is complete; the diagonal scratch is read
  GDR_PPROF(2);

  // ---- off-diagonal tiles (J < I) ----------------------------------------------
  f32x4 aqT[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) aqT[j] = zero4();
  if (I > 0) {
    for (int J = 0; J < I; ++J) {
      const float* cf = sCf + (I * (I - 1) / 2 + J) * K;
      f32x4 akk = zero4(), aq = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const frag_t fe = sKE[(J * KB + kb) * 64 + lane];
        const f32x4 ca = *reinterpret_cast<const f32x4*>(cf + 32 * kb + 8 * grp);
        const f32x4 cb = *reinterpret_cast<const f32x4*>(cf + 32 * kb + 8 * grp + 4);
        float fv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) fv[j] = (float)fe[j] * (j < 4 ? ca[j] : cb[j - 4]);
        const frag_t F = P::make(fv);
        akk = mma32(kLf[kb], F, akk);   // rows i (block I), columns j (block J)
        aq = mma32(F, qLf[kb], aq);     // rows c' (block J), columns i (block I)
      }
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int ii = 16 * I + 4 * grp + j4, jj = 16 * J + r;
        sL[ii * LP + jj] = a.linear ? 0.f : akk[j4] * sBeta[jj];   // linear rule: M = I
        aq[j4] *= sBeta[16 * J + 4 * grp + j4] * a.scale;
      }
      aqT[J] = aq;
    }
  }
  // diagonal tiles: masks, beta, scale
#pragma unroll
  for (int j4 = 0; j4 < 4; ++j4) {
    const int rr = 16 * I + 4 * grp + j4, cc = 16 * I + r;
    sL[rr * LP + cc] = (rr > cc && !a.linear) ? dkk[j4] * sBeta[cc] : 0.f;
    aqT[I][j4] = rr <= cc ? dqk[j4] * sBeta[rr] * a.scale : 0.f;
  }

  lds_barrier();   // sL complete; sKE and the tables are dead
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) store_frag16(sSK + i * SP + 32 * kb + 8 * grp, wxf[kb]);
  lds_barrier();   // sSK complete
  GDR_PPROF(3);

  if constexpr (DUMP) {
    if (a.d_akk) dump_akk<C>(a.d_akk + (size_t)cid * C * C, sL, tid);
    if (a.d_aqk) dump_aqk<C>(a.d_aqk + (size_t)cid * C * C, aqT, wave, r, grp);
    lds_barrier();   // sL is read before the inverse overwrites it
  }

  // ---- M^-1 (M^-T replaces A_kk in sL), then the folded operands -------------
  // (the linear rule: M = I, the identity written only for the dump, and the
  // folds element by element)
  if (a.linear) {
    if constexpr (DUMP) identity_inverse<C>(sL, tid);
  } else {
    unit_lower_inverse<C, P>(sL, wave, r, grp);
  }
  GDR_PPROF(4);
  if constexpr (DUMP) {
    if (a.d_minv) dump_minv<C>(a.d_minv + (size_t)cid * C * C, sL, tid);
  }
  ws_t* const wt_chunk = static_cast<ws_t*>(a.wt) + (size_t)cid * K * C;
  auto sk_at = [&](int c, int d) { return (float)sSK[c * SP + d]; };
  auto unit = [&](int) { return 1.f; };
  if (a.linear)
    fold_w_identity<K, C, P, false>(wt_chunk, wave, lane, r, grp, sk_at, unit);
  else
    fold_w<K, C, P, false>(sL, wt_chunk, wave, lane, r, grp, sk_at, unit);
  GDR_PPROF(5);
  ws_t* const ah_chunk = static_cast<ws_t*>(a.ah) + (size_t)cid * ah_frags(C) * 512;
  if (a.linear)
    fold_aqk_identity<C, P>(aqT, ah_chunk, wave, lane);
  else
    fold_aqk<C, P>(aqT, sL, ah_chunk, wave, lane, r, grp);
  GDR_PPROF(6);
  GDR_PPROF_FLUSH;
}

}  // namespace gdr
