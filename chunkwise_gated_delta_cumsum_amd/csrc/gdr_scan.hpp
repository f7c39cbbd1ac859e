// State scan kernel: the serial inter-chunk recurrence (sec-03 notes,
// "inter-chunk recurrence").
//
// One workgroup per (batch, value head, slab of BV value columns); each wave
// owns 16 columns and keeps its K x 16 slice of the fp32 state S in
// registers, as MFMA accumulator tiles, for the whole sequence.  Per chunk:
//   Y = k S                       (exp(gamma) applied to the fp32 rows)
//   Z = v - exp(gamma) Y          = M r, with r = U - W S
//   o = exp(gamma) scale q S + A^ Z            (= (q exp(gamma)) S + A_qk r)
//   S <- diag(exp(gamma_last)) S + W^T Z       (= ... + K~^T diag(beta) r)
// The accumulator tiles of S and Z are already B operands (see
// gdr_device.hpp), so the chain S -> Y -> Z -> S never leaves registers.
// For per-channel decay the prep kernel supplies q exp(gamma) scale and
// k exp(gamma) as ready fragments.
#pragma once
#include "gdr_device.hpp"

namespace gdr {

struct ScanArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* s0;
  float* o;
  float* sT;
  const void* wt;
  const void* ah;
  const float* rs;
  const void* qh;
  const void* kh;
  int B, T, H, HV, N;
  float scale;
};

template <int K, int V, int BV, bool PERCH, class P>
__global__ __launch_bounds__(BV / 16 * 64) void chunk_scan_kernel(ScanArgs a) {
  using in_t = typename P::in_t;
  using frag_t = typename P::frag_t;
  using ws_t = typename P::ws_t;
  constexpr int C = kChunk;
  constexpr int NSLAB = V / BV;
  constexpr int KT = K / 16;
  constexpr int KB = K / 32;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int bh = blockIdx.x / NSLAB, sv = blockIdx.x % NSLAB;
  const int b = bh / a.HV, hv = bh % a.HV;
  const int h = hv / (a.HV / a.H);
  const int col = sv * BV + wave * 16 + r;
  const int T = a.T;

  const in_t* qg = static_cast<const in_t*>(a.q);
  const in_t* kg = static_cast<const in_t*>(a.k);
  const in_t* vg = static_cast<const in_t*>(a.v);
  const ws_t* wtg = static_cast<const ws_t*>(a.wt);
  const ws_t* ahg = static_cast<const ws_t*>(a.ah);
  const ws_t* qhg = static_cast<const ws_t*>(a.qh);
  const ws_t* khg = static_cast<const ws_t*>(a.kh);

  f32x4 S[KT];
#pragma unroll
  for (int rt = 0; rt < KT; ++rt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 16 * rt + 4 * grp + j;
      S[rt][j] = a.s0 ? a.s0[((size_t)bh * K + d) * V + col] : 0.f;
    }
  }

  float zf[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const frag_t fzero = P::make(zf);

  for (int n = 0; n < a.N; ++n) {
    const size_t cid = (size_t)bh * a.N + n;
    const int t0 = n * C;
    const float* rs = a.rs + cid * 256;

    frag_t Sf[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) Sf[kb] = P::make2(S[2 * kb], S[2 * kb + 1]);

    // Y = k S, O = q S (rows of this chunk; tiles of 16 rows)
    f32x4 Y[4], O[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Y[rt] = zero4();
      O[rt] = zero4();
      const int t = t0 + 16 * rt + r;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        frag_t ka, qa;
        if constexpr (PERCH) {
          const size_t off = ((cid * 4 + rt) * KB + kb) * 512 + lane * 8;
          ka = frag_ws(khg + off);
          qa = frag_ws(qhg + off);
        } else {
          if (t < T) {
            const size_t off = (((size_t)b * T + t) * a.H + h) * K + 32 * kb;
            ka = frag_row_in(kg + off, grp, P{});
            qa = frag_row_in(qg + off, grp, P{});
          } else {
            ka = fzero;
            qa = fzero;
          }
        }
        Y[rt] = mma32(ka, Sf[kb], Y[rt]);
        O[rt] = mma32(qa, Sf[kb], O[rt]);
      }
    }

    // Z = v - exp(gamma) Y ; O <- exp(gamma) scale O
    f32x4 Z[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 16 * rt + 4 * grp + j, t = t0 + c;
        const float vv = (t < T) ? P::in_to_f32(vg[(((size_t)b * T + t) * a.HV + hv) * V + col]) : 0.f;
        if constexpr (PERCH) {
          Z[rt][j] = vv - Y[rt][j];
        } else {
          const float eg = rs[c];
          Z[rt][j] = vv - eg * Y[rt][j];
          O[rt][j] *= eg * a.scale;
        }
      }
    }
    const frag_t Zf0 = P::make2(Z[0], Z[1]);
    const frag_t Zf1 = P::make2(Z[2], Z[3]);

    // o = O + A^ Z
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const ws_t* ap = ahg + (cid * 4 + rt) * 2 * 512 + lane * 8;
      O[rt] = mma32(frag_ws(ap), Zf0, O[rt]);
      if (rt >= 2) O[rt] = mma32(frag_ws(ap + 512), Zf1, O[rt]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = t0 + 16 * rt + 4 * grp + j;
        if (t < T) a.o[(((size_t)b * T + t) * a.HV + hv) * V + col] = O[rt][j];
      }
    }

    // S <- diag(exp(gamma_last)) S + W^T Z
#pragma unroll
    for (int rt = 0; rt < KT; ++rt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) S[rt][j] *= rs[64 + 16 * rt + 4 * grp + j];
      const ws_t* wp = wtg + (cid * KT + rt) * 2 * 512 + lane * 8;
      S[rt] = mma32(frag_ws(wp), Zf0, S[rt]);
      S[rt] = mma32(frag_ws(wp + 512), Zf1, S[rt]);
    }
  }

  if (a.sT) {
#pragma unroll
    for (int rt = 0; rt < KT; ++rt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 16 * rt + 4 * grp + j;
        a.sT[((size_t)bh * K + d) * V + col] = S[rt][j];
      }
    }
  }
}

}  // namespace gdr
