// State scan kernels: the serial inter-chunk recurrence (sec-03 notes,
// "inter-chunk recurrence"), optionally split into sequence segments.
//
// Per chunk, with r = U - W S = M^-1 Z folded into the prep outputs:
//   Y = k S                       (exp(gamma) applied to the fp32 rows)
//   Z = v - exp(gamma) Y          (= M r)
//   o = exp(gamma) scale q S + A^ Z             (= (q exp(gamma)) S + A_qk r)
//   S <- diag(exp(gamma_last)) S + W^T Z        (= ... + K~^T diag(beta) r)
// (per-channel decay: the prep kernel folds exp(gamma) into the q, k
// fragments, so the row scales are 1.)  For the decayed linear attention
// (no erase term) M = I, so W^ = diag(beta exp(gamma_last - gamma)) k and
// A^ = A_qk, and Z = v: the same loop with the prediction dropped.  With
// 64-column slabs that rule has its own instantiation (LIN): Z = v needs
// no state, so it is staged a step ahead and a step has one barrier.
//
// The state update is affine in S: S_{n+1} = A_n S_n + B_n.  A sequence cut
// into segments is therefore run in two passes:
//   chain mode  : per (head, segment) the segment's transition Phi = prod A_n
//                 (the scan run on an identity state with v = 0) and its
//                 zero-start end state E (the scan run from S = 0), in
//                 parallel over segments;
//   full mode   : the scan of every segment from its true start state,
//                 writing o, in parallel over segments; segment p first
//                 runs the combine S_{q+1} = Phi_q S_q + E_q, q < p, itself
//                 (combine_prefix).
// With one segment only the full mode runs.
//
// Work split in a workgroup of NW waves (4, or 8 for 128-row chunks with
// K = 128) over BV = 32 or 64 state columns (a "slab"): wave w owns chunk
// rows [C/NW w, C/NW (w+1)) of Y, Z and o and state rows [K/NW w,
// K/NW (w+1)).  Every A-operand fragment (k, q, W^T and A^ rows)
// belongs to exactly one wave, which loads it straight into registers.  The
// next chunk's operands are double-buffered and their loads are issued one
// at a time between the current chunk's products: issued in a burst they
// stall the wave (in-order issue) while the memory pipeline drains them.
// Only the B operands S and Z cross between waves, through LDS in fragment
// order (accumulator tiles are B fragments, see gdr_device.hpp), with two
// barriers per chunk (one for LIN).  The output is formed transposed,
// o^T = S^T q^T + Z^T A^T: the B fragments of S and Z are also A fragments of
// S^T and Z^T, and the q and A^ fragments are B fragments of q^T and A^T, so
// no operand moves, and each lane ends up with four consecutive columns of
// one o row.  Those rows pass through a per-wave LDS area so that they leave
// as whole 256-byte rows, stored at the end of the chunk's step once every
// load of the step is issued (so no wait for loads also waits for them); v
// arrives as 16-byte row pieces and reaches accumulator layout through a
// per-wave LDS tile, filled at the end of the step before.  The LDS work
// that belongs to no product thus sits after the last product of a step
// instead of between the barrier and the first.  The fp32 state never
// leaves registers except at segment ends.
//
// Every global operand is stored in the order its lanes consume it, 16
// contiguous bytes per lane: the vector memory path serves a 16-lane access
// that touches 16 rows at a quarter of its contiguous rate.  The k and q
// fragments are the prep kernel's copies (q and k with one decay per row,
// k exp(gamma) and q exp(gamma) scale per channel).
#pragma once
#include <type_traits>
#include "gdr_device.hpp"

namespace gdr {

struct ScanArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* s0;
  void* o;           // [B, T, HV, V] in the format o_fmt
  float* sT;
  const void* wt;
  const void* ah;
  const float* rs;
  const void* qh;
  const void* kh;
  int B, T, H, HV, N;
  float scale;
  int linear;        // 1: decayed linear attention: Z = v (no prediction term)
  // segment p covers chunks [p * seg_len, min((p + 1) * seg_len, N))
  int seg_len, nseg;
  void* phi;         // transitions [BH][nseg-1], each K x K in A-fragment order
                     // [K/16 row tiles][K/32 k blocks][64 lanes][8], workspace type
  float* eend;       // zero-start end states, tile order [BH][nseg-1][K*V]
  int o_fmt;         // kOutF32, kOutBF16 or kOutF16
  float* s0_copy;    // chain pass: when set, copy s0 here [BH][K][V] (the full
                     // pass then reads this copy: the state is updated in place)
};

#ifdef GDR_SCAN_PROFILE
// clock marks of one chunk step, kept in registers and written out at the
// end of the step (a store per mark would add waits of its own)
__device__ long long gdr_scan_prof[64 * 16 * 8];
#define GDR_PROF_DECL long long pt_[16] = {}
#define GDR_PROF(ph) pt_[ph] = clock64()
#define GDR_PROF_FLUSH                                                             \
  do {                                                                             \
    if (MODE == kScanFull && bh == 0 && p == 0 && sv == 0 && lane == 0 && n < 64)   \
      for (int i_ = 0; i_ < 16; ++i_) gdr_scan_prof[(n * 16 + i_) * 8 + w] = pt_[i_]; \
  } while (0)
#else
#define GDR_PROF_DECL do {} while (0)
#define GDR_PROF(ph) do {} while (0)
#define GDR_PROF_FLUSH do {} while (0)
#endif

constexpr int kScanFull = 0;
constexpr int kScanChain = 1;

// Waves per scan workgroup: one 16-row tile of the chunk and K/16/NW state
// row tiles each; 128-row chunks with K = 128 take 8 waves (one chunk row
// tile and one state row tile each), 32-row chunks 2, everything else 4.
template <int K, int C>
constexpr int scan_waves() { return C == 32 ? 2 : (C == 128 && K == 128) ? 8 : 4; }


// Calls f(std::integral_constant<int, I>{}) for I = B .. E-1.
template <int B, int E, class F>
__device__ __forceinline__ void static_for_scan(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for_scan<B + 1, E>(f);
  }
}

// Half of a fragment (4 consecutive k slots) in LDS.
template <class F>
__device__ __forceinline__ void store_half(F* frag, int half, f32x4 v);
template <>
__device__ __forceinline__ void store_half<half8>(half8* frag, int half, f32x4 v) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  h4 x = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
  reinterpret_cast<h4*>(frag)[half] = x;
}
template <>
__device__ __forceinline__ void store_half<f32x8>(f32x8* frag, int half, f32x4 v) {
  reinterpret_cast<f32x4*>(frag)[half] = v;
}

// XCD-aware placement: workgroups are dealt to the 8 XCDs round-robin.  A
// group is one (batch, q/k head, segment); its G value heads and their slabs
// get the same (id % 8) and consecutive slots, so every operand they share
// (the q/k rows of the head, and each value head's W^ and A^ across its
// slabs) is read through one L2.  unit = (batch * HV + value head) * nsegu
// + segment.
__device__ __forceinline__ bool unit_block(int B, int H, int G, int nsegu, int nslab, int& unit,
                                           int& sv) {
  const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
  sv = slot % nslab;
  const int gi = (slot / nslab) % G;
  const long group = (long)(slot / nslab / G) * 8 + xcd;   // (b, h, segment)
  if (group >= (long)B * H * nsegu) return false;
  const int p = (int)(group % nsegu);
  const long bhq = group / nsegu;
  const long bh = (bhq / H) * (H * G) + (bhq % H) * G + gi;
  unit = (int)(bh * nsegu + p);
  return true;
}

// Offset (floats) of accumulator tile (state row tile dt, column tile ct) of
// slab sv inside one K x V state kept in tile order:
// [slab][row tile][column tile][64 lanes][4].
template <int K, int BV>
__device__ __forceinline__ size_t state_tile(int sv, int dt, int ct) {
  return (((size_t)sv * (K / 16) + dt) * (BV / 16) + ct) * 256;
}

// Bytes of one wave's staging area for its fp32 o rows (full mode only).
template <int MODE, int BV, int C, int NW>
constexpr int scan_stage_bytes() {
  return MODE == kScanFull ? (C / NW) * (BV * 4 + 16) : 16;
}

// The start state of segment p from the chain pass's results:
// S_{q+1} = Phi_q S_q + E_q for q = 0 .. p-1, from S_0 = the initial state
// (in S on entry).  Each segment's workgroup runs its own prefix of this
// short serial recurrence before its chunk loop, so no separate pass and no
// round trip of the segment states through memory sits between the chain
// and full passes.  Wave w owns state rows 16(SRT w + st) + 4grp + j (its
// accumulator tiles); S crosses waves through LDS as B fragments, Phi_q
// arrives as A fragments and E_q as accumulator tiles, both 16 contiguous
// bytes per lane, the next step's loaded while this one computes.
template <int K, int V, class P, int SRT, int BV>
__device__ __forceinline__ void combine_prefix(const ScanArgs& a, typename P::frag_t* sS, int bh,
                                               int p, int sv, int w, int lane,
                                               f32x4 (&S)[SRT][BV / 16]) {
  using frag_t = typename P::frag_t;
  using ws_t = typename P::ws_t;
  constexpr int NCT = BV / 16;
  constexpr int KB = K / 32;
  struct Ops {
    frag_t ph[SRT][KB];     // Phi rows 16(SRT w + st) + r, columns 32kb + kslot(grp, .)
    f32x4 e[SRT][NCT];
  };
  const int nstep = a.nseg - 1;
  auto load = [&](int q, Ops& op) {
    const ws_t* ph = static_cast<const ws_t*>(a.phi) + ((size_t)bh * nstep + q) * K * K;
    const float* e = a.eend + ((size_t)bh * nstep + q) * K * V;
#pragma unroll
    for (int st = 0; st < SRT; ++st) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        op.ph[st][kb] = frag_ws(ph + (((size_t)(SRT * w + st) * KB + kb) * 64 + lane) * 8);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        op.e[st][ct] = *reinterpret_cast<const f32x4*>(
            e + state_tile<K, BV>(sv, SRT * w + st, ct) + lane * 4);
    }
  };
  auto step = [&](const Ops& cur) {
#pragma unroll
    for (int st = 0; st < SRT; ++st) {
      const int tile = SRT * w + st;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        store_half(&sS[((tile >> 1) * NCT + ct) * 64 + lane], tile & 1, S[st][ct]);
    }
    lds_barrier();
#pragma unroll
    for (int st = 0; st < SRT; ++st)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) S[st][ct] = cur.e[st][ct];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const frag_t fb = sS[(kb * NCT + ct) * 64 + lane];
#pragma unroll
        for (int st = 0; st < SRT; ++st) S[st][ct] = mma32(cur.ph[st][kb], fb, S[st][ct]);
      }
    lds_barrier();   // every wave has read sS before it is rewritten
  };
  Ops oa, ob;
  load(0, oa);
  int q = 0;
  for (; q + 1 < p; q += 2) {
    load(q + 1, ob);
    step(oa);
    if (q + 2 < p) load(q + 2, oa);
    step(ob);
  }
  if (q < p) step(oa);
}

// One wave of a scan workgroup.  W (the wave index) and PHI (chain mode:
// transition slab, identity start and no v) are template arguments so that
// every choice between waves and slab kinds folds at compile time.
template <int K, int V, bool PERCH, class P, int MODE, int BV, int C, int NW, int W, bool PHI,
          bool LIN>
__device__ __forceinline__ void scan_wave(const ScanArgs& a, typename P::frag_t* sS,
                                          typename P::frag_t* sZ, typename P::in_t* sVw,
                                          unsigned char* stg, int unit, int sv) {
  using in_t = typename P::in_t;
  using frag_t = typename P::frag_t;
  using ws_t = typename P::ws_t;
  constexpr bool FULL = MODE == kScanFull;
  constexpr int NCT = BV / 16;     // column tiles
  constexpr int KT = K / 16;       // state row tiles
  constexpr int KB = K / 32;       // 32-wide k blocks over K
  constexpr int CB = C / 32;       // 32-wide k blocks over the chunk rows
  constexpr int SRT = KT / NW;     // state row tiles per wave
  constexpr int CT = C / 16 / NW;  // chunk row tiles per wave
  constexpr int CR = 16 * CT;      // chunk rows per wave
  static_assert(SRT * NW == KT && CT * NW == C / 16, "scan wave split");
  constexpr int VVEC = 16 / (int)sizeof(in_t);       // v elements per 16 bytes
  constexpr int VPR = BV / VVEC;                     // 16-byte pieces per v row
  constexpr int VRI = 64 / VPR;                      // v rows per load instruction
  constexpr int VNI = CR / VRI;                      // load instructions per wave
  constexpr int VP = BV + VVEC;                      // padded LDS v row
  constexpr int w = W;
  // k blocks of c (32 rows) that meet this wave's rows in A^ (lower triangular)
  constexpr int AKB = (CR * (w + 1) + 31) / 32;
  // o rows leave through the wave's staging area: fp32, BV columns, padded
  // so that the 16 rows of an accumulator tile land on distinct banks
  constexpr int ORB = BV * 4 + 16;
  constexpr int OLPR = BV * 4 / 16;            // lanes per o row
  constexpr int ORPI = 64 / OLPR;              // o rows per store instruction
  constexpr int ONI = CR / ORPI;               // o store instructions
  static_assert(CR % ORPI == 0, "o row staging shape");

  const int nsegu = FULL ? a.nseg : a.nseg - 1;
  const int bh = unit / nsegu, p = unit % nsegu;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, grp = lane >> 4;
  const int b = bh / a.HV, hv = bh % a.HV;
  const int h = hv / (a.HV / a.H);
  const int T = a.T;
  // chain mode: slabs [0, K/64) carry columns of the transition, the rest the
  // zero-start end state
  const int v0 = FULL ? sv * BV : (PHI ? 0 : (sv - K / BV) * BV);
  const int n0 = p * a.seg_len;
  const int n1 = min(n0 + a.seg_len, a.N);

  const in_t* vg = static_cast<const in_t*>(a.v);
  const ws_t* wtg = static_cast<const ws_t*>(a.wt);
  const ws_t* ahg = static_cast<const ws_t*>(a.ah);

  // ---- per-chunk operands of this wave, reloaded right after their use -----
  // k, q and v are reloaded as soon as their last use is issued; the rest is
  // double-buffered and loaded early in the previous chunk, so that no wait
  // at the top of the chunk loop (where the compiler's accounting of loads in
  // flight is conservative) finds a load issued late.
  u32x4 vr[VNI];
  struct WA {
    frag_t kf[CT][KB], qf[CT][KB];
    frag_t wf[SRT][CB], af[CT][AKB];
    f32x4 eg[CT];                        // exp(gamma), rows CR w + 16ct + 4grp + j
    float ego[CT];                       // exp(gamma), row CR w + 16ct + r
    f32x4 dl[PERCH ? SRT : 1];           // exp(gamma_last) per state row (one value
                                         // for every row with scalar decay)
  };
  // k / q fragments from the prep kernel's copies, 16 contiguous bytes per
  // lane: per value head with per-channel decay, per query head otherwise.
  // Rows past T are zero there; their Z rows meet zero rows of W^ and zero
  // columns of A^ (beta = 0 there), and their o is not stored.
  const size_t qkb = PERCH ? (size_t)bh * a.N : ((size_t)b * a.H + h) * a.N;
  auto kq_load = [&](const ws_t* wsb, int n, int ct, int kb) -> frag_t {
    return frag_ws(wsb + (((qkb + n) * (C / 16) + CT * w + ct) * KB + kb) * 512 + lane * 8);
  };
  auto load_v = [&](int n) {
    if constexpr (!PHI) {
#pragma unroll
      for (int i = 0; i < VNI; ++i) {
        // tail rows read row T-1 (see kq_load_raw)
        const int t = min(n * C + CR * w + VRI * i + lane / VPR, T - 1);
        vr[i] = *reinterpret_cast<const u32x4*>(
            vg + (((size_t)b * T + t) * a.HV + hv) * V + v0 + (lane % VPR) * VVEC);
      }
    }
  };
  // The next chunk's operands as a list of load items, issued one at a time
  // between the products of the current chunk: a burst of them would stall
  // the wave at issue (in order) while the memory pipeline drains it.
  constexpr int NKQ = CT * KB;                  // load items per k / q operand
  constexpr int IT_K = 0;
  constexpr int IT_Q = IT_K + (LIN ? 0 : NKQ);  // the linear rule never reads k here
  constexpr int IT_W = IT_Q + (FULL ? NKQ : 0);
  constexpr int IT_A = IT_W + ((LIN && PHI) ? 0 : SRT * CB);
  constexpr int IT_R = IT_A + (FULL ? CT * AKB : 0);
  constexpr int NITEMS = IT_R + 1;
  auto load_item = [&](int i, int n, WA& x) {
    const size_t cid = (size_t)bh * a.N + n;
    const float* rs = a.rs + cid * 256;
    if (i < IT_Q) {
      const int ct = (i - IT_K) / KB, kb = (i - IT_K) % KB;
      x.kf[ct][kb] = kq_load(static_cast<const ws_t*>(a.kh), n, ct, kb);
    } else if (i < IT_W) {
      if constexpr (FULL) {
        const int ct = (i - IT_Q) / KB, kb = (i - IT_Q) % KB;
        x.qf[ct][kb] = kq_load(static_cast<const ws_t*>(a.qh), n, ct, kb);
      }
    } else if (i < IT_A) {
      const int st = (i - IT_W) / CB, kb = (i - IT_W) % CB;
      x.wf[st][kb] = frag_ws(wtg + ((cid * KT + SRT * w + st) * CB + kb) * 512 + lane * 8);
    } else if (i < IT_R) {
      if constexpr (FULL) {
        const int ct = (i - IT_A) / AKB, kb = (i - IT_A) % AKB;
        x.af[ct][kb] = frag_ws(ahg + (cid * ah_frags(C) + ah_frag(CT * w + ct, kb)) * 512 +
                               lane * 8);
      }
    } else {
      if constexpr (PERCH) {
#pragma unroll
        for (int st = 0; st < SRT; ++st)
          x.dl[st] = *reinterpret_cast<const f32x4*>(rs + C + 16 * (SRT * w + st) + 4 * grp);
      } else {
        x.dl[0][0] = rs[C];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          x.eg[ct] = *reinterpret_cast<const f32x4*>(rs + CR * w + 16 * ct + 4 * grp);
          if constexpr (FULL) x.ego[ct] = rs[CR * w + 16 * ct + r];
        }
      }
    }
  };
  auto load_wa = [&](int n, WA& x) {
#pragma unroll
    for (int i = 0; i < NITEMS; ++i) load_item(i, n, x);
  };

  // ---- state: rows 16(SRT w + st) + 4grp + j, columns v0 + 16ct + r ----------
  f32x4 S[SRT][NCT];
#pragma unroll
  for (int st = 0; st < SRT; ++st)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) S[st][ct] = zero4();
  if constexpr (FULL) {
    if (a.s0) {
#pragma unroll
      for (int st = 0; st < SRT; ++st)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d = 16 * (SRT * w + st) + 4 * grp + j;
            S[st][ct][j] = a.s0[((size_t)bh * K + chan_of_row(d)) * V + v0 + 16 * ct + r];
          }
    }
    if (p > 0) combine_prefix<K, V, P, SRT, BV>(a, sS, bh, p, sv, w, lane, S);
  } else if constexpr (PHI) {
    // identity columns [64 sv, 64 sv + 64) of I_K
#pragma unroll
    for (int st = 0; st < SRT; ++st)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 16 * (SRT * w + st) + 4 * grp + j;
          S[st][ct][j] = (d == sv * BV + 16 * ct + r) ? 1.f : 0.f;
        }
  }

  // v rows of this wave into its LDS tile (the first chunk's here, every
  // later chunk's at the end of the step before it)
  auto stage_v = [&]() {
    if constexpr (!PHI) {
#pragma unroll
      for (int i = 0; i < VNI; ++i) {
        const int row = VRI * i + lane / VPR;
        *reinterpret_cast<u32x4*>(sVw + row * VP + (lane % VPR) * VVEC) = vr[i];
      }
    }
  };
  // The linear rule (LIN): Z = v does not depend on the state, so the v rows
  // of a chunk go to the Z fragments at the end of the step before it (two
  // alternating buffers), and the barrier at the top of the step publishes
  // them with the state: one barrier per step instead of two, and no Y.
  auto publish_vz = [&](int n) {
    if constexpr (LIN && !PHI) {
      frag_t* zb = sZ + (n & 1) * (CB * NCT * 64);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int c2 = 0; c2 < CT; ++c2) {
          f32x4 z;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            z[j] = P::in_to_f32(sVw[(16 * c2 + 4 * grp + j) * VP + 16 * ct + r]);
          const int tile = CT * w + c2;
          store_half(&zb[((tile >> 1) * NCT + ct) * 64 + lane], tile & 1, z);
        }
    }
  };
  load_v(n0);
  stage_v();
  publish_vz(n0);

  // o^T of a chunk leaves at the end of its step, after its last product and
  // after every load of the step is issued (so that no later wait for those
  // loads also waits for the stores): its accumulator tiles (lane: o row
  // CR w + 16 c2 + r, columns v0 + 16ct + 4grp .. +3) go to the staging area
  // as fp32 rows and come back as whole-row pieces.
  f32x4 OT[NCT][CT];
  f32x4 orow_v[ONI];
  auto stage_o = [&]() {
#pragma unroll
    for (int c2 = 0; c2 < CT; ++c2)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        *reinterpret_cast<f32x4*>(stg + (16 * c2 + r) * ORB + (16 * ct + 4 * grp) * 4) =
            OT[ct][c2];
#pragma unroll
    for (int i = 0; i < ONI; ++i)
      orow_v[i] = *reinterpret_cast<const f32x4*>(stg + (ORPI * i + lane / OLPR) * ORB +
                                                 (lane % OLPR) * 16);
  };
  auto store_o = [&](int n) {
#pragma unroll
    for (int i = 0; i < ONI; ++i) {
      const int t = n * C + CR * w + ORPI * i + lane / OLPR;
      if (t < T)
        store_o4(a.o, (((size_t)b * T + t) * a.HV + hv) * V + v0 + (lane % OLPR) * 4,
                 orow_v[i], a.o_fmt);
    }
  };

  auto step = [&](int n, const WA& cur, WA& nxt) {
    const int nn = min(n + 1, n1 - 1);   // the last chunk reloads itself
    GDR_PROF_DECL;
    GDR_PROF(0);
    // the next chunk's v (into the LDS tile at the end of this step)
    if constexpr (!PHI) load_v(nn);
    // this wave's state rows as halves of the B fragments of S (the linear
    // rule's chain pass reads no state across waves: no Y and no o).  With
    // one barrier per step (LIN) a wave may still read the state of the step
    // before while another writes this one, so S alternates between two
    // buffers as Z does; the barrier of step n orders the reads of step n-1
    // before the writes of step n + 1 to the same buffer.
    frag_t* sSb = LIN ? sS + (n & 1) * (KB * NCT * 64) : sS;
    if constexpr (!(LIN && !FULL)) {
#pragma unroll
      for (int st = 0; st < SRT; ++st) {
        const int tile = SRT * w + st;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          store_half(&sSb[((tile >> 1) * NCT + ct) * 64 + lane], tile & 1, S[st][ct]);
      }
    }
    GDR_PROF(11);
    lds_barrier();
    GDR_PROF(1);
    int item = 0;
    GDR_PROF(6);

    // Y = k S and o^T = S^T q^T for chunk rows [CR w, CR (w+1)): each B fragment
    // of S serves both (it is also the A fragment of S^T)
    f32x4 Y[CT][NCT];
#pragma unroll
    for (int c2 = 0; c2 < CT; ++c2)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        Y[c2][ct] = zero4();
        OT[ct][c2] = zero4();
      }
    if constexpr (!(LIN && !FULL)) {
      // every B fragment of S at once, so the LDS latency is paid once
      frag_t bS[KB][NCT];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) bS[kb][ct] = sSb[(kb * NCT + ct) * 64 + lane];
      GDR_PROF(7);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        frag_t fk[CT], fq[CT];
#pragma unroll
        for (int c2 = 0; c2 < CT; ++c2) {
          if constexpr (!LIN) fk[c2] = cur.kf[c2][kb];
          if constexpr (FULL) fq[c2] = cur.qf[c2][kb];
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
          for (int c2 = 0; c2 < CT; ++c2) {
            if constexpr (!LIN) Y[c2][ct] = mma32(fk[c2], bS[kb][ct], Y[c2][ct]);
            if constexpr (FULL) OT[ct][c2] = mma32(bS[kb][ct], fq[c2], OT[ct][c2]);
          }
          if (item < NITEMS) load_item(item++, nn, nxt);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    GDR_PROF(2);

    // Z = v - exp(gamma) Y, published as halves of the B fragments of Z
    // (the linear rule published Z = v at the end of the step before)
    if constexpr (!LIN) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 z[CT];
#pragma unroll
      for (int c2 = 0; c2 < CT; ++c2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float vv =
              PHI ? 0.f : P::in_to_f32(sVw[(16 * c2 + 4 * grp + j) * VP + 16 * ct + r]);
          if constexpr (PERCH)
            z[c2][j] = a.linear ? vv : vv - Y[c2][ct][j];
          else
            z[c2][j] = a.linear ? vv : vv - cur.eg[c2][j] * Y[c2][ct][j];
        }
#pragma unroll
      for (int c2 = 0; c2 < CT; ++c2) {
        const int tile = CT * w + c2;
        store_half(&sZ[((tile >> 1) * NCT + ct) * 64 + lane], tile & 1, z[c2]);
      }
    }
    lds_barrier();
    }
    GDR_PROF(3);

    // S <- diag(exp(gamma_last)) S + W^T Z, and o^T = exp(gamma) scale o^T + Z^T A^T
    float sc[CT];
#pragma unroll
    for (int c2 = 0; c2 < CT; ++c2) sc[c2] = (FULL && !PERCH) ? cur.ego[c2] * a.scale : 1.f;
    frag_t bZ[CB][NCT];
    const frag_t* zr = LIN ? sZ + (n & 1) * (CB * NCT * 64) : sZ;
    if constexpr (!(LIN && PHI)) {
#pragma unroll
      for (int kb = 0; kb < CB; ++kb)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) bZ[kb][ct] = zr[(kb * NCT + ct) * 64 + lane];
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int st = 0; st < SRT; ++st) {
        if constexpr (PERCH)
          S[st][ct] *= cur.dl[st];
        else
          S[st][ct] *= cur.dl[0][0];
        if constexpr (!(LIN && PHI)) {   // (the linear rule's transition: Z = 0)
#pragma unroll
          for (int kb = 0; kb < CB; ++kb) S[st][ct] = mma32(cur.wf[st][kb], bZ[kb][ct], S[st][ct]);
        }
        if (item < NITEMS) load_item(item++, nn, nxt);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (FULL) {
#pragma unroll
        for (int c2 = 0; c2 < CT; ++c2) {
          if constexpr (!PERCH) OT[ct][c2] *= sc[c2];
#pragma unroll
          for (int kb = 0; kb < AKB; ++kb)
            OT[ct][c2] = mma32(bZ[kb][ct], cur.af[c2][kb], OT[ct][c2]);
        }
      }
    }
#pragma unroll
    for (; item < NITEMS; ++item) load_item(item, nn, nxt);
    GDR_PROF(12);
    // this chunk's o, then the next chunk's v rows into the LDS tile (this
    // chunk's were last read for Z)
    if constexpr (FULL) {
      stage_o();
      GDR_PROF(9);
      store_o(n);
    }
    stage_v();
    publish_vz(n + 1);
    GDR_PROF(4);

    GDR_PROF(5);
    GDR_PROF_FLUSH;
  };

  // two chunks per iteration with the operand buffers in swapped roles
  WA bufA, bufB;
  int n = n0;
  load_wa(n0, bufA);
  for (; n + 1 < n1; n += 2) {
    step(n, bufA, bufB);
    step(n + 1, bufB, bufA);
  }
  if (n < n1) step(n, bufA, bufB);

  if constexpr (FULL) {
    if (a.sT && p == a.nseg - 1) {
#pragma unroll
      for (int st = 0; st < SRT; ++st)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d = 16 * (SRT * w + st) + 4 * grp + j;
            a.sT[((size_t)bh * K + chan_of_row(d)) * V + v0 + 16 * ct + r] = S[st][ct][j];
          }
    }
  } else if constexpr (PHI) {
    // Phi columns [64 sv, 64 sv + 64) in the workspace type, in the order in
    // which the combine reads them as A fragments: element (row d, column c)
    // goes to fragment (row tile d / 16, k block c / 32), lane
    // d % 16 + 16 g, slot i with c % 32 = kslot(g, i).  Here c % 32 =
    // 16 (ct & 1) + r, so g = r / 4 and i = 4 (ct & 1) + r % 4.
    ws_t* dst = static_cast<ws_t*>(a.phi) + ((size_t)bh * (a.nseg - 1) + p) * K * K;
#pragma unroll
    for (int st = 0; st < SRT; ++st)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int kb = (sv * BV + 16 * ct) / 32;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int fl = 4 * grp + j + 16 * (r >> 2);
          dst[(((size_t)(SRT * w + st) * KB + kb) * 64 + fl) * 8 + 4 * (ct & 1) + (r & 3)] =
              (ws_t)S[st][ct][j];
        }
      }
  } else {
    float* dst = a.eend + ((size_t)bh * (a.nseg - 1) + p) * K * V;
#pragma unroll
    for (int st = 0; st < SRT; ++st)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        *reinterpret_cast<f32x4*>(dst + state_tile<K, BV>(sv - K / BV, SRT * w + st, ct) +
                                  lane * 4) = S[st][ct];
  }
}

template <int K, int V, bool PERCH, class P, int MODE, int BV, int C, bool LIN = false>
__global__ __launch_bounds__((scan_waves<K, C>() * 64)) void chunk_scan_kernel(ScanArgs a) {
  using in_t = typename P::in_t;
  using frag_t = typename P::frag_t;
  constexpr int NW = scan_waves<K, C>();
  constexpr bool FULL = MODE == kScanFull;
  constexpr int NSLAB = FULL ? V / BV : (K + V) / BV;
  constexpr int NCT = BV / 16;
  constexpr int KB = K / 32;
  constexpr int CB = C / 32;
  constexpr int VVEC = 16 / (int)sizeof(in_t);
  constexpr int VP = BV + VVEC;
  __shared__ frag_t sS[(LIN ? 2 : 1) * KB * NCT * 64];  // B fragments of S (2 buffers: LIN)
  __shared__ frag_t sZ[(LIN ? 2 : 1) * CB * NCT * 64];  // B fragments of Z (2 buffers: LIN)
  __shared__ __attribute__((aligned(16))) in_t sV[NW][(C / NW) * VP];
  __shared__ __attribute__((aligned(16))) unsigned char
      sStg[NW][scan_stage_bytes<MODE, BV, C, NW>()];

  const int nsegu = FULL ? a.nseg : a.nseg - 1;       // segments handled by this pass
  int unit, sv;
  if (!unit_block(a.B, a.H, a.HV / a.H, nsegu, NSLAB, unit, sv)) return;
  const int wv = wave_id();
  if constexpr (!FULL) {
    // in-place state: the first segment's first slab copies the head's
    // initial state before the full pass (a later launch) overwrites it
    if (a.s0_copy && a.s0 && unit % nsegu == 0 && sv == 0) {
      const size_t base = (size_t)(unit / nsegu) * K * V;
      for (int e = threadIdx.x * 4; e < K * V; e += NW * 64 * 4)
        *reinterpret_cast<f32x4*>(a.s0_copy + base + e) =
            *reinterpret_cast<const f32x4*>(a.s0 + base + e);
    }
  }
  GDR_WGT(FULL ? 3 : 1, 0);
  auto run = [&](auto phi) {
    constexpr bool PHI = decltype(phi)::value;
    static_for_scan<0, NW>([&](auto wc) {
      constexpr int W = decltype(wc)::value;
      if (wv == W)
        scan_wave<K, V, PERCH, P, MODE, BV, C, NW, W, PHI, LIN>(a, sS, sZ, sV[W], sStg[W], unit,
                                                                 sv);
    });
  };
  if (FULL || sv >= K / BV)
    run(std::false_type{});
  else if constexpr (!FULL)
    run(std::true_type{});
  GDR_WGT(FULL ? 3 : 1, 1);
}

}  // namespace gdr
