// State scan kernels: the serial inter-chunk recurrence (sec-03 notes,
// "inter-chunk recurrence"), optionally split into sequence segments.
//
// Per chunk, with r = U - W S = M^-1 Z folded into the prep outputs:
//   Y = k S                       (exp(gamma) applied to the fp32 rows)
//   Z = v - exp(gamma) Y          (= M r)
//   o = exp(gamma) scale q S + A^ Z             (= (q exp(gamma)) S + A_qk r)
//   S <- diag(exp(gamma_last)) S + W^T Z        (= ... + K~^T diag(beta) r)
// (per-channel decay: the prep kernel folds exp(gamma) into the q, k
// fragments, so the row scales are 1.)
//
// The state update is affine in S: S_{n+1} = A_n S_n + B_n.  A sequence cut
// into segments is therefore run in three passes:
//   chain mode  : per (head, segment) the segment's transition Phi = prod A_n
//                 (the scan run on an identity state with v = 0) and its
//                 zero-start end state E (the scan run from S = 0), in
//                 parallel over segments;
//   combine     : S_{p+1} = Phi_p S_p + E_p, serial over segments;
//   full mode   : the scan of every segment from its true start state,
//                 writing o, in parallel over segments.
// With one segment only the full mode runs.
//
// Work split in a workgroup of 4 waves (64 state columns): wave w owns chunk
// rows [16w, 16w+16) of Y, Z and o and state rows [K/4 w, K/4 (w+1)).  Every
// A-operand fragment (q, k, W^T and A^ rows) belongs to exactly one wave,
// which loads it from the workspace straight into registers one chunk ahead,
// 16 bytes per lane and 1 KB per instruction, interleaved with the MFMAs so
// the memory and matrix pipes run together.  Only the B operands S and Z are
// shared, through LDS in fragment order (accumulator tiles are B fragments,
// see gdr_device.hpp), with two barriers per chunk.  v arrives as 16-byte
// row pieces and is turned into accumulator layout through a per-wave LDS
// tile; o leaves the same way.  The fp32 state never leaves registers
// except at segment ends.
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
  // segment p covers chunks [p * seg_len, min((p + 1) * seg_len, N))
  int seg_len, nseg;
  float* seg_state;  // start states of the segments, tile order [BH][nseg][K*V]
  float* phi;        // transitions, row-major [BH][nseg-1][K][K]
  float* eend;       // zero-start end states, tile order [BH][nseg-1][K*V]
};

#ifdef GDR_SCAN_PROFILE
__device__ long long gdr_scan_prof[64 * 8 * 4];
#define GDR_PROF(ph)                                                               \
  do {                                                                             \
    if (MODE == kScanFull && bh == 0 && p == 0 && sv == 0 && lane == 0 && n < 64)   \
      gdr_scan_prof[(n * 8 + (ph)) * 4 + w] = clock64();                           \
  } while (0)
#else
#define GDR_PROF(ph) do {} while (0)
#endif

constexpr int kScanFull = 0;
constexpr int kScanChain = 1;
constexpr int kScanBV = 64;   // state columns per workgroup
constexpr int kScanWaves = 4;

// Barrier for LDS traffic only: wait for this wave's LDS operations, then
// the workgroup barrier.  Outstanding global loads (the next chunk's
// prefetch) stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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

// XCD-aware placement: workgroups are dealt to the 8 XCDs round-robin, so
// give every slab of one unit (head or head segment) the same (id % 8) and
// they share an L2.
__device__ __forceinline__ bool unit_block(int nunits, int nslab, int& unit, int& sv) {
  const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
  unit = (slot / nslab) * 8 + xcd;
  sv = slot % nslab;
  return unit < nunits;
}

// Offset of the state tiles owned by (slab sv, wave w) inside one K x V state
// stored in tile order: [slab][wave][SRT][NCT][64 lanes][4].
template <int K, int V>
__device__ __forceinline__ size_t tile_off(int sv, int w) {
  return ((size_t)sv * kScanWaves + w) * (K / 64) * (kScanBV / 16) * 256;
}

template <int K, int V, bool PERCH, class P, int MODE>
__global__ __launch_bounds__(256) void chunk_scan_kernel(ScanArgs a) {
  using in_t = typename P::in_t;
  using frag_t = typename P::frag_t;
  using ws_t = typename P::ws_t;
  constexpr bool FULL = MODE == kScanFull;
  constexpr int C = kChunk;
  constexpr int BV = kScanBV;
  constexpr int NSLAB = FULL ? V / BV : (K + V) / BV;   // chain: Phi slabs, then E slabs
  constexpr int NCT = BV / 16;     // column tiles
  constexpr int KT = K / 16;       // state row tiles
  constexpr int KB = K / 32;       // 32-wide k blocks over K
  constexpr int SRT = KT / 4;      // state row tiles per wave
  constexpr int VVEC = 16 / (int)sizeof(in_t);       // v elements per 16 bytes
  constexpr int VPR = BV / VVEC;                     // 16-byte pieces per v row
  constexpr int VRI = 64 / VPR;                      // v rows per load instruction
  constexpr int VNI = 16 / VRI;                      // load instructions per wave
  constexpr int VP = BV + VVEC;                      // padded LDS v row
  constexpr int OP = BV + 4;                         // padded LDS o row (fp32)

  __shared__ frag_t sS[KB * NCT * 64];                // B fragments of S
  __shared__ frag_t sZ[2 * NCT * 64];                 // B fragments of Z
  __shared__ __attribute__((aligned(16))) in_t sV[kScanWaves][16 * VP];
  __shared__ __attribute__((aligned(16))) float sO[FULL ? kScanWaves : 1][FULL ? 16 * OP : 4];

  const int nsegu = FULL ? a.nseg : a.nseg - 1;       // segments handled by this pass
  int unit, sv;
  if (!unit_block(a.B * a.HV * nsegu, NSLAB, unit, sv)) return;
  const int bh = unit / nsegu, p = unit % nsegu;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int b = bh / a.HV, hv = bh % a.HV;
  const int h = hv / (a.HV / a.H);
  const int T = a.T;
  // chain mode: slabs [0, K/64) carry columns of the transition (identity
  // start, no v), the rest the zero-start end state
  const bool isphi = !FULL && sv < K / BV;
  const int v0 = FULL ? sv * BV : (isphi ? 0 : (sv - K / BV) * BV);
  const int n0 = p * a.seg_len;
  const int n1 = min(n0 + a.seg_len, a.N);

  const in_t* vg = static_cast<const in_t*>(a.v);
  const ws_t* wtg = static_cast<const ws_t*>(a.wt);
  const ws_t* ahg = static_cast<const ws_t*>(a.ah);
  const ws_t* qhg = static_cast<const ws_t*>(a.qh);
  const ws_t* khg = static_cast<const ws_t*>(a.kh);

  float zf[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const frag_t fzero = P::make(zf);

  // Per-chunk operands of this wave, as loaded.
  struct Ops {
    frag_t kf[KB], qf[KB];
    frag_t wf[SRT][2], af[2];
    uint4 vr[VNI];
    f32x4 eg;
    f32x4 dl[SRT];
  };

  // The operand loads of one chunk as a list of items; the chunk loop issues
  // them one at a time between MFMAs so that the memory pipe and the matrix
  // pipe stay busy together (a wave issues in order).
  constexpr int IT_V = 0, IT_K = IT_V + VNI, IT_Q = IT_K + KB, IT_EG = IT_Q + KB;
  constexpr int IT_W = IT_EG + 1, IT_A = IT_W + 2 * SRT, IT_DL = IT_A + 2;
  constexpr int NITEMS = IT_DL + SRT;
  auto load_item = [&](int i, int n, Ops& op) {
    const size_t cid = (size_t)bh * a.N + n;
    const size_t fid = PERCH ? cid : ((size_t)b * a.H + h) * a.N + n;
    const int t0 = n * C;
    const float* rs = a.rs + cid * 256;
    if (i < IT_K) {
      if (!isphi) {
        // v rows; tail rows read a valid row and are zeroed in the LDS write
        const int t = min(t0 + 16 * w + VRI * (i - IT_V) + lane / VPR, T - 1);
        op.vr[i - IT_V] = *reinterpret_cast<const uint4*>(
            vg + (((size_t)b * T + t) * a.HV + hv) * V + v0 + (lane % VPR) * VVEC);
      }
    } else if (i < IT_Q) {
      op.kf[i - IT_K] = frag_ws(khg + ((fid * 4 + w) * KB + (i - IT_K)) * 512 + lane * 8);
    } else if (i < IT_EG) {
      if constexpr (FULL)
        op.qf[i - IT_Q] = frag_ws(qhg + ((fid * 4 + w) * KB + (i - IT_Q)) * 512 + lane * 8);
    } else if (i < IT_W) {
      op.eg = *reinterpret_cast<const f32x4*>(rs + 16 * w + 4 * grp);
    } else if (i < IT_A) {
      const int st = (i - IT_W) >> 1, kb = (i - IT_W) & 1;
      op.wf[st][kb] = frag_ws(wtg + ((cid * KT + SRT * w + st) * 2 + kb) * 512 + lane * 8);
    } else if (i < IT_DL) {
      if constexpr (FULL) {
        const int kb = i - IT_A;
        op.af[kb] = (kb == 0 || w >= 2)
                        ? frag_ws(ahg + ((cid * 4 + w) * 2 + kb) * 512 + lane * 8)
                        : fzero;
      }
    } else {
      const int st = i - IT_DL;
      op.dl[st] = *reinterpret_cast<const f32x4*>(rs + 64 + 16 * (SRT * w + st) + 4 * grp);
    }
  };
  auto load = [&](int n, Ops& op) {
#pragma unroll
    for (int i = 0; i < NITEMS; ++i) load_item(i, n, op);
  };

  // state rows 16*(SRT*w + st) + 4*grp + j, columns v0 + 16*ct + r
  f32x4 S[SRT][NCT];
#pragma unroll
  for (int st = 0; st < SRT; ++st)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) S[st][ct] = zero4();
  if constexpr (FULL) {
    if (p > 0) {
      const float* src = a.seg_state + ((size_t)bh * a.nseg + p) * K * V + tile_off<K, V>(sv, w);
#pragma unroll
      for (int st = 0; st < SRT; ++st)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          S[st][ct] = *reinterpret_cast<const f32x4*>(src + ((st * NCT + ct) * 64 + lane) * 4);
    } else if (a.s0) {
#pragma unroll
      for (int st = 0; st < SRT; ++st)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d = 16 * (SRT * w + st) + 4 * grp + j;
            S[st][ct][j] = a.s0[((size_t)bh * K + d) * V + v0 + 16 * ct + r];
          }
    }
  } else if (isphi) {
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

  in_t* sVw = sV[w];
  float* sOw = sO[FULL ? w : 0];

  // One chunk: consume `cur`, prefetch chunk n+1 into `nxt`.  The loop below
  // alternates two operand sets, so the prefetch never waits for the loads
  // it replaces.
  auto body = [&](int n, const Ops& cur, Ops& nxt) {
    GDR_PROF(0);
    const int t0 = n * C;
    const int nn = min(n + 1, n1 - 1);   // the last chunk reloads itself
    int item = 0;
    GDR_PROF(1);

    // v rows of this wave into its LDS tile (zero past T)
    if (!isphi) {
#pragma unroll
      for (int i = 0; i < VNI; ++i) {
        const int row = VRI * i + lane / VPR;
        const bool ok = t0 + 16 * w + row < T;
        *reinterpret_cast<uint4*>(sVw + row * VP + (lane % VPR) * VVEC) =
            ok ? cur.vr[i] : uint4{0u, 0u, 0u, 0u};
      }
    }
    // publish this wave's state rows as halves of the S B-fragments
#pragma unroll
    for (int st = 0; st < SRT; ++st) {
      const int tile = SRT * w + st;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        store_half(&sS[((tile >> 1) * NCT + ct) * 64 + lane], tile & 1, S[st][ct]);
    }
    lds_barrier();
    GDR_PROF(2);

    // Y = k S (and O = q S) for chunk rows [16w, 16w+16)
    frag_t bS[KB][NCT];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) bS[kb][ct] = sS[(kb * NCT + ct) * 64 + lane];
    f32x4 Y[NCT], O[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) { Y[ct] = zero4(); O[ct] = zero4(); }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        Y[ct] = mma32(cur.kf[kb], bS[kb][ct], Y[ct]);
        if constexpr (FULL) O[ct] = mma32(cur.qf[kb], bS[kb][ct], O[ct]);
        if (item < NITEMS) load_item(item++, nn, nxt);
        __builtin_amdgcn_sched_barrier(0);
      }
    GDR_PROF(3);

    // Z = v - exp(gamma) Y, published as halves of the Z B-fragments
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 z;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float vv = isphi ? 0.f : P::in_to_f32(sVw[(4 * grp + j) * VP + 16 * ct + r]);
        if constexpr (PERCH) {
          z[j] = vv - Y[ct][j];
        } else {
          z[j] = vv - cur.eg[j] * Y[ct][j];
          if constexpr (FULL) O[ct][j] *= cur.eg[j] * a.scale;
        }
      }
      store_half(&sZ[((w >> 1) * NCT + ct) * 64 + lane], w & 1, z);
    }
    GDR_PROF(4);
    lds_barrier();
    GDR_PROF(5);

    frag_t zb[2][NCT];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) zb[kb][ct] = sZ[(kb * NCT + ct) * 64 + lane];

    // S <- diag(exp(gamma_last)) S + W^T Z
#pragma unroll
    for (int st = 0; st < SRT; ++st)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int j = 0; j < 4; ++j) S[st][ct][j] *= cur.dl[st][j];
        S[st][ct] = mma32(cur.wf[st][0], zb[0][ct], S[st][ct]);
        S[st][ct] = mma32(cur.wf[st][1], zb[1][ct], S[st][ct]);
        if (item < NITEMS) load_item(item++, nn, nxt);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
    for (; item < NITEMS; ++item) load_item(item, nn, nxt);
    GDR_PROF(6);

    if constexpr (FULL) {
      // o = O + A^ Z
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        O[ct] = mma32(cur.af[0], zb[0][ct], O[ct]);
        if (w >= 2) O[ct] = mma32(cur.af[1], zb[1][ct], O[ct]);
      }
      // o rows through this wave's LDS tile, then 16-byte row stores
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) sOw[(4 * grp + j) * OP + 16 * ct + r] = O[ct][j];
      constexpr int OPR = BV / 4;          // 16-byte pieces per o row
      constexpr int ORI = 64 / OPR;        // rows per store instruction
#pragma unroll
      for (int i = 0; i < 16 / ORI; ++i) {
        const int row = ORI * i + lane / OPR, c4 = (lane % OPR) * 4;
        const int t = t0 + 16 * w + row;
        const f32x4 x = *reinterpret_cast<const f32x4*>(sOw + row * OP + c4);
        if (t < T)
          *reinterpret_cast<f32x4*>(a.o + (((size_t)b * T + t) * a.HV + hv) * V + v0 + c4) = x;
      }
    }
    GDR_PROF(7);
  };

  Ops bufA, bufB;
  load(n0, bufA);
  int n = n0;
  for (; n + 1 < n1; n += 2) {
    body(n, bufA, bufB);
    body(n + 1, bufB, bufA);
  }
  if (n < n1) body(n, bufA, bufB);

  if constexpr (FULL) {
    if (a.sT && p == a.nseg - 1) {
#pragma unroll
      for (int st = 0; st < SRT; ++st)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d = 16 * (SRT * w + st) + 4 * grp + j;
            a.sT[((size_t)bh * K + d) * V + v0 + 16 * ct + r] = S[st][ct][j];
          }
    }
  } else if (isphi) {
    // Phi columns [64 sv, 64 sv + 64), row-major
    float* dst = a.phi + ((size_t)bh * (a.nseg - 1) + p) * K * K;
#pragma unroll
    for (int st = 0; st < SRT; ++st)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 16 * (SRT * w + st) + 4 * grp + j;
          dst[(size_t)d * K + sv * BV + 16 * ct + r] = S[st][ct][j];
        }
  } else {
    float* dst = a.eend + ((size_t)bh * (a.nseg - 1) + p) * K * V +
                 tile_off<K, V>(sv - K / BV, w);
#pragma unroll
    for (int st = 0; st < SRT; ++st)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        *reinterpret_cast<f32x4*>(dst + ((st * NCT + ct) * 64 + lane) * 4) = S[st][ct];
  }
}

// Combine pass: S_{p+1} = Phi_p S_p + E_p over the segments of one head,
// one workgroup per (head, 64-column slab), same tile ownership as the scan.
// Writes the start state of every segment p >= 1 in tile order.
template <int K, int V, class P>
__global__ __launch_bounds__(256) void seg_combine_kernel(ScanArgs a) {
  using frag_t = typename P::frag_t;
  constexpr int BV = kScanBV;
  constexpr int NSLAB = V / BV;
  constexpr int NCT = BV / 16;
  constexpr int KT = K / 16;
  constexpr int KB = K / 32;
  constexpr int SRT = KT / 4;

  __shared__ frag_t sS[KB * NCT * 64];

  int bh, sv;
  if (!unit_block(a.B * a.HV, NSLAB, bh, sv)) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int v0 = sv * BV;

  f32x4 S[SRT][NCT];
#pragma unroll
  for (int st = 0; st < SRT; ++st)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) S[st][ct] = zero4();
  if (a.s0) {
#pragma unroll
    for (int st = 0; st < SRT; ++st)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 16 * (SRT * w + st) + 4 * grp + j;
          S[st][ct][j] = a.s0[((size_t)bh * K + d) * V + v0 + 16 * ct + r];
        }
  }

  for (int p = 0; p + 1 < a.nseg; ++p) {
#pragma unroll
    for (int st = 0; st < SRT; ++st) {
      const int tile = SRT * w + st;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        store_half(&sS[((tile >> 1) * NCT + ct) * 64 + lane], tile & 1, S[st][ct]);
    }
    lds_barrier();
    const float* ph = a.phi + ((size_t)bh * (a.nseg - 1) + p) * K * K;
    const float* e = a.eend + ((size_t)bh * (a.nseg - 1) + p) * K * V + tile_off<K, V>(sv, w);
    f32x4 acc[SRT][NCT];
#pragma unroll
    for (int st = 0; st < SRT; ++st)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        acc[st][ct] = *reinterpret_cast<const f32x4*>(e + ((st * NCT + ct) * 64 + lane) * 4);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int st = 0; st < SRT; ++st) {
        const int d = 16 * (SRT * w + st) + r;
        const frag_t fa = frag_row_f32<P>(ph + (size_t)d * K + 32 * kb, grp);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          acc[st][ct] = mma32(fa, sS[(kb * NCT + ct) * 64 + lane], acc[st][ct]);
      }
    }
    float* dst = a.seg_state + ((size_t)bh * a.nseg + p + 1) * K * V + tile_off<K, V>(sv, w);
#pragma unroll
    for (int st = 0; st < SRT; ++st)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        S[st][ct] = acc[st][ct];
        *reinterpret_cast<f32x4*>(dst + ((st * NCT + ct) * 64 + lane) * 4) = acc[st][ct];
      }
    lds_barrier();   // every wave has read sS before it is rewritten
  }
}

}  // namespace gdr
