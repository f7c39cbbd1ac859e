// C ABI of the chunkwise gated delta rule forward pass (declared in gdr.h).
//
// Host side only: argument validation (no HIP call before it passes), the
// workspace layout, the gfx950 check, and the launches of the kernels on the
// caller's stream (the launchers, one translation unit per kernel family,
// are declared in gdr_launch.hpp).  The library allocates nothing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "gdr.h"
#include "gdr_launch.hpp"

// The workspace of gdr_chunk_fwd_noalloc: one array per device, loaded with
// the library's code object.  In host code `scratch` names a host-side
// stand-in, not device memory: the device address comes from
// hipGetSymbolAddress (scratch_address below) and only that address is
// handed to kernels.
static __device__ __align__(256) unsigned char scratch[GDR_NOALLOC_SCRATCH_BYTES];

using namespace gdr;

namespace {

// Cost of the state scan, in 64-column full-pass chunk steps, with P
// segments of L chunks and BV-column slabs.  One segment runs the serial scan
// over all N chunks with B*HV*V/BV workgroups.  P segments run a chain pass
// (B*HV*(P-1)*(K+V)/BV workgroups of L chunks, each chunk step about 0.7 of a
// full-pass step), a serial combine (P-1 steps of about 1.7 full-pass steps
// each) and the full pass (B*HV*P*V/BV workgroups of L chunks).  A pass with
// up to 256 workgroups (one per compute unit of an MI355X) takes L steps;
// beyond that two workgroups share a compute unit at about 1.6x the step
// time, in rounds of 512.  A 32-column step costs about 0.7 of a 64-column
// one (half the products and state, the same operand stream).  The constants
// are fitted to measured scan times of the 4096-, 8192-, 16000- and
// 65536-token workloads and of batched variants (12 to 256 scans) over forced
// segment counts and both widths.  The estimate uses problem sizes only, so
// the workspace size query needs no device query.
double scan_cost(int BH, int K, int V, int BV, int P, int L) {
  constexpr double kCU = 256.0, kShare = 1.6, kChain = 0.7, kComb = 1.7, kStep32 = 0.7;
  auto pass = [&](double wgs, double steps) {
    return wgs <= kCU ? steps : steps * kShare * std::ceil(wgs / (2.0 * kCU));
  };
  double t = pass((double)BH * P * (V / BV), L);
  if (P > 1) t += pass((double)BH * (P - 1) * ((K + V) / BV), L) * kChain + (P - 1) * kComb;
  return BV == 32 ? t * kStep32 : t;
}

// Segment count for BV-column slabs (and its cost).
int choose_segments(int BH, int N, int K, int V, int BV, int& seg_len, double& cost) {
  double best = 1e300;
  int bestP = 1;
  seg_len = N;
  for (int P = 1; P <= 256 && P <= N; ++P) {
    const int L = (N + P - 1) / P;
    const int Pe = (N + L - 1) / L;
    if (Pe != P) continue;
    const double t = scan_cost(BH, K, V, BV, P, L);
    // more segments also move more bytes (the chain pass reads k, v and W^
    // once more), which the step counts above do not see: a larger P must
    // win by 5%
    if (t < best * 0.95) {
      best = t;
      bestP = P;
      seg_len = L;
    }
  }
  cost = best;
  return bestP;
}

gdr_status validate(const gdr_problem* p, Prob* out) {
  if (!p) return GDR_ERR_NULL;
  if (p->B < 1 || p->T < 1 || p->H < 1 || p->HV < 1 || p->K < 1 || p->V < 1 ||
      p->HV % p->H != 0)
    return GDR_ERR_SHAPE;
  if (p->qkv_dtype != GDR_F32 && p->qkv_dtype != GDR_BF16 && p->qkv_dtype != GDR_F16)
    return GDR_ERR_DTYPE;
  if (p->o_dtype != GDR_F32 && p->o_dtype != GDR_BF16 && p->o_dtype != GDR_F16)
    return GDR_ERR_DTYPE;
  if (p->g_per_channel != 0 && p->g_per_channel != 1) return GDR_ERR_ARG;
  if (p->qk_l2norm != 0 && p->qk_l2norm != 1) return GDR_ERR_ARG;
  if (p->rule != GDR_RULE_DELTA && p->rule != GDR_RULE_LINEAR) return GDR_ERR_ARG;
  if (!std::isfinite(p->scale)) return GDR_ERR_ARG;
  if (p->chunk < 0) return GDR_ERR_ARG;
  if (p->chunk != 0 && p->chunk != 32 && p->chunk != 64 && p->chunk != 128)
    return GDR_ERR_UNSUPPORTED;
  if ((p->K != 64 && p->K != 128) || (p->V != 64 && p->V != 128)) return GDR_ERR_UNSUPPORTED;
  Prob r;
  r.B = p->B; r.T = p->T; r.H = p->H; r.HV = p->HV; r.K = p->K; r.V = p->V;
  // chunk 0: the automatic choice.  64-row chunks measured faster than
  // 128-row ones on every workload tried (the prep's C^2 work doubles per
  // token while the scan's serial steps only halve) and than 32-row ones
  // (twice the serial steps), so it is 64.
  r.C = p->chunk == 0 ? 64 : p->chunk;
  r.N = (int)(((int64_t)p->T + r.C - 1) / r.C);   // T + C - 1 may pass INT_MAX
  // grid sizes must fit a 32-bit launch dimension: B HV N workgroups and
  // more; B HV is bounded first, so that no product here can wrap
  const uint64_t bhv = (uint64_t)p->B * (uint64_t)p->HV;   // < 2^62
  if (bhv > 0x7fffffffull || bhv * (uint64_t)r.N + 8ull * (uint64_t)p->HV > 0x7fffffffull)
    return GDR_ERR_SHAPE;
  r.perch = p->g_per_channel == 1;
  r.f32 = p->qkv_dtype == GDR_F32;
  r.h16 = p->qkv_dtype == GDR_F16;
  r.scale = p->scale;
  r.l2norm = p->qk_l2norm == 1;
  r.linear = p->rule == GDR_RULE_LINEAR;
  r.es = r.f32 ? 4 : 2;
  r.ofmt = p->o_dtype;   // GDR_F32, GDR_BF16, GDR_F16 = kOutF32, kOutBF16, kOutF16
  if (p->scan_segments < 0) return GDR_ERR_ARG;
  if (p->scan_slab != 0 && p->scan_slab != 32 && p->scan_slab != 64) return GDR_ERR_ARG;
  // 128-row chunks are built with one slab width per key dimension: 32
  // columns for K = 128 (8 waves), 64 for K = 64 (4 waves)
  const int bv128 = r.K == 128 ? 32 : 64;
  if (r.C == 128 && p->scan_slab != 0 && p->scan_slab != bv128) return GDR_ERR_UNSUPPORTED;
  // The automatic width: 64 columns, or 32 where the cost model prices them
  // at least 15% cheaper.  The model overrates the narrow slabs by about 10%
  // when few workgroups run: on the 4096-token, 12-head workload it prices
  // them 11% cheaper (5 segments against 6) and the two measure the same;
  // on 48 to 64 scans it prices them 18-20% cheaper and they measure 8-18%
  // faster.  Both widths were measured only with 16-bit operands,
  // K = V = 128 and the delta rule (the linear rule's 64-column kernel is a
  // faster instantiation of its own), so elsewhere the choice stays at 64.
  const bool try32 =
      p->scan_slab == 0 && r.C == 64 && !r.f32 && !r.linear && r.K == 128 && r.V == 128;
  const int BH = r.B * r.HV;
  r.bv = r.C == 128 ? bv128 : (p->scan_slab != 0 ? p->scan_slab : 64);
  if (p->scan_segments == 0) {
    double cost = 0.0, cost32 = 0.0;
    int len32 = 0;
    r.nseg = choose_segments(BH, r.N, r.K, r.V, r.bv, r.seg_len, cost);
    if (try32) {
      const int nseg32 = choose_segments(BH, r.N, r.K, r.V, 32, len32, cost32);
      if (cost32 < cost * 0.85) {
        r.bv = 32;
        r.nseg = nseg32;
        r.seg_len = len32;
      }
    }
  } else {
    const int want = p->scan_segments < r.N ? p->scan_segments : r.N;
    r.seg_len = (r.N + want - 1) / want;
    r.nseg = (r.N + r.seg_len - 1) / r.seg_len;
    if (try32 && scan_cost(BH, r.K, r.V, 32, r.nseg, r.seg_len) <
                     scan_cost(BH, r.K, r.V, 64, r.nseg, r.seg_len) * 0.85)
      r.bv = 32;
  }
  if (out) *out = r;
  return GDR_OK;
}

size_t nchunks(const Prob& r) { return (size_t)r.B * r.HV * r.N; }

WsLayout layout(const Prob& r) {
  // q/k fragments: per value head with the per-channel decay folded in, per
  // query head (shared by its value heads) with one decay per row
  const size_t qk = r.perch ? nchunks(r) : (size_t)r.B * r.H * r.N;
  return ws_layout(nchunks(r), qk, r.C, r.K, r.V, r.es, (size_t)r.B * r.HV, r.nseg);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Span {
  const void* p;
  size_t n;
};

bool overlap(Span a, Span b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

struct Spans {
  Span q, k, v, g, beta, s0, o, sT, ws;
};

Spans spans(const Prob& r, const void* q, const void* k, const void* v, const float* g,
            const float* beta, const float* s0, const void* o, const float* sT,
            const void* ws, size_t ws_bytes) {
  const size_t tok = (size_t)r.B * r.T;
  Spans s;
  s.q = {q, tok * r.H * r.K * r.es};
  s.k = {k, tok * r.H * r.K * r.es};
  s.v = {v, tok * r.HV * r.V * r.es};
  s.g = {g, tok * r.HV * (r.perch ? r.K : 1) * sizeof(float)};
  s.beta = {beta, tok * r.HV * sizeof(float)};
  s.s0 = {s0, (size_t)r.B * r.HV * r.K * r.V * sizeof(float)};
  s.o = {o, tok * r.HV * r.V * (r.ofmt != kOutF32 ? 2 : 4)};
  s.sT = {sT, (size_t)r.B * r.HV * r.K * r.V * sizeof(float)};
  s.ws = {ws, ws_bytes};
  return s;
}

// An output span must not overlap any input span.
bool out_overlaps(Span out, std::initializer_list<Span> ins) {
  for (const Span& in : ins)
    if (overlap(out, in)) return true;
  return false;
}

gdr_status check_device() {
  static std::atomic<int> arch_state[64];  // 0 unknown, 1 gfx950, 2 other (per device ordinal)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GDR_ERR_HIP;
  if (dev >= 0 && dev < 64) {
    const int v = arch_state[dev].load(std::memory_order_relaxed);
    if (v == 1) return GDR_OK;
    if (v == 2) return GDR_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GDR_ERR_HIP;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) arch_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? GDR_OK : GDR_ERR_DEVICE;
}

gdr_status launch_scan(const Prob& r, ScanArgs& a, hipStream_t s) {
  if (r.h16) {
    if (r.C == 128) return launch_scan128_h16(r, a, s);
    if (r.C == 32) return launch_scan32_h16(r, a, s);
    if (r.linear && r.bv == 64) return launch_scan_h16_linear(r, a, s);
    return launch_scan_h16(r, a, s);
  }
  if (r.C == 128) return r.f32 ? launch_scan128_f32(r, a, s) : launch_scan128_f16(r, a, s);
  if (r.C == 32) return r.f32 ? launch_scan32_f32(r, a, s) : launch_scan32_f16(r, a, s);
  if (r.f32) return launch_scan_f32(r, a, s);
  if (r.linear && r.bv == 64) return launch_scan_f16_linear(r, a, s);
  return launch_scan_f16(r, a, s);
}

PrepArgs prep_args(const Prob& r, const void* q, const void* k, const float* g,
                   const float* beta, void* ws) {
  const WsLayout L = layout(r);
  char* base = static_cast<char*>(ws);
  PrepArgs a;
  a.q = q; a.k = k; a.g = g; a.beta = beta;
  a.B = r.B; a.T = r.T; a.H = r.H; a.HV = r.HV; a.N = r.N;
  a.scale = r.scale;
  a.wt = base + L.wt; a.ah = base + L.ah; a.rs = reinterpret_cast<float*>(base + L.rs);
  a.qh = base + L.qh; a.kh = base + L.kh;
  a.l2norm = r.l2norm ? 1 : 0;
  a.linear = r.linear ? 1 : 0;
  a.d_gamma = a.d_akk = a.d_aqk = a.d_minv = nullptr;
  return a;
}

ScanArgs scan_args(const Prob& r, const void* q, const void* k, const void* v,
                   const float* s0, void* o, float* sT, const void* ws) {
  const WsLayout L = layout(r);
  char* base = static_cast<char*>(const_cast<void*>(ws));
  ScanArgs a;
  a.q = q; a.k = k; a.v = v; a.s0 = s0; a.o = o; a.sT = sT;
  a.o_fmt = r.ofmt;
  // In place (final_state == initial_state) with sequence segments, the
  // last segment's workgroups write the final state while workgroups of
  // other segments may not yet have read their columns of the initial
  // state.  The chain pass, which runs first, then copies the initial state
  // into the workspace, and the full pass reads the copy.
  a.s0_copy = (s0 && s0 == sT && r.nseg > 1) ? reinterpret_cast<float*>(base + L.s0c) : nullptr;
  a.wt = base + L.wt; a.ah = base + L.ah; a.rs = reinterpret_cast<const float*>(base + L.rs);
  a.qh = base + L.qh; a.kh = base + L.kh;
  a.B = r.B; a.T = r.T; a.H = r.H; a.HV = r.HV; a.N = r.N;
  a.scale = r.scale;
  a.seg_len = r.seg_len; a.nseg = r.nseg;
  a.linear = r.linear ? 1 : 0;
  a.phi = base + L.phi;
  a.eend = reinterpret_cast<float*>(base + L.eend);
  return a;
}

gdr_status check_ws(const Prob& r, const void* ws, size_t ws_bytes) {
  if (!ws || ws_bytes < layout(r).total) return GDR_ERR_WORKSPACE;
  if (!aligned16(ws)) return GDR_ERR_ALIGN;
  return GDR_OK;
}

// Device address of this device's `scratch` array, looked up on the
// device's first call (with that device current) and kept per device.
gdr_status scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GDR_ERR_HIP;
  if (dev < 0 || dev >= 64) return GDR_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return GDR_ERR_HIP;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return GDR_OK;
}

// Checks shared by gdr_chunk_fwd and gdr_chunk_fwd_noalloc after validation:
// the required pointers and their alignment, then (once the workspace is
// known) overlaps between buffers.  ws may be NULL: the library's own
// scratch array overlaps none of the caller's buffers.
gdr_status check_fwd_pointers(const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const float* initial_state, const void* o,
                              const float* final_state) {
  if (!q || !k || !v || !g || !beta || !o) return GDR_ERR_NULL;
  for (const void* ptr : {(const void*)q, (const void*)k, (const void*)v, (const void*)g,
                          (const void*)beta, (const void*)initial_state, (const void*)o,
                          (const void*)final_state})
    if (ptr && !aligned16(ptr)) return GDR_ERR_ALIGN;
  return GDR_OK;
}

gdr_status check_fwd_overlaps(const Prob& r, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const float* initial_state,
                              const void* o, const float* final_state, const void* ws,
                              size_t ws_bytes) {
  const Spans s = spans(r, q, k, v, g, beta, initial_state, o, final_state, ws, ws_bytes);
  if (out_overlaps(s.o, {s.q, s.k, s.v, s.g, s.beta, s.s0, s.sT, s.ws})) return GDR_ERR_ALIAS;
  if (out_overlaps(s.ws, {s.q, s.k, s.v, s.g, s.beta, s.s0, s.sT})) return GDR_ERR_ALIAS;
  if (out_overlaps(s.sT, {s.q, s.k, s.v, s.g, s.beta})) return GDR_ERR_ALIAS;
  if (initial_state && final_state && initial_state != final_state && overlap(s.sT, s.s0))
    return GDR_ERR_ALIAS;
  return GDR_OK;
}

// The launches of the whole forward pass on a checked problem.
gdr_status launch_fwd(const Prob& r, const void* q, const void* k, const void* v,
                      const float* g, const float* beta, const float* initial_state, void* o,
                      float* final_state, void* ws, hipStream_t hs) {
  PrepArgs pa = prep_args(r, q, k, g, beta, ws);
  gdr_status st = launch_prep(r, pa, false, hs);
  if (st != GDR_OK) return st;
  ScanArgs sa = scan_args(r, q, k, v, initial_state, o, final_state, ws);
  return launch_scan(r, sa, hs);
}

// State columns per decode workgroup: 0 chooses (see decode_columns).
int decode_columns(const gdr_problem* p) {
  if (p->scan_slab != 0) return p->scan_slab < p->V ? p->scan_slab : p->V;
  return p->V;   // whole rows: measured best or equal on the decode batches
}

}  // namespace

extern "C" {

gdr_status gdr_decode_step(const gdr_problem* p, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, const float* state_in,
                           float* state_out, void* o, void* stream) {
  if (!p) return GDR_ERR_NULL;
  if (p->B < 1 || p->T != 1 || p->H < 1 || p->HV < 1 || p->K < 1 || p->V < 1 ||
      p->HV % p->H != 0)
    return GDR_ERR_SHAPE;
  if (p->qkv_dtype != GDR_F32 && p->qkv_dtype != GDR_BF16 && p->qkv_dtype != GDR_F16)
    return GDR_ERR_DTYPE;
  if (p->o_dtype != GDR_F32 && p->o_dtype != GDR_BF16 && p->o_dtype != GDR_F16)
    return GDR_ERR_DTYPE;
  if ((p->g_per_channel != 0 && p->g_per_channel != 1) ||
      (p->qk_l2norm != 0 && p->qk_l2norm != 1) ||
      (p->rule != GDR_RULE_DELTA && p->rule != GDR_RULE_LINEAR) || !std::isfinite(p->scale))
    return GDR_ERR_ARG;
  if ((p->K != 64 && p->K != 128) || (p->V != 64 && p->V != 128)) return GDR_ERR_UNSUPPORTED;
  if (p->scan_slab != 0 && p->scan_slab != 32 && p->scan_slab != 64 && p->scan_slab != 128)
    return GDR_ERR_ARG;
  if ((uint64_t)p->B * p->HV * 4 > 0x7fffffffull) return GDR_ERR_SHAPE;
  if (!q || !k || !v || !g || !beta || !state_out || !o) return GDR_ERR_NULL;
  for (const void* ptr : {(const void*)q, (const void*)k, (const void*)v, (const void*)g,
                          (const void*)beta, (const void*)state_in, (const void*)state_out,
                          (const void*)o})
    if (ptr && !aligned16(ptr)) return GDR_ERR_ALIGN;
  const size_t es = p->qkv_dtype == GDR_F32 ? 4 : 2;
  const size_t heads = (size_t)p->B * p->HV;
  const Span sq = {q, (size_t)p->B * p->H * p->K * es}, sk = {k, sq.n};
  const Span sv = {v, heads * p->V * es};
  const Span sg = {g, heads * (p->g_per_channel ? p->K : 1) * sizeof(float)};
  const Span sb = {beta, heads * sizeof(float)};
  const Span si = {state_in, heads * p->K * p->V * sizeof(float)};
  const Span so = {state_out, si.n};
  const Span sO = {o, heads * p->V * (p->o_dtype != GDR_F32 ? 2 : 4)};
  if (out_overlaps(sO, {sq, sk, sv, sg, sb, si, so})) return GDR_ERR_ALIAS;
  if (out_overlaps(so, {sq, sk, sv, sg, sb})) return GDR_ERR_ALIAS;
  if (state_in && state_in != state_out && overlap(si, so)) return GDR_ERR_ALIAS;
  gdr_status st = check_device();
  if (st != GDR_OK) return st;
  DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.s_in = state_in; a.s_out = state_out; a.o = o;
  a.o_fmt = p->o_dtype;
  a.B = p->B; a.H = p->H; a.HV = p->HV;
  a.scale = p->scale;
  a.l2norm = p->qk_l2norm;
  a.linear = p->rule == GDR_RULE_LINEAR;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int vb = decode_columns(p);
  return launch_decode(p->K, p->V, vb, p->g_per_channel == 1, p->qkv_dtype, a, hs);
}

gdr_status gdr_check_inputs(const gdr_problem* p, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, uint32_t* flags,
                            void* stream) {
  Prob r;
  gdr_status st = validate(p, &r);
  if (st != GDR_OK) return st;
  if (!q || !k || !v || !g || !beta || !flags) return GDR_ERR_NULL;
  for (const void* ptr : {(const void*)q, (const void*)k, (const void*)v, (const void*)g,
                          (const void*)beta})
    if (!aligned16(ptr)) return GDR_ERR_ALIGN;
  if (((uintptr_t)flags & 3u) != 0) return GDR_ERR_ALIGN;
  const Spans sp = spans(r, q, k, v, g, beta, nullptr, nullptr, nullptr, nullptr, 0);
  if (out_overlaps({flags, sizeof(uint32_t)}, {sp.q, sp.k, sp.v, sp.g, sp.beta}))
    return GDR_ERR_ALIAS;
  st = check_device();
  if (st != GDR_OK) return st;
  CheckArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.flags = flags;
  const size_t tok = (size_t)r.B * r.T;
  a.nqk = tok * r.H * r.K;
  a.nv = tok * r.HV * r.V;
  a.nbeta = tok * r.HV;
  a.B = r.B; a.T = r.T; a.HV = r.HV; a.K = r.K; a.C = r.C; a.N = r.N;
  a.perch = r.perch;
  a.fmt = r.f32 ? 0 : (r.h16 ? 2 : 1);
  a.qk_range = a.fmt == 1 && !r.l2norm;   // bf16 values can exceed the fp16 range
  a.decay = !r.f32;
  return launch_check(r, a, static_cast<hipStream_t>(stream));
}

size_t gdr_chunk_fwd_workspace_size(const gdr_problem* p) {
  Prob r;
  if (validate(p, &r) != GDR_OK) return 0;
  return layout(r).total;
}

gdr_status gdr_chunk_fwd(const gdr_problem* p, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* initial_state,
                         void* o, float* final_state, void* workspace,
                         size_t workspace_bytes, void* stream) {
  Prob r;
  gdr_status st = validate(p, &r);
  if (st != GDR_OK) return st;
  if ((st = check_fwd_pointers(q, k, v, g, beta, initial_state, o, final_state)) != GDR_OK)
    return st;
  if ((st = check_ws(r, workspace, workspace_bytes)) != GDR_OK) return st;
  if ((st = check_fwd_overlaps(r, q, k, v, g, beta, initial_state, o, final_state, workspace,
                               workspace_bytes)) != GDR_OK)
    return st;
  if ((st = check_device()) != GDR_OK) return st;
  return launch_fwd(r, q, k, v, g, beta, initial_state, o, final_state, workspace,
                    static_cast<hipStream_t>(stream));
}

gdr_status gdr_chunk_fwd_noalloc(const gdr_problem* p, const void* q, const void* k,
                                 const void* v, const float* g, const float* beta,
                                 const float* initial_state, void* o, float* final_state,
                                 void* stream) {
  Prob r;
  gdr_status st = validate(p, &r);
  if (st != GDR_OK) return st;
  if ((st = check_fwd_pointers(q, k, v, g, beta, initial_state, o, final_state)) != GDR_OK)
    return st;
  if (layout(r).total > GDR_NOALLOC_SCRATCH_BYTES) return GDR_ERR_SCRATCH;
  if ((st = check_fwd_overlaps(r, q, k, v, g, beta, initial_state, o, final_state, nullptr,
                               0)) != GDR_OK)
    return st;
  if ((st = check_device()) != GDR_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != GDR_OK) return st;
  return launch_fwd(r, q, k, v, g, beta, initial_state, o, final_state, ws,
                    static_cast<hipStream_t>(stream));
}

gdr_status gdr_chunk_prep(const gdr_problem* p, const void* q, const void* k, const float* g,
                          const float* beta, void* workspace, size_t workspace_bytes,
                          float* gamma, float* a_kk, float* a_qk, float* m_inv, void* stream) {
  Prob r;
  gdr_status st = validate(p, &r);
  if (st != GDR_OK) return st;
  if (!q || !k || !g || !beta) return GDR_ERR_NULL;
  for (const void* ptr : {(const void*)q, (const void*)k, (const void*)g, (const void*)beta,
                          (const void*)gamma, (const void*)a_kk, (const void*)a_qk,
                          (const void*)m_inv})
    if (ptr && !aligned16(ptr)) return GDR_ERR_ALIGN;
  if ((st = check_ws(r, workspace, workspace_bytes)) != GDR_OK) return st;
  const Spans s = spans(r, q, k, nullptr, g, beta, nullptr, nullptr, nullptr, workspace,
                        workspace_bytes);
  if (out_overlaps(s.ws, {s.q, s.k, s.g, s.beta})) return GDR_ERR_ALIAS;
  const size_t nc = nchunks(r);
  const Span dg = {gamma, nc * r.C * (r.perch ? r.K : 1) * sizeof(float)};
  const Span dm = {a_kk, nc * r.C * r.C * sizeof(float)};
  const Span da = {a_qk, nc * r.C * r.C * sizeof(float)};
  const Span di = {m_inv, nc * r.C * r.C * sizeof(float)};
  for (const Span& out : {dg, dm, da, di})
    if (out_overlaps(out, {s.q, s.k, s.g, s.beta, s.ws})) return GDR_ERR_ALIAS;
  if (overlap(dg, dm) || overlap(dg, da) || overlap(dg, di) || overlap(dm, da) ||
      overlap(dm, di) || overlap(da, di))
    return GDR_ERR_ALIAS;
  if ((st = check_device()) != GDR_OK) return st;

  PrepArgs pa = prep_args(r, q, k, g, beta, workspace);
  pa.d_gamma = gamma; pa.d_akk = a_kk; pa.d_aqk = a_qk; pa.d_minv = m_inv;
  const bool dump = gamma || a_kk || a_qk || m_inv;
  return launch_prep(r, pa, dump, static_cast<hipStream_t>(stream));
}

gdr_status gdr_chunk_scan(const gdr_problem* p, const void* q, const void* k, const void* v,
                          const float* initial_state, void* o, float* final_state,
                          void* workspace, size_t workspace_bytes, void* stream) {
  Prob r;
  gdr_status st = validate(p, &r);
  if (st != GDR_OK) return st;
  if (!q || !k || !v || !o) return GDR_ERR_NULL;
  for (const void* ptr : {(const void*)q, (const void*)k, (const void*)v,
                          (const void*)initial_state, (const void*)o, (const void*)final_state})
    if (ptr && !aligned16(ptr)) return GDR_ERR_ALIGN;
  if ((st = check_ws(r, workspace, workspace_bytes)) != GDR_OK) return st;
  const Spans s = spans(r, q, k, v, nullptr, nullptr, initial_state, o, final_state,
                        workspace, workspace_bytes);
  if (out_overlaps(s.o, {s.q, s.k, s.v, s.s0, s.sT, s.ws})) return GDR_ERR_ALIAS;
  if (out_overlaps(s.sT, {s.q, s.k, s.v, s.ws})) return GDR_ERR_ALIAS;
  if (out_overlaps(s.ws, {s.q, s.k, s.v, s.s0})) return GDR_ERR_ALIAS;
  if (initial_state && final_state && initial_state != final_state && overlap(s.sT, s.s0))
    return GDR_ERR_ALIAS;
  if ((st = check_device()) != GDR_OK) return st;
  ScanArgs sa = scan_args(r, q, k, v, initial_state, o, final_state, workspace);
  return launch_scan(r, sa, static_cast<hipStream_t>(stream));
}

const char* gdr_status_string(int status) {
  switch (status) {
    case GDR_OK: return "GDR_OK: success";
    case GDR_ERR_NULL: return "GDR_ERR_NULL: a required pointer is NULL";
    case GDR_ERR_SHAPE: return "GDR_ERR_SHAPE: B, T, H, HV, K, V must be >= 1 and HV % H == 0";
    case GDR_ERR_DTYPE: return "GDR_ERR_DTYPE: qkv_dtype must be GDR_F32 or GDR_BF16";
    case GDR_ERR_UNSUPPORTED: return "GDR_ERR_UNSUPPORTED: built for chunk 64 or 128 and K, V in {64, 128}; chunk 128 takes scan_slab 0 or its one width (32 for K = 128, 64 for K = 64)";
    case GDR_ERR_ALIGN: return "GDR_ERR_ALIGN: tensors and workspace must be 16-byte aligned";
    case GDR_ERR_WORKSPACE: return "GDR_ERR_WORKSPACE: workspace NULL or smaller than gdr_chunk_fwd_workspace_size";
    case GDR_ERR_DEVICE: return "GDR_ERR_DEVICE: the current HIP device is not gfx950";
    case GDR_ERR_HIP: return "GDR_ERR_HIP: a HIP query or kernel launch failed";
    case GDR_ERR_ARG: return "GDR_ERR_ARG: scale must be finite, g_per_channel and qk_l2norm 0 or 1, rule a gdr_rule, scan_segments >= 0, scan_slab 0, 32 or 64 (128 for decode)";
    case GDR_ERR_ALIAS: return "GDR_ERR_ALIAS: an output overlaps an input or another output";
    case GDR_ERR_SCRATCH: return "GDR_ERR_SCRATCH: the problem needs more workspace than gdr_chunk_fwd_noalloc's GDR_NOALLOC_SCRATCH_BYTES";
    default: return "GDR_ERR_UNKNOWN: unknown status value";
  }
}

int gdr_chunk_scan_segments(const gdr_problem* p) {
  Prob r;
  if (validate(p, &r) != GDR_OK) return 0;
  return r.nseg;
}

int gdr_chunk_scan_slab(const gdr_problem* p) {
  Prob r;
  if (validate(p, &r) != GDR_OK) return 0;
  return r.bv;
}

int gdr_version(void) { return 500; }   // 0.5.0: fp16 inputs and o (GDR_F16)

}  // extern "C"
