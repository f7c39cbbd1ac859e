/*
 * gdr_oracle.c -- fp64 per-token recurrence of the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP path.
 *
 * What it computes (the "naive recurrent" form that the chunkwise algorithm
 * reproduces exactly; sec-03 notes, "Why chunk?" and the closing summary; the
 * delta rule of the "Chunkwise parallel algorithms" page, section 2.1, written
 * there in the transposed d_v x d_k convention):
 *
 *   for every batch b and value head hv (q/k head h = hv / (HV/H), the
 *   repeat_interleave grouping of the sec-03 listing):
 *     S = initial_state[b,hv] (K x V), or 0
 *     for t = 0 .. T-1:
 *       S <- diag(exp(g_t)) S                    decay first (sec-03,
 *                                                 inter-chunk loop: decay old
 *                                                 state, then write)
 *       S <- S + beta_t k_t (v_t - S^T k_t)^T    delta-rule write
 *       o_t = scale * S^T q_t                    read after the write: A_qk
 *                                                 keeps its diagonal
 *     final_state[b,hv] = S
 *
 * g_t is one scalar per (b, t, hv) or, for the per-channel (KDA) form, one
 * value per key channel; exp(g_t) then scales row d of S by exp(g_t[d]).
 *
 * With linear = 1 the write has no prediction term (no erase):
 *       S <- S + beta_t k_t v_t^T
 * the decayed linear attention of the Mamba2 state-space-duality section of
 * the "Chunkwise parallel algorithms" page (section 1.1: S_t = alpha_t
 * S_{t-1} + v_t k_t^T, o_t = S_t q_t, with alpha_t = exp(g_t) and beta_t as
 * an input scale; beta = 1 and scale = 1 give the page's form exactly).
 *
 * Layouts (row-major, contiguous):
 *   q, k   [B, T, H, K]      v, o  [B, T, HV, V]
 *   g      [B, T, HV] or [B, T, HV, K]
 *   beta   [B, T, HV]        s0, s_final [B, HV, K, V]   (s0 may be NULL)
 *
 * Parallel over the B*HV independent scans with OpenMP; each scan is the plain
 * serial loop above, in fp64, with no blocking or reordering.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int gdr_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation failure. */
int gdr_oracle_recurrence_rule(int B, int T, int H, int HV, int K, int V,
                               int g_per_channel, int linear, double scale,
                               const double* q, const double* k, const double* v,
                               const double* g, const double* beta,
                               const double* s0, double* o, double* s_final,
                               int num_threads) {
  if (B < 1 || T < 0 || H < 1 || HV < 1 || K < 1 || V < 1 || HV % H != 0)
    return -1;
  if (!q || !k || !v || !g || !beta || !o || !s_final) return -1;
  const int G = HV / H;
  const long nscan = (long)B * HV;
  int failed = 0;
#ifdef _OPENMP
  if (num_threads < 1) num_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads)
#endif
  for (long bh = 0; bh < nscan; ++bh) {
    const int b = (int)(bh / HV), hv = (int)(bh % HV), h = hv / G;
    double* S = (double*)malloc(sizeof(double) * (size_t)K * V);
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    double* dec = (double*)malloc(sizeof(double) * (size_t)K);
    if (!S || !p || !dec) {
      failed = 1;
      free(S); free(p); free(dec);
      continue;
    }
    if (s0)
      memcpy(S, s0 + (size_t)bh * K * V, sizeof(double) * (size_t)K * V);
    else
      memset(S, 0, sizeof(double) * (size_t)K * V);

    for (int t = 0; t < T; ++t) {
      const size_t tok = (size_t)b * T + t;
      const double* qt = q + (tok * H + h) * K;
      const double* kt = k + (tok * H + h) * K;
      const double* vt = v + (tok * HV + hv) * V;
      const double bt = beta[tok * HV + hv];
      double* ot = o + (tok * HV + hv) * V;

      /* decay: S <- diag(exp(g_t)) S */
      if (g_per_channel) {
        const double* gt = g + (tok * HV + hv) * K;
        for (int d = 0; d < K; ++d) dec[d] = exp(gt[d]);
      } else {
        const double e = exp(g[tok * HV + hv]);
        for (int d = 0; d < K; ++d) dec[d] = e;
      }
      for (int d = 0; d < K; ++d)
        for (int j = 0; j < V; ++j) S[(size_t)d * V + j] *= dec[d];

      /* prediction p = S^T k_t (none for the linear rule) */
      for (int j = 0; j < V; ++j) p[j] = 0.0;
      if (!linear)
        for (int d = 0; d < K; ++d)
          for (int j = 0; j < V; ++j) p[j] += S[(size_t)d * V + j] * kt[d];

      /* write: S <- S + beta_t k_t (v_t - p)^T */
      for (int j = 0; j < V; ++j) p[j] = bt * (vt[j] - p[j]);
      for (int d = 0; d < K; ++d)
        for (int j = 0; j < V; ++j) S[(size_t)d * V + j] += kt[d] * p[j];

      /* read: o_t = scale * S^T q_t */
      for (int j = 0; j < V; ++j) ot[j] = 0.0;
      for (int d = 0; d < K; ++d)
        for (int j = 0; j < V; ++j) ot[j] += S[(size_t)d * V + j] * qt[d];
      for (int j = 0; j < V; ++j) ot[j] *= scale;
    }
    memcpy(s_final + (size_t)bh * K * V, S, sizeof(double) * (size_t)K * V);
    free(S); free(p); free(dec);
  }
  return failed ? -2 : 0;
}

/* The gated delta rule (linear = 0). */
int gdr_oracle_recurrence(int B, int T, int H, int HV, int K, int V,
                          int g_per_channel, double scale,
                          const double* q, const double* k, const double* v,
                          const double* g, const double* beta,
                          const double* s0, double* o, double* s_final,
                          int num_threads) {
  return gdr_oracle_recurrence_rule(B, T, H, HV, K, V, g_per_channel, 0, scale, q, k, v, g,
                                    beta, s0, o, s_final, num_threads);
}
