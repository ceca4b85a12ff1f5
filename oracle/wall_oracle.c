/*
 * Wall Attention — plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the package smoke check and the benchmark's CPU-baseline leg may build,
 * load or call it.  It shares no code, header, table or helper with the HIP
 * library and must never be used as a fallback for it.
 *
 * What it computes (Wall Attention README, introduction, "Usage" and
 * "Decode" sections; the sliding-window/document rule from the FlexAttention
 * article, section "score_mod and mask_mod"):
 *
 *   P[t,hq,n]  = sum_{u=bos..t} g[u,hq,n]              (inclusive prefix, natural log units)
 *   Gs[t,hq]   = sum_{u=bos..t} g_scalar[u,hq]         (0 when absent)
 *   S_i        = { j : bos <= j <= i  and  (W <= 0 or i - j < W) }
 *   s_ij       = scale * sum_n q[i,hq,n] k[j,h,n] exp(P[i,hq,n] - P[j,hq,n]) + Gs[i] - Gs[j]
 *   m_i        = max( max_{j in S_i} s_ij , sink[hq] if present )
 *   Z_i        = sum_{j in S_i} exp(s_ij - m_i) + [sink] exp(sink[hq] - m_i)
 *   o[i,hq,:]  = sum_{j in S_i} exp(s_ij - m_i) v[j,h,:] / Z_i,   lse[i,hq] = m_i + ln Z_i
 *
 * with h = floor(hq / (HQ/H)) (contiguous GQA groups).  A segment [bos,eos)
 * is one batch row when no cu_seqlens is given, else one packed sequence.
 *
 * Decode side (README "Decode"): P2 = P / ln 2 (log2 units), chunk anchors
 * R_c = P2 at the last token of chunk c, k_tilde[j] = k[j] * 2^(R_c - P2[j]),
 * and the single-step decode over that cache scores key j with
 * scale * sum_n q[n] 2^(p_curr[n] - R_{c(j)}[n]) k_tilde[j,n].
 *
 * Every loop runs in the order of the formulas above; nothing is blocked,
 * fused or reordered.  Inputs arrive as float (exact for bf16 and fp32
 * tensors) and are promoted to double; all arithmetic is double.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads the loops below use from now on (n > 0); returns the count in force.
   Only the timing of the oracle changes, not what it computes. */
int oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* Segment s of the packed token axis: [bos, eos). */
static void segment(int64_t s, int64_t T, const int32_t *cu, int64_t *bos, int64_t *eos) {
  if (cu) {
    *bos = cu[s];
    *eos = cu[s + 1];
  } else {
    *bos = s * T;
    *eos = (s + 1) * T;
  }
}

/* Inclusive running sums of g (per channel) and g_scalar, restarted at every
 * segment start.  Output P and Gs are double, natural-log units. */
static void prefix_sums(const float *g, const float *gs, int64_t nseg, int64_t T,
                        const int32_t *cu, int64_t HQ, int64_t K, double *P, double *Gs) {
  #pragma omp parallel for collapse(2) schedule(static)
  for (int64_t s = 0; s < nseg; ++s) {
    for (int64_t hq = 0; hq < HQ; ++hq) {
      int64_t bos, eos;
      segment(s, T, cu, &bos, &eos);
      for (int64_t n = 0; n < K; ++n) {
        double acc = 0.0;
        for (int64_t t = bos; t < eos; ++t) {
          acc += (double)g[(t * HQ + hq) * K + n];
          P[(t * HQ + hq) * K + n] = acc;
        }
      }
      double accs = 0.0;
      for (int64_t t = bos; t < eos; ++t) {
        if (gs) accs += (double)gs[t * HQ + hq];
        Gs[t * HQ + hq] = accs;
      }
    }
  }
}

/*
 * Forward (prefill) rows.  Shapes, all contiguous, token axis packed:
 *   q [Ntok,HQ,K]  k [Ntok,H,K]  v [Ntok,H,V]  g [Ntok,HQ,K]  g_scalar [Ntok,HQ] or NULL
 *   sink [HQ] or NULL, cu_seqlens [nseq+1] or NULL (then Ntok = B*T, one segment per b).
 * rows: global token indices to evaluate (NULL = every token, nrows ignored).
 * o [nrows,HQ,V] and lse [nrows,HQ] (lse may be NULL).
 * Returns 0, or -1 on a bad argument.
 */
int oracle_wall_attn_fwd(const float *q, const float *k, const float *v, const float *g,
                         const float *g_scalar, const float *sink,
                         int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                         const int32_t *cu_seqlens, int64_t nseq, int64_t window, double scale,
                         const int64_t *rows, int64_t nrows, double *o, double *lse) {
  if (H <= 0 || HQ <= 0 || HQ % H != 0 || K <= 0 || V <= 0) return -1;
  int64_t nseg = cu_seqlens ? nseq : B;
  int64_t ntok = cu_seqlens ? (int64_t)cu_seqlens[nseq] : B * T;
  if (cu_seqlens && B != 1) return -1;
  int64_t group = HQ / H;

  double *P = (double *)malloc(sizeof(double) * (size_t)(ntok * HQ * K));
  double *Gs = (double *)malloc(sizeof(double) * (size_t)(ntok * HQ));
  if (!P || !Gs) { free(P); free(Gs); return -1; }
  prefix_sums(g, g_scalar, nseg, T, cu_seqlens, HQ, K, P, Gs);

  if (!rows) nrows = ntok;
  /* segment index of each requested row */
  int64_t *rseg = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nrows > 0 ? nrows : 1));
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t i = rows ? rows[r] : r;
    int64_t s = 0;
    if (cu_seqlens) {
      while (s + 1 < nseg && i >= cu_seqlens[s + 1]) ++s;
    } else {
      s = i / T;
    }
    rseg[r] = s;
  }

  #pragma omp parallel
  {
    double *sc = NULL;
    int64_t cap = 0;
    #pragma omp for collapse(2) schedule(dynamic, 4)
    for (int64_t r = 0; r < nrows; ++r) {
      for (int64_t hq = 0; hq < HQ; ++hq) {
        int64_t i = rows ? rows[r] : r;
        int64_t bos, eos;
        segment(rseg[r], T, cu_seqlens, &bos, &eos);
        int64_t h = hq / group;
        int64_t jlo = bos;
        if (window > 0 && i - window + 1 > jlo) jlo = i - window + 1;
        int64_t L = i - jlo + 1;
        if (L > cap) { free(sc); cap = L; sc = (double *)malloc(sizeof(double) * (size_t)cap); }
        const float *qi = q + (i * HQ + hq) * K;
        const double *Pi = P + (i * HQ + hq) * K;
        double m = -INFINITY;
        for (int64_t j = jlo; j <= i; ++j) {
          const float *kj = k + (j * H + h) * K;
          const double *Pj = P + (j * HQ + hq) * K;
          double dot = 0.0;
          for (int64_t n = 0; n < K; ++n)
            dot += (double)qi[n] * (double)kj[n] * exp(Pi[n] - Pj[n]);
          double s = scale * dot + (Gs[i * HQ + hq] - Gs[j * HQ + hq]);
          sc[j - jlo] = s;
          if (s > m) m = s;
        }
        if (sink && (double)sink[hq] > m) m = (double)sink[hq];
        double Z = 0.0;
        for (int64_t j = jlo; j <= i; ++j) Z += exp(sc[j - jlo] - m);
        if (sink) Z += exp((double)sink[hq] - m);
        double *oi = o + (r * HQ + hq) * V;
        for (int64_t c = 0; c < V; ++c) oi[c] = 0.0;
        for (int64_t j = jlo; j <= i; ++j) {
          double w = exp(sc[j - jlo] - m) / Z;
          const float *vj = v + (j * H + h) * V;
          for (int64_t c = 0; c < V; ++c) oi[c] += w * (double)vj[c];
        }
        if (lse) lse[r * HQ + hq] = m + log(Z);
      }
    }
    free(sc);
  }
  free(rseg);
  free(P);
  free(Gs);
  return 0;
}

/*
 * P2 = log2(e) * inclusive prefix of g, restarted at each segment start
 * (README "Decode": the prefix is taken with scale RCP_LN2 = 1/ln 2).
 * g [Ntok,HQ,K] -> P2 [Ntok,HQ,K] (double).
 */
int oracle_prefix_log2(const float *g, int64_t B, int64_t T, int64_t HQ, int64_t K,
                       const int32_t *cu_seqlens, int64_t nseq, double *P2) {
  int64_t nseg = cu_seqlens ? nseq : B;
  #pragma omp parallel for collapse(2) schedule(static)
  for (int64_t s = 0; s < nseg; ++s) {
    for (int64_t hq = 0; hq < HQ; ++hq) {
      int64_t bos, eos;
      segment(s, T, cu_seqlens, &bos, &eos);
      for (int64_t n = 0; n < K; ++n) {
        double acc = 0.0;
        for (int64_t t = bos; t < eos; ++t) {
          acc += (double)g[(t * HQ + hq) * K + n];
          P2[(t * HQ + hq) * K + n] = acc / log(2.0);
        }
      }
    }
  }
  return 0;
}

/*
 * Decode cache build (README "Decode"): chunk c of C tokens has anchor
 * R_c = P2 at its last token, min((c+1)C, T) - 1; the rescaled key is
 * k_tilde[j,hq,:] = k[j,h,:] * 2^(R_{c(j)} - P2[j,hq,:]).
 *   k [B,T,H,K], P2 [B,T,HQ,K] (float, as the caller stores it)
 *   -> k_tilde [B,T,HQ,K] (double, unrounded), r_cache [B,ceil(T/C),HQ,K] (double)
 */
int oracle_build_kv_cache(const float *k, const float *P2, int64_t B, int64_t T, int64_t HQ,
                          int64_t H, int64_t K, int64_t C, double *k_tilde, double *r_cache) {
  if (H <= 0 || HQ % H != 0 || C <= 0) return -1;
  int64_t group = HQ / H;
  int64_t nc = (T + C - 1) / C;
  #pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t c = 0; c < nc; ++c) {
      int64_t last = (c + 1) * C < T ? (c + 1) * C - 1 : T - 1;
      for (int64_t hq = 0; hq < HQ; ++hq) {
        const float *R = P2 + ((b * T + last) * HQ + hq) * K;
        double *rc = r_cache + ((b * nc + c) * HQ + hq) * K;
        for (int64_t n = 0; n < K; ++n) rc[n] = (double)R[n];
        for (int64_t j = c * C; j <= last; ++j) {
          const float *kj = k + ((b * T + j) * H + hq / group) * K;
          const float *pj = P2 + ((b * T + j) * HQ + hq) * K;
          double *kt = k_tilde + ((b * T + j) * HQ + hq) * K;
          for (int64_t n = 0; n < K; ++n)
            kt[n] = (double)kj[n] * exp2((double)R[n] - (double)pj[n]);
        }
      }
    }
  }
  return 0;
}

/*
 * Single-step decode over a pre-rescaled cache (README "Decode").  The query
 * is the newest token; it attends to all T_kv cached positions, itself
 * included.  Key j of chunk c = floor(j/C) is scored as
 *   s_j = scale * sum_n q[n] * 2^(p_curr[n] - r_cache[c,n]) * k_tilde[j,n]
 * and the softmax (with the optional sink logit) runs over j = 0..T_kv-1.
 *   q [B,HQ,K], v [B,T,H,V], p_curr [B,HQ,K], k_tilde [B,T,HQ,K],
 *   r_cache [B,ceil(T/C),HQ,K], sink [HQ] or NULL -> o [B,HQ,V], lse [B,HQ]
 */
int oracle_decode_cache(const float *q, const float *v, const float *p_curr, const float *k_tilde,
                        const float *r_cache, const float *sink, int64_t B, int64_t T, int64_t HQ,
                        int64_t H, int64_t K, int64_t V, int64_t C, double scale, double *o,
                        double *lse) {
  if (H <= 0 || HQ % H != 0 || C <= 0) return -1;
  int64_t group = HQ / H;
  int64_t nc = (T + C - 1) / C;
  #pragma omp parallel
  {
    double *sc = (double *)malloc(sizeof(double) * (size_t)T);
    #pragma omp for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b) {
      for (int64_t hq = 0; hq < HQ; ++hq) {
        int64_t h = hq / group;
        const float *qv = q + (b * HQ + hq) * K;
        const float *pc = p_curr + (b * HQ + hq) * K;
        double m = -INFINITY;
        for (int64_t j = 0; j < T; ++j) {
          int64_t c = j / C;
          const float *r = r_cache + ((b * nc + c) * HQ + hq) * K;
          const float *kt = k_tilde + ((b * T + j) * HQ + hq) * K;
          double dot = 0.0;
          for (int64_t n = 0; n < K; ++n)
            dot += (double)qv[n] * exp2((double)pc[n] - (double)r[n]) * (double)kt[n];
          sc[j] = scale * dot;
          if (sc[j] > m) m = sc[j];
        }
        if (sink && (double)sink[hq] > m) m = (double)sink[hq];
        double Z = 0.0;
        for (int64_t j = 0; j < T; ++j) Z += exp(sc[j] - m);
        if (sink) Z += exp((double)sink[hq] - m);
        double *ov = o + (b * HQ + hq) * V;
        for (int64_t c = 0; c < V; ++c) ov[c] = 0.0;
        for (int64_t j = 0; j < T; ++j) {
          double w = exp(sc[j] - m) / Z;
          const float *vj = v + ((b * T + j) * H + h) * V;
          for (int64_t c = 0; c < V; ++c) ov[c] += w * (double)vj[c];
        }
        if (lse) lse[b * HQ + hq] = m + log(Z);
      }
    }
    free(sc);
  }
  return 0;
}

/*
 * Decode over a pre-rescaled cache with the serving options (README "Decode"
 * formula; the window rule of the FlexAttention article, section "score_mod
 * and mask_mod"; the gate is the forward's Gs[i] - Gs[j] of README "Usage").
 * Row b holds lens[b] cached tokens (lens NULL: all T) and its query sits at
 * position i = lens[b] - 1; key j counts if j < lens[b] and (W <= 0 or
 * i - j < W).  With a gate cache (running sums of g_scalar in log2 units)
 * the score of key j gains (gate_curr[b,hq] - gate_cache[b,j,hq]) * ln 2:
 *   s_j = scale * sum_n q[n] 2^(p_curr[n] - r_cache[c(j),n]) k_tilde[j,n]
 *         + (gate_curr - gate_cache[j]) * ln 2
 * then the softmax over the counted keys (and the optional sink logit).  A
 * row with no counted key gets o = 0 and lse = sink (or -inf).
 *   q [B,HQ,K], v [B,T,H,V], p_curr [B,HQ,K], k_tilde [B,T,HQ,K],
 *   r_cache [B,ceil(T/C),HQ,K], sink [HQ] or NULL, gate_cache [B,T,HQ] and
 *   gate_curr [B,HQ] or NULL, lens [B] or NULL -> o [B,HQ,V], lse [B,HQ]
 */
int oracle_decode_cache_ext(const float *q, const float *v, const float *p_curr,
                            const float *k_tilde, const float *r_cache, const float *sink,
                            const float *gate_cache, const float *gate_curr, const int32_t *lens,
                            int64_t window, int64_t B, int64_t T, int64_t HQ, int64_t H,
                            int64_t K, int64_t V, int64_t C, double scale, double *o,
                            double *lse) {
  if (H <= 0 || HQ % H != 0 || C <= 0) return -1;
  int64_t group = HQ / H;
  int64_t nc = (T + C - 1) / C;
  #pragma omp parallel
  {
    double *sc = (double *)malloc(sizeof(double) * (size_t)T);
    #pragma omp for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b) {
      for (int64_t hq = 0; hq < HQ; ++hq) {
        int64_t h = hq / group;
        int64_t L = lens ? (int64_t)lens[b] : T;
        int64_t jlo = 0;
        if (window > 0 && L - window > 0) jlo = L - window;
        const float *qv = q + (b * HQ + hq) * K;
        const float *pc = p_curr + (b * HQ + hq) * K;
        double m = -INFINITY;
        for (int64_t j = jlo; j < L; ++j) {
          int64_t c = j / C;
          const float *r = r_cache + ((b * nc + c) * HQ + hq) * K;
          const float *kt = k_tilde + ((b * T + j) * HQ + hq) * K;
          double dot = 0.0;
          for (int64_t n = 0; n < K; ++n)
            dot += (double)qv[n] * exp2((double)pc[n] - (double)r[n]) * (double)kt[n];
          double s = scale * dot;
          if (gate_cache)
            s += ((double)gate_curr[b * HQ + hq] - (double)gate_cache[(b * T + j) * HQ + hq]) * log(2.0);
          sc[j] = s;
          if (s > m) m = s;
        }
        if (sink && (double)sink[hq] > m) m = (double)sink[hq];
        double *ov = o + (b * HQ + hq) * V;
        for (int64_t c = 0; c < V; ++c) ov[c] = 0.0;
        if (m == -INFINITY) {
          if (lse) lse[b * HQ + hq] = -INFINITY;
          continue;
        }
        double Z = 0.0;
        for (int64_t j = jlo; j < L; ++j) Z += exp(sc[j] - m);
        if (sink) Z += exp((double)sink[hq] - m);
        for (int64_t j = jlo; j < L; ++j) {
          double w = exp(sc[j] - m) / Z;
          const float *vj = v + ((b * T + j) * H + h) * V;
          for (int64_t c = 0; c < V; ++c) ov[c] += w * (double)vj[c];
        }
        if (lse) lse[b * HQ + hq] = m + log(Z);
      }
    }
    free(sc);
  }
  return 0;
}

/*
 * Gradients of the forward (Wall Attention README, introduction: "fused
 * forward + backward kernels with analytic gradients for q, k, v, g"; its
 * tests check the gradients of g and g_scalar against central finite
 * differences).  For a loss L with dL/do = dO, written from the forward's
 * definition above:
 *   p_ij   = exp(s_ij - lse_i)  (j in S_i),   p_sink_i = exp(sink - lse_i)
 *   dv_j   = sum_i p_ij dO_i                             (summed over the query heads of v's head)
 *   dp_ij  = dO_i . v_j,   D_i = sum_j p_ij dp_ij,   ds_ij = p_ij (dp_ij - D_i)
 *   dsink  = -sum_i p_sink_i D_i                         (the sink logit has no value)
 *   a_ijn  = scale q_in k_jn exp(P_in - P_jn)             (so s_ij = sum_n a_ijn + Gs_i - Gs_j)
 *   dq_in  = sum_j ds_ij a_ijn / q_in  = scale sum_j ds_ij k_jn exp(P_in - P_jn)
 *   dk_jn  = scale sum_i ds_ij q_in exp(P_in - P_jn)      (summed over the query heads of k's head)
 *   dP_tn  = sum_j ds_tj a_tjn - sum_i ds_it a_itn        (P_t enters as the query's and the key's prefix)
 *   dGs_t  = sum_j ds_tj - sum_i ds_it
 *   dg_un  = sum_{t >= u, same segment} dP_tn,   dg_scalar_u = sum_{t >= u} dGs_t
 * Every array is double; inputs as oracle_wall_attn_fwd; dO [Ntok,HQ,V].
 * dg_scalar and dsink may be NULL.  Returns 0, or -1 on a bad argument.
 */
int oracle_wall_attn_bwd(const float *q, const float *k, const float *v, const float *g,
                         const float *g_scalar, const float *sink, const float *dO,
                         int64_t B, int64_t T, int64_t HQ, int64_t H, int64_t K, int64_t V,
                         const int32_t *cu_seqlens, int64_t nseq, int64_t window, double scale,
                         double *dq, double *dk, double *dv, double *dg, double *dg_scalar,
                         double *dsink) {
  if (H <= 0 || HQ <= 0 || HQ % H != 0 || K <= 0 || V <= 0) return -1;
  if (cu_seqlens && B != 1) return -1;
  int64_t nseg = cu_seqlens ? nseq : B;
  int64_t ntok = cu_seqlens ? (int64_t)cu_seqlens[nseq] : B * T;
  int64_t group = HQ / H;
  double *P = (double *)malloc(sizeof(double) * (size_t)(ntok * HQ * K));
  double *Gs = (double *)malloc(sizeof(double) * (size_t)(ntok * HQ));
  double *dP = (double *)calloc((size_t)(ntok * HQ * K), sizeof(double));
  double *dGs = (double *)calloc((size_t)(ntok * HQ), sizeof(double));
  double *dsk = (double *)calloc((size_t)HQ, sizeof(double));
  if (!P || !Gs || !dP || !dGs || !dsk) { free(P); free(Gs); free(dP); free(dGs); free(dsk); return -1; }
  prefix_sums(g, g_scalar, nseg, T, cu_seqlens, HQ, K, P, Gs);
  memset(dq, 0, sizeof(double) * (size_t)(ntok * HQ * K));
  memset(dk, 0, sizeof(double) * (size_t)(ntok * H * K));
  memset(dv, 0, sizeof(double) * (size_t)(ntok * H * V));
  /* Sequential over (segment, query head, row): the key-side sums (dk, dv,
   * the key's share of dP and dGs) accumulate from many rows. */
  for (int64_t s = 0; s < nseg; ++s) {
    int64_t bos, eos;
    segment(s, T, cu_seqlens, &bos, &eos);
    for (int64_t hq = 0; hq < HQ; ++hq) {
      int64_t h = hq / group;
      for (int64_t i = bos; i < eos; ++i) {
        int64_t jlo = bos;
        if (window > 0 && i - window + 1 > jlo) jlo = i - window + 1;
        int64_t n_j = i - jlo + 1;
        double *sc = (double *)malloc(sizeof(double) * (size_t)n_j);
        double *dp = (double *)malloc(sizeof(double) * (size_t)n_j);
        const float *qi = q + (i * HQ + hq) * K;
        const double *Pi = P + (i * HQ + hq) * K;
        const float *dOi = dO + (i * HQ + hq) * V;
        /* forward statistics of row i */
        double m = -INFINITY;
        for (int64_t j = jlo; j <= i; ++j) {
          const float *kj = k + (j * H + h) * K;
          const double *Pj = P + (j * HQ + hq) * K;
          double dot = 0.0;
          for (int64_t n = 0; n < K; ++n) dot += (double)qi[n] * (double)kj[n] * exp(Pi[n] - Pj[n]);
          sc[j - jlo] = scale * dot + (Gs[i * HQ + hq] - Gs[j * HQ + hq]);
          if (sc[j - jlo] > m) m = sc[j - jlo];
        }
        if (sink && (double)sink[hq] > m) m = (double)sink[hq];
        double Z = 0.0;
        for (int64_t j = jlo; j <= i; ++j) Z += exp(sc[j - jlo] - m);
        if (sink) Z += exp((double)sink[hq] - m);
        double lse = m + log(Z);
        /* dp, D */
        double D = 0.0;
        for (int64_t j = jlo; j <= i; ++j) {
          const float *vj = v + (j * H + h) * V;
          double t = 0.0;
          for (int64_t c = 0; c < V; ++c) t += (double)dOi[c] * (double)vj[c];
          dp[j - jlo] = t;
          D += exp(sc[j - jlo] - lse) * t;
        }
        if (sink) dsk[hq] -= exp((double)sink[hq] - lse) * D;
        for (int64_t j = jlo; j <= i; ++j) {
          const float *kj = k + (j * H + h) * K;
          const float *vj = v + (j * H + h) * V;
          const double *Pj = P + (j * HQ + hq) * K;
          double p = exp(sc[j - jlo] - lse);
          double ds = p * (dp[j - jlo] - D);
          for (int64_t c = 0; c < V; ++c) dv[(j * H + h) * V + c] += p * (double)dOi[c];
          for (int64_t n = 0; n < K; ++n) {
            double a = scale * (double)qi[n] * (double)kj[n] * exp(Pi[n] - Pj[n]);
            dq[(i * HQ + hq) * K + n] += ds * scale * (double)kj[n] * exp(Pi[n] - Pj[n]);
            dk[(j * H + h) * K + n] += ds * scale * (double)qi[n] * exp(Pi[n] - Pj[n]);
            dP[(i * HQ + hq) * K + n] += ds * a;
            dP[(j * HQ + hq) * K + n] -= ds * a;
          }
          dGs[i * HQ + hq] += ds;
          dGs[j * HQ + hq] -= ds;
        }
        free(sc);
        free(dp);
      }
      /* reverse running sums within the segment */
      for (int64_t n = 0; n < K; ++n) {
        double acc = 0.0;
        for (int64_t t = eos - 1; t >= bos; --t) {
          acc += dP[(t * HQ + hq) * K + n];
          dg[(t * HQ + hq) * K + n] = acc;
        }
      }
      if (dg_scalar) {
        double acc = 0.0;
        for (int64_t t = eos - 1; t >= bos; --t) {
          acc += dGs[t * HQ + hq];
          dg_scalar[t * HQ + hq] = acc;
        }
      }
    }
  }
  if (dsink)
    for (int64_t hq = 0; hq < HQ; ++hq) dsink[hq] = sink ? dsk[hq] : 0.0;
  free(P);
  free(Gs);
  free(dP);
  free(dGs);
  free(dsk);
  return 0;
}
