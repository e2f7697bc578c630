/*
 * Gated delta rule (GDN) oracle: plain fp64 token-by-token recurrence, forward
 * and reverse-mode backward, on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference for the
 * HIP path.  It shares no code, header, table or helper with the HIP library;
 * only tests, the smoke check and the CPU-baseline leg of the benchmark may
 * load it.  Nothing in the product path calls it.
 *
 * What it computes (FlashQLA article, "高级 API 示例" and "底层 API" sections:
 * q,k [B,T,H_q,K], v [B,T,H_v,V], gate g and beta [B,T,H_v], scale, optional
 * initial state, optional cu_seqlens; outputs o and final_state, and the
 * backward's dq, dk, dv, dbeta, dg, dh0).  The pages name the operator (the
 * GDN chunked prefill) but print no formula; the recurrence below is the
 * gated delta rule with the state stored K x V:
 *
 *   S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *   o_t = scale * S_t^T q_t          (the state after the token's update)
 *
 * computed in the order  S~ = e^g S;  p = S~^T k;  d = beta (v - p);
 * S = S~ + k d^T;  o = scale S^T q.
 *
 * The v-head h reads q/k head  h / (H_v / H_q)  (consecutive v-heads share a
 * q/k head).  With cu_seqlens (B must be 1) sequence n covers tokens
 * [cu[n], cu[n+1]) and owns initial/final state row n; without it, N = B and
 * sequence n is batch row n.
 *
 * Backward: reverse mode of the same loop.  Forward states are checkpointed
 * every CKPT tokens and recomputed inside each window.  dq and dk are first
 * produced per v-head and then summed over the v-heads of each q/k group in
 * increasing v-head order.
 *
 * Sampling: unit_mask (N*H_v bytes, or NULL for all) selects which
 * (sequence, v-head) units are computed; outputs of unselected units are left
 * as they were.  dq/dk of a q/k head sum only over its selected v-heads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define CKPT 64

typedef struct {
  int B, T, Hq, Hv, K, V, N;
  const int64_t *cu;
} dims_t;

static void unit_range(const dims_t *d, int n, int64_t *tok0, int64_t *len) {
  if (d->cu) {
    *tok0 = d->cu[n];
    *len = d->cu[n + 1] - d->cu[n];
  } else {
    *tok0 = (int64_t)n * d->T;
    *len = d->T;
  }
}

/* One forward token step on state S (K x V, row-major).  Writes o (may be
 * NULL).  Uses scratch p (V). */
static void token_fwd(int K, int V, double *S, const double *q, const double *k,
                      const double *v, double g, double beta, double scale,
                      double *o, double *p) {
  const double a = exp(g);
  for (int j = 0; j < V; ++j) p[j] = 0.0;
  for (int i = 0; i < K; ++i) {
    double *Si = S + (size_t)i * V;
    const double ki = k[i];
    for (int j = 0; j < V; ++j) {
      Si[j] *= a;
      p[j] += Si[j] * ki;
    }
  }
  for (int j = 0; j < V; ++j) p[j] = beta * (v[j] - p[j]); /* p := delta */
  if (o)
    for (int j = 0; j < V; ++j) o[j] = 0.0;
  for (int i = 0; i < K; ++i) {
    double *Si = S + (size_t)i * V;
    const double ki = k[i];
    const double qi = q ? q[i] : 0.0;
    for (int j = 0; j < V; ++j) {
      Si[j] += ki * p[j];
      if (o) o[j] += Si[j] * qi;
    }
  }
  if (o)
    for (int j = 0; j < V; ++j) o[j] *= scale;
}

int gdn_oracle_fwd(int B, int T, int Hq, int Hv, int K, int V, int N,
                   const int64_t *cu_seqlens, const double *q, const double *k,
                   const double *v, const double *g, const double *beta,
                   double scale, const double *h0, double *o, double *ht,
                   const uint8_t *unit_mask, int nthreads) {
  if (Hq <= 0 || Hv <= 0 || Hv % Hq != 0 || K <= 0 || V <= 0) return 1;
  dims_t d = {B, T, Hq, Hv, K, V, N, cu_seqlens};
  const int grp = Hv / Hq;
  const int units = N * Hv;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double *S = (double *)malloc(sizeof(double) * (size_t)K * V);
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int u = 0; u < units; ++u) {
      if (unit_mask && !unit_mask[u]) continue;
      const int n = u / Hv, h = u % Hv, hq = h / grp;
      int64_t tok0, len;
      unit_range(&d, n, &tok0, &len);
      if (h0)
        memcpy(S, h0 + (size_t)u * K * V, sizeof(double) * (size_t)K * V);
      else
        memset(S, 0, sizeof(double) * (size_t)K * V);
      for (int64_t t = tok0; t < tok0 + len; ++t) {
        const double *qt = q + ((size_t)t * Hq + hq) * K;
        const double *kt = k + ((size_t)t * Hq + hq) * K;
        const double *vt = v + ((size_t)t * Hv + h) * V;
        const size_t gi = (size_t)t * Hv + h;
        double *ot = o ? o + ((size_t)t * Hv + h) * V : NULL;
        token_fwd(K, V, S, qt, kt, vt, g[gi], beta[gi], scale, ot, p);
      }
      if (ht) memcpy(ht + (size_t)u * K * V, S, sizeof(double) * (size_t)K * V);
    }
    free(S);
    free(p);
  }
  return 0;
}

int gdn_oracle_bwd(int B, int T, int Hq, int Hv, int K, int V, int N,
                   const int64_t *cu_seqlens, const double *q, const double *k,
                   const double *v, const double *g, const double *beta,
                   double scale, const double *h0, const double *dout,
                   const double *dht, double *dq, double *dk, double *dv,
                   double *dbeta, double *dg, double *dh0,
                   const uint8_t *unit_mask, int nthreads) {
  if (Hq <= 0 || Hv <= 0 || Hv % Hq != 0 || K <= 0 || V <= 0) return 1;
  dims_t d = {B, T, Hq, Hv, K, V, N, cu_seqlens};
  const int grp = Hv / Hq;
  const int units = N * Hv;
  int64_t total_tokens = cu_seqlens ? cu_seqlens[N] : (int64_t)B * T;
  const size_t KV = (size_t)K * V;
  /* per-v-head dq / dk, reduced over each group afterwards */
  double *dqv = (double *)calloc((size_t)total_tokens * Hv * K, sizeof(double));
  double *dkv = (double *)calloc((size_t)total_tokens * Hv * K, sizeof(double));
  if (!dqv || !dkv) {
    free(dqv);
    free(dkv);
    return 2;
  }
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double *S = (double *)malloc(sizeof(double) * KV);
    double *dS = (double *)malloc(sizeof(double) * KV);
    double *win = (double *)malloc(sizeof(double) * KV * (CKPT + 1));
    double *p = (double *)malloc(sizeof(double) * V);
    double *dd = (double *)malloc(sizeof(double) * V);
    double *dp = (double *)malloc(sizeof(double) * V);
    double *ck = NULL;
    size_t ck_cap = 0;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int u = 0; u < units; ++u) {
      if (unit_mask && !unit_mask[u]) continue;
      const int n = u / Hv, h = u % Hv, hq = h / grp;
      int64_t tok0, len;
      unit_range(&d, n, &tok0, &len);
      const int64_t nck = (len + CKPT - 1) / CKPT;
      if ((size_t)(nck + 1) > ck_cap) {
        free(ck);
        ck_cap = (size_t)nck + 1;
        ck = (double *)malloc(sizeof(double) * KV * ck_cap);
      }
      /* forward sweep, checkpoint the state entering every window */
      if (h0)
        memcpy(S, h0 + (size_t)u * KV, sizeof(double) * KV);
      else
        memset(S, 0, sizeof(double) * KV);
      for (int64_t c = 0; c < nck; ++c) {
        memcpy(ck + (size_t)c * KV, S, sizeof(double) * KV);
        const int64_t a0 = tok0 + c * CKPT;
        const int64_t a1 = (c + 1) * CKPT < len ? a0 + CKPT : tok0 + len;
        for (int64_t t = a0; t < a1; ++t) {
          const size_t gi = (size_t)t * Hv + h;
          token_fwd(K, V, S, NULL, k + ((size_t)t * Hq + hq) * K,
                    v + ((size_t)t * Hv + h) * V, g[gi], beta[gi], scale, NULL,
                    p);
        }
      }
      /* reverse sweep */
      if (dht)
        memcpy(dS, dht + (size_t)u * KV, sizeof(double) * KV);
      else
        memset(dS, 0, sizeof(double) * KV);
      for (int64_t c = nck - 1; c >= 0; --c) {
        const int64_t a0 = tok0 + c * CKPT;
        const int64_t a1 = (c + 1) * CKPT < len ? a0 + CKPT : tok0 + len;
        const int64_t wl = a1 - a0;
        /* win[i] = state before token a0+i (i = 0..wl) */
        memcpy(win, ck + (size_t)c * KV, sizeof(double) * KV);
        for (int64_t i = 0; i < wl; ++i) {
          const int64_t t = a0 + i;
          const size_t gi = (size_t)t * Hv + h;
          memcpy(win + (size_t)(i + 1) * KV, win + (size_t)i * KV,
                 sizeof(double) * KV);
          token_fwd(K, V, win + (size_t)(i + 1) * KV, NULL,
                    k + ((size_t)t * Hq + hq) * K,
                    v + ((size_t)t * Hv + h) * V, g[gi], beta[gi], scale, NULL,
                    p);
        }
        for (int64_t i = wl - 1; i >= 0; --i) {
          const int64_t t = a0 + i;
          const size_t gi = (size_t)t * Hv + h;
          const double *qt = q + ((size_t)t * Hq + hq) * K;
          const double *kt = k + ((size_t)t * Hq + hq) * K;
          const double *vt = v + ((size_t)t * Hv + h) * V;
          const double *dot = dout + ((size_t)t * Hv + h) * V;
          const double *Sp = win + (size_t)i * KV;      /* S_{t-1} */
          const double *St = win + (size_t)(i + 1) * KV; /* S_t */
          const double a = exp(g[gi]), bt = beta[gi];
          double *dqt = dqv + ((size_t)t * Hv + h) * K;
          double *dkt = dkv + ((size_t)t * Hv + h) * K;
          /* o_t = scale S_t^T q_t */
          for (int r = 0; r < K; ++r) {
            double acc = 0.0;
            const double *Sr = St + (size_t)r * V;
            for (int j = 0; j < V; ++j) acc += Sr[j] * dot[j];
            dqt[r] = scale * acc;
          }
          for (int r = 0; r < K; ++r) {
            double *dSr = dS + (size_t)r * V;
            const double sq = scale * qt[r];
            for (int j = 0; j < V; ++j) dSr[j] += sq * dot[j];
          }
          /* recompute p = S~^T k with S~ = a S_{t-1}, and delta */
          for (int j = 0; j < V; ++j) p[j] = 0.0;
          for (int r = 0; r < K; ++r) {
            const double *Sr = Sp + (size_t)r * V;
            const double kr = a * kt[r];
            for (int j = 0; j < V; ++j) p[j] += Sr[j] * kr;
          }
          /* S_t = S~ + k delta^T:  dk = dS delta,  d(delta) = dS^T k */
          for (int j = 0; j < V; ++j) dd[j] = 0.0;
          for (int r = 0; r < K; ++r) {
            const double *dSr = dS + (size_t)r * V;
            double acc = 0.0;
            const double kr = kt[r];
            for (int j = 0; j < V; ++j) {
              const double delta = bt * (vt[j] - p[j]);
              acc += dSr[j] * delta;
              dd[j] += dSr[j] * kr;
            }
            dkt[r] = acc;
          }
          /* delta = beta (v - p) */
          double db = 0.0;
          double *dvt = dv + ((size_t)t * Hv + h) * V;
          for (int j = 0; j < V; ++j) {
            db += dd[j] * (vt[j] - p[j]);
            dvt[j] = bt * dd[j];
            dp[j] = -bt * dd[j];
          }
          dbeta[gi] = db;
          /* p = S~^T k:  dS~ = dS + k dp^T,  dk += S~ dp */
          for (int r = 0; r < K; ++r) {
            const double *Sr = Sp + (size_t)r * V;
            double acc = 0.0;
            for (int j = 0; j < V; ++j) acc += Sr[j] * dp[j];
            dkt[r] += a * acc;
          }
          double dga = 0.0;
          for (int r = 0; r < K; ++r) {
            double *dSr = dS + (size_t)r * V;
            const double *Sr = Sp + (size_t)r * V;
            const double kr = kt[r];
            for (int j = 0; j < V; ++j) {
              const double dst = dSr[j] + kr * dp[j];
              dga += dst * (a * Sr[j]); /* <dS~, S~> */
              dSr[j] = a * dst;         /* S~ = a S_{t-1} */
            }
          }
          dg[gi] = dga;
        }
      }
      if (dh0) memcpy(dh0 + (size_t)u * KV, dS, sizeof(double) * KV);
    }
    free(S);
    free(dS);
    free(win);
    free(p);
    free(dd);
    free(dp);
    free(ck);
  }
  /* group reduction of dq, dk over selected v-heads, fixed order */
  for (int n = 0; n < N; ++n) {
    int64_t tok0, len;
    unit_range(&d, n, &tok0, &len);
    for (int hq = 0; hq < Hq; ++hq) {
      int any = 0;
      for (int h = hq * grp; h < (hq + 1) * grp; ++h)
        if (!unit_mask || unit_mask[n * Hv + h]) any = 1;
      if (!any) continue;
      for (int64_t t = tok0; t < tok0 + len; ++t) {
        double *dqt = dq + ((size_t)t * Hq + hq) * K;
        double *dkt = dk + ((size_t)t * Hq + hq) * K;
        for (int r = 0; r < K; ++r) {
          dqt[r] = 0.0;
          dkt[r] = 0.0;
        }
        for (int h = hq * grp; h < (hq + 1) * grp; ++h) {
          if (unit_mask && !unit_mask[n * Hv + h]) continue;
          const double *a = dqv + ((size_t)t * Hv + h) * K;
          const double *b = dkv + ((size_t)t * Hv + h) * K;
          for (int r = 0; r < K; ++r) {
            dqt[r] += a[r];
            dkt[r] += b[r];
          }
        }
      }
    }
  }
  free(dqv);
  free(dkv);
  return 0;
}

int gdn_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
