/*
 * la_oracle.c -- plain fp64 CPU oracle for the Lightning Attention layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP path.
 *
 * What is computed.  The Ling & Ring 2.6 Technical Report pages ("Hybrid
 * Linear Attention: Balancing Long-Context Efficiency and Model Quality")
 * describe Lightning Attention as sequence mixing of O(n) cost with a
 * recursive dependency along the sequence ("Long-Context Training: Context
 * Parallel for Lightning Attention": per-shard hidden states combined by local
 * recursion plus a global correction).  The pages never print the formula; the
 * reading used here (decayed causal linear attention) is
 *
 *     lambda_h = exp(-s_h)                       (per-head decay)
 *     S_t      = lambda S_{t-1} + k_t v_t^T      (S_{-1} = S0, d_k x d_v)
 *     o_t      = q_t^T S_t,  i.e.  o_t[j] = sum_i q_t[i] S_t[i][j]
 *
 * which equals o_t = sum_{s<=t} lambda^(t-s) (q_t . k_s) v_s + lambda^(t+1) q_t^T S0.
 * Every function below evaluates that definition one token at a time (the
 * recurrent form), in double precision, over independent (b, h) pairs.
 *
 * Layouts (row-major, contiguous):
 *   q, k, v, o, dout, dq, dk, dv : [B][H][N][d]
 *   state, S0, S_out             : [B][H][d][d]   (S[i][j], i = key feature)
 *   slope                        : [H], fp32 as handed to the GPU; the decay
 *                                  is exp(-(double)slope[h]).
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#define IDX4(b, h, t, i, H, N, d) ((((size_t)(b) * (H) + (h)) * (N) + (t)) * (d) + (i))

/* Forward, recurrent.  S0 may be NULL (zero state); S_out may be NULL. */
void lao_fwd(int B, int H, int N, int d, const double *q, const double *k,
             const double *v, const float *slope, const double *S0, double *o,
             double *S_out) {
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      const double lam = exp(-(double)slope[h]);
      double *S = (double *)malloc(sizeof(double) * (size_t)d * d);
      const size_t sb = ((size_t)b * H + h) * (size_t)d * d;
      if (S0)
        memcpy(S, S0 + sb, sizeof(double) * (size_t)d * d);
      else
        memset(S, 0, sizeof(double) * (size_t)d * d);
      for (int t = 0; t < N; ++t) {
        const double *qt = q + IDX4(b, h, t, 0, H, N, d);
        const double *kt = k + IDX4(b, h, t, 0, H, N, d);
        const double *vt = v + IDX4(b, h, t, 0, H, N, d);
        double *ot = o + IDX4(b, h, t, 0, H, N, d);
        /* S <- lambda S + k_t v_t^T */
        for (int i = 0; i < d; ++i)
          for (int j = 0; j < d; ++j)
            S[(size_t)i * d + j] = lam * S[(size_t)i * d + j] + kt[i] * vt[j];
        /* o_t = q_t^T S */
        for (int j = 0; j < d; ++j) ot[j] = 0.0;
        for (int i = 0; i < d; ++i)
          for (int j = 0; j < d; ++j) ot[j] += qt[i] * S[(size_t)i * d + j];
      }
      if (S_out) memcpy(S_out + sb, S, sizeof(double) * (size_t)d * d);
      free(S);
    }
  }
}

/* One decode step on a carried state: S <- lambda S + k v^T, then o = q^T S.
 * q, k, v, o : [B][H][d];  state : [B][H][d][d], updated in place. */
void lao_decode(int B, int H, int d, const double *q, const double *k,
                const double *v, const float *slope, double *state, double *o) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      const double lam = exp(-(double)slope[h]);
      double *S = state + ((size_t)b * H + h) * (size_t)d * d;
      const double *qb = q + ((size_t)b * H + h) * d;
      const double *kb = k + ((size_t)b * H + h) * d;
      const double *vb = v + ((size_t)b * H + h) * d;
      double *ob = o + ((size_t)b * H + h) * d;
      for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j)
          S[(size_t)i * d + j] = lam * S[(size_t)i * d + j] + kb[i] * vb[j];
      for (int j = 0; j < d; ++j) ob[j] = 0.0;
      for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) ob[j] += qb[i] * S[(size_t)i * d + j];
    }
  }
}

/* Backward of L = sum_t o_t . dout_t with respect to q, k, v (no gradient
 * flows into S0 or lambda).  S0 may be NULL.
 *   forward sweep : rebuild S_t, dq_t = S_t dout_t      (dq_t[i] = sum_j S_t[i][j] dout_t[j])
 *   reverse sweep : G <- lambda G + q_t dout_t^T, then
 *                   dk_t = G v_t  (dk_t[i] = sum_j G[i][j] v_t[j])
 *                   dv_t = G^T k_t (dv_t[j] = sum_i G[i][j] k_t[i])
 * G_t = sum_{u>=t} lambda^(u-t) q_u dout_u^T is the adjoint of S_t. */
void lao_bwd(int B, int H, int N, int d, const double *q, const double *k,
             const double *v, const double *dout, const float *slope,
             const double *S0, double *dq, double *dk, double *dv) {
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      const double lam = exp(-(double)slope[h]);
      double *S = (double *)malloc(sizeof(double) * (size_t)d * d);
      const size_t sb = ((size_t)b * H + h) * (size_t)d * d;
      if (S0)
        memcpy(S, S0 + sb, sizeof(double) * (size_t)d * d);
      else
        memset(S, 0, sizeof(double) * (size_t)d * d);
      for (int t = 0; t < N; ++t) {
        const double *kt = k + IDX4(b, h, t, 0, H, N, d);
        const double *vt = v + IDX4(b, h, t, 0, H, N, d);
        const double *gt = dout + IDX4(b, h, t, 0, H, N, d);
        double *dqt = dq + IDX4(b, h, t, 0, H, N, d);
        for (int i = 0; i < d; ++i)
          for (int j = 0; j < d; ++j)
            S[(size_t)i * d + j] = lam * S[(size_t)i * d + j] + kt[i] * vt[j];
        for (int i = 0; i < d; ++i) {
          double acc = 0.0;
          for (int j = 0; j < d; ++j) acc += S[(size_t)i * d + j] * gt[j];
          dqt[i] = acc;
        }
      }
      double *G = S; /* reuse the buffer for the adjoint state */
      memset(G, 0, sizeof(double) * (size_t)d * d);
      for (int t = N - 1; t >= 0; --t) {
        const double *qt = q + IDX4(b, h, t, 0, H, N, d);
        const double *kt = k + IDX4(b, h, t, 0, H, N, d);
        const double *vt = v + IDX4(b, h, t, 0, H, N, d);
        const double *gt = dout + IDX4(b, h, t, 0, H, N, d);
        double *dkt = dk + IDX4(b, h, t, 0, H, N, d);
        double *dvt = dv + IDX4(b, h, t, 0, H, N, d);
        for (int i = 0; i < d; ++i)
          for (int j = 0; j < d; ++j)
            G[(size_t)i * d + j] = lam * G[(size_t)i * d + j] + qt[i] * gt[j];
        for (int i = 0; i < d; ++i) {
          double acc = 0.0;
          for (int j = 0; j < d; ++j) acc += G[(size_t)i * d + j] * vt[j];
          dkt[i] = acc;
        }
        for (int j = 0; j < d; ++j) dvt[j] = 0.0;
        for (int i = 0; i < d; ++i)
          for (int j = 0; j < d; ++j) dvt[j] += G[(size_t)i * d + j] * kt[i];
      }
      free(S);
    }
  }
}

/* Forward in the chunked order (chunk length C; the last chunk may be short).
 * Within chunk c starting at token t0 with n rows (local index i, j):
 *   o_i   = sum_{j<=i} lambda^(i-j) (q_i . k_j) v_j + lambda^(i+1) q_i^T S_prev
 *   S_new = lambda^n S_prev + sum_j lambda^(n-1-j) k_j v_j^T
 * This is only another evaluation order of the same definition; it exists so
 * that the tests can check that chunked, recurrent and quadratic forms agree.
 * Every power of lambda is exp(-s * exponent), never a repeated product. */
void lao_fwd_chunked(int B, int H, int N, int d, int C, const double *q,
                     const double *k, const double *v, const float *slope,
                     const double *S0, double *o, double *S_out) {
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      const double s = (double)slope[h];
      double *S = (double *)malloc(sizeof(double) * (size_t)d * d);
      double *Snew = (double *)malloc(sizeof(double) * (size_t)d * d);
      const size_t sb = ((size_t)b * H + h) * (size_t)d * d;
      if (S0)
        memcpy(S, S0 + sb, sizeof(double) * (size_t)d * d);
      else
        memset(S, 0, sizeof(double) * (size_t)d * d);
      for (int t0 = 0; t0 < N; t0 += C) {
        const int n = (N - t0 < C) ? (N - t0) : C;
        for (int i = 0; i < n; ++i) {
          const double *qi = q + IDX4(b, h, t0 + i, 0, H, N, d);
          double *oi = o + IDX4(b, h, t0 + i, 0, H, N, d);
          for (int jj = 0; jj < d; ++jj) oi[jj] = 0.0;
          /* intra-chunk: masked scores times V */
          for (int j = 0; j <= i; ++j) {
            const double *kj = k + IDX4(b, h, t0 + j, 0, H, N, d);
            const double *vj = v + IDX4(b, h, t0 + j, 0, H, N, d);
            double sc = 0.0;
            for (int x = 0; x < d; ++x) sc += qi[x] * kj[x];
            sc *= exp(-s * (double)(i - j));
            for (int jj = 0; jj < d; ++jj) oi[jj] += sc * vj[jj];
          }
          /* inter-chunk: the carried state, decayed to row i */
          const double a = exp(-s * (double)(i + 1));
          for (int x = 0; x < d; ++x)
            for (int jj = 0; jj < d; ++jj)
              oi[jj] += a * qi[x] * S[(size_t)x * d + jj];
        }
        /* state update */
        const double g = exp(-s * (double)n);
        for (int x = 0; x < d * d; ++x) Snew[x] = g * S[x];
        for (int j = 0; j < n; ++j) {
          const double bj = exp(-s * (double)(n - 1 - j));
          const double *kj = k + IDX4(b, h, t0 + j, 0, H, N, d);
          const double *vj = v + IDX4(b, h, t0 + j, 0, H, N, d);
          for (int x = 0; x < d; ++x)
            for (int jj = 0; jj < d; ++jj)
              Snew[(size_t)x * d + jj] += bj * kj[x] * vj[jj];
        }
        double *tmp = S;
        S = Snew;
        Snew = tmp;
      }
      if (S_out) memcpy(S_out + sb, S, sizeof(double) * (size_t)d * d);
      free(S);
      free(Snew);
    }
  }
}

int lao_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
