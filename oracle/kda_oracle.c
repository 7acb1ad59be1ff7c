/*
 * kda_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU implementation of the Kimi Delta Attention (KDA)
 * recurrence, written to be checked by eye against the pages.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.  It
 * shares no code, header, table or helper with the GPU library, and the GPU
 * library never calls it.
 *
 * Source of the arithmetic: page "Kimi Delta Attention (KDA)" (brain.bigb.es),
 * the opening update equation and section "KDA: a separate gate per key
 * channel".  Per head, with a state S of shape d_v x d_k (it maps keys to
 * values, so key channels are the columns of S):
 *
 *   forget : S~_t = S_{t-1} Diag(alpha_t)        (alpha_t in [0,1]^{d_k})
 *   predict: vhat_t = S~_t k_t
 *   correct: e_t = beta_t (v_t - vhat_t)          (beta_t in [0,1])
 *   write  : S_t = S~_t + e_t k_t^T
 *   read   : o_t = scale * S_t q_t                (scale defaults to d_k^-1/2)
 *
 * Forget comes before predict (section "Gated DeltaNet: sometimes everything
 * must be erased" stresses the order), and the read happens after the write
 * (the same page's chunkwise section: a token sees its own write).
 *
 * Inputs are fp64 (callers upcast bf16 / fp32 exactly).  k is used exactly as
 * given: it is not renormalised.  alpha = 0 is allowed and clears a column.
 *
 * Readings of points the pages leave open:
 *  - layout: q,k,alpha [tokens, H, d_k], v [tokens, H, d_v], beta [tokens, H],
 *    state [units, H, d_v, d_k] row-major (d_k fastest);
 *  - packed variable-length batches: sequence n owns tokens
 *    [cu[n], cu[n+1]); no state flows between sequences.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* One token of the recurrence on one head.  S is d_v x d_k, row-major.
 * tmp must hold d_v doubles.  Writes the d_v outputs to o. */
static void kda_token(double *S, const double *q, const double *k,
                      const double *v, const double *alpha, double beta,
                      int dk, int dv, double scale, double *o, double *tmp) {
  /* forget: S~ = S Diag(alpha) scales column c by alpha[c] */
  for (int r = 0; r < dv; ++r)
    for (int c = 0; c < dk; ++c)
      S[(size_t)r * dk + c] *= alpha[c];

  /* predict: vhat = S~ k ; correct: e = beta (v - vhat) */
  for (int r = 0; r < dv; ++r) {
    double vhat = 0.0;
    for (int c = 0; c < dk; ++c)
      vhat += S[(size_t)r * dk + c] * k[c];
    tmp[r] = beta * (v[r] - vhat);
  }

  /* write: S = S~ + e k^T */
  for (int r = 0; r < dv; ++r)
    for (int c = 0; c < dk; ++c)
      S[(size_t)r * dk + c] += tmp[r] * k[c];

  /* read (after the write): o = scale * S q */
  for (int r = 0; r < dv; ++r) {
    double acc = 0.0;
    for (int c = 0; c < dk; ++c)
      acc += S[(size_t)r * dk + c] * q[c];
    o[r] = scale * acc;
  }
}

/*
 * Whole-sequence forward.
 *
 *   q, k, alpha : [Ttot, H, dk]     v : [Ttot, H, dv]     beta : [Ttot, H]
 *   S0          : [N, H, dv, dk] or NULL (zero state)
 *   cu_seqlens  : [N+1] token offsets, or NULL: then N sequences of T tokens
 *                 each, sequence n starting at token n*T (a dense [N, T] batch)
 *   o           : [Ttot, H, dv]     S_final : [N, H, dv, dk]
 *
 * Ttot = cu_seqlens[N] with offsets, else N*T.  scale <= 0 selects dk^-1/2.
 * Units (sequence, head) are independent and run in parallel with OpenMP when
 * n_threads > 1.  Returns 0, or -1 on a bad argument.
 */
int kda_oracle_fwd(const double *q, const double *k, const double *v,
                   const double *alpha, const double *beta, const double *S0,
                   const int64_t *cu_seqlens, int N, int T, int H, int dk,
                   int dv, double scale, double *o, double *S_final,
                   int n_threads) {
  if (N < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  if (!S_final) return -1;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)dk);
  const size_t sq = (size_t)dv * dk;
  int n_units = N * H;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
  for (int u = 0; u < n_units; ++u) {
    int n = u / H, h = u % H;
    int64_t t0, t1;
    if (cu_seqlens) { t0 = cu_seqlens[n]; t1 = cu_seqlens[n + 1]; }
    else { t0 = (int64_t)n * T; t1 = t0 + T; }
    double *S = S_final + ((size_t)n * H + h) * sq;
    if (S0) memcpy(S, S0 + ((size_t)n * H + h) * sq, sq * sizeof(double));
    else memset(S, 0, sq * sizeof(double));
    double *tmp = (double *)malloc((size_t)dv * sizeof(double));
    for (int64_t t = t0; t < t1; ++t) {
      size_t th = (size_t)t * H + h;
      kda_token(S, q + th * dk, k + th * dk, v + th * dv, alpha + th * dk,
                beta[th], dk, dv, scale, o + th * dv, tmp);
    }
    free(tmp);
  }
  return 0;
}

/*
 * One decode step for N independent sequences: each (n, h) state in S
 * ([N, H, dv, dk], updated in place) takes one token.
 *   q, k, alpha : [N, H, dk]   v : [N, H, dv]   beta : [N, H]   o : [N, H, dv]
 */
int kda_oracle_decode(const double *q, const double *k, const double *v,
                      const double *alpha, const double *beta, double *S,
                      int N, int H, int dk, int dv, double scale, double *o,
                      int n_threads) {
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !S) return -1;
  if (scale <= 0.0) scale = 1.0 / sqrt((double)dk);
  const size_t sq = (size_t)dv * dk;
  int n_units = N * H;
#pragma omp parallel for schedule(static) num_threads(n_threads > 0 ? n_threads : 1)
  for (int u = 0; u < n_units; ++u) {
    double *tmp = (double *)malloc((size_t)dv * sizeof(double));
    kda_token(S + (size_t)u * sq, q + (size_t)u * dk, k + (size_t)u * dk,
              v + (size_t)u * dv, alpha + (size_t)u * dk, beta[u], dk, dv,
              scale, o + (size_t)u * dv, tmp);
    free(tmp);
  }
  return 0;
}
