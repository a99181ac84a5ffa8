/*
 * fp64 CPU oracle for the Kimi Delta Attention (KDA) core.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this library.  The HIP library never links, includes
 * or calls anything here, and this file includes nothing of the HIP library.
 *
 * What it computes (plain definitions, written out; no blocking, no chunking):
 *
 *   Gate.  Per token t, head h, key channel c:
 *       g[t,h,c]  = -exp(A_log[h]) * softplus(x[t,h,c] + dt_bias[h,c])
 *       beta[t,h] = 1 / (1 + exp(-b[t,h]))
 *   A_log is one value per head and dt_bias one per (head, channel)
 *   (Kimi K3 artifact audit, §4.1 KDA tensor table and §5.2 shape table:
 *   dt_bias [12288] = [96,128], A_log [H]); beta is a sigmoid taken in full
 *   precision (Model-Optimizer PR #2749 review, the KDA beta fix).
 *   softplus(z) = max(z,0) + log1p(exp(-|z|)).
 *
 *   Recurrence.  Kimi Delta Attention is the per-channel gated delta rule
 *       S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *       o_t = scale * S_t^T q_t,      alpha_t = exp(g_t),
 *   with S a d_k x d_v matrix per (sequence, head), S[c][j] (c key channel,
 *   j value channel).  The code audit page (finding "dual-kda-execution-
 *   regimes") names its two execution forms, chunked for prefill and fused
 *   recurrent for one-token decode; this oracle is the token-by-token form
 *   that both must equal.  Order inside one step: decay first, then the
 *   delta correction against the decayed state, then the readout of the
 *   updated state.
 *
 *   Varlen.  Sequences are packed along the token axis; cu[n]..cu[n+1]-1 are
 *   the tokens of sequence n.  A missing initial state means zeros.
 *
 * Layouts (row-major, last index fastest): q,k,g [T,H,dk]; v,o [T,H,dv];
 * beta [T,H]; states [N,H,dk,dv].  All arithmetic is fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double softplus(double z) { return fmax(z, 0.0) + log1p(exp(-fabs(z))); }

void kdao_gate(int64_t n_tok, int32_t H, int32_t d, const double* x, const double* b,
               const double* A_log, int32_t a_per_channel, const double* dt_bias, double* g,
               double* beta) {
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int32_t h = 0; h < H; ++h) {
      for (int32_t c = 0; c < d; ++c) {
        const int64_t i = (t * H + h) * (int64_t)d + c;
        /* A_log per head [H], or per (head, channel) [H, d] */
        const double a = exp(a_per_channel ? A_log[(int64_t)h * d + c] : A_log[h]);
        g[i] = -a * softplus(x[i] + dt_bias[(int64_t)h * d + c]);
      }
      beta[t * H + h] = 1.0 / (1.0 + exp(-b[t * H + h]));
    }
  }
}

/* One step of the recurrence on S (dk x dv) for one token of one head. */
static void step(int32_t dk, int32_t dv, double* S, double* e, const double* q,
                 const double* k, const double* v, const double* g, double beta,
                 double scale, double* o) {
  for (int32_t c = 0; c < dk; ++c) {          /* S <- Diag(alpha) S */
    const double a = exp(g[c]);
    for (int32_t j = 0; j < dv; ++j) S[(int64_t)c * dv + j] *= a;
  }
  for (int32_t j = 0; j < dv; ++j) e[j] = v[j]; /* e <- v - S^T k */
  for (int32_t c = 0; c < dk; ++c)
    for (int32_t j = 0; j < dv; ++j) e[j] -= k[c] * S[(int64_t)c * dv + j];
  for (int32_t c = 0; c < dk; ++c) {          /* S <- S + beta k e^T */
    const double kb = beta * k[c];
    for (int32_t j = 0; j < dv; ++j) S[(int64_t)c * dv + j] += kb * e[j];
  }
  for (int32_t j = 0; j < dv; ++j) o[j] = 0.0; /* o <- scale S^T q */
  for (int32_t c = 0; c < dk; ++c)
    for (int32_t j = 0; j < dv; ++j) o[j] += q[c] * S[(int64_t)c * dv + j];
  for (int32_t j = 0; j < dv; ++j) o[j] *= scale;
}

/* Returns the number of threads the parallel region used. */
int32_t kdao_prefill(int32_t N, const int32_t* cu, int32_t H, int32_t dk, int32_t dv,
                     const double* q, const double* k, const double* v, const double* g,
                     const double* beta, double scale, const double* S0, double* o,
                     double* S_final, int32_t nthreads) {
  int32_t used = 1;
  const int64_t pairs = (int64_t)N * H;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
#ifdef _OPENMP
#pragma omp single
    used = omp_get_num_threads();
#endif
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* e = (double*)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
      const int32_t n = (int32_t)(p / H), h = (int32_t)(p % H);
      const int64_t sidx = p * (int64_t)dk * dv;
      if (S0) memcpy(S, S0 + sidx, sizeof(double) * (size_t)dk * dv);
      else memset(S, 0, sizeof(double) * (size_t)dk * dv);
      for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
        const int64_t r = t * H + h;
        step(dk, dv, S, e, q + r * dk, k + r * dk, v + r * dv, g + r * dk, beta[r], scale,
             o + r * dv);
      }
      if (S_final) memcpy(S_final + sidx, S, sizeof(double) * (size_t)dk * dv);
    }
    free(S);
    free(e);
  }
  return used;
}

/* One decode step: one token per sequence, state updated in place. */
int32_t kdao_decode(int32_t N, int32_t H, int32_t dk, int32_t dv, const double* q,
                    const double* k, const double* v, const double* g, const double* beta,
                    double scale, double* S, double* o, int32_t nthreads) {
  int32_t used = 1;
  const int64_t pairs = (int64_t)N * H;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
#ifdef _OPENMP
#pragma omp single
    used = omp_get_num_threads();
#endif
    double* e = (double*)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(static)
    for (int64_t p = 0; p < pairs; ++p) {
      step(dk, dv, S + p * (int64_t)dk * dv, e, q + p * dk, k + p * dk, v + p * dv,
           g + p * dk, beta[p], scale, o + p * dv);
    }
    free(e);
  }
  return used;
}
