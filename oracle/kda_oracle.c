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

/*
 * Gradient of kdao_gate.  With z = x + dt_bias, a = exp(A_log) (per head or
 * per (head, channel)) and g = -a softplus(z), beta = sigmoid(b):
 *   dx = dg * (-a sigmoid(z)),  ddt_bias[h,c] = sum_t dx[t,h,c],
 *   dA_log = sum of dg * g over the entries that share the parameter,
 *   db = dbeta * beta (1 - beta).
 * dA_log has A_log's shape; ddt_bias is [H, d].
 */
void kdao_gate_backward(int64_t n_tok, int32_t H, int32_t d, const double* x, const double* b,
                        const double* A_log, int32_t a_per_channel, const double* dt_bias,
                        const double* dg, const double* dbeta, double* dx, double* db,
                        double* dA_log, double* ddt_bias) {
  memset(dA_log, 0, sizeof(double) * (size_t)(a_per_channel ? (int64_t)H * d : H));
  memset(ddt_bias, 0, sizeof(double) * (size_t)((int64_t)H * d));
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int32_t h = 0; h < H; ++h) {
      for (int32_t c = 0; c < d; ++c) {
        const int64_t i = (t * H + h) * (int64_t)d + c;
        const int64_t ai = a_per_channel ? (int64_t)h * d + c : h;
        const double a = exp(A_log[ai]);
        const double z = x[i] + dt_bias[(int64_t)h * d + c];
        const double sig = 1.0 / (1.0 + exp(-z));
        const double g = -a * softplus(z);
        dx[i] = dg[i] * (-a * sig);
        ddt_bias[(int64_t)h * d + c] += dx[i];
        dA_log[ai] += dg[i] * g;
      }
      const double be = 1.0 / (1.0 + exp(-b[t * H + h]));
      db[t * H + h] = dbeta[t * H + h] * be * (1.0 - be);
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

/*
 * Reverse-mode gradient of kdao_prefill (the same recurrence), written out
 * step by step.  For one token, with S' = Diag(exp(g)) S_prev,
 * e = v - S'^T k, S = S' + beta k e^T and o = scale S^T q, and dS the
 * gradient arriving at S (from later tokens, or dS_final at the end):
 *   dS     += scale q do^T;            dq  = scale S do
 *   dbeta   = k^T dS e;                de  = beta dS^T k;     dv = de
 *   dk      = beta dS e - S' de;       dS' = dS - k de^T
 *   dg[c]   = sum_j dS'[c,j] S'[c,j];  dS_prev = Diag(exp(g)) dS'
 * and dS after the first token is the gradient of the initial state.  The
 * states are recomputed forward from checkpoints taken every 64 tokens.
 * do, dS_final may be NULL (zero); dS0 may be NULL (not wanted).
 */
int32_t kdao_prefill_backward(int32_t N, const int32_t* cu, int32_t H, int32_t dk, int32_t dv,
                              const double* q, const double* k, const double* v,
                              const double* g, const double* beta, double scale,
                              const double* S0, const double* d_o, const double* dS_final,
                              double* dq, double* dk_out, double* dv_out, double* dg,
                              double* dbeta, double* dS0, int32_t nthreads) {
  enum { CK = 64 };
  int32_t used = 1;
  const int64_t pairs = (int64_t)N * H;
  const size_t SS = (size_t)dk * dv;
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
    double* de = (double*)malloc(sizeof(double) * (size_t)dv);
    double* otmp = (double*)malloc(sizeof(double) * (size_t)dv);
    double* dS = (double*)malloc(sizeof(double) * SS);
    double* Sp = (double*)malloc(sizeof(double) * SS);
    double* seg = (double*)malloc(sizeof(double) * SS * (CK + 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
      const int32_t n = (int32_t)(p / H), h = (int32_t)(p % H);
      const int64_t t0 = cu[n], L = cu[n + 1] - cu[n];
      const int64_t nck = (L + CK - 1) / CK;
      /* forward: the state before each segment of CK tokens */
      double* ck = (double*)malloc(sizeof(double) * SS * (size_t)(nck > 0 ? nck : 1));
      double* S = seg;
      if (S0) memcpy(S, S0 + p * SS, sizeof(double) * SS);
      else memset(S, 0, sizeof(double) * SS);
      for (int64_t t = 0; t < L; ++t) {
        if (t % CK == 0) memcpy(ck + (t / CK) * SS, S, sizeof(double) * SS);
        const int64_t r = (t0 + t) * H + h;
        step(dk, dv, S, e, q + r * dk, k + r * dk, v + r * dv, g + r * dk, beta[r], scale, otmp);
      }
      if (dS_final) memcpy(dS, dS_final + p * SS, sizeof(double) * SS);
      else memset(dS, 0, sizeof(double) * SS);
      for (int64_t b = nck - 1; b >= 0; --b) {
        const int64_t ta = b * CK, tb = (ta + CK < L) ? ta + CK : L;
        /* seg[i] = state before token ta + i, i = 0 .. tb - ta */
        memcpy(seg, ck + b * SS, sizeof(double) * SS);
        for (int64_t t = ta; t < tb; ++t) {
          const int64_t r = (t0 + t) * H + h;
          memcpy(seg + (t - ta + 1) * SS, seg + (t - ta) * SS, sizeof(double) * SS);
          step(dk, dv, seg + (t - ta + 1) * SS, e, q + r * dk, k + r * dk, v + r * dv,
               g + r * dk, beta[r], scale, otmp);
        }
        for (int64_t t = tb - 1; t >= ta; --t) {
          const int64_t r = (t0 + t) * H + h;
          const double* Sprev = seg + (t - ta) * SS;
          const double* Snew = seg + (t - ta + 1) * SS;
          const double* qt = q + r * dk;
          const double* kt = k + r * dk;
          const double* vt = v + r * dv;
          const double* gt = g + r * dk;
          const double bt = beta[r];
          const double* dot = d_o ? d_o + r * dv : NULL;
          /* o = scale S^T q */
          for (int32_t c = 0; c < dk; ++c) {
            double acc = 0.0;
            if (dot)
              for (int32_t j = 0; j < dv; ++j) acc += Snew[(int64_t)c * dv + j] * dot[j];
            dq[r * dk + c] = scale * acc;
            if (dot)
              for (int32_t j = 0; j < dv; ++j) dS[(int64_t)c * dv + j] += scale * qt[c] * dot[j];
          }
          /* S' = Diag(exp(g)) S_prev and e = v - S'^T k, recomputed */
          for (int32_t c = 0; c < dk; ++c) {
            const double a = exp(gt[c]);
            for (int32_t j = 0; j < dv; ++j) Sp[(int64_t)c * dv + j] = a * Sprev[(int64_t)c * dv + j];
          }
          for (int32_t j = 0; j < dv; ++j) {
            double acc = vt[j];
            for (int32_t c = 0; c < dk; ++c) acc -= kt[c] * Sp[(int64_t)c * dv + j];
            e[j] = acc;
          }
          /* S = S' + beta k e^T */
          double db = 0.0;
          for (int32_t c = 0; c < dk; ++c) {
            double dse = 0.0;
            for (int32_t j = 0; j < dv; ++j) dse += dS[(int64_t)c * dv + j] * e[j];
            db += kt[c] * dse;
            dk_out[r * dk + c] = bt * dse;
          }
          dbeta[r] = db;
          for (int32_t j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int32_t c = 0; c < dk; ++c) acc += dS[(int64_t)c * dv + j] * kt[c];
            de[j] = bt * acc;
            dv_out[r * dv + j] = de[j];
          }
          /* e = v - S'^T k:  dS' = dS - k de^T,  dk -= S' de */
          for (int32_t c = 0; c < dk; ++c) {
            double acc = 0.0;
            for (int32_t j = 0; j < dv; ++j) {
              acc += Sp[(int64_t)c * dv + j] * de[j];
              dS[(int64_t)c * dv + j] -= kt[c] * de[j];
            }
            dk_out[r * dk + c] -= acc;
          }
          /* S' = Diag(exp(g)) S_prev */
          for (int32_t c = 0; c < dk; ++c) {
            const double a = exp(gt[c]);
            double acc = 0.0;
            for (int32_t j = 0; j < dv; ++j) {
              acc += dS[(int64_t)c * dv + j] * Sp[(int64_t)c * dv + j];
              dS[(int64_t)c * dv + j] *= a;
            }
            dg[r * dk + c] = acc;
          }
        }
      }
      if (dS0) memcpy(dS0 + p * SS, dS, sizeof(double) * SS);
      free(ck);
    }
    free(e);
    free(de);
    free(otmp);
    free(dS);
    free(Sp);
    free(seg);
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
