/*
 * kda_oracle.c -- plain fp64 CPU oracle for the Kimi Delta Attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or constant with the GPU library and never calls it.
 *
 * What it computes (one function per passage):
 *
 *  kda_oracle_gate -- the bounded gate of "Kimi K3 模型结构（2）：序列维度（下）",
 *      section "K3 的改动：下界衰减", equation (5):
 *          g = g_min * Sigmoid(exp(A_h) * z),   alpha = exp(g).
 *      A_h is one scalar per head; z and g are per key channel.
 *
 *  kda_oracle_gate_softplus -- the unbounded gate that the same section gives
 *      for Kimi Linear (as in GDN and Mamba-2), the map the bound replaces:
 *          g = -exp(A_h) * Softplus(z),   Softplus(z) = log(1 + exp(z)),
 *      so g ranges over (-inf, 0) with no lower bound.
 *
 *  kda_oracle_recurrent -- the token recurrence of "Kimi K3 模型结构（7）：
 *      结构决定系统", section "KDA 上下文并行", equation (1):
 *          S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *      evaluated in the equivalent delta form printed on the SemiAnalysis page
 *      "Kimi K3 ...", section "FlashKDA 算法 / 算法":
 *          u_t = beta_t (v_t - (D_t S_{t-1})^T k_t),
 *          S_t = D_t S_{t-1} + k_t u_t^T,
 *          o_t = S_t^T q_t          (the output reads the state after the update),
 *      with D_t = Diag(alpha_t).  Each packed document (cu_seqlens) starts from
 *      its own initial state (zero if none is given); the state is reset at
 *      document starts as stated in the systems page, section "文档边界".
 *
 *  The state S is d_k x d_v, row i = key channel i.  Columns of S never
 *  interact in the update, so the loops run (document, head) in parallel.
 *  Everything is double precision; inputs are the exact values the GPU reads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* g[t,h,c] = g_min * sigmoid(exp(A_log[h]) * z[t,h,c]); A_log may be NULL (= 0). */
void kda_oracle_gate(const double *z, const double *A_log, double g_min, int64_t T,
                     int32_t H, int32_t dk, double *g) {
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t h = 0; h < H; ++h) {
      const double scale = exp(A_log ? A_log[h] : 0.0);
      const double *zr = z + (t * H + h) * (int64_t)dk;
      double *gr = g + (t * H + h) * (int64_t)dk;
      for (int32_t c = 0; c < dk; ++c) {
        const double x = scale * zr[c];
        gr[c] = g_min * (1.0 / (1.0 + exp(-x)));
      }
    }
  }
}

/* g[t,h,c] = -exp(A_log[h]) * softplus(z[t,h,c]); A_log may be NULL (= 0).
 * softplus(x) is evaluated as max(x, 0) + log1p(exp(-|x|)), which equals
 * log(1 + exp(x)) and never overflows. */
void kda_oracle_gate_softplus(const double *z, const double *A_log, int64_t T, int32_t H,
                              int32_t dk, double *g) {
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t h = 0; h < H; ++h) {
      const double scale = exp(A_log ? A_log[h] : 0.0);
      const double *zr = z + (t * H + h) * (int64_t)dk;
      double *gr = g + (t * H + h) * (int64_t)dk;
      for (int32_t c = 0; c < dk; ++c) {
        const double x = zr[c];
        const double sp = (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
        gr[c] = -scale * sp;
      }
    }
  }
}

/*
 * One (document, head): run tokens [t0, t1) from the state in S (d_k x d_v,
 * row-major, updated in place).  g is the per-step log-decay (alpha = exp(g)).
 * Writes o rows for the same tokens.
 */
static void recur_one(const double *q, const double *k, const double *v, const double *g,
                      const double *beta, int64_t t0, int64_t t1, int32_t H, int32_t h,
                      int32_t dk, int32_t dv, double *S, double *o, double *u) {
  for (int64_t t = t0; t < t1; ++t) {
    const int64_t row = t * H + h;
    const double *qt = q + row * dk;
    const double *kt = k + row * dk;
    const double *vt = v + row * dv;
    const double *gt = g + row * dk;
    const double bt = beta[row];
    /* decay first: S <- Diag(alpha_t) S */
    for (int32_t i = 0; i < dk; ++i) {
      const double a = exp(gt[i]);
      double *Si = S + (int64_t)i * dv;
      for (int32_t j = 0; j < dv; ++j) Si[j] *= a;
    }
    /* u = beta (v - S^T k), against the decayed state */
    for (int32_t j = 0; j < dv; ++j) u[j] = 0.0;
    for (int32_t i = 0; i < dk; ++i) {
      const double ki = kt[i];
      const double *Si = S + (int64_t)i * dv;
      for (int32_t j = 0; j < dv; ++j) u[j] += Si[j] * ki;
    }
    for (int32_t j = 0; j < dv; ++j) u[j] = bt * (vt[j] - u[j]);
    /* erase-and-write: S <- S + k u^T */
    for (int32_t i = 0; i < dk; ++i) {
      const double ki = kt[i];
      double *Si = S + (int64_t)i * dv;
      for (int32_t j = 0; j < dv; ++j) Si[j] += ki * u[j];
    }
    /* o_t = S_t^T q_t */
    double *ot = o + row * dv;
    for (int32_t j = 0; j < dv; ++j) ot[j] = 0.0;
    for (int32_t i = 0; i < dk; ++i) {
      const double qi = qt[i];
      const double *Si = S + (int64_t)i * dv;
      for (int32_t j = 0; j < dv; ++j) ot[j] += Si[j] * qi;
    }
  }
}

/*
 * q,k,g: [T, H, dk]; v: [T, H, dv]; beta: [T, H]; all double.
 * cu_seqlens: [N+1] document offsets (cu[0] = 0, cu[N] = T).
 * S0: [N, H, dk, dv] or NULL (zero initial states).
 * o: [T, H, dv] (written); S_final: [N, H, dk, dv] or NULL.
 * nthreads <= 0 lets OpenMP decide.  Returns 0 on success, -1 on bad input.
 */
int kda_oracle_recurrent(const double *q, const double *k, const double *v, const double *g,
                         const double *beta, const double *S0, const int32_t *cu_seqlens,
                         int32_t N, int32_t H, int32_t dk, int32_t dv, double *o,
                         double *S_final, int32_t nthreads) {
  if (!q || !k || !v || !g || !beta || !cu_seqlens || !o || N < 0 || H <= 0 || dk <= 0 ||
      dv <= 0)
    return -1;
  if (cu_seqlens[0] != 0) return -1;
  for (int32_t n = 0; n < N; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  const int64_t SS = (int64_t)dk * dv;
  const int64_t units = (int64_t)N * H;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double *S = (double *)malloc(sizeof(double) * SS);
    double *u = (double *)malloc(sizeof(double) * dv);
    if (!S || !u) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      bad = 1;
    }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t w = 0; w < units; ++w) {
      if (!S || !u) continue;
      const int32_t n = (int32_t)(w / H), h = (int32_t)(w % H);
      if (S0)
        memcpy(S, S0 + w * SS, sizeof(double) * SS);
      else
        memset(S, 0, sizeof(double) * SS);
      recur_one(q, k, v, g, beta, cu_seqlens[n], cu_seqlens[n + 1], H, h, dk, dv, S, o, u);
      if (S_final) memcpy(S_final + w * SS, S, sizeof(double) * SS);
    }
    free(S);
    free(u);
  }
  return bad ? -1 : 0;
}

/* Number of OpenMP threads the recurrence would use (1 without OpenMP). */
int kda_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
