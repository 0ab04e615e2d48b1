/*
 * kda_c_consumer.c -- the C ABI of libkda.so driven from plain C11, with the
 * HIP runtime's C API for device memory and no Python or PyTorch in the
 * process.  It runs three calls on seeded synthetic inputs and checks each
 * against the fp64 CPU oracle (test infrastructure, oracle/kda_oracle.c):
 *
 *   1. kda_chunk_fwd, fp32 inputs (fp32 arithmetic): two packed documents with
 *      initial states;
 *   2. kda_chunk_fwd, bf16 inputs, with a caller-allocated workspace (the
 *      two-kernel path), on the same inputs rounded to bf16;
 *   3. kda_decode_step, fp32 inputs: replay of 0..4 accepted cached drafts
 *      plus the bonus token from saved states, checked as a recurrence over
 *      those tokens from the saved state (o of the bonus token, state after).
 *
 * Prints one line per check and exits 0 when every relative L2 error is
 * within its tolerance (fp32 arithmetic 1e-4, bf16 operands 1e-2), 1 when one
 * is not, 2 on an API or HIP error.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda.h"

/* fp64 oracle (oracle/kda_oracle.c) */
void kda_oracle_gate(const double *z, const double *A_log, double g_min, int64_t T, int32_t H,
                     int32_t dk, double *g);
int kda_oracle_recurrent(const double *q, const double *k, const double *v, const double *g,
                         const double *beta, const double *S0, const int32_t *cu_seqlens,
                         int32_t N, int32_t H, int32_t dk, int32_t dv, double *o,
                         double *S_final, int32_t nthreads);

#define D 128

/* splitmix64 -> uniform (0, 1) -> normal (Box-Muller) */
static uint64_t rng_state;
static double uniform01(void) {
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return ((double)(z >> 11) + 0.5) / 9007199254740992.0;
}
static double normal(void) {
  const double u = uniform01(), w = uniform01();
  return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * w);
}

/* round-to-nearest-even fp32 -> bf16 bits, and back */
static uint16_t to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float x;
  memcpy(&x, &u, 4);
  return x;
}

static int fail_hip(hipError_t e, const char *what) {
  fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  exit(2);
}
#define HIP(call) do { hipError_t e_ = (call); if (e_ != hipSuccess) fail_hip(e_, #call); } while (0)
#define KDA(call) do { int r_ = (call); if (r_ != KDA_OK) { \
    fprintf(stderr, "%s: %s (%s)\n", #call, kda_status_string(r_), kda_last_error()); exit(2); } } while (0)

static void *dev_copy(const void *h, size_t bytes) {
  void *d = NULL;
  HIP(hipMalloc(&d, bytes));
  HIP(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  return d;
}
static void *dev_alloc(size_t bytes) {
  void *d = NULL;
  HIP(hipMalloc(&d, bytes));
  return d;
}

/* relative L2 error of float values against double references */
static double rel_l2_f(const float *x, const double *ref, size_t n) {
  double num = 0.0, den = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double e = (double)x[i] - ref[i];
    num += e * e;
    den += ref[i] * ref[i];
  }
  return sqrt(num / (den > 0.0 ? den : 1.0));
}

static int report(const char *name, double err, double tol) {
  const int ok = err <= tol && err == err;
  printf("%-40s rel L2 %.3e (tolerance %.0e) %s\n", name, err, tol, ok ? "ok" : "FAIL");
  return ok;
}

/* unit L2 norm per row of D values */
static void normalise_rows(double *x, size_t rows) {
  for (size_t r = 0; r < rows; ++r) {
    double s = 0.0;
    for (int c = 0; c < D; ++c) s += x[r * D + c] * x[r * D + c];
    s = 1.0 / sqrt(s);
    for (int c = 0; c < D; ++c) x[r * D + c] *= s;
  }
}

int main(void) {
  int ok = 1;
  rng_state = 20240611ull;
  const float g_min = -5.0f;

  /* ---------------- prefill: two documents, T = 300, H = 2 ---------------- */
  {
    const int32_t N = 2, H = 2;
    const int64_t T = 300;
    const int32_t cu[3] = {0, 130, 300};
    const size_t nx = (size_t)T * H * D, nb = (size_t)T * H, ns = (size_t)N * H * D * D;
    double *q = malloc(nx * 8), *k = malloc(nx * 8), *v = malloc(nx * 8), *z = malloc(nx * 8);
    double *beta = malloc(nb * 8), *S0 = malloc(ns * 8), A_log[2], *g = malloc(nx * 8);
    double *o_ref = malloc(nx * 8), *S_ref = malloc(ns * 8);
    for (size_t i = 0; i < nx; ++i) { q[i] = normal(); k[i] = normal(); v[i] = normal(); z[i] = normal(); }
    normalise_rows(q, nb);
    normalise_rows(k, nb);
    for (size_t i = 0; i < nb; ++i) beta[i] = 1.0 / (1.0 + exp(-normal()));
    for (size_t i = 0; i < ns; ++i) S0[i] = 0.02 * normal();
    for (int h = 0; h < H; ++h) A_log[h] = 0.5 * normal();

    for (int pass = 0; pass < 2; ++pass) {  /* 0: fp32 inputs; 1: bf16 inputs, workspace */
      const int bf16 = pass == 1;
      const size_t es = bf16 ? 2 : 4;
      /* the values the GPU reads, as float, and the oracle's copy of them */
      float *hq = malloc(nx * 4), *hk = malloc(nx * 4), *hv = malloc(nx * 4), *hz = malloc(nx * 4);
      float *hb = malloc(nb * 4), *hS0 = malloc(ns * 4), hA[2];
      double *dq = malloc(nx * 8), *dk = malloc(nx * 8), *dv = malloc(nx * 8), *dz = malloc(nx * 8);
      double *db = malloc(nb * 8), *dS0 = malloc(ns * 8), dA[2];
      for (size_t i = 0; i < nx; ++i) {
        hq[i] = (float)q[i]; hk[i] = (float)k[i]; hv[i] = (float)v[i]; hz[i] = (float)z[i];
        if (bf16) {
          hq[i] = from_bf16(to_bf16(hq[i])); hk[i] = from_bf16(to_bf16(hk[i]));
          hv[i] = from_bf16(to_bf16(hv[i])); hz[i] = from_bf16(to_bf16(hz[i]));
        }
        dq[i] = hq[i]; dk[i] = hk[i]; dv[i] = hv[i]; dz[i] = hz[i];
      }
      for (size_t i = 0; i < nb; ++i) {
        hb[i] = (float)beta[i];
        if (bf16) hb[i] = from_bf16(to_bf16(hb[i]));
        db[i] = hb[i];
      }
      for (size_t i = 0; i < ns; ++i) { hS0[i] = (float)S0[i]; dS0[i] = hS0[i]; }
      for (int h = 0; h < H; ++h) { hA[h] = (float)A_log[h]; dA[h] = hA[h]; }
      kda_oracle_gate(dz, dA, (double)g_min, T, H, D, g);
      if (kda_oracle_recurrent(dq, dk, dv, g, db, dS0, cu, N, H, D, D, o_ref, S_ref, 0) != 0) {
        fprintf(stderr, "oracle failed\n");
        return 2;
      }
      /* device inputs in the call's dtype */
      void *d_in[5];
      const float *src[5] = {hq, hk, hv, hz, hb};
      const size_t cnt[5] = {nx, nx, nx, nx, nb};
      for (int a = 0; a < 5; ++a) {
        if (bf16) {
          uint16_t *tmp = malloc(cnt[a] * 2);
          for (size_t i = 0; i < cnt[a]; ++i) tmp[i] = to_bf16(src[a][i]);
          d_in[a] = dev_copy(tmp, cnt[a] * 2);
          free(tmp);
        } else {
          d_in[a] = dev_copy(src[a], cnt[a] * 4);
        }
      }
      float *d_A = dev_copy(hA, sizeof hA), *d_S0 = dev_copy(hS0, ns * 4);
      int32_t *d_cu = dev_copy(cu, sizeof cu);
      void *d_o = dev_alloc(nx * es);
      float *d_S = dev_alloc(ns * 4);
      size_t ws_bytes = 0;
      void *d_ws = NULL;
      if (bf16) {
        ws_bytes = kda_chunk_fwd_workspace_size(N, T, H, D, D);
        d_ws = dev_alloc(ws_bytes);
      }
      KDA(kda_chunk_fwd(d_in[0], d_in[1], d_in[2], d_in[3], d_in[4], d_A, g_min, d_S0, d_cu, cu,
                        N, T, H, D, D, bf16 ? KDA_BF16 : KDA_F32, KDA_COMPUTE_AUTO, d_o, d_S, d_ws,
                        ws_bytes, NULL));
      HIP(hipDeviceSynchronize());
      float *ho = malloc(nx * 4), *hS = malloc(ns * 4);
      if (bf16) {
        uint16_t *tmp = malloc(nx * 2);
        HIP(hipMemcpy(tmp, d_o, nx * 2, hipMemcpyDeviceToHost));
        for (size_t i = 0; i < nx; ++i) ho[i] = from_bf16(tmp[i]);
        free(tmp);
      } else {
        HIP(hipMemcpy(ho, d_o, nx * 4, hipMemcpyDeviceToHost));
      }
      HIP(hipMemcpy(hS, d_S, ns * 4, hipMemcpyDeviceToHost));
      const double tol = bf16 ? 1e-2 : 1e-4;
      ok &= report(bf16 ? "kda_chunk_fwd bf16 (two kernels): O" : "kda_chunk_fwd fp32: O",
                   rel_l2_f(ho, o_ref, nx), tol);
      ok &= report(bf16 ? "kda_chunk_fwd bf16 (two kernels): state" : "kda_chunk_fwd fp32: state",
                   rel_l2_f(hS, S_ref, ns), tol);
      for (int a = 0; a < 5; ++a) HIP(hipFree(d_in[a]));
      HIP(hipFree(d_A)); HIP(hipFree(d_S0)); HIP(hipFree(d_cu)); HIP(hipFree(d_o)); HIP(hipFree(d_S));
      if (d_ws) HIP(hipFree(d_ws));
      free(hq); free(hk); free(hv); free(hz); free(hb); free(hS0); free(ho); free(hS);
      free(dq); free(dk); free(dv); free(dz); free(db); free(dS0);
    }
    free(q); free(k); free(v); free(z); free(beta); free(S0); free(g); free(o_ref); free(S_ref);
  }

  /* ---------------- decode: N = 6 sequences, W = 4 cached drafts, fp32 ---------------- */
  {
    const int32_t N = 6, H = 2, W = 4;
    const int32_t accepted[6] = {0, 1, 2, 3, 4, 2};
    const size_t nc = (size_t)N * W * H * D, ncb = (size_t)N * W * H, nn = (size_t)N * H * D;
    const size_t nnb = (size_t)N * H, ns = (size_t)N * H * D * D;
    float *cq = malloc(nc * 4), *ck = malloc(nc * 4), *cv = malloc(nc * 4), *cz = malloc(nc * 4);
    float *cb = malloc(ncb * 4), *nq = malloc(nn * 4), *nk = malloc(nn * 4), *nv = malloc(nn * 4);
    float *nz = malloc(nn * 4), *nbt = malloc(nnb * 4), *state = malloc(ns * 4), hA[2];
    double *tmp = malloc((nc > nn ? nc : nn) * 8);
    /* cached drafts, then the bonus tokens: q, k unit rows, v, z normal, beta in (0, 1) */
    for (size_t i = 0; i < nc; ++i) tmp[i] = normal();
    normalise_rows(tmp, nc / D);
    for (size_t i = 0; i < nc; ++i) cq[i] = (float)tmp[i];
    for (size_t i = 0; i < nc; ++i) tmp[i] = normal();
    normalise_rows(tmp, nc / D);
    for (size_t i = 0; i < nc; ++i) ck[i] = (float)tmp[i];
    for (size_t i = 0; i < nc; ++i) { cv[i] = (float)normal(); cz[i] = (float)normal(); }
    for (size_t i = 0; i < ncb; ++i) cb[i] = (float)(1.0 / (1.0 + exp(-normal())));
    for (size_t i = 0; i < nn; ++i) tmp[i] = normal();
    normalise_rows(tmp, nn / D);
    for (size_t i = 0; i < nn; ++i) nq[i] = (float)tmp[i];
    for (size_t i = 0; i < nn; ++i) tmp[i] = normal();
    normalise_rows(tmp, nn / D);
    for (size_t i = 0; i < nn; ++i) nk[i] = (float)tmp[i];
    for (size_t i = 0; i < nn; ++i) { nv[i] = (float)normal(); nz[i] = (float)normal(); }
    for (size_t i = 0; i < nnb; ++i) nbt[i] = (float)(1.0 / (1.0 + exp(-normal())));
    for (size_t i = 0; i < ns; ++i) state[i] = (float)(0.02 * normal());
    for (int h = 0; h < H; ++h) hA[h] = (float)(0.5 * normal());
    free(tmp);

    /* oracle: each sequence's accepted drafts then its bonus token, one packed
     * document per sequence starting from its saved state */
    int32_t cu[7];
    cu[0] = 0;
    for (int n = 0; n < N; ++n) cu[n + 1] = cu[n] + accepted[n] + 1;
    const int64_t T = cu[N];
    const size_t nx = (size_t)T * H * D, nb = (size_t)T * H;
    double *q = malloc(nx * 8), *k = malloc(nx * 8), *v = malloc(nx * 8), *z = malloc(nx * 8);
    double *g = malloc(nx * 8), *beta = malloc(nb * 8), *S0 = malloc(ns * 8), dA[2];
    double *o_ref = malloc(nx * 8), *S_ref = malloc(ns * 8);
    for (int n = 0; n < N; ++n)
      for (int t = 0; t <= accepted[n]; ++t) {
        const int64_t row = cu[n] + t;
        for (int h = 0; h < H; ++h) {
          const size_t dst = ((size_t)row * H + h) * D;
          const size_t src = t < accepted[n] ? (((size_t)n * W + t) * H + h) * D : ((size_t)n * H + h) * D;
          const int bonus = t == accepted[n];
          for (int c = 0; c < D; ++c) {
            q[dst + c] = bonus ? nq[src + c] : cq[src + c];
            k[dst + c] = bonus ? nk[src + c] : ck[src + c];
            v[dst + c] = bonus ? nv[src + c] : cv[src + c];
            z[dst + c] = bonus ? nz[src + c] : cz[src + c];
          }
          beta[(size_t)row * H + h] = bonus ? nbt[(size_t)n * H + h] : cb[((size_t)n * W + t) * H + h];
        }
      }
    for (size_t i = 0; i < ns; ++i) S0[i] = state[i];
    for (int h = 0; h < H; ++h) dA[h] = hA[h];
    kda_oracle_gate(z, dA, (double)g_min, T, H, D, g);
    if (kda_oracle_recurrent(q, k, v, g, beta, S0, cu, N, H, D, D, o_ref, S_ref, 0) != 0) {
      fprintf(stderr, "oracle failed\n");
      return 2;
    }
    double *ob_ref = malloc(nn * 8);  /* the bonus token's output per sequence */
    for (int n = 0; n < N; ++n)
      memcpy(ob_ref + (size_t)n * H * D, o_ref + (size_t)(cu[n + 1] - 1) * H * D, (size_t)H * D * 8);

    float *d_state = dev_copy(state, ns * 4);
    void *d_cq = dev_copy(cq, nc * 4), *d_ck = dev_copy(ck, nc * 4), *d_cv = dev_copy(cv, nc * 4);
    void *d_cz = dev_copy(cz, nc * 4), *d_cb = dev_copy(cb, ncb * 4), *d_nq = dev_copy(nq, nn * 4);
    void *d_nk = dev_copy(nk, nn * 4), *d_nv = dev_copy(nv, nn * 4), *d_nz = dev_copy(nz, nn * 4);
    void *d_nb = dev_copy(nbt, nnb * 4);
    int32_t *d_acc = dev_copy(accepted, sizeof accepted);
    float *d_A = dev_copy(hA, sizeof hA);
    void *d_o = dev_alloc(nn * 4);
    KDA(kda_decode_step(d_state, N, NULL, d_cq, d_ck, d_cv, d_cz, d_cb, d_acc, W, d_nq, d_nk, d_nv,
                        d_nz, d_nb, d_A, g_min, d_o, NULL, N, H, D, D, KDA_F32, NULL));
    HIP(hipDeviceSynchronize());
    float *ho = malloc(nn * 4), *hS = malloc(ns * 4);
    HIP(hipMemcpy(ho, d_o, nn * 4, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(hS, d_state, ns * 4, hipMemcpyDeviceToHost));
    ok &= report("kda_decode_step fp32: bonus output", rel_l2_f(ho, ob_ref, nn), 1e-4);
    ok &= report("kda_decode_step fp32: state", rel_l2_f(hS, S_ref, ns), 1e-4);
    void *bufs[] = {d_state, d_cq, d_ck, d_cv, d_cz, d_cb, d_nq, d_nk, d_nv, d_nz, d_nb, d_acc, d_A, d_o};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP(hipFree(bufs[i]));
    free(cq); free(ck); free(cv); free(cz); free(cb); free(nq); free(nk); free(nv); free(nz);
    free(nbt); free(state); free(q); free(k); free(v); free(z); free(g); free(beta); free(S0);
    free(o_ref); free(S_ref); free(ob_ref); free(ho); free(hS);
  }
  printf("%s\n", ok ? "all checks ok" : "a check failed");
  return ok ? 0 : 1;
}
