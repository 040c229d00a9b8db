/*
 * abi_check.c — TEST PROGRAM: uses libkda.so through include/kda.h from plain
 * C (no Python, no torch) and checks the results against the fp64 oracle
 * (oracle/kda_oracle.c, linked in as test infrastructure).
 *
 * It allocates every buffer with hipMalloc, sizes the prefill workspace with
 * kda_chunk_fwd_workspace_bytes, and runs on the null stream:
 *   1. kda_chunk_fwd, fp32, two packed sequences (300 and 77 tokens), H = 3,
 *      initial state given, final state returned;
 *   2. kda_decode_step on the prefill's final state, one token;
 *   3. kda_decode_replay, 5 cached tokens per sequence, ragged counts, in-place
 *      commit;
 *   4. kda_chunk_fwd again with kda_fused_opts.unbounded_decay = 1 and
 *      log_alpha = -20 softplus(z) (far below the -5 bound), one sequence;
 *   5. kda_chunk_fwd_save on step 1's inputs (its o and final state must equal
 *      step 1's bit for bit), then kda_chunk_bwd_saved from its workspace for
 *      random d_o and d_final_state, against the oracle's backward;
 * and compares each output slice (per sequence and head) with the oracle by
 * max|y - r| / max|r| against 1e-4.  Exit status 0 when everything passes.
 * Inputs come from a fixed linear congruential generator (q, k normalised
 * per row, log_alpha in (-5, 0), beta in (0, 1)).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kda.h"

int kda_oracle_chunk_fwd(const double*, const double*, const double*, const double*, const double*, const double*,
                         const int64_t*, int, int64_t, int, int, int, const double*, const double*, const double*,
                         const double*, double, double, double*, double*, int);
int kda_oracle_chunk_bwd(const double*, const double*, const double*, const double*, const double*, const double*,
                         const int64_t*, int, int64_t, int, int, int, const double*, const double*, double*, double*,
                         double*, double*, double*, double*, int);
int kda_oracle_decode_step(double*, const double*, const double*, const double*, const double*, const double*, int,
                           int, int, int, double*, int);
int kda_oracle_decode_multi(const double*, const double*, const double*, const double*, const double*, const double*,
                            const int64_t*, int, int, int, int, int, const double*, const double*, const double*,
                            const double*, const double*, const double*, double, double, double*, double*, double*,
                            double*, int);

#define D 128

static uint64_t lcg_state = 0x4B444143ull;
static double uniform(void) {
  lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(lcg_state >> 11) * (1.0 / 9007199254740992.0);
}
static double normal(void) {
  const double u1 = uniform() + 1e-12, u2 = uniform();
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

/* rows x D values, normalised per row when unit != 0 */
static void fill_rows(float* x, size_t rows, int unit) {
  for (size_t r = 0; r < rows; ++r) {
    double ss = 0.0;
    for (int j = 0; j < D; ++j) {
      x[r * D + j] = (float)normal();
      ss += (double)x[r * D + j] * x[r * D + j];
    }
    if (unit)
      for (int j = 0; j < D; ++j) x[r * D + j] = (float)(x[r * D + j] / sqrt(ss));
  }
}
static void fill_decay(float* x, size_t n) {
  for (size_t i = 0; i < n; ++i) x[i] = (float)(-5.0 / (1.0 + exp(-normal())));
}
static void fill_beta(float* x, size_t n) {
  for (size_t i = 0; i < n; ++i) x[i] = (float)(1.0 / (1.0 + exp(-normal())));
}
static double* widen(const float* x, size_t n) {
  double* y = (double*)malloc(n * sizeof(double));
  for (size_t i = 0; i < n; ++i) y[i] = x[i];
  return y;
}

static int failures = 0;
static void check(const char* what, const float* y, const double* r, size_t n) {
  double num = 0.0, den = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double e = fabs((double)y[i] - r[i]);
    if (!(e <= num)) num = e; /* also catches NaN */
    if (fabs(r[i]) > den) den = fabs(r[i]);
  }
  const double err = den > 0.0 ? num / den : num;
  const int ok = err <= 1e-4;
  if (!ok) ++failures;
  printf("%-44s err %.3e %s\n", what, err, ok ? "ok" : "FAIL");
}

#define HIP_OK(x)                                                  \
  do {                                                             \
    hipError_t e_ = (x);                                           \
    if (e_ != hipSuccess) {                                        \
      printf("HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
      return 2;                                                    \
    }                                                              \
  } while (0)
#define KDA_OK_(x)                                                              \
  do {                                                                          \
    kda_status s_ = (x);                                                        \
    if (s_ != KDA_OK) {                                                         \
      printf("kda error %d (%s) at %s:%d\n", (int)s_, kda_status_string(s_), __FILE__, __LINE__); \
      return 3;                                                                 \
    }                                                                           \
  } while (0)

/* device copy of h (or uninitialised device memory when h is NULL); NULL and a message on failure */
static void* dev_copy(const void* h, size_t bytes) {
  void* d = NULL;
  hipError_t e = hipMalloc(&d, bytes);
  if (e == hipSuccess && h) e = hipMemcpy(d, h, bytes, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    printf("device allocation or copy of %zu bytes failed: %s\n", bytes, hipGetErrorString(e));
    return NULL;
  }
  return d;
}

int main(void) {
  const int H = 3, N = 2;
  const int lens[2] = {300, 77};
  const int T = lens[0] + lens[1];
  const size_t tok = (size_t)T * H, st = (size_t)N * H * D * D;
  int32_t cu[3] = {0, lens[0], T};
  int64_t cu64[3] = {0, lens[0], T};

  /* ---- 1. prefill ---- */
  float *q = malloc(tok * D * 4), *k = malloc(tok * D * 4), *v = malloc(tok * D * 4), *la = malloc(tok * D * 4);
  float *b = malloc(tok * 4), *s0 = malloc(st * 4), *o = malloc(tok * D * 4), *fs = malloc(st * 4);
  fill_rows(q, tok, 1);
  fill_rows(k, tok, 1);
  fill_rows(v, tok, 0);
  fill_decay(la, tok * D);
  fill_beta(b, tok);
  for (size_t i = 0; i < st; ++i) s0[i] = (float)(0.3 * normal());
  void *dq = dev_copy(q, tok * D * 4), *dk = dev_copy(k, tok * D * 4), *dv = dev_copy(v, tok * D * 4);
  void *dla = dev_copy(la, tok * D * 4), *db = dev_copy(b, tok * 4), *ds0 = dev_copy(s0, st * 4);
  void *dcu = dev_copy(cu, sizeof(cu)), *dout = dev_copy(NULL, tok * D * 4), *dfs = dev_copy(NULL, st * 4);
  if (!dq || !dk || !dv || !dla || !db || !ds0 || !dcu || !dout || !dfs) return 2;
  const size_t wsb = kda_chunk_fwd_workspace_bytes(N, T, H, D, D, KDA_DTYPE_F32, NULL);
  void* dws = wsb ? dev_copy(NULL, wsb) : NULL;
  KDA_OK_(kda_chunk_fwd(dq, dk, dv, dla, db, ds0, dcu, N, T, H, D, D, KDA_DTYPE_F32, NULL, dout, dfs, dws, wsb, 0));
  HIP_OK(hipMemcpy(o, dout, tok * D * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(fs, dfs, st * 4, hipMemcpyDeviceToHost));
  {
    double *wq = widen(q, tok * D), *wk = widen(k, tok * D), *wv = widen(v, tok * D), *wla = widen(la, tok * D);
    double *wb = widen(b, tok), *ws0 = widen(s0, st);
    double *ro = malloc(tok * D * 8), *rfs = malloc(st * 8);
    if (kda_oracle_chunk_fwd(wq, wk, wv, wla, wb, ws0, cu64, N, T, H, D, D, NULL, NULL, NULL, NULL, 1e-6, 1e-6, ro,
                             rfs, 0) != 0)
      return 4;
    for (int n = 0; n < N; ++n)
      for (int h = 0; h < H; ++h) {
        /* gather the (n, h) slices */
        size_t m = (size_t)lens[n] * D;
        float* y = malloc(m * 4);
        double* r = malloc(m * 8);
        for (int t = 0; t < lens[n]; ++t)
          for (int j = 0; j < D; ++j) {
            const size_t at = ((size_t)(cu[n] + t) * H + h) * D + j;
            y[(size_t)t * D + j] = o[at];
            r[(size_t)t * D + j] = ro[at];
          }
        char name[64];
        snprintf(name, sizeof name, "chunk_fwd o    (seq %d, head %d)", n, h);
        check(name, y, r, m);
        snprintf(name, sizeof name, "chunk_fwd S_T  (seq %d, head %d)", n, h);
        check(name, fs + ((size_t)n * H + h) * D * D, rfs + ((size_t)n * H + h) * D * D, (size_t)D * D);
        free(y);
        free(r);
      }
    free(wq); free(wk); free(wv); free(wla); free(wb); free(ws0); free(ro); free(rfs);
  }

  /* ---- 2. one decode step on the final state, in place ---- */
  const size_t un = (size_t)N * H;
  float *dq1 = malloc(un * D * 4), *dk1 = malloc(un * D * 4), *dv1 = malloc(un * D * 4), *dla1 = malloc(un * D * 4);
  float *db1 = malloc(un * 4), *do1 = malloc(un * D * 4), *st1 = malloc(st * 4);
  fill_rows(dq1, un, 1);
  fill_rows(dk1, un, 1);
  fill_rows(dv1, un, 0);
  fill_decay(dla1, un * D);
  fill_beta(db1, un);
  void *gq = dev_copy(dq1, un * D * 4), *gk = dev_copy(dk1, un * D * 4), *gv = dev_copy(dv1, un * D * 4);
  void *gla = dev_copy(dla1, un * D * 4), *gb = dev_copy(db1, un * 4), *go = dev_copy(NULL, un * D * 4);
  if (!gq || !gk || !gv || !gla || !gb || !go) return 2;
  KDA_OK_(kda_decode_step((float*)dfs, gq, gk, gv, gla, gb, N, H, D, D, KDA_DTYPE_F32, go, 0));
  HIP_OK(hipMemcpy(do1, go, un * D * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(st1, dfs, st * 4, hipMemcpyDeviceToHost));
  {
    double *rs = widen(fs, st), *ro = malloc(un * D * 8);
    double *wq = widen(dq1, un * D), *wk = widen(dk1, un * D), *wv = widen(dv1, un * D), *wla = widen(dla1, un * D);
    double* wb = widen(db1, un);
    if (kda_oracle_decode_step(rs, wq, wk, wv, wla, wb, N, H, D, D, ro, 0) != 0) return 4;
    check("decode_step o", do1, ro, un * D);
    check("decode_step state", st1, rs, st);
    free(rs); free(ro); free(wq); free(wk); free(wv); free(wla); free(wb);
  }

  /* ---- 3. replay: 5 cached tokens, counts {5, 2}, in-place commit ---- */
  const int L = 5;
  int32_t counts[2] = {5, 2};
  int64_t counts64[2] = {5, 2};
  const size_t rt = (size_t)N * L * H;
  float *rq = malloc(rt * D * 4), *rk = malloc(rt * D * 4), *rv = malloc(rt * D * 4), *rla = malloc(rt * D * 4);
  float *rb = malloc(rt * 4), *ro = malloc(rt * D * 4), *st2 = malloc(st * 4);
  fill_rows(rq, rt, 1);
  fill_rows(rk, rt, 1);
  fill_rows(rv, rt, 0);
  fill_decay(rla, rt * D);
  fill_beta(rb, rt);
  void *hq = dev_copy(rq, rt * D * 4), *hk = dev_copy(rk, rt * D * 4), *hv = dev_copy(rv, rt * D * 4);
  void *hla = dev_copy(rla, rt * D * 4), *hb = dev_copy(rb, rt * 4), *hc = dev_copy(counts, sizeof(counts));
  void* ho = dev_copy(NULL, rt * D * 4);
  if (!hq || !hk || !hv || !hla || !hb || !hc || !ho) return 2;
  HIP_OK(hipMemset(ho, 0, rt * D * 4));
  KDA_OK_(kda_decode_replay((float*)dfs, (float*)dfs, hq, hk, hv, hla, hb, hc, N, L, H, D, D, KDA_DTYPE_F32, NULL,
                            NULL, NULL, ho, 0));
  HIP_OK(hipMemcpy(ro, ho, rt * D * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(st2, dfs, st * 4, hipMemcpyDeviceToHost));
  {
    double *ws = widen(st1, st), *rro = calloc(rt * D, 8), *rst = malloc(st * 8);
    double *wq = widen(rq, rt * D), *wk = widen(rk, rt * D), *wv = widen(rv, rt * D), *wla = widen(rla, rt * D);
    double* wb = widen(rb, rt);
    if (kda_oracle_decode_multi(ws, wq, wk, wv, wla, wb, counts64, N, L, H, D, D, NULL, NULL, NULL, NULL, NULL, NULL,
                                1e-6, 1e-6, rro, rst, NULL, NULL, 0) != 0)
      return 4;
    check("decode_replay o", ro, rro, rt * D);
    check("decode_replay state", st2, rst, st);
    free(ws); free(rro); free(rst); free(wq); free(wk); free(wv); free(wla); free(wb);
  }

  /* ---- 4. prefill with unbounded decay, set through the options struct ---- */
  {
    const int Tu = 150;
    const size_t tu = (size_t)Tu * H;
    float *uq = malloc(tu * D * 4), *uk = malloc(tu * D * 4), *uv = malloc(tu * D * 4), *ula = malloc(tu * D * 4);
    float *ub = malloc(tu * 4), *uo = malloc(tu * D * 4), *ufs = malloc((size_t)H * D * D * 4);
    fill_rows(uq, tu, 1);
    fill_rows(uk, tu, 1);
    fill_rows(uv, tu, 0);
    for (size_t i = 0; i < tu * D; ++i) ula[i] = (float)(-20.0 * log1p(exp(normal())));
    fill_beta(ub, tu);
    void *eq = dev_copy(uq, tu * D * 4), *ek = dev_copy(uk, tu * D * 4), *ev = dev_copy(uv, tu * D * 4);
    void *ela = dev_copy(ula, tu * D * 4), *eb = dev_copy(ub, tu * 4), *eo = dev_copy(NULL, tu * D * 4);
    void* efs = dev_copy(NULL, (size_t)H * D * D * 4);
    if (!eq || !ek || !ev || !ela || !eb || !eo || !efs) return 2;
    kda_fused_opts opts;
    memset(&opts, 0, sizeof opts);
    opts.l2_eps = 1e-6f;
    opts.rms_eps = 1e-6f;
    opts.unbounded_decay = 1;
    const size_t wsu = kda_chunk_fwd_workspace_bytes(1, Tu, H, D, D, KDA_DTYPE_F32, &opts);
    void* dwsu = wsu ? dev_copy(NULL, wsu) : NULL;
    KDA_OK_(kda_chunk_fwd(eq, ek, ev, ela, eb, NULL, NULL, 1, Tu, H, D, D, KDA_DTYPE_F32, &opts, eo, efs, dwsu, wsu, 0));
    HIP_OK(hipMemcpy(uo, eo, tu * D * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ufs, efs, (size_t)H * D * D * 4, hipMemcpyDeviceToHost));
    double *wq = widen(uq, tu * D), *wk = widen(uk, tu * D), *wv = widen(uv, tu * D), *wla = widen(ula, tu * D);
    double *wb = widen(ub, tu), *ro = malloc(tu * D * 8), *rfs = malloc((size_t)H * D * D * 8);
    int64_t cu1[2] = {0, Tu};
    if (kda_oracle_chunk_fwd(wq, wk, wv, wla, wb, NULL, cu1, 1, Tu, H, D, D, NULL, NULL, NULL, NULL, 1e-6, 1e-6, ro,
                             rfs, 0) != 0)
      return 4;
    for (int h = 0; h < H; ++h) {
      size_t m = (size_t)Tu * D;
      float* y = malloc(m * 4);
      double* r = malloc(m * 8);
      for (int t = 0; t < Tu; ++t)
        for (int j = 0; j < D; ++j) {
          y[(size_t)t * D + j] = uo[((size_t)t * H + h) * D + j];
          r[(size_t)t * D + j] = ro[((size_t)t * H + h) * D + j];
        }
      char name[64];
      snprintf(name, sizeof name, "unbounded chunk_fwd o   (head %d)", h);
      check(name, y, r, m);
      snprintf(name, sizeof name, "unbounded chunk_fwd S_T (head %d)", h);
      check(name, ufs + (size_t)h * D * D, rfs + (size_t)h * D * D, (size_t)D * D);
      free(y);
      free(r);
    }
    free(wq); free(wk); free(wv); free(wla); free(wb); free(ro); free(rfs);
  }

  /* ---- 5. the training forward and the backward from its residuals, on step 1's inputs ---- */
  {
    const size_t bwb = kda_chunk_bwd_workspace_bytes(N, T, H, D, D, KDA_DTYPE_F32);
    void *dwb = bwb ? dev_copy(NULL, bwb) : NULL, *so = dev_copy(NULL, tok * D * 4), *sfs = dev_copy(NULL, st * 4);
    if (!dwb || !so || !sfs) return 2;
    KDA_OK_(kda_chunk_fwd_save(dq, dk, dv, dla, db, ds0, dcu, N, T, H, D, D, KDA_DTYPE_F32, so, sfs, dwb, bwb, 0));
    float *o2 = malloc(tok * D * 4), *fs2 = malloc(st * 4);
    HIP_OK(hipMemcpy(o2, so, tok * D * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(fs2, sfs, st * 4, hipMemcpyDeviceToHost));
    const int same = memcmp(o2, o, tok * D * 4) == 0 && memcmp(fs2, fs, st * 4) == 0;
    if (!same) ++failures;
    printf("%-44s %s\n", "chunk_fwd_save o, S_T = chunk_fwd bit for bit", same ? "ok" : "FAIL");
    float *gdo = malloc(tok * D * 4), *gds = malloc(st * 4);
    fill_rows(gdo, tok, 0);
    for (size_t i = 0; i < st; ++i) gds[i] = (float)normal();
    void *ddo = dev_copy(gdo, tok * D * 4), *dds = dev_copy(gds, st * 4), *xq = dev_copy(NULL, tok * D * 4);
    void *xk = dev_copy(NULL, tok * D * 4), *xv = dev_copy(NULL, tok * D * 4), *xla = dev_copy(NULL, tok * D * 4);
    void *xb = dev_copy(NULL, tok * 4), *xs0 = dev_copy(NULL, st * 4);
    if (!ddo || !dds || !xq || !xk || !xv || !xla || !xb || !xs0) return 2;
    KDA_OK_(kda_chunk_bwd_saved(dq, dk, dv, dla, db, ds0, dcu, ddo, dds, N, T, H, D, D, KDA_DTYPE_F32, xq, xk, xv, xla,
                                xb, xs0, dwb, bwb, 0));
    const size_t sizes[6] = {tok * D, tok * D, tok * D, tok * D, tok, st};
    void* devs[6] = {xq, xk, xv, xla, xb, xs0};
    const char* names[6] = {"chunk_bwd_saved dq", "chunk_bwd_saved dk", "chunk_bwd_saved dv",
                            "chunk_bwd_saved dlog_alpha", "chunk_bwd_saved dbeta", "chunk_bwd_saved d_initial_state"};
    double *wq = widen(q, tok * D), *wk = widen(k, tok * D), *wv = widen(v, tok * D), *wla = widen(la, tok * D);
    double *wb = widen(b, tok), *ws0 = widen(s0, st), *wdo = widen(gdo, tok * D), *wds = widen(gds, st);
    double* ref[6];
    for (int i = 0; i < 6; ++i) ref[i] = malloc(sizes[i] * 8);
    if (kda_oracle_chunk_bwd(wq, wk, wv, wla, wb, ws0, cu64, N, T, H, D, D, wdo, wds, ref[0], ref[1], ref[2], ref[3],
                             ref[4], ref[5], 0) != 0)
      return 4;
    for (int i = 0; i < 6; ++i) {
      float* y = malloc(sizes[i] * 4);
      HIP_OK(hipMemcpy(y, devs[i], sizes[i] * 4, hipMemcpyDeviceToHost));
      check(names[i], y, ref[i], sizes[i]);
      free(y);
      free(ref[i]);
    }
    free(wq); free(wk); free(wv); free(wla); free(wb); free(ws0); free(wdo); free(wds);
    free(o2); free(fs2); free(gdo); free(gds);
  }

  /* an argument error comes back before anything is launched */
  if (kda_decode_step(NULL, gq, gk, gv, gla, gb, N, H, D, D, KDA_DTYPE_F32, go, 0) != KDA_ERR_INVALID_ARG) {
    printf("expected KDA_ERR_INVALID_ARG for a NULL state\n");
    ++failures;
  }
  printf("%s\n", failures ? "FAILED" : "all checks passed");
  return failures ? 1 : 0;
}
