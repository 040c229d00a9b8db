/*
 * kda_oracle.c — TEST INFRASTRUCTURE ONLY.  A plain, slow, fp64 CPU reference
 * of the Kimi Delta Attention recurrence.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the library's
 * compute path never does.  It shares no code with the HIP library.
 *
 * What it computes, token by token, for one (sequence, head):
 *
 *   a_j   = exp(log_alpha_t[j])                         per key channel j
 *   S'    = Diag(a) S                                   row j of S scaled by a_j
 *   vhat  = S'^T k_t                                    old prediction at key k_t
 *   u     = beta_t (v_t - vhat)                         delta-rule correction
 *   S     = S' + k_t u^T
 *         = (I - beta_t k_t k_t^T) Diag(a) S + beta_t k_t v_t^T
 *   o_t   = S^T q_t                                     read after the write
 *
 * Sources: "Kimi K3" study notes (dimensionstp.github.io/study-concept/kimi_k3),
 * section 3-2 item 2) Kimi Delta Attention: the update and read-out equations.
 * "Kimi K3 架构、训练与系统全景解析", section 4.2.2: the three sub-steps in this
 * order (per-key-channel decay, erase along k, write beta k v^T) and the read
 * o = S^T q.  "AI-Workshop 文献分享 #15", section 7.2 ("Delta" paragraph): the
 * correction form  S' + beta k (v - vhat)^T ; the talk's own simplified
 * formula reads vhat from the undecayed state and is a teaching shortcut it
 * labels as such; here vhat is read from the decayed state, which is what the
 * exact update above implies.
 *
 * Optional prologue ("Kimi K3 架构…" section 4.2.3; study notes section 3-2,
 * "ShortConv, Swish and L2 normalization on Q and K"): for q and k,
 *   c_t[j] = sum_{m=0..3} w[h*dk+j][m] x_{t-3+m}[j]    (zeros before the sequence start)
 *   s      = c * sigmoid(c)                              (SiLU / Swish)
 *   x'_t   = s / sqrt(sum_j s_j^2 + l2_eps)
 * Optional epilogue ("Kimi K3 架构…" section 4.2.6): head-wise RMSNorm of o_t,
 * times norm_w, times sigmoid(gate_t) channel-wise.
 *
 * Layouts (all double): q,k,log_alpha [T,H,dk]; v,gate,o [T,H,dv];
 * beta [T,H]; states [N,H,dk,dv] row-major; cu_seqlens int64 [N+1].
 * Any dk, dv >= 1.  OpenMP over (sequence, head) pairs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads of one parallel region: num_threads if positive, else the OpenMP
 * default (set per region, so a call never changes the default of the next). */
static int team_size(int num_threads) {
#ifdef _OPENMP
  return num_threads > 0 ? num_threads : omp_get_max_threads();
#else
  (void)num_threads;
  return 1;
#endif
}

/* One token of the recurrence on a dk x dv state S (row-major). */
static void kda_token(double* S, int dk, int dv, const double* q, const double* k, const double* v,
                      const double* log_alpha, double beta, double* vhat, double* o) {
  for (int i = 0; i < dk; ++i) {
    const double a = exp(log_alpha[i]);
    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;
  }
  for (int j = 0; j < dv; ++j) vhat[j] = 0.0;
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) vhat[j] += S[(size_t)i * dv + j] * k[i];
  for (int j = 0; j < dv; ++j) vhat[j] = beta * (v[j] - vhat[j]); /* now u */
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += k[i] * vhat[j];
  for (int j = 0; j < dv; ++j) o[j] = 0.0;
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) o[j] += S[(size_t)i * dv + j] * q[i];
}

/* ShortConv(4) + SiLU + L2 of one token: rows[m] is the raw row x_{t-3+m}
 * (NULL before the sequence start, i.e. zero), w the head's taps [d][4]. */
static void conv_silu_l2(const double* const rows[4], const double* w, int d, double eps, double* out) {
  double ss = 0.0;
  for (int j = 0; j < d; ++j) {
    double c = 0.0;
    for (int m = 0; m < 4; ++m) {
      if (!rows[m]) continue;
      c += w[(size_t)j * 4 + m] * rows[m][j];
    }
    const double s = c / (1.0 + exp(-c));
    out[j] = s;
    ss += s * s;
  }
  const double inv = 1.0 / sqrt(ss + eps);
  for (int j = 0; j < d; ++j) out[j] *= inv;
}

/* The prologue for token t (absolute index) of a packed sequence starting at bos. */
static void prologue(const double* x, const double* w, int64_t bos, int64_t t, int H, int h, int d,
                     double eps, double* out) {
  const double* rows[4];
  for (int m = 0; m < 4; ++m) {
    const int64_t src = t - 3 + m;
    rows[m] = src < bos ? NULL : x + ((size_t)src * H + h) * d;
  }
  conv_silu_l2(rows, w + (size_t)h * d * 4, d, eps, out);
}

static void epilogue(double* o, const double* gate, const double* norm_w, int dv, double eps) {
  double ms = 0.0;
  for (int j = 0; j < dv; ++j) ms += o[j] * o[j];
  ms /= (double)dv;
  const double inv = 1.0 / sqrt(ms + eps);
  for (int j = 0; j < dv; ++j) {
    const double w = norm_w ? norm_w[j] : 1.0;
    o[j] = o[j] * inv * w * (1.0 / (1.0 + exp(-gate[j])));
  }
}

int kda_oracle_chunk_fwd(const double* q, const double* k, const double* v, const double* log_alpha,
                         const double* beta, const double* initial_state, const int64_t* cu_seqlens,
                         int num_seqs, int64_t total_tokens, int H, int dk, int dv,
                         const double* conv_q_w, const double* conv_k_w, const double* gate,
                         const double* norm_w, double l2_eps, double rms_eps, double* o,
                         double* final_state, int num_threads) {
  if (num_seqs < 1 || H < 1 || dk < 1 || dv < 1 || total_tokens < 0) return 1;
  if (!cu_seqlens && num_seqs != 1) return 1;
  const int64_t units = (int64_t)num_seqs * H;
  const int nth = team_size(num_threads);
  (void)nth; /* used by the parallel-for clause */
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nth)
  for (int64_t u = 0; u < units; ++u) {
    const int n = (int)(u / H), h = (int)(u % H);
    const int64_t bos = cu_seqlens ? cu_seqlens[n] : 0;
    const int64_t eos = cu_seqlens ? cu_seqlens[n + 1] : total_tokens;
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)dv);
    double* qb = (double*)malloc(sizeof(double) * (size_t)dk);
    double* kb = (double*)malloc(sizeof(double) * (size_t)dk);
    if (!S || !tmp || !qb || !kb) {
#pragma omp atomic write
      err = 2;
      free(S); free(tmp); free(qb); free(kb);
      continue;
    }
    const size_t soff = ((size_t)n * H + h) * (size_t)dk * dv;
    if (initial_state)
      memcpy(S, initial_state + soff, sizeof(double) * (size_t)dk * dv);
    else
      memset(S, 0, sizeof(double) * (size_t)dk * dv);
    for (int64_t t = bos; t < eos; ++t) {
      const size_t tk = ((size_t)t * H + h) * dk, tv = ((size_t)t * H + h) * dv;
      const double* qt = q + tk;
      const double* kt = k + tk;
      if (conv_q_w) { prologue(q, conv_q_w, bos, t, H, h, dk, l2_eps, qb); qt = qb; }
      if (conv_k_w) { prologue(k, conv_k_w, bos, t, H, h, dk, l2_eps, kb); kt = kb; }
      kda_token(S, dk, dv, qt, kt, v + tv, log_alpha + tk, beta[(size_t)t * H + h], tmp, o + tv);
      if (gate) epilogue(o + tv, gate + tv, norm_w, dv, rms_eps);
    }
    if (final_state) memcpy(final_state + soff, S, sizeof(double) * (size_t)dk * dv);
    free(S); free(tmp); free(qb); free(kb);
  }
  return err;
}

/* One decode token per (n, h): the same token body, state updated in place. */
int kda_oracle_decode_step(double* state, const double* q, const double* k, const double* v,
                           const double* log_alpha, const double* beta, int num_seqs, int H, int dk,
                           int dv, double* o, int num_threads) {
  if (num_seqs < 1 || H < 1 || dk < 1 || dv < 1) return 1;
  const int64_t units = (int64_t)num_seqs * H;
  const int nth = team_size(num_threads);
  (void)nth; /* used by the parallel-for clause */
  int err = 0;
#pragma omp parallel for schedule(static) num_threads(nth)
  for (int64_t u = 0; u < units; ++u) {
    double* tmp = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!tmp) {
#pragma omp atomic write
      err = 2;
      continue;
    }
    kda_token(state + (size_t)u * dk * dv, dk, dv, q + (size_t)u * dk, k + (size_t)u * dk,
              v + (size_t)u * dv, log_alpha + (size_t)u * dk, beta[u], tmp, o + (size_t)u * dv);
    free(tmp);
  }
  return err;
}

/* Multi-token decode from cached per-token inputs: the replay of accepted
 * draft tokens in speculative decoding ("Kimi K3 架构、训练与系统全景解析",
 * section 7.4, KDA state replay under speculative decoding: keep the small
 * per-token inputs instead of one state per draft position, replay the
 * accepted prefix from the verified state, write back only the final state;
 * the short convolution, the norms, the gate and the recurrence run together).
 *
 * For each (n, h): from state_in (zeros if NULL), the token body above over
 * tokens 0 .. nt-1 of sequence n's L cached tokens, nt = ntok[n] clamped to
 * [0, L] (L when ntok is NULL).  The prologue's convolution of token t reads
 * raw rows t-3 .. t; rows before token 0 come from the history [N, 3, H, dk]
 * (oldest first; a NULL history is zeros, as at a sequence start).
 * Layouts: q, k, log_alpha [N, L, H, dk]; v, gate, o [N, L, H, dv];
 * beta [N, L, H]; states [N, H, dk, dv].  Writes o for the tokens run (the
 * other rows are not touched), the state after them (state_out, if given) and
 * the raw rows just before token nt (conv_*_out, if given: the history the
 * next call continues from). */
static const double* raw_row(const double* x, const double* hist, int n, int L, int H, int h, int d, int pos) {
  if (pos >= 0) return x + (((size_t)n * L + pos) * H + h) * d;
  if (!hist) return NULL;
  return hist + (((size_t)n * 3 + (3 + pos)) * H + h) * d;
}

int kda_oracle_decode_multi(const double* state_in, const double* q, const double* k, const double* v,
                            const double* log_alpha, const double* beta, const int64_t* ntok, int num_seqs,
                            int L, int H, int dk, int dv, const double* conv_q_w, const double* conv_k_w,
                            const double* conv_q_hist, const double* conv_k_hist, const double* gate,
                            const double* norm_w, double l2_eps, double rms_eps, double* o, double* state_out,
                            double* conv_q_out, double* conv_k_out, int num_threads) {
  if (num_seqs < 1 || L < 1 || H < 1 || dk < 1 || dv < 1) return 1;
  const int64_t units = (int64_t)num_seqs * H;
  const int nth = team_size(num_threads);
  (void)nth; /* used by the parallel-for clause */
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nth)
  for (int64_t u = 0; u < units; ++u) {
    const int n = (int)(u / H), h = (int)(u % H);
    int nt = L;
    if (ntok) nt = ntok[n] < 0 ? 0 : (ntok[n] > L ? L : (int)ntok[n]);
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)dv);
    double* qb = (double*)malloc(sizeof(double) * (size_t)dk);
    double* kb = (double*)malloc(sizeof(double) * (size_t)dk);
    if (!S || !tmp || !qb || !kb) {
#pragma omp atomic write
      err = 2;
      free(S); free(tmp); free(qb); free(kb);
      continue;
    }
    const size_t soff = (size_t)u * dk * dv;
    if (state_in)
      memcpy(S, state_in + soff, sizeof(double) * (size_t)dk * dv);
    else
      memset(S, 0, sizeof(double) * (size_t)dk * dv);
    for (int t = 0; t < nt; ++t) {
      const size_t tk = (((size_t)n * L + t) * H + h) * dk, tv = (((size_t)n * L + t) * H + h) * dv;
      const double* qt = q + tk;
      const double* kt = k + tk;
      const double* rows[4];
      if (conv_q_w) {
        for (int m = 0; m < 4; ++m) rows[m] = raw_row(q, conv_q_hist, n, L, H, h, dk, t - 3 + m);
        conv_silu_l2(rows, conv_q_w + (size_t)h * dk * 4, dk, l2_eps, qb);
        qt = qb;
      }
      if (conv_k_w) {
        for (int m = 0; m < 4; ++m) rows[m] = raw_row(k, conv_k_hist, n, L, H, h, dk, t - 3 + m);
        conv_silu_l2(rows, conv_k_w + (size_t)h * dk * 4, dk, l2_eps, kb);
        kt = kb;
      }
      kda_token(S, dk, dv, qt, kt, v + tv, log_alpha + tk, beta[((size_t)n * L + t) * H + h], tmp, o + tv);
      if (gate) epilogue(o + tv, gate + tv, norm_w, dv, rms_eps);
    }
    if (state_out) memcpy(state_out + soff, S, sizeof(double) * (size_t)dk * dv);
    for (int r = 0; r < 3; ++r) {
      const size_t hoff = (((size_t)n * 3 + r) * H + h) * dk;
      const double* sq = raw_row(q, conv_q_hist, n, L, H, h, dk, nt - 3 + r);
      const double* sk = raw_row(k, conv_k_hist, n, L, H, h, dk, nt - 3 + r);
      for (int j = 0; j < dk; ++j) {
        if (conv_q_out) conv_q_out[hoff + j] = sq ? sq[j] : 0.0;
        if (conv_k_out) conv_k_out[hoff + j] = sk ? sk[j] : 0.0;
      }
    }
    free(S); free(tmp); free(qb); free(kb);
  }
  return err;
}

/* Backward pass (gradients) of the per-token recurrence above, without the
 * prologue and epilogue.  "Kimi K3 架构、训练与系统全景解析", section 7.1
 * (FlashKDA): the chunked KDA kernel serves training as well as prefill, so
 * the recurrence needs its gradients.  The pages give no formula for them;
 * this is the exact derivative of the forward definition for the loss
 *
 *   L = sum_t <do_t, o_t> + <dS_T, S_T>        (dS_T = d_final_state, or 0)
 *
 * taken by reverse accumulation through the token body's own steps.  With
 * S the state before token t, Sp = Diag(a) S, vhat = Sp^T k, u = beta (v - vhat),
 * S_t = Sp + k u^T and o_t = S_t^T q, and dS the gradient reaching S_t:
 *
 *   dq   = S_t do                     dS  += q do^T
 *   dk   = dS u                       du   = dS^T k
 *   dbeta = <du, v - vhat>            dv   = beta du          dvhat = -beta du
 *   dSp  = dS + k dvhat^T             dk  += Sp dvhat
 *   dlog_alpha_i = a_i sum_j dSp[i][j] S[i][j]                (a_i = exp(log_alpha_i))
 *   gradient reaching S:  Diag(a) dSp
 *
 * and d_initial_state is the gradient that reaches S_0.  States are
 * recomputed forward from checkpoints every BWD_SEG tokens (the recurrence
 * cannot be run backwards: beta = 1 erases).  Layouts as the forward;
 * d_o [T,H,dv], d_final_state [N,H,dk,dv] or NULL (zero); outputs dq, dk,
 * dlog_alpha [T,H,dk], dv [T,H,dv], dbeta [T,H], d_initial_state
 * [N,H,dk,dv] (or NULL: not written).  OpenMP over (sequence, head). */
#define BWD_SEG 64

int kda_oracle_chunk_bwd(const double* q, const double* k, const double* v, const double* log_alpha,
                         const double* beta, const double* initial_state, const int64_t* cu_seqlens,
                         int num_seqs, int64_t total_tokens, int H, int dk, int dv, const double* d_o,
                         const double* d_final_state, double* dq, double* dkk, double* dvv, double* dlog_alpha,
                         double* dbeta, double* d_initial_state, int num_threads) {
  if (num_seqs < 1 || H < 1 || dk < 1 || dv < 1 || total_tokens < 0) return 1;
  if (!cu_seqlens && num_seqs != 1) return 1;
  const int64_t units = (int64_t)num_seqs * H;
  const size_t SZ = (size_t)dk * dv;
  const int nth = team_size(num_threads);
  (void)nth; /* used by the parallel-for clause */
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nth)
  for (int64_t un = 0; un < units; ++un) {
    const int n = (int)(un / H), h = (int)(un % H);
    const int64_t bos = cu_seqlens ? cu_seqlens[n] : 0;
    const int64_t eos = cu_seqlens ? cu_seqlens[n + 1] : total_tokens;
    const int64_t len = eos - bos;
    const int64_t nseg = (len + BWD_SEG - 1) / BWD_SEG;
    /* checkpoints: the state before each segment; states of one segment */
    double* ck = (double*)malloc(sizeof(double) * SZ * (size_t)(nseg > 0 ? nseg : 1));
    double* st = (double*)malloc(sizeof(double) * SZ * (BWD_SEG + 1));
    double* dS = (double*)malloc(sizeof(double) * SZ);
    double* Sp = (double*)malloc(sizeof(double) * SZ);
    double* w = (double*)malloc(sizeof(double) * (size_t)(3 * dv + dk));
    if (!ck || !st || !dS || !Sp || !w) {
#pragma omp atomic write
      err = 2;
      free(ck); free(st); free(dS); free(Sp); free(w);
      continue;
    }
    double *vhat = w, *u = w + dv, *du = w + 2 * dv, *dvhat = du; /* dvhat reuses du's slot after use */
    double* scratch_k = w + 3 * dv;
    (void)scratch_k;
    const size_t soff = ((size_t)n * H + h) * SZ;
    /* forward sweep: checkpoints only */
    double* S = st;
    if (initial_state)
      memcpy(S, initial_state + soff, sizeof(double) * SZ);
    else
      memset(S, 0, sizeof(double) * SZ);
    for (int64_t sg = 0; sg < nseg; ++sg) {
      memcpy(ck + (size_t)sg * SZ, S, sizeof(double) * SZ);
      const int64_t t1 = bos + (sg + 1) * BWD_SEG < eos ? bos + (sg + 1) * BWD_SEG : eos;
      for (int64_t t = bos + sg * BWD_SEG; t < t1; ++t) {
        const size_t tk = ((size_t)t * H + h) * dk, tv = ((size_t)t * H + h) * dv;
        kda_token(S, dk, dv, q + tk, k + tk, v + tv, log_alpha + tk, beta[(size_t)t * H + h], vhat, u);
      }
    }
    /* reverse sweep */
    if (d_final_state)
      memcpy(dS, d_final_state + soff, sizeof(double) * SZ);
    else
      memset(dS, 0, sizeof(double) * SZ);
    for (int64_t sg = nseg - 1; sg >= 0; --sg) {
      const int64_t t0 = bos + sg * BWD_SEG;
      const int64_t t1 = t0 + BWD_SEG < eos ? t0 + BWD_SEG : eos;
      /* st[i] = state before token t0 + i, st[i + 1] = after it */
      memcpy(st, ck + (size_t)sg * SZ, sizeof(double) * SZ);
      for (int64_t t = t0; t < t1; ++t) {
        const size_t tk = ((size_t)t * H + h) * dk, tv = ((size_t)t * H + h) * dv;
        double* nxt = st + (size_t)(t - t0 + 1) * SZ;
        memcpy(nxt, st + (size_t)(t - t0) * SZ, sizeof(double) * SZ);
        kda_token(nxt, dk, dv, q + tk, k + tk, v + tv, log_alpha + tk, beta[(size_t)t * H + h], vhat, u);
      }
      for (int64_t t = t1 - 1; t >= t0; --t) {
        const size_t tk = ((size_t)t * H + h) * dk, tv = ((size_t)t * H + h) * dv;
        const double* S0 = st + (size_t)(t - t0) * SZ;     /* before token t */
        const double* S1 = st + (size_t)(t - t0 + 1) * SZ; /* after token t  */
        const double* qt = q + tk;
        const double* kt = k + tk;
        const double* vt = v + tv;
        const double* la = log_alpha + tk;
        const double* dot = d_o + tv;
        const double bt = beta[(size_t)t * H + h];
        /* recompute Sp, vhat, u of this token */
        for (int i = 0; i < dk; ++i) {
          const double a = exp(la[i]);
          for (int j = 0; j < dv; ++j) Sp[(size_t)i * dv + j] = a * S0[(size_t)i * dv + j];
        }
        for (int j = 0; j < dv; ++j) vhat[j] = 0.0;
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < dv; ++j) vhat[j] += Sp[(size_t)i * dv + j] * kt[i];
        for (int j = 0; j < dv; ++j) u[j] = bt * (vt[j] - vhat[j]);
        /* o_t = S_t^T q:  dq = S_t do,  dS += q do^T */
        for (int i = 0; i < dk; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) acc += S1[(size_t)i * dv + j] * dot[j];
          dq[tk + i] = acc;
          for (int j = 0; j < dv; ++j) dS[(size_t)i * dv + j] += qt[i] * dot[j];
        }
        /* S_t = Sp + k u^T:  dk = dS u,  du = dS^T k */
        for (int j = 0; j < dv; ++j) du[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) {
            acc += dS[(size_t)i * dv + j] * u[j];
            du[j] += dS[(size_t)i * dv + j] * kt[i];
          }
          dkk[tk + i] = acc;
        }
        /* u = beta (v - vhat) */
        double db = 0.0;
        for (int j = 0; j < dv; ++j) {
          db += du[j] * (vt[j] - vhat[j]);
          dvv[tv + j] = bt * du[j];
          dvhat[j] = -bt * du[j]; /* overwrites du in place */
        }
        dbeta[(size_t)t * H + h] = db;
        /* vhat = Sp^T k:  dSp = dS + k dvhat^T,  dk += Sp dvhat */
        for (int i = 0; i < dk; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) acc += Sp[(size_t)i * dv + j] * dvhat[j];
          dkk[tk + i] += acc;
          for (int j = 0; j < dv; ++j) dS[(size_t)i * dv + j] += kt[i] * dvhat[j];
        }
        /* Sp = Diag(a) S:  dlog_alpha_i = a_i <dSp[i], S[i]>,  dS <- Diag(a) dSp */
        for (int i = 0; i < dk; ++i) {
          const double a = exp(la[i]);
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) acc += dS[(size_t)i * dv + j] * S0[(size_t)i * dv + j];
          dlog_alpha[tk + i] = a * acc;
          for (int j = 0; j < dv; ++j) dS[(size_t)i * dv + j] *= a;
        }
      }
    }
    if (d_initial_state) memcpy(d_initial_state + soff, dS, sizeof(double) * SZ);
    free(ck); free(st); free(dS); free(Sp); free(w);
  }
  return err;
}

/* Number of threads an OpenMP parallel region would use (1 without OpenMP). */
int kda_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
