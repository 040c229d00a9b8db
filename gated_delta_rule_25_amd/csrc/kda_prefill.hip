// kda_prefill.hip — chunkwise-parallel KDA prefill for gfx950.
//
// Method ("Kimi K3 架构、训练与系统全景解析", section 4.2.4: inside a chunk the
// causal token interactions become lower-triangular matrix products, across
// chunks the state is carried recurrently, and the output is a history term
// plus an intra-chunk term; section 4.2.5: the decay is bounded below so the
// cumulative log-decay over a 16-token tile stays in [-80, 0] and every tile,
// diagonal ones included, can use dense matrix-core products).
//
// For a chunk of n <= C tokens with incoming state S and per-channel
// cumulative log-decay g_r = sum_{i<=r} log_alpha_i (within the chunk):
//   Kt = K (.) e^{g},  Qt = Q (.) e^{g},  Kh = K (.) e^{-g},  Kb = K (.) e^{g_n - g}
//   A  = strictly-lower( Diag(beta) Kt Kh^T ),   T = (I + A)^{-1} Diag(beta)
//   W  = T Kt,   U' = T V,   U = U' - W S
//   O  = Qt S + lower-incl( Qt Kh^T ) U
//   S <- Diag(e^{g_n}) S + Kb^T U
// This is the per-token update of the header kda.h summed over the chunk in
// closed form (the triangular solve is the UT/WY transform the analysis page
// attributes to Kimi Linear; derivation in the design notes).  The products
// Kt Kh^T and Qt Kh^T are formed per 16-token tile pair (a, b <= a) relative
// to rho_a, the cumulative decay just before tile a: the row factor
// e^{g_r - rho_a} is <= 1 and the column factor e^{rho_a - g_i} is <= 1 off
// the diagonal and <= e^{80} on it, so nothing overflows in fp32 or bf16.
//
// Mapping.  One 256-thread workgroup (4 waves) per (sequence, head, value
// column block); the block's slice of the 128 x DV fp32 state lives in MFMA
// accumulators for the whole sequence (wave w owns DV/4 columns, all 128
// rows).  Chunks are walked in order.  Per chunk: (1) prep, independent of S:
// decay prefix sums, scaled operand tiles in LDS, the Gram tiles on MFMA, the
// unit-triangular inverse in fp32, W and U' on MFMA; (2) the carried part:
// U, O and the new S, with S and U fed to the matrix cores straight from
// registers (d-permuted operand order, see kda_device.h).
// Work items are ordered longest sequence first, and the column blocks of one
// (sequence, head) land on the same XCD so they share its L2 for K, Q and the
// decay.
#include "kda_chunk_util.h"

namespace kda {

template <typename E, int C, int DV, bool PRO, bool EPI>
__global__ __launch_bounds__(256) void prefill_kernel(const PrefillArgs p) {
  using L = PrefillLayout<E, C, DV>;
  constexpr bool SPLIT = L::SPLIT;
  constexpr int NT = C / 16;     // 16-token tiles per chunk
  constexpr int KT = C / 32;     // 32-deep token steps per chunk
  constexpr int NCW = DV / 4;    // value columns per wave
  constexpr int NCT = NCW / 16;  // 16-wide column tiles per wave
  constexpr int LDK = L::LDK, LDT = L::LDT;
  static_assert(!EPI || DV == D, "the epilogue normalises whole heads");
  static_assert(NCT >= 1 && KT >= 1 && NT <= 4, "unsupported tile shape");

  extern __shared__ __align__(16) unsigned char smem[];
  E* sKrel = reinterpret_cast<E*>(smem + L::S_KR);
  E* sKih = reinterpret_cast<E*>(smem + L::S_KIH);
  E* sKil = reinterpret_cast<E*>(smem + L::S_KIL);   // used only when SPLIT
  E* sQrh = reinterpret_cast<E*>(smem + L::S_QRH);   // Q_rel, then Qt in place
  E* sQrl = reinterpret_cast<E*>(smem + L::S_QRL);   // used only when SPLIT
  E* sP = reinterpret_cast<E*>(smem + L::R_P);
  E* sM = reinterpret_cast<E*>(smem + L::R_M);
  float* sAd = reinterpret_cast<float*>(smem + L::O_AD);
  E* sW = reinterpret_cast<E*>(smem + L::R_W);
  E* sKtt = reinterpret_cast<E*>(smem + L::O_KTT);   // beta * Kt, channel-major
  E* sKbt = reinterpret_cast<E*>(smem + L::O_KBT);
  E* sVt = reinterpret_cast<E*>(smem + L::O_VT);     // beta * V, column-major
  E* sQt = L::QT_OWN ? reinterpret_cast<E*>(smem + L::O_QT) : sQrh;
  float* sTot = reinterpret_cast<float*>(smem + L::O_TOT);
  float* sEf = reinterpret_cast<float*>(smem + L::O_EF);
  float* sEra = reinterpret_cast<float*>(smem + L::O_ERA);
  float* sGam = reinterpret_cast<float*>(smem + L::O_GAM);
  float* sBeta = reinterpret_cast<float*>(smem + L::O_BETA);
  float* sSS = reinterpret_cast<float*>(smem + L::O_SS);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, g = lane >> 4;
  // XCD-aware decode of the work item: blocks b and b + 8 run on the same XCD.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int cb = slot % p.col_split;
  const int u = (slot / p.col_split) * 8 + xcd;
  if (u >= p.units) return;
  const int H = p.num_heads;
  const int rnk = u / H, h = u % H;
  int n = rnk, seg = 0;
  if (p.mode == 0) {
    if (p.order) n = p.order[rnk];
  } else {
    if (rnk >= *p.seg_count) return;
    n = p.seg_list[2 * rnk];
    seg = p.seg_list[2 * rnk + 1];
  }
  const int64_t seq_bos = p.cu ? (int64_t)p.cu[n] : 0;
  const int64_t seq_eos = p.cu ? (int64_t)p.cu[n + 1] : p.total_tokens;
  // this work item's token range: the whole sequence, or one segment of it
  const int64_t bos = p.mode == 0 ? seq_bos : seq_bos + (int64_t)seg * p.seg_len;
  const int64_t eos = p.mode == 0 ? seq_eos : min(seq_eos, bos + (int64_t)p.seg_len);
  const int64_t rs = (int64_t)H * D;  // elements between consecutive tokens
  const int64_t hoff = (int64_t)h * D;
  // mode 1: blocks [0, col_split/2) carry V from a zero state (B); the others
  // carry the identity with V = 0 (M)
  const int half = p.mode == 1 ? p.col_split / 2 : p.col_split;
  const int cbv = cb % half;
  const bool mpart = p.mode == 1 && cb >= half;
  const bool write_o = p.mode != 1;
  const size_t pair_base = ((size_t)rnk * H + h) * (size_t)(2 * D * D);
  const int col0 = cbv * DV + wv * NCW;  // first value column owned by this wave

  const E* gq = static_cast<const E*>(p.q);
  const E* gk = static_cast<const E*>(p.k);
  const E* gv = static_cast<const E*>(p.v);
  E* go = static_cast<E*>(p.o);

  // State slice: tile (rt8, ct) holds rows 16 rt8 + 4g + i, column col0 + 16 ct + l16.
  f32x4 accS[8][NCT];
  const size_t sbase = ((size_t)n * H + h) * (size_t)(D * D);
  const float* init = p.mode == 0 ? (p.init ? p.init + sbase : nullptr)
                    : p.mode == 2 ? p.pairs + pair_base : nullptr;
  float* fin = p.mode == 0 ? (p.fin ? p.fin + sbase : nullptr)
             : p.mode == 1 ? p.pairs + pair_base + (mpart ? D * D : 0) : nullptr;
#pragma unroll
  for (int rt8 = 0; rt8 < 8; ++rt8)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * rt8 + 4 * g + i, col = col0 + 16 * ct + l16;
        accS[rt8][ct][i] = init ? init[(size_t)row * D + col] : ((mpart && row == col) ? 1.f : 0.f);
      }

  // Prep role: channel group cg (channels 8cg .. 8cg+7) and token group tg
  // (chunk rows TPL*tg .. +TPL-1).  The 16 lanes of a lane group hold one set
  // of rows across all 128 channels; wave w holds rows 4*TPL*w .. +4*TPL-1,
  // i.e. one 16-token tile (C = 64) or half of one (C = 32).
  constexpr int TPL = C / 16;       // rows per prep thread
  constexpr int WPT = 4 / TPL;      // waves per 16-token tile
  const int cg = tid & 15, tg = tid >> 4, lg = g;
  const int c8 = 8 * cg, r0 = TPL * tg;
  float wq[8][4], wk[8][4];
  if (PRO) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        wq[j][m] = p.conv_q_w ? p.conv_q_w[(hoff + c8 + j) * 4 + m] : (m == 3 ? 1.f : 0.f);
        wk[j][m] = p.conv_k_w ? p.conv_k_w[(hoff + c8 + j) * 4 + m] : (m == 3 ? 1.f : 0.f);
      }
  }

  // Global inputs of one chunk held by this thread (see Raw8).
  constexpr int QR = TPL + (PRO ? 3 : 0);  // q / k rows (with conv history)
  constexpr int VCG = DV / 8, VTPL = C * VCG / 256;
  const int vcg = tid % VCG, vtg = tid / VCG;
  Raw8<float> rla[TPL];
  Raw8<E> rq[QR], rk[QR], rv[VTPL];
  float rvb[VTPL], rb = 0.f;
  auto issue_loads = [&](int64_t tc) {
    const int nvc = (int)((eos - tc) < C ? (eos - tc) : C);
    const int64_t cb0 = tc * rs + hoff;
#pragma unroll
    for (int i = 0; i < TPL; ++i) ld_raw8(rla[i], p.log_alpha + cb0 + (int64_t)min(r0 + i, nvc - 1) * rs + c8);
    const int64_t back = seq_bos - tc;  // <= 0
    const int loc = back < -3 ? -3 : (int)back;
#pragma unroll
    for (int i = 0; i < QR; ++i) {
      const int row = PRO ? min(max(r0 - 3 + i, loc), nvc - 1) : min(r0 + i, nvc - 1);
      ld_raw8(rq[i], gq + cb0 + (int64_t)row * rs + c8);
      ld_raw8(rk[i], gk + cb0 + (int64_t)row * rs + c8);
    }
#pragma unroll
    for (int i = 0; i < VTPL; ++i) {
      const int row = min(VTPL * vtg + i, nvc - 1);
      ld_raw8(rv[i], gv + cb0 + (int64_t)row * rs + cbv * DV + 8 * vcg);
      rvb[i] = p.beta[(tc + row) * H + h];
    }
    if (tid < C) rb = p.beta[(tc + min(tid, nvc - 1)) * H + h];
  };
  if (bos < eos) issue_loads(bos);

  for (int64_t t0 = bos; t0 < eos; t0 += C) {
    const int nv = (int)((eos - t0) < C ? (eos - t0) : C);
    // Per-lane indices are re-derived from an opaque copy of the thread id in
    // every chunk, so the LDS address arithmetic of the unrolled stages stays
    // inside the loop instead of being hoisted into registers for the whole
    // sequence.
    int tidv = tid;
    asm volatile("" : "+v"(tidv));
    const int lane = tidv & 63, l16 = lane & 15, g = lane >> 4;
    const int cg = tidv & 15, tg = tidv >> 4, lg = g;
    const int c8 = 8 * cg, r0 = TPL * tg;
    const int vcg = tidv % VCG, vtg = tidv / VCG;

    // ---- P1: log-decay prefix sums relative to the first row of this wave ----
    // decay kept in log2 units: every factor below is one exp2
    const bool full = (nv == C);
    float dl[TPL][8];
    rows_from_raw<float, TPL>(dl, rla, r0, nv, full);
#pragma unroll
    for (int i = 0; i < TPL; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) dl[i][j] *= 1.4426950408889634f;
    {
#pragma unroll
      for (int i = 1; i < TPL; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) dl[i][j] += dl[i - 1][j];
      // exclusive prefix over the four lane groups (same channels, earlier rows)
      float inc[8], tot[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        tot[j] = dl[TPL - 1][j];
        float x = tot[j];
        const float y1 = __shfl_up(x, 16);
        if (lg >= 1) x += y1;
        const float y2 = __shfl_up(x, 32);
        if (lg >= 2) x += y2;
        inc[j] = x;
      }
#pragma unroll
      for (int i = 0; i < TPL; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) dl[i][j] += inc[j] - tot[j];
      if (lg == 3) st8(sTot + wv * D + c8, inc);  // total of this wave's rows
    }

    // ---- P2: q and k rows (raw, or through the prologue), beta V^T, beta ----
    float qv[TPL][8], kv[TPL][8];
    {
      if (PRO) {
        const int64_t back = seq_bos - t0;  // <= 0
        const int lo = back < -3 ? -3 : (int)back;
        if (p.conv_q_w)
          prologue_from_raw<E, TPL>(qv, rq, r0, nv, lo, wq, p.l2_eps);
        else
          rows_from_raw<E, TPL>(qv, rq + (QR - TPL), r0, nv, full);
        if (p.conv_k_w)
          prologue_from_raw<E, TPL>(kv, rk, r0, nv, lo, wk, p.l2_eps);
        else
          rows_from_raw<E, TPL>(kv, rk + (QR - TPL), r0, nv, full);
      } else {
        rows_from_raw<E, TPL>(qv, rq, r0, nv, full);
        rows_from_raw<E, TPL>(kv, rk, r0, nv, full);
      }
      // beta V^T: thread (vcg, vtg) moves columns 8 vcg .. +7 of rows VTPL*vtg .. +VTPL-1
      float vv[VTPL][8];
      rows_from_raw<E, VTPL>(vv, rv, VTPL * vtg, nv, full);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float col[VTPL];
#pragma unroll
        for (int i = 0; i < VTPL; ++i) col[i] = mpart ? 0.f : vv[i][j] * rvb[i];   // rows past nv are already zero
        stN<VTPL>(sVt + cm_off<C, LDT>(8 * vcg + j, VTPL * vtg), col);
      }
      if (tid < C) sBeta[tid] = (tid < nv) ? rb : 0.f;
    }
    __syncthreads();

    // ---- P3: scaled operand tiles ----
    {
      // rho_a = cumulative log-decay before tile a, for this thread's 8 channels
      float wt[4][8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(sTot + w * D + c8);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(sTot + w * D + c8 + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wt[w][j] = x0[j];
          wt[w][j + 4] = x1[j];
        }
      }
      float rho[NT + 1][8];
#pragma unroll
      for (int j = 0; j < 8; ++j) rho[0][j] = 0.f;
#pragma unroll
      for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float t = 0.f;
#pragma unroll
          for (int w = a * WPT; w < (a + 1) * WPT; ++w) t += wt[w][j];
          rho[a + 1][j] = rho[a][j] + t;
        }
      const int my_a = wv / WPT;
      float ra[8], intra[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ra[j] = rho[0][j];
        intra[j] = 0.f;
      }
#pragma unroll
      for (int a = 1; a < NT; ++a)
        if (a == my_a)
#pragma unroll
          for (int j = 0; j < 8; ++j) ra[j] = rho[a][j];
      if (WPT == 2 && (wv & 1))
#pragma unroll
        for (int j = 0; j < 8; ++j) intra[j] = wt[wv - 1][j];
      float ea[8], eb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ea[j] = exp2_fast(ra[j]);                  // e^{rho_a} <= 1
        eb[j] = exp2_fast(rho[NT][j] - ra[j]);     // e^{g_n - rho_a} <= 1
      }
      float ktt[8][TPL], kbt[8][TPL];
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        const int rr = r0 + i;
        const float br = sBeta[rr];
        float xq[8], xk[8], xi[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float d = dl[i][j] + intra[j];   // g_r - rho_a, in [-80, 0]
          const float ep = exp2_fast(d), en = exp2_fast(-d);
          xq[j] = qv[i][j] * ep;
          xk[j] = kv[i][j] * ep;
          xi[j] = kv[i][j] * en;
          ktt[j][i] = xk[j] * ea[j] * br;   // beta Kt = beta K e^{g}
          kbt[j][i] = xi[j] * eb[j];   // Kb = K e^{g_n - g}
        }
        st8_split(sQrh + rr * LDK + c8, sQrl + rr * LDK + c8, xq);
        if constexpr (L::QT_OWN) {
          float xt[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) xt[j] = xq[j] * ea[j];   // Qt = Q e^{g}
          st8(sQt + rr * LDK + c8, xt);
        }
        st8_split(sKih + rr * LDK + c8, sKil + rr * LDK + c8, xi);
        st8(sKrel + rr * LDK + c8, xk);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        stN<TPL>(sKtt + cm_off<C, LDT>(c8 + j, r0), ktt[j]);
        stN<TPL>(sKbt + cm_off<C, LDT>(c8 + j, r0), kbt[j]);
      }
      if (tg == 0) {
        float v8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v8[j] = exp2_fast(rho[NT][j]);
        st8(sGam + c8, v8);
#pragma unroll
        for (int a = 0; a < NT; ++a) {
#pragma unroll
          for (int j = 0; j < 8; ++j) v8[j] = exp2_fast(rho[a][j]);
          st8(sEra + a * D + c8, v8);
        }
#pragma unroll
        for (int a = 1; a < NT; ++a)
#pragma unroll
          for (int b = 0; b < a; ++b) {
#pragma unroll
            for (int j = 0; j < 8; ++j) v8[j] = exp2_fast(rho[a][j] - rho[b][j]);
            st8(sEf + off_idx(a, b) * D + c8, v8);
          }
      }
    }
    __syncthreads();

    // ---- P5: Gram tiles per 16-token tile pair (a, b <= a):
    //      A_ab = Krel_a Kh_ab^T,  P_ab = Qrel_a Kh_ab^T  with Kh_ab = K_inv_b (.) e^{rho_a - rho_b}.
    //      Wave w takes the diagonal pair (w, w) and the strictly-lower pairs q = w, w + 4.
    //      With bf16 operands P is formed from the hi + lo parts of Q_rel, and of
    //      K_inv on the diagonal (where it is not rescaled).
    // ---- P6: each wave then inverts its own diagonal block, (I + A_ww)^{-1},
    //      by fp32 forward substitution (lane j < 16 solves column j) while the
    //      other waves are still on their Gram products.
    {
      constexpr int NOFF = L::NOFF;
      constexpr int PPW = 1 + (NOFF + 3) / 4;  // pairs per wave (first one diagonal)
      f32x4 ga[PPW], gp[PPW];
      int pa[PPW], pb[PPW];
#pragma unroll
      for (int j = 0; j < PPW; ++j) {
        ga[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        gp[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        const int q = wv + 4 * (j - 1);
        const bool valid = (j == 0) ? (wv < NT) : (q < NOFF);
        pa[j] = -1;
        pb[j] = -1;
        if (valid) {
          const int a = (j == 0) ? wv : off_a(q), b = (j == 0) ? wv : off_b(q);
          pa[j] = a;
          pb[j] = b;
          const int arow = (16 * a + l16) * LDK + 8 * g, brow = (16 * b + l16) * LDK + 8 * g;
          const float* ef = sEf + (b < a ? off_idx(a, b) : 0) * D + 8 * g;
#pragma unroll
          for (int s = 0; s < D / 32; ++s) {
            Frag<E> fk, fq, fbh;
            ld_frag(fk, sKrel + arow + 32 * s);
            ld_frag(fq, sQrh + arow + 32 * s);
            ld_frag(fbh, sKih + brow + 32 * s);
            if (b < a) {
              float x[8];
              frag_unpack(fbh, x);
#pragma unroll
              for (int jj = 0; jj < 8; ++jj) x[jj] *= ef[32 * s + jj];
              frag_from_f32(fbh, x);
            }
            ga[j] = mma(ga[j], fk, fbh);
            gp[j] = mma(gp[j], fq, fbh);
            if constexpr (SPLIT) {
              Frag<E> fql;
              ld_frag(fql, sQrl + arow + 32 * s);
              gp[j] = mma(gp[j], fql, fbh);
              if (b == a) {
                Frag<E> fbl;
                ld_frag(fbl, sKil + brow + 32 * s);
                gp[j] = mma(gp[j], fq, fbl);
              }
            }
          }
          if (j == 0) {
            // Diag(beta) A_ww, strictly lower, to this wave's own fp32 block
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 16 * a + 4 * g + i;
              sAd[(a * 16 + 4 * g + i) * L::AST + l16] = (l16 < 4 * g + i) ? ga[0][i] * sBeta[r] : 0.f;
            }
          }
        }
      }
      float xinv[16];  // column `lane` of (I + A_ww)^{-1} (lanes < 16 of waves < NT)
      if (wv < NT && lane < 16) {
        const float* ab = sAd + wv * 16 * L::AST;
        f32x4 av[16][4];
#pragma unroll
        for (int r = 1; r < 16; ++r)
#pragma unroll
          for (int q4 = 0; q4 < (r + 3) / 4; ++q4) av[r][q4] = *reinterpret_cast<const f32x4*>(ab + r * L::AST + 4 * q4);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // four partial sums keep the dependency chains short
          float part[4] = {(r == lane) ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q4 = 0; q4 < (r + 3) / 4; ++q4)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (4 * q4 + e < r) part[e] -= av[r][q4][e] * xinv[4 * q4 + e];
          xinv[r] = (part[0] + part[1]) + (part[2] + part[3]);
        }
      }
      __syncthreads();  // every wave is done reading the Gram operands
      if (wv < NT && lane < 16)
#pragma unroll
        for (int r = 0; r < 16; ++r) sM[(16 * wv + r) * LDT + 16 * wv + lane] = from_f32<E>(xinv[r]);
#pragma unroll
      for (int j = 0; j < PPW; ++j) {
        const int a = pa[j], b = pb[j];
        if (a >= 0) {
          const int c = 16 * b + l16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * a + 4 * g + i;
            if (b < a) sM[r * LDT + c] = from_f32<E>(-ga[j][i] * sBeta[r]);   // -(Diag(beta) A)_ab
            sP[r * LDT + c] = from_f32<E>(((b < a) || (c <= r)) ? gp[j][i] : 0.f);
          }
        }
      }
      // strictly-upper tiles of P are read by the 32-deep token steps: zero them
      for (int e = tid; e < NOFF * 256; e += 256) {
        const int q = e >> 8, a = off_a(q), b = off_b(q);
        sP[(16 * b + ((e >> 4) & 15)) * LDT + 16 * a + (e & 15)] = from_f32<E>(0.f);
      }
      // Qt = (Q_rel hi + lo) e^{rho_a}, in place over the Q_rel slot (8 elements per step)
      if constexpr (!L::QT_OWN)
      for (int e = tid; e < C * (D / 8); e += 256) {
        const int r = e / (D / 8), c8 = (e % (D / 8)) * 8;
        float x[8];
        Frag<E> f;
        ld_frag(f, sQrh + r * LDK + c8);
        frag_unpack(f, x);
        if constexpr (SPLIT) {
          float lv[8];
          Frag<E> fl;
          ld_frag(fl, sQrl + r * LDK + c8);
          frag_unpack(fl, lv);
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) x[jj] += lv[jj];
        }
        const float* er = sEra + (r >> 4) * D + c8;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) x[jj] *= er[jj];
        frag_from_f32(f, x);
        st_frag(sQrh + r * LDK + c8, f);
      }
    }
    __syncthreads();

    // ---- P7: blocked forward substitution on the matrix cores,
    //      (I + A) [W | U'] = Diag(beta) [Kt | V], tile row by tile row:
    //      Y_a = (I + A_aa)^{-1} (beta R_a - sum_{b<a} A_ab Y_b).
    //      Wave w solves W columns 32w .. 32w+31 and its own U' columns, so
    //      every Y_b it needs is already in its registers.  W is stored
    //      negated for the carried stage. ----
    f32x4 accU[NT][NCT];
    {
      constexpr int NOWN = 2 + NCT;
      // all LDS operands of the solve are fetched up front
      Frag16<E> mfr[NT][NT], rfr[NOWN][NT];
#pragma unroll
      for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int b = 0; b <= a; ++b) ld_frag16(mfr[a][b], sM + (16 * a + l16) * LDT + 16 * b + 4 * g);
#pragma unroll
      for (int o = 0; o < NOWN; ++o)
#pragma unroll
        for (int a = 0; a < NT; ++a) {
          const E* src = (o < 2) ? sKtt + cm_off<C, LDT>(32 * wv + 16 * o + l16, 16 * a + 4 * g)
                                 : sVt + cm_off<C, LDT>(wv * NCW + 16 * (o - 2) + l16, 16 * a + 4 * g);
          ld_frag16(rfr[o][a], src);
        }
      f32x4 Y[NOWN][NT];
      Frag16<E> Yb[NOWN][NT];
#pragma unroll
      for (int a = 0; a < NT; ++a) {
        f32x4 z[NOWN];
#pragma unroll
        for (int o = 0; o < NOWN; ++o) z[o] = frag16_to_f32(rfr[o][a]);
#pragma unroll
        for (int b = 0; b < a; ++b)
#pragma unroll
          for (int o = 0; o < NOWN; ++o) z[o] = mma16(z[o], mfr[a][b], Yb[o][b]);
#pragma unroll
        for (int o = 0; o < NOWN; ++o) {
          Frag16<E> zb;
          frag16_from_acc(zb, z[o]);
          Y[o][a] = mma16((f32x4){0.f, 0.f, 0.f, 0.f}, mfr[a][a], zb);
          frag16_from_acc(Yb[o][a], Y[o][a]);
        }
      }
#pragma unroll
      for (int o = 0; o < 2; ++o)
#pragma unroll
        for (int a = 0; a < NT; ++a)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sW[(16 * a + 4 * g + i) * LDK + 32 * wv + 16 * o + l16] = from_f32<E>(-Y[o][a][i]);
#pragma unroll
      for (int a = 0; a < NT; ++a)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) accU[a][ct] = Y[2 + ct][a];
    }
    __syncthreads();  // W visible to every wave

    // the next chunk's inputs are loaded while this chunk's carried stage runs
    if (t0 + C < eos) issue_loads(t0 + C);

    // ---- S1: U = U' - W S ----
    Frag<E> sf[4][NCT];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) frag_from_acc(sf[ks][ct], accS[2 * ks][ct], accS[2 * ks + 1][ct]);
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        Frag<E> fa;
        ld_frag_perm(fa, sW + (16 * rt + l16) * LDK + 32 * ks + 4 * g);   // W is stored negated
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) accU[rt][ct] = mma(accU[rt][ct], fa, sf[ks][ct]);
      }

    // ---- S2: O = Qt S + P U ----
    f32x4 accO[NT][NCT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) accO[rt][ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        Frag<E> fa;
        ld_frag_perm(fa, sQt + (16 * rt + l16) * LDK + 32 * ks + 4 * g);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) accO[rt][ct] = mma(accO[rt][ct], fa, sf[ks][ct]);
      }
    Frag<E> uf[KT][NCT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) frag_from_acc(uf[kt][ct], accU[2 * kt][ct], accU[2 * kt + 1][ct]);
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        if (kt <= (16 * rt + 15) / 32) {
          Frag<E> fa;
          ld_frag_perm(fa, sP + (16 * rt + l16) * LDT + 32 * kt + 4 * g);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) accO[rt][ct] = mma(accO[rt][ct], fa, uf[kt][ct]);
        }
      }

    if (EPI && write_o) {
      // head-wise RMSNorm over the 128 value channels, then the sigmoid gate
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float ss = 0.f;
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) ss += accO[rt][ct][i] * accO[rt][ct][i];
#pragma unroll
          for (int m = 1; m < 16; m <<= 1) ss += __shfl_xor(ss, m);
          if (l16 == 0) sSS[wv * C + 16 * rt + 4 * g + i] = ss;
        }
      __syncthreads();
      const E* gg = static_cast<const E*>(p.gate);
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 16 * rt + 4 * g + i;
          const float ms = (sSS[tok] + sSS[C + tok] + sSS[2 * C + tok] + sSS[3 * C + tok]) * (1.f / D);
          const float inv = rsqrtf(ms + p.rms_eps);
          if (tok < nv) {
            const int64_t row = (t0 + tok) * rs + hoff;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
              const int col = col0 + 16 * ct + l16;
              const float w = p.norm_w ? p.norm_w[col] : 1.f;
              const float y = accO[rt][ct][i] * inv * w * sigmoidf_fast(to_f32(gg[row + col]));
              go[row + col] = from_f32<E>(y);
            }
          }
        }
    } else if (write_o) {
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 16 * rt + 4 * g + i;
          if (tok < nv) {
            const int64_t row = (t0 + tok) * rs + hoff;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) go[row + col0 + 16 * ct + l16] = from_f32<E>(accO[rt][ct][i]);
          }
        }
    }

    // ---- S3: S <- Diag(e^{g_n}) S + Kb^T U ----
#pragma unroll
    for (int rt8 = 0; rt8 < 8; ++rt8) {
      const f32x4 gam = *reinterpret_cast<const f32x4*>(sGam + 16 * rt8 + 4 * g);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) accS[rt8][ct] *= gam;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        Frag<E> fa;
        ld_frag_pair(fa, sKbt + cm_off<C, LDT>(16 * rt8 + l16, 32 * kt + 4 * g),
                     sKbt + cm_off<C, LDT>(16 * rt8 + l16, 32 * kt + 16 + 4 * g));
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) accS[rt8][ct] = mma(accS[rt8][ct], fa, uf[kt][ct]);
      }
    }
  }

  if (fin) {
#pragma unroll
    for (int rt8 = 0; rt8 < 8; ++rt8)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          fin[(size_t)(16 * rt8 + 4 * g + i) * D + col0 + 16 * ct + l16] = accS[rt8][ct][i];
  }
}

// ---------------------------------------------------------------------------
// Varlen work list: sequence indices ordered longest first (ties by index),
// so the longest chains start first.  One workgroup; O(N^2 / 1024) compares.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void worklist_kernel(const int32_t* __restrict__ cu, int N,
                                                         int32_t* __restrict__ order, int sort) {
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    if (!sort) {
      order[i] = i;
      continue;
    }
    const int Li = cu[i + 1] - cu[i];
    int rank = 0;
    for (int m = 0; m < N; ++m) {
      const int Lm = cu[m + 1] - cu[m];
      rank += (Lm > Li) || (Lm == Li && m < i);
    }
    order[rank] = i;
  }
}

hipError_t launch_worklist(const int32_t* cu, int num_seqs, int32_t* order, hipStream_t stream) {
  const int sort = num_seqs <= 16384 ? 1 : 0;
  hipLaunchKernelGGL(worklist_kernel, dim3(1), dim3(1024), 0, stream, cu, num_seqs, order, sort);
  return hipGetLastError();
}

template <typename E, int C, int DV, bool PRO, bool EPI>
static hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  constexpr size_t lds = PrefillLayout<E, C, DV>::BYTES;
  static_assert(lds <= 160 * 1024, "LDS budget exceeded");
  auto fn = prefill_kernel<E, C, DV, PRO, EPI>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int groups = (a.units + 7) / 8;
  const unsigned grid = (unsigned)(8 * a.col_split * groups);
  hipLaunchKernelGGL(fn, dim3(grid), dim3(256), lds, stream, a);
  return hipGetLastError();
}

template <typename E, int C>
static hipError_t launch_dtype(const PrefillArgs& a, hipStream_t stream) {
  const bool pro = a.conv_q_w != nullptr || a.conv_k_w != nullptr;
  const bool epi = a.gate != nullptr && a.mode != 1;
  // value-column blocks per work item (mode 1 runs two sets: B and M)
  const int blocks = a.mode == 1 ? a.col_split / 2 : a.col_split;
  if (blocks == 2) {
    if (epi) return hipErrorInvalidValue;
    return pro ? launch_t<E, C, 64, true, false>(a, stream) : launch_t<E, C, 64, false, false>(a, stream);
  }
  if (epi) return pro ? launch_t<E, C, 128, true, true>(a, stream) : launch_t<E, C, 128, false, true>(a, stream);
  return pro ? launch_t<E, C, 128, true, false>(a, stream) : launch_t<E, C, 128, false, false>(a, stream);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.bf16) return launch_dtype<__bf16, 64>(a, stream);
  return launch_dtype<float, 32>(a, stream);
}

}  // namespace kda
