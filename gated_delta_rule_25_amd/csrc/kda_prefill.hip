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
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

__host__ __device__ constexpr size_t al16(size_t x) { return (x + 15) & ~(size_t)15; }
__host__ __device__ constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

template <typename E, int C, int DV>
struct PrefillLayout {
  // bf16 operands keep a low-order bf16 part of Q_rel and K_inv so that the
  // output Gram tiles P are formed to ~16 significant bits (three products).
  static constexpr bool SPLIT = sizeof(E) == 2;
  static constexpr int NT = C / 16;
  static constexpr int NOFF = NT * (NT - 1) / 2;  // strictly-lower tile pairs
  static constexpr int PAD = 16 / (int)sizeof(E);
  static constexpr int LDK = D + PAD;   // token-major [C][D] operand tiles
  static constexpr int LDT = C + PAD;   // channel-major [D][C] / [DV][C] tiles, and [C][C] tiles
  static constexpr int LDA = C + 1;     // [C][C] fp32 work tiles
  static constexpr size_t TOK = (size_t)C * LDK * sizeof(E);
  static constexpr size_t CHM = (size_t)D * LDT * sizeof(E);
  static constexpr size_t VTB = (size_t)DV * LDT * sizeof(E);
  static constexpr size_t CCE = (size_t)C * LDT * sizeof(E);
  static constexpr size_t CCF = (size_t)C * LDA * 4;
  // Region R, during the Gram products: K_rel | K_inv (hi) | [K_inv lo] | Q_rel (hi) | [Q_rel lo].
  static constexpr size_t S_KR = 0;
  static constexpr size_t S_KIH = TOK;
  static constexpr size_t S_KIL = 2 * TOK;
  static constexpr size_t S_QRH = (SPLIT ? 3 : 2) * TOK;
  static constexpr size_t S_QRL = 4 * TOK;
  static constexpr size_t R_BYTES = (SPLIT ? 5 : 3) * TOK;
  // After them, [0, S_QRH) holds P | T | A (later W) | X, and the Q_rel slot is
  // turned into Qt = Q (.) e^{g} in place.
  static constexpr size_t R_P = 0;
  static constexpr size_t R_T = al16(CCE);
  static constexpr size_t R_A = R_T + al16(CCE);
  static constexpr size_t R_W = R_A;
  static constexpr size_t R_X = R_A + al16(CCF);
  static_assert(cmax(R_X + CCF, R_W + TOK) <= S_QRH, "post-Gram tiles overflow their region");
  static constexpr size_t O_KTT = R_BYTES;
  static constexpr size_t O_KBT = O_KTT + CHM;
  static constexpr size_t O_VT = O_KBT + CHM;
  static constexpr size_t O_TOT = al16(O_VT + VTB);                 // f32 [NT][D]
  static constexpr size_t O_EF = O_TOT + (size_t)NT * D * 4;         // f32 [NOFF][D]
  static constexpr size_t O_ERA = O_EF + (size_t)(NOFF > 0 ? NOFF : 1) * D * 4;  // f32 [NT][D]
  static constexpr size_t O_GAM = O_ERA + (size_t)NT * D * 4;        // f32 [D]
  static constexpr size_t O_BETA = O_GAM + (size_t)D * 4;            // f32 [C]
  static constexpr size_t O_Y = O_BETA + (size_t)C * 4;              // f32 [NT-1][256]
  static constexpr size_t O_NRM = O_Y + (size_t)(NT > 1 ? NT - 1 : 1) * 256 * 4;  // f32 [2][2][C]
  static constexpr size_t O_SS = O_NRM + (size_t)4 * C * 4;          // f32 [4][C]
  static constexpr size_t BYTES = O_SS + (size_t)4 * C * 4;
};

// Tile pairs (a, b <= a) in the order (0,0) (1,0) (1,1) (2,0) ...
__device__ __forceinline__ int pair_a(int p) { return p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3; }
__device__ __forceinline__ int pair_b(int p) { const int a = pair_a(p); return p - a * (a + 1) / 2; }
// Strictly-lower pairs (a, b < a) in the order (1,0) (2,0) (2,1) (3,0) ...
__device__ __forceinline__ int off_a(int q) { return q < 1 ? 1 : q < 3 ? 2 : 3; }
__device__ __forceinline__ int off_b(int q) { const int a = off_a(q); return q - a * (a - 1) / 2; }
__device__ __forceinline__ int off_idx(int a, int b) { return a * (a - 1) / 2 + b; }

// Reduce-scatter of V per-lane values over the 64 lanes of a wave: on return
// x[0] of every lane holds the 64-lane sum of value (lane / (64 / V)) % V
// after the trailing xor steps in butterfly_sum.
template <int V, int M>
__device__ __forceinline__ void bfly_step(float* x, int lane) {
  if constexpr (V > 1) {
    constexpr int N = V / 2;
    const bool up = (lane & M) != 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float send = up ? x[i] : x[i + N];
      const float keep = up ? x[i + N] : x[i];
      x[i] = keep + __shfl_xor(send, M);
    }
    bfly_step<N, M / 2>(x, lane);
  }
}
template <int V>
__device__ __forceinline__ float butterfly_sum(float* x, int lane) {
  bfly_step<V, 32>(x, lane);
  float r = x[0];
#pragma unroll
  for (int m = (64 / V) / 2; m >= 1; m >>= 1) r += __shfl_xor(r, m);
  return r;
}

// Rows r0 .. r0+N-1 of a chunk (row stride rs elements) as fp32.  Rows at or
// past nv read row nv-1 instead and are then zeroed, so the loads carry no
// branches and are issued back to back.
template <typename T, int N>
__device__ __forceinline__ void load_rows(float* dst, const T* cbase, int64_t rs, int r0, int nv) {
  T raw[N];
#pragma unroll
  for (int i = 0; i < N; ++i) raw[i] = cbase[(int64_t)min(r0 + i, nv - 1) * rs];
#pragma unroll
  for (int i = 0; i < N; ++i) dst[i] = (r0 + i < nv) ? to_f32(raw[i]) : 0.f;
}

// Prologue for rows r0 .. r0+N-1: causal depthwise conv (4 taps; zero history
// before the sequence start, chunk row `lo` = max(-3, bos - t0)) and SiLU.
template <typename T, int N>
__device__ __forceinline__ void load_conv_silu(float* dst, const T* cbase, int64_t rs, int r0, int nv, int lo,
                                               const float* w) {
  T raw[N + 3];
#pragma unroll
  for (int i = 0; i < N + 3; ++i) {
    const int row = r0 - 3 + i;
    raw[i] = cbase[(int64_t)min(max(row, lo), nv - 1) * rs];
  }
  float x[N + 3];
#pragma unroll
  for (int i = 0; i < N + 3; ++i) {
    const int row = r0 - 3 + i;
    x[i] = (row >= lo && row < nv) ? to_f32(raw[i]) : 0.f;
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float c = w[0] * x[i] + w[1] * x[i + 1] + w[2] * x[i + 2] + w[3] * x[i + 3];
    dst[i] = c * sigmoidf_fast(c);
  }
}

template <typename E, int C, int DV, bool PRO, bool EPI>
__global__ __launch_bounds__(256) void prefill_kernel(const PrefillArgs p) {
  using L = PrefillLayout<E, C, DV>;
  constexpr bool SPLIT = L::SPLIT;
  constexpr int NT = C / 16;     // 16-token tiles per chunk
  constexpr int KT = C / 32;     // 32-deep token steps per chunk
  constexpr int HALF = C / 2;    // tokens per prep thread
  constexpr int HT = HALF / 16;  // tiles per prep thread
  constexpr int NCW = DV / 4;    // value columns per wave
  constexpr int NCT = NCW / 16;  // 16-wide column tiles per wave
  constexpr int LDK = L::LDK, LDT = L::LDT, LDA = L::LDA;
  static_assert(!EPI || DV == D, "the epilogue normalises whole heads");
  static_assert(NCT >= 1 && KT >= 1 && NT <= 4, "unsupported tile shape");

  extern __shared__ __align__(16) unsigned char smem[];
  E* sKrel = reinterpret_cast<E*>(smem + L::S_KR);
  E* sKih = reinterpret_cast<E*>(smem + L::S_KIH);
  E* sKil = reinterpret_cast<E*>(smem + L::S_KIL);   // used only when SPLIT
  E* sQrh = reinterpret_cast<E*>(smem + L::S_QRH);   // Q_rel, then Qt in place
  E* sQrl = reinterpret_cast<E*>(smem + L::S_QRL);   // used only when SPLIT
  E* sP = reinterpret_cast<E*>(smem + L::R_P);
  E* sT = reinterpret_cast<E*>(smem + L::R_T);
  float* sA = reinterpret_cast<float*>(smem + L::R_A);
  float* sX = reinterpret_cast<float*>(smem + L::R_X);
  E* sW = reinterpret_cast<E*>(smem + L::R_W);
  E* sKtt = reinterpret_cast<E*>(smem + L::O_KTT);
  E* sKbt = reinterpret_cast<E*>(smem + L::O_KBT);
  E* sVt = reinterpret_cast<E*>(smem + L::O_VT);
  float* sTot = reinterpret_cast<float*>(smem + L::O_TOT);
  float* sEf = reinterpret_cast<float*>(smem + L::O_EF);
  float* sEra = reinterpret_cast<float*>(smem + L::O_ERA);
  float* sGam = reinterpret_cast<float*>(smem + L::O_GAM);
  float* sBeta = reinterpret_cast<float*>(smem + L::O_BETA);
  float* sY = reinterpret_cast<float*>(smem + L::O_Y);
  float* sNrm = reinterpret_cast<float*>(smem + L::O_NRM);
  float* sSS = reinterpret_cast<float*>(smem + L::O_SS);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, g = lane >> 4;
  // XCD-aware decode of the work item: blocks b and b + 8 run on the same XCD.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int cb = slot % p.col_split;
  const int u = (slot / p.col_split) * 8 + xcd;
  if (u >= p.units) return;
  const int H = p.num_heads;
  const int rnk = u / H, h = u % H;
  const int n = p.order ? p.order[rnk] : rnk;
  const int64_t bos = p.cu ? (int64_t)p.cu[n] : 0;
  const int64_t eos = p.cu ? (int64_t)p.cu[n + 1] : p.total_tokens;
  const int64_t rs = (int64_t)H * D;  // elements between consecutive tokens
  const int64_t hoff = (int64_t)h * D;
  const int col0 = cb * DV + wv * NCW;  // first value column owned by this wave

  const E* gq = static_cast<const E*>(p.q);
  const E* gk = static_cast<const E*>(p.k);
  const E* gv = static_cast<const E*>(p.v);
  E* go = static_cast<E*>(p.o);

  // State slice: tile (rt8, ct) holds rows 16 rt8 + 4g + i, column col0 + 16 ct + l16.
  f32x4 accS[8][NCT];
  const size_t sbase = ((size_t)n * H + h) * (size_t)(D * D);
#pragma unroll
  for (int rt8 = 0; rt8 < 8; ++rt8)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        accS[rt8][ct][i] =
            p.init ? p.init[sbase + (size_t)(16 * rt8 + 4 * g + i) * D + col0 + 16 * ct + l16] : 0.f;

  // Prep role: key channel ch, chunk tokens [rbase, rbase + HALF).
  const int ch = tid & (D - 1), th = tid >> 7, rbase = th * HALF;
  float wq[4] = {0.f, 0.f, 0.f, 1.f}, wk[4] = {0.f, 0.f, 0.f, 1.f};
  if (PRO) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (p.conv_q_w) wq[m] = p.conv_q_w[(hoff + ch) * 4 + m];
      if (p.conv_k_w) wk[m] = p.conv_k_w[(hoff + ch) * 4 + m];
    }
  }

  for (int64_t t0 = bos; t0 < eos; t0 += C) {
    const int nv = (int)((eos - t0) < C ? (eos - t0) : C);
    const int64_t cbase = t0 * rs + hoff;  // element offset of (token t0, head h, channel 0)

    // ---- P1: in-tile inclusive prefix sums of the log-decay ----
    float dl[HALF];
    load_rows<float, HALF>(dl, p.log_alpha + cbase + ch, rs, rbase, nv);
#pragma unroll
    for (int i = 0; i < HALF; ++i)
      if (i & 15) dl[i] += dl[i - 1];
#pragma unroll
    for (int j = 0; j < HT; ++j) sTot[(rbase / 16 + j) * D + ch] = dl[16 * j + 15];

    // ---- P2: q and k columns (raw, or through conv + SiLU), V^T, beta ----
    float qv[HALF], kv[HALF];
    {
      const E* qs = gq + cbase + ch;
      const E* ks = gk + cbase + ch;
      if (PRO) {
        const int64_t back = bos - t0;  // <= 0
        const int lo = back < -3 ? -3 : (int)back;
        const int qh = wv & 1;  // which 64-channel half of the head this wave holds
        if (p.conv_q_w) {
          load_conv_silu<E, HALF>(qv, qs, rs, rbase, nv, lo, wq);
          float sq[HALF];
#pragma unroll
          for (int i = 0; i < HALF; ++i) sq[i] = qv[i] * qv[i];
          const float r = butterfly_sum<HALF>(sq, lane);
          if ((lane % (64 / HALF)) == 0) sNrm[(0 * 2 + qh) * C + rbase + (lane / (64 / HALF)) % HALF] = r;
        } else {
          load_rows<E, HALF>(qv, qs, rs, rbase, nv);
        }
        if (p.conv_k_w) {
          load_conv_silu<E, HALF>(kv, ks, rs, rbase, nv, lo, wk);
          float sk[HALF];
#pragma unroll
          for (int i = 0; i < HALF; ++i) sk[i] = kv[i] * kv[i];
          const float r = butterfly_sum<HALF>(sk, lane);
          if ((lane % (64 / HALF)) == 0) sNrm[(1 * 2 + qh) * C + rbase + (lane / (64 / HALF)) % HALF] = r;
        } else {
          load_rows<E, HALF>(kv, ks, rs, rbase, nv);
        }
      } else {
        load_rows<E, HALF>(qv, qs, rs, rbase, nv);
        load_rows<E, HALF>(kv, ks, rs, rbase, nv);
      }
      constexpr int VPARTS = 256 / DV, VTOK = C / VPARTS;
      const int vc = tid % DV, vp = tid / DV;
      float vv[VTOK];
      load_rows<E, VTOK>(vv, gv + cbase + cb * DV + vc, rs, vp * VTOK, nv);
#pragma unroll
      for (int i = 0; i < VTOK; ++i) sVt[vc * LDT + vp * VTOK + i] = from_f32<E>(vv[i]);
      if (tid < C) {
        const float bb = p.beta[(t0 + min(tid, nv - 1)) * H + h];
        sBeta[tid] = (tid < nv) ? bb : 0.f;
      }
    }
    __syncthreads();

    // ---- P3: scaled operand tiles ----
    {
      float rho[NT + 1];
      rho[0] = 0.f;
#pragma unroll
      for (int a = 0; a < NT; ++a) rho[a + 1] = rho[a] + sTot[a * D + ch];
      const float gn = rho[NT];
      float iq[HALF], ik[HALF];
#pragma unroll
      for (int i = 0; i < HALF; ++i) {
        iq[i] = 1.f;
        ik[i] = 1.f;
      }
      if (PRO) {
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
          const int rr = rbase + i;
          if (p.conv_q_w) iq[i] = rsqrtf(sNrm[0 * C + rr] + sNrm[1 * C + rr] + p.l2_eps);
          if (p.conv_k_w) ik[i] = rsqrtf(sNrm[2 * C + rr] + sNrm[3 * C + rr] + p.l2_eps);
        }
      }
#pragma unroll
      for (int j = 0; j < HT; ++j) {
        const int a = rbase / 16 + j;
        float ra = rho[0];
#pragma unroll
        for (int aa = 1; aa < NT; ++aa)
          if (aa == a) ra = rho[aa];
        const float ea = __expf(ra);       // e^{rho_a} <= 1
        const float eb = __expf(gn - ra);  // e^{g_n - rho_a} <= 1
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int idx = 16 * j + i, rr = rbase + idx;
          const float qn = qv[idx] * iq[idx], kn = kv[idx] * ik[idx];
          const float ep = __expf(dl[idx]);   // e^{g_r - rho_a}  in (e^-80, 1]
          const float en = __expf(-dl[idx]);  // e^{rho_a - g_r}  in [1, e^80)
          const float xq = qn * ep, xk = kn * ep, xi = kn * en;
          const E qhi = from_f32<E>(xq), ihi = from_f32<E>(xi);
          sQrh[rr * LDK + ch] = qhi;
          sKih[rr * LDK + ch] = ihi;
          if constexpr (SPLIT) {
            sQrl[rr * LDK + ch] = from_f32<E>(xq - to_f32(qhi));
            sKil[rr * LDK + ch] = from_f32<E>(xi - to_f32(ihi));
          }
          sKrel[rr * LDK + ch] = from_f32<E>(xk);
          sKtt[ch * LDT + rr] = from_f32<E>(xk * ea);   // Kt = K e^{g}
          sKbt[ch * LDT + rr] = from_f32<E>(xi * eb);   // Kb = K e^{g_n - g}
        }
      }
      if (th == 0) {
        sGam[ch] = __expf(gn);
#pragma unroll
        for (int a = 0; a < NT; ++a) sEra[a * D + ch] = __expf(rho[a]);
#pragma unroll
        for (int a = 1; a < NT; ++a)
#pragma unroll
          for (int b = 0; b < a; ++b) sEf[off_idx(a, b) * D + ch] = __expf(rho[a] - rho[b]);
      }
    }
    __syncthreads();

    // ---- P5: Gram tiles per tile pair (a, b <= a), pair p on wave p % 4:
    //      A_ab = K_rel_a Kh_ab^T (bf16),  P_ab = Q_rel_a Kh_ab^T (hi/lo when SPLIT)
    {
      constexpr int NPAIR = NT * (NT + 1) / 2;
      constexpr int PPW = (NPAIR + 3) / 4;
      f32x4 ga[PPW], gp[PPW];
#pragma unroll
      for (int j = 0; j < PPW; ++j) {
        ga[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        gp[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        const int pr = wv + 4 * j;
        if (pr < NPAIR) {
          const int a = pair_a(pr), b = pair_b(pr);
          const int arow = (16 * a + l16) * LDK + 8 * g, brow = (16 * b + l16) * LDK + 8 * g;
          const float* ef = sEf + (b < a ? off_idx(a, b) : 0) * D + 8 * g;
#pragma unroll
          for (int s = 0; s < D / 32; ++s) {
            Frag<E> fk, fq, fbh;
            ld_frag(fk, sKrel + arow + 32 * s);
            ld_frag(fq, sQrh + arow + 32 * s);
            ld_frag(fbh, sKih + brow + 32 * s);
            if constexpr (SPLIT) {
              Frag<E> fql, fbl;
              ld_frag(fql, sQrl + arow + 32 * s);
              ld_frag(fbl, sKil + brow + 32 * s);
              if (b < a) {
                float hv[8], lv[8], x[8];
                frag_unpack(fbh, hv);
                frag_unpack(fbl, lv);
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) x[jj] = (hv[jj] + lv[jj]) * ef[32 * s + jj];
                frag_split(fbh, fbl, x);
              }
              ga[j] = mma(ga[j], fk, fbh);
              gp[j] = mma(gp[j], fq, fbh);
              gp[j] = mma(gp[j], fq, fbl);
              gp[j] = mma(gp[j], fql, fbh);
            } else {
              if (b < a) {
                float x[8];
                frag_unpack(fbh, x);
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) x[jj] *= ef[32 * s + jj];
                frag_from_f32(fbh, x);
              }
              ga[j] = mma(ga[j], fk, fbh);
              gp[j] = mma(gp[j], fq, fbh);
            }
          }
        }
      }
      __syncthreads();  // every wave is done reading the Gram operands
#pragma unroll
      for (int j = 0; j < PPW; ++j) {
        const int pr = wv + 4 * j;
        if (pr < NPAIR) {
          const int a = pair_a(pr), b = pair_b(pr);
          const int c = 16 * b + l16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * a + 4 * g + i;
            sA[r * LDA + c] = ((b < a) || (c < r)) ? ga[j][i] * sBeta[r] : 0.f;
            sP[r * LDT + c] = from_f32<E>(((b < a) || (c <= r)) ? gp[j][i] : 0.f);
          }
        }
      }
      // strictly-upper tiles of P are read by the 32-deep token steps: zero them
      for (int e = tid; e < L::NOFF * 256; e += 256) {
        const int q = e >> 8, a = off_a(q), b = off_b(q);
        sP[(16 * b + ((e >> 4) & 15)) * LDT + 16 * a + (e & 15)] = from_f32<E>(0.f);
      }
      // Qt = (Q_rel hi + lo) e^{rho_a}, in place over the Q_rel slot (8 elements per step)
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

    // ---- P6: T = (I + A)^{-1} Diag(beta), blocked by 16-token tiles, fp32 ----
    if (tid < 16 * NT) {
      const int a = tid >> 4, j = tid & 15;
      float x[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float* arow = sA + (16 * a + rr) * LDA + 16 * a;
        float s = (rr == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < rr; ++i) s -= arow[i] * x[i];
        x[rr] = s;
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sX[(16 * a + rr) * LDA + 16 * a + j] = x[rr];
    }
    __syncthreads();
#pragma unroll
    for (int dist = 1; dist < NT; ++dist) {
      const int nb = NT - dist;
      for (int e = tid; e < nb * 256; e += 256) {
        const int blk = e >> 8, i = (e >> 4) & 15, jj = e & 15, b = blk, a = blk + dist;
        float y = 0.f;
        for (int c = b; c < a; ++c)
#pragma unroll
          for (int m = 0; m < 16; ++m) y += sA[(16 * a + i) * LDA + 16 * c + m] * sX[(16 * c + m) * LDA + 16 * b + jj];
        sY[blk * 256 + i * 16 + jj] = y;
      }
      __syncthreads();
      for (int e = tid; e < nb * 256; e += 256) {
        const int blk = e >> 8, i = (e >> 4) & 15, jj = e & 15, b = blk, a = blk + dist;
        float xx = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m) xx -= sX[(16 * a + i) * LDA + 16 * a + m] * sY[blk * 256 + m * 16 + jj];
        sX[(16 * a + i) * LDA + 16 * b + jj] = xx;
      }
      __syncthreads();
    }
    for (int e = tid; e < C * C; e += 256) {
      const int rr = e / C, cc = e % C;
      sT[rr * LDT + cc] = from_f32<E>(cc <= rr ? sX[rr * LDA + cc] * sBeta[cc] : 0.f);
    }
    __syncthreads();

    // ---- P7: W = T Kt  (C x 128), stored token-major for the carried stage ----
    {
      constexpr int TPW = 2 * NT;  // tiles per wave: (C/16) * 8 / 4
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        const int tile = wv * TPW + j, rt = tile >> 3, ct = tile & 7;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const int nks = (16 * rt + 15) / 32 + 1;
        for (int ks = 0; ks < nks; ++ks) {
          Frag<E> fa, fb;
          ld_frag(fa, sT + (16 * rt + l16) * LDT + 32 * ks + 8 * g);
          ld_frag(fb, sKtt + (16 * ct + l16) * LDT + 32 * ks + 8 * g);
          acc = mma(acc, fa, fb);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sW[(16 * rt + 4 * g + i) * LDK + 16 * ct + l16] = from_f32<E>(acc[i]);
      }
    }
    // ---- P8: U' = T V for this wave's columns (kept in registers) ----
    f32x4 accU[NT][NCT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) accU[rt][ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
      const int nks = (16 * rt + 15) / 32 + 1;
#pragma unroll
      for (int ks = 0; ks < KT; ++ks) {
        if (ks < nks) {
          Frag<E> fa;
          ld_frag(fa, sT + (16 * rt + l16) * LDT + 32 * ks + 8 * g);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            Frag<E> fb;
            ld_frag(fb, sVt + (wv * NCW + 16 * ct + l16) * LDT + 32 * ks + 8 * g);
            accU[rt][ct] = mma(accU[rt][ct], fa, fb);
          }
        }
      }
    }
    __syncthreads();  // W visible to every wave

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
        ld_frag_perm(fa, sW + (16 * rt + l16) * LDK + 32 * ks + 4 * g);
        fa = frag_neg(fa);
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
        ld_frag_perm(fa, sQrh + (16 * rt + l16) * LDK + 32 * ks + 4 * g);
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

    if (EPI) {
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
    } else {
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
        ld_frag_perm(fa, sKbt + (16 * rt8 + l16) * LDT + 32 * kt + 4 * g);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) accS[rt8][ct] = mma(accS[rt8][ct], fa, uf[kt][ct]);
      }
    }
  }

  if (p.fin) {
#pragma unroll
    for (int rt8 = 0; rt8 < 8; ++rt8)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          p.fin[sbase + (size_t)(16 * rt8 + 4 * g + i) * D + col0 + 16 * ct + l16] = accS[rt8][ct][i];
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
  const bool epi = a.gate != nullptr;
  if (a.col_split == 2) {
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
