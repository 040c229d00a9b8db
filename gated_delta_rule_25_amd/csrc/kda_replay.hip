// kda_replay.hip — multi-token decode from cached per-token inputs: the
// replay step of speculative decoding.
//
// "Kimi K3 架构、训练与系统全景解析", section 7.4 (KDA state replay under
// speculative decoding): rolling the recurrent state back over rejected draft
// tokens would need one saved state per draft position.  Instead the small
// per-token inputs are kept; after verification the accepted prefix is
// replayed from the verified state on chip, in one kernel that also runs the
// short convolution, the norms and the output gate, and only the final state
// is written back.  The same kernel without the state write is the
// verification pass over every draft token.
//
// The nt <= 16 tokens of one (sequence n, head h) are taken as one block of
// the chunkwise form (section 4.2.4): with D_t = prod_{s<=t} alpha_s per key
// channel, K~ = D k, Q~ = D q, K^ = k / D, Kb = (D_last / D) k,
//     X = K~ S0,  Y = Q~ S0,  G = [K~; Q~] K^^T            (matrix products)
//     u_t = beta_t (v_t - X_t - sum_{s<t} G[t][s] u_s)       (forward substitution)
//     o_t = Y_t + sum_{s<=t} G[LP+t][s] u_s
//     S   = Diag(D_last) S0 + Kb^T U
// which is the token-by-token recurrence regrouped.  The decay lower bound
// (log alpha >= -5, section 4.2.5: over 16 tokens the reciprocal stays
// below e^80, inside the fp32 range) keeps every factor finite; that bound is
// why a block holds at most 16 tokens.  With the unbounded decay (Kimi
// Linear's negative softplus, section 4.2.5) 1 / D can overflow, so that
// mode never forms it: G[t][s] = sum_i x_t[i] k_s[i] prod_{s<r<=t} alpha_r[i]
// is built pair by pair from running sums of log alpha over the tokens
// between the two (same-sign sums, factors <= 1) and reduced over the
// channels with wave sums, and Kb_t = k_t prod_{r>t} alpha_r from suffix sums.
//
// One 256-thread workgroup per (n, h).  Wave w owns value columns 32w..32w+31
// as two 16-column MFMA tiles (tile C holds columns 32w + 2c + C, c = lane %
// 16) over all 128 rows, so the state sits in registers in the MFMA
// accumulator layout; that layout is also the B operand of a 16-deep fp32
// MFMA step, so X, Y and the state update read the state where it is.
// Steps:
//   1. the state load (8-byte pieces, two columns) and every cached input of
//      the tokens run (16-byte pieces: q and k rows with their three history
//      rows when the convolution runs, v, log_alpha, gate), all in flight
//      together; the inputs are staged in LDS;
//   2. per channel: the prologue (ShortConv4 + SiLU, then L2 over the head's
//      channels; section 4.2.3) and the decay products D_t, giving K~, Q~,
//      K^ (and Kb, D_last when committing);
//   3. [X; Y] = [K~; Q~] S0 and G on fp32 MFMA (v_mfma_f32_16x16x4_f32);
//      the substitution solved once for all columns (T and M below), the
//      outputs O = Y + M (V - X), then RMSNorm x sigmoid(gate) (section 4.2.6);
//   4. when a state output is given: S = Diag(D_last) S0 + Kb^T U on MFMA,
//      the state store, and the three raw rows before the next token.
// All arithmetic is fp32.  The state is read once and written at most once
// however many tokens run.
#include "kda_chunk_util.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kNonTemporal = 2;  // cache-policy operand of a streaming buffer access
constexpr int PS = D + 4;   // padded row stride (floats) of the MFMA A / B operand arrays

// Dynamic LDS of one workgroup for L cached tokens, LP = 8 or 16 block rows
// (byte offsets, all multiples of 16).
struct ReplayLayout {
  uint32_t RQ, RK, SGP, SG, RV, RG, RLA, PX, PY, SP, SKH, SGAM, SSC, BYTES;
  __host__ __device__ ReplayLayout(int L, int es, bool gate, int LP) {
    const uint32_t rb = 128u * (uint32_t)es;
    RQ = 0;                                       // E [3 + L][128]: raw q, history rows then tokens
    RK = RQ + (3u + L) * rb;                      // E [3 + L][128]: raw k
    // once the prologue has read the raw rows, the same bytes hold the Gram products
    SGP = 0;                                      // f32 [4 waves][2LP][16] partial G
    SG = SGP + 4u * (uint32_t)(2 * LP) * 64u;     // f32 [2LP][16] G
    const uint32_t u0 = 2u * (3u + L) * rb, u1 = SG + (uint32_t)(2 * LP) * 64u;
    RV = u0 > u1 ? u0 : u1;                       // E [L][128]
    RG = RV + (uint32_t)L * rb;                   // E [L][128] gate logits
    RLA = RG + (gate ? (uint32_t)L * rb : 0u);    // f32 [L][128] log_alpha
    PX = RLA + (uint32_t)L * 512u;                // f32 [LP][128] q before L2, then X
    PY = PX + (uint32_t)LP * 512u;                // f32 [LP][128] k before L2, then Y
    SP = PY + (uint32_t)LP * 512u;                // f32 [2LP][PS] K~ then Q~; later U [LP][128]
    SKH = SP + (uint32_t)(2 * LP) * PS * 4u;      // f32 [LP][PS] K^, or Kb with unbounded decay (rows >= nt zero)
    SGAM = SKH + (uint32_t)LP * PS * 4u;          // f32 [128] D_last
    SSC = SGAM + 512u;                            // f32 [LP][4] 1/|q|, 1/|k|, -, beta
    BYTES = SSC + (uint32_t)LP * 16u;
  }
};

// Sum over the 64 lanes of a wave, returned in every lane: prefix sums
// within each 16-lane row (DPP row shifts), then row 0 into row 1 and row 2
// into row 3 (row_bcast:15), then lane 31 into rows 2 and 3 (row_bcast:31);
// lane 63 ends with the total.  Every lane of the wave must be active.
__device__ __forceinline__ float wave_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xa, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x143, 0xc, 0xf, false));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

template <typename E>
__device__ __forceinline__ float lds_elem(const unsigned char* base, int row, int j) {
  return to_f32(reinterpret_cast<const E*>(base)[row * D + j]);
}

template <typename E, int LP, bool PRO, bool EPI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(LP == 8 ? 3 : 1))) void replay_kernel(const ReplayArgs p) {
  constexpr int ES = (int)sizeof(E);
  constexpr int RP = D * ES / 16;  // 16-byte pieces of one row in the I/O dtype
  constexpr int LP4 = D * 4 / 16;  // pieces of one log_alpha row
  constexpr int NR = 2 * LP / 16;  // MFMA row tiles of [K~; Q~]
  constexpr float LOG2E = 1.4426950408889634f;
  extern __shared__ __align__(16) unsigned char smem[];

  const int L = p.max_tokens, H = p.num_heads;
  const ReplayLayout lay(L, ES, EPI, LP);
  const int64_t u = blockIdx.x;  // n * H + h
  const int n = (int)(u / H), h = (int)(u % H);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c16 = lane & 15, g4 = lane >> 4;  // MFMA lane coordinates
  int nt = p.num_tokens ? p.num_tokens[n] : L;
  nt = min(max(nt, 0), L);
  const bool commit = p.state_out != nullptr;

  // ---- 1. token inputs, then the state, all in flight together ----
  const bool cq = PRO && p.conv_q_w, ck = PRO && p.conv_k_w;
  const size_t rowb = (size_t)D * ES;
  // The cached inputs go straight from global memory into LDS (16-byte
  // pieces, piece pc of an input at byte 16 pc of its LDS array, so one
  // instruction of wave w writes 64 consecutive pieces at a wave-uniform
  // base).  q / k: staged row r holds the history (rows 0..2, oldest first)
  // or token r - 3; without the convolution only rows 3 .. 3 + nt - 1 are
  // loaded.
  constexpr int QKS = ((3 + kReplayMaxTokens) * RP + kThreads - 1) / kThreads;
  constexpr int VS = (kReplayMaxTokens * RP + kThreads - 1) / kThreads;
  constexpr int LS = (kReplayMaxTokens * LP4 + kThreads - 1) / kThreads;
  const int wu = __builtin_amdgcn_readfirstlane(wv);
  auto qk_src = [&](const void* tok, const void* hist, int r, int w) {
    const char* b = r < 3 ? static_cast<const char*>(hist) + ((size_t)(n * 3 + r) * H + h) * rowb
                          : static_cast<const char*>(tok) + ((size_t)(n * L + r - 3) * H + h) * rowb;
    return b + w * 16;
  };
  auto tok_src = [&](const void* base, size_t rb, int t, int w) {
    return static_cast<const char*>(base) + ((size_t)(n * L + t) * H + h) * rb + w * 16;
  };
  auto to_lds = [&](const char* g, uint32_t wave_base) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(smem + wave_base), 16, 0, 0);
  };
  const int q0 = cq ? 0 : 3, k0 = ck ? 0 : 3;  // first staged row
  const int nq = (3 + nt - q0) * RP, nk = (3 + nt - k0) * RP, ntp = nt * RP, nlp = nt * LP4;
#pragma unroll
  for (int i = 0; i < QKS; ++i) {
    const int pc = tid + kThreads * i;
    const uint32_t pw = (uint32_t)(kThreads * i + 64 * wu) * 16u;  // this wave's first piece
    if (pc < nq) to_lds(qk_src(p.q, p.conv_q_state, q0 + pc / RP, pc % RP), lay.RQ + (uint32_t)(q0 * RP) * 16u + pw);
    if (pc < nk) to_lds(qk_src(p.k, p.conv_k_state, k0 + pc / RP, pc % RP), lay.RK + (uint32_t)(k0 * RP) * 16u + pw);
  }
#pragma unroll
  for (int i = 0; i < VS; ++i) {
    const int pc = tid + kThreads * i;
    const uint32_t pw = (uint32_t)(kThreads * i + 64 * wu) * 16u;
    if (pc < ntp) to_lds(tok_src(p.v, rowb, pc / RP, pc % RP), lay.RV + pw);
    if (EPI && pc < ntp) to_lds(tok_src(p.gate, rowb, pc / RP, pc % RP), lay.RG + pw);
  }
#pragma unroll
  for (int i = 0; i < LS; ++i) {
    const int pc = tid + kThreads * i;
    const uint32_t pw = (uint32_t)(kThreads * i + 64 * wu) * 16u;
    if (pc < nlp) to_lds(tok_src(p.log_alpha, D * 4, pc / LP4, pc % LP4), lay.RLA + pw);
  }
  float bt = 0.f;
  if (tid < nt) bt = p.beta[((size_t)n * L + tid) * H + h];
  // RMSNorm weights of the four value columns this thread outputs (read
  // here so that the output stores at the end never wait behind a late load)
  const int cc = 4 * (tid & 31);
  float nw[4] = {1.f, 1.f, 1.f, 1.f};
  if (EPI && p.norm_w)
#pragma unroll
    for (int e = 0; e < 4; ++e) nw[e] = p.norm_w[cc + e];
  // convolution taps of channel j of the branch this thread forms (q: threads 0..127, k: 128..255)
  const int j = tid & 127;
  const bool isk = tid >= 128;
  const bool conv = isk ? ck : cq;
  float w4[4] = {0.f, 0.f, 0.f, 0.f};
  if (conv) {
    const float* cw = (isk ? p.conv_k_w : p.conv_q_w) + ((size_t)h * D + j) * 4;
#pragma unroll
    for (int m = 0; m < 4; ++m) w4[m] = cw[m];
  }
  // The state, issued last: its 32 loads per lane stay in flight through the
  // prologue while the wait below covers only what was issued before them.
  // st[T][C][e] = S0[16T + 4 g4 + e][32 wv + 2 c16 + C]
  __builtin_amdgcn_sched_barrier(0);
  f32x4 st[8][2];
  const int col0 = 32 * wv + 2 * c16;
  {
    // a buffer view of the (n, h) state; with no state given its range is
    // empty and every load returns zero
    const Rsrc rs = make_rsrc(p.state_in ? p.state_in + u * (D * D) : nullptr, p.state_in ? D * D * 4 : 0);
#pragma unroll
    for (int T = 0; T < 8; ++T)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 x = __builtin_bit_cast(
            f32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, ((16 * T + 4 * g4 + e) * D + col0) * 4, 0, kNonTemporal));
        st[T][0][e] = x[0];
        st[T][1][e] = x[1];
      }
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(32));
  float* sX = reinterpret_cast<float*>(smem + lay.PX);  // pre-norm q, then X
  float* sY = reinterpret_cast<float*>(smem + lay.PY);  // pre-norm k, then Y
  float* sP = reinterpret_cast<float*>(smem + lay.SP);
  float* sKh = reinterpret_cast<float*>(smem + lay.SKH);
  float* sGam = reinterpret_cast<float*>(smem + lay.SGAM);
  float* sSC = reinterpret_cast<float*>(smem + lay.SSC);
  float* sGP = reinterpret_cast<float*>(smem + lay.SGP);
  float* sG = reinterpret_cast<float*>(smem + lay.SG);
  const float* sLA = reinterpret_cast<const float*>(smem + lay.RLA);
  if (tid < nt) sSC[4 * tid + 3] = bt;
  __syncthreads();

  // ---- 2. per-channel operands ----
  // raw rows t-3, t-2, t-1 of channel j; after the loop the three rows
  // before token nt, which a commit writes back as the new history
  float x0 = 0.f, x1 = 0.f, x2 = 0.f;
  {
    const unsigned char* rows = smem + (isk ? lay.RK : lay.RQ);
    float* pre = isk ? sY : sX;  // before the L2 scale
    if (conv) {
      x0 = lds_elem<E>(rows, 0, j);
      x1 = lds_elem<E>(rows, 1, j);
      x2 = lds_elem<E>(rows, 2, j);
    }
    for (int t = 0; t < nt; ++t) {
      const float x3 = lds_elem<E>(rows, 3 + t, j);
      float s = x3;
      if (conv) {
        const float c = w4[0] * x0 + w4[1] * x1 + w4[2] * x2 + w4[3] * x3;
        s = c * sigmoidf_fast(c);
        x0 = x1;
        x1 = x2;
        x2 = x3;
      }
      pre[t * D + j] = s;
    }
  }
  __syncthreads();
  // squared norms of every token's q and k (wave wv takes tokens wv, wv + 4, ...)
  if (cq || ck) {
    for (int t = wv; t < nt; t += 4) {
      const float q0v = sX[t * D + lane], q1v = sX[t * D + 64 + lane];
      const float k0v = sY[t * D + lane], k1v = sY[t * D + 64 + lane];
      const float sq = wave_sum(q0v * q0v + q1v * q1v), sk = wave_sum(k0v * k0v + k1v * k1v);
      if (lane == 0) {
        sSC[4 * t] = cq ? rsqrtf(sq + p.l2_eps) : 1.f;
        sSC[4 * t + 1] = ck ? rsqrtf(sk + p.l2_eps) : 1.f;
      }
    }
    __syncthreads();
  }
  {
    // D_t = prod_{s<=t} alpha_s and its reciprocal, from exp2 of each step
    float Dt = 1.f, Di = 1.f;
    if (!isk) {
#pragma unroll
      for (int t = 0; t < LP; ++t) {
        float qt = 0.f;
        if (t < nt) {
          Dt *= exp2_fast(sLA[t * D + j] * LOG2E);
          qt = sX[t * D + j] * ((cq || ck) ? sSC[4 * t] : 1.f) * Dt;
        }
        sP[(LP + t) * PS + j] = qt;
      }
    } else if (!p.unbounded) {
#pragma unroll
      for (int t = 0; t < LP; ++t) {
        float kt = 0.f, kh = 0.f;
        if (t < nt) {
          const float x = sLA[t * D + j] * LOG2E;
          Dt *= exp2_fast(x);
          Di *= exp2_fast(-x);
          const float kv = sY[t * D + j] * ((cq || ck) ? sSC[4 * t + 1] : 1.f);
          kt = kv * Dt;
          kh = kv * Di;
        }
        sP[t * PS + j] = kt;
        sKh[t * PS + j] = kh;
      }
      sGam[j] = Dt;  // D_last: the decay over all tokens run
    } else {
      // unbounded decay: K~ = D k, and Kb (not K^) from suffix sums of log alpha
#pragma unroll
      for (int t = 0; t < LP; ++t) {
        float kt = 0.f;
        if (t < nt) {
          Dt *= exp2_fast(sLA[t * D + j] * LOG2E);
          kt = sY[t * D + j] * ((cq || ck) ? sSC[4 * t + 1] : 1.f) * Dt;
        }
        sP[t * PS + j] = kt;
      }
      sGam[j] = Dt;
      float suf = 0.f;  // sum of log alpha over the tokens after t
#pragma unroll
      for (int t = LP - 1; t >= 0; --t) {
        float kb = 0.f;
        if (t < nt) {
          kb = sY[t * D + j] * ((cq || ck) ? sSC[4 * t + 1] : 1.f) * exp2_fast(suf * LOG2E);
          suf += sLA[t * D + j];
        }
        sKh[t * PS + j] = kb;
      }
    }
  }
  if (p.unbounded) {
    // pairwise Gram entries: waves 0-1 (q channels) form the Q~ rows, waves
    // 2-3 (k channels) the K~ rows; each wave's 64-channel partial sums go to
    // its own block of the partial-Gram array, the other rows zero
    float* mine = sGP + wv * 2 * LP * 16;
    for (int i = lane; i < 2 * LP * 16; i += 64) mine[i] = 0.f;
    for (int s = 0; s < nt; ++s) {
      const float ks = sY[s * D + j] * ((cq || ck) ? sSC[4 * s + 1] : 1.f);
      float cum = 0.f;  // sum of log alpha over tokens s+1 .. t
      for (int t = s; t < nt; ++t) {
        if (t > s) cum += sLA[t * D + j];
        const float xt = isk ? sY[t * D + j] * ((cq || ck) ? sSC[4 * t + 1] : 1.f)
                             : sX[t * D + j] * ((cq || ck) ? sSC[4 * t] : 1.f);
        const float v = xt * ks * exp2_fast(cum * LOG2E);
        const float sum = wave_sum(v);
        if (lane == 0) mine[((isk ? 0 : LP) + t) * 16 + s] = sum;
      }
    }
  }
  __syncthreads();

  // ---- 3. [X; Y] = [K~; Q~] S0 and the partial Gram products on MFMA ----
  {
    f32x4 acc[NR][2], gacc[NR];
#pragma unroll
    for (int R = 0; R < NR; ++R) acc[R][0] = acc[R][1] = gacc[R] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int T = 0; T < 8; ++T) {
      Frag16<float> a[NR];
#pragma unroll
      for (int R = 0; R < NR; ++R)
        a[R].v = *reinterpret_cast<const f32x4*>(sP + (16 * R + c16) * PS + 16 * T + 4 * g4);
#pragma unroll
      for (int C = 0; C < 2; ++C) {
        Frag16<float> b;
        b.v = st[T][C];
#pragma unroll
        for (int R = 0; R < NR; ++R) acc[R][C] = mma16(acc[R][C], a[R], b);
      }
      if (!p.unbounded && (T >> 1) == wv) {  // this wave's quarter of the Gram contraction
        Frag16<float> b;
        b.v = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (c16 < LP) b.v = *reinterpret_cast<const f32x4*>(sKh + c16 * PS + 16 * T + 4 * g4);
#pragma unroll
        for (int R = 0; R < NR; ++R) gacc[R] = mma16(gacc[R], a[R], b);
      }
    }
    // rows 0..LP-1 of the block are X (K~ rows), LP..2LP-1 are Y (Q~ rows)
#pragma unroll
    for (int R = 0; R < NR; ++R)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * R + 4 * g4 + e;
        float* dst = row < LP ? sX + row * D : sY + (row - LP) * D;
        *reinterpret_cast<f32x2*>(dst + col0) = (f32x2){acc[R][0][e], acc[R][1][e]};
        if (!p.unbounded) sGP[(wv * 2 * LP + row) * 16 + c16] = gacc[R][e];
      }
  }
  __syncthreads();
  for (int i = tid; i < 2 * LP * 16; i += kThreads)
    sG[i] = sGP[i] + sGP[2 * LP * 16 + i] + sGP[4 * LP * 16 + i] + sGP[6 * LP * 16 + i];
  __syncthreads();

  // ---- the block's triangular system, for every value column at once ----
  // u_t = beta_t (v_t - X_t - sum_{r<t} G_K[t][r] u_r) reads U = T (V - X)
  // with T = (I + Diag(beta) G_K)^{-1} Diag(beta), and o_t = Y_t +
  // sum_{r<=t} G_Q[t][r] u_r reads O = Y + M (V - X) with M = G_Q T.  Lane j
  // of wave 0 solves column j of T by forward substitution and forms column
  // j of M; rows past nt are zero, their beta being zero.  Then every thread
  // takes value columns cc .. cc + 3 of token rows tr, tr + 8, ...: independent
  // dot products over the LP block rows (T and M are lower triangular, so the
  // terms above the diagonal are exact zeros), a token's RMS sum over the 32
  // lanes that hold its row, and one 8- or 16-byte store per output row.
  E* go = static_cast<E*>(p.o);
  const E* sV = reinterpret_cast<const E*>(smem + lay.RV);
  const E* sGt = reinterpret_cast<const E*>(smem + lay.RG);
  float* sU = sP;           // [LP][128]: the [K~; Q~] block is no longer read
  float* sT = sGP;          // [LP][16]: the partial Gram products are summed
  float* sM = sGP + LP * 16;  // [LP][16]
  float* sW = sX;           // [LP][128] V - X over X, zero past nt
  if (wv == 0) {
    const int jc = lane;
    float x[LP];
#pragma unroll
    for (int t = 0; t < LP; ++t) {
      float s = (t == jc) ? 1.f : 0.f;
#pragma unroll
      for (int r = 0; r < t; ++r) s -= sG[t * 16 + r] * x[r];
      x[t] = t < nt ? s * sSC[4 * t + 3] : 0.f;
    }
    if (jc < LP)
#pragma unroll
      for (int t = 0; t < LP; ++t) {
        float m = 0.f;
#pragma unroll
        for (int r = 0; r <= t; ++r) m += sG[(LP + t) * 16 + r] * x[r];
        sT[t * 16 + jc] = x[t];
        sM[t * 16 + jc] = m;
      }
  }
  constexpr int TPT = LP / 8;  // token rows per thread
  const int tr = tid >> 5;
#pragma unroll
  for (int q = 0; q < TPT; ++q) {
    const int t = tr + 8 * q;
    f32x4 w = {0.f, 0.f, 0.f, 0.f};
    if (t < nt) {  // V's rows past nt were never loaded
      Frag16<E> vf;
      ld_frag16(vf, sV + t * D + cc);
      w = frag16_to_f32(vf) - *reinterpret_cast<const f32x4*>(sX + t * D + cc);
    }
    *reinterpret_cast<f32x4*>(sW + t * D + cc) = w;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < TPT; ++q) {
    const int t = tr + 8 * q;
    f32x4 o = *reinterpret_cast<const f32x4*>(sY + t * D + cc);
    f32x4 uu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < LP; ++r) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(sW + r * D + cc);
      o += sM[t * 16 + r] * w;
      if (commit) uu += sT[t * 16 + r] * w;
    }
    if (commit) *reinterpret_cast<f32x4*>(sU + t * D + cc) = uu;
    if (go) {
      if constexpr (EPI) {
        float ss = (o[0] * o[0] + o[1] * o[1]) + (o[2] * o[2] + o[3] * o[3]);
#pragma unroll
        for (int m = 1; m < 32; m <<= 1) ss += __shfl_xor(ss, m);
        const float inv = rsqrtf(ss * (1.f / D) + p.rms_eps);
        if (t < nt) {
          Frag16<E> gf;
          ld_frag16(gf, sGt + t * D + cc);
          const f32x4 gl = frag16_to_f32(gf);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] *= inv * nw[e] * sigmoidf_fast(gl[e]);
        }
      }
      if (t < nt) store_row4(go + ((size_t)(n * L + t) * H + h) * D + cc, o);
    }
  }
  if (commit) __syncthreads();  // U is read across the threads below

  // ---- 4. commit: S = Diag(D_last) S0 + Kb^T U ----
  // The contraction runs over the LP block rows, four per instruction: lane
  // group g4 carries rows g4 + 4 jj.  Kb^T[i][t] = K^[t][i] D_last[i] (with
  // unbounded decay the array already holds Kb).
  if (commit) {
    constexpr int NJ = LP / 4;
    float bu[2][NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const f32x2 x = *reinterpret_cast<const f32x2*>(sU + (g4 + 4 * jj) * D + col0);
      bu[0][jj] = x[0];
      bu[1][jj] = x[1];
    }
    float* S = p.state_out + u * (D * D) + col0;
#pragma unroll
    for (int T = 0; T < 8; ++T) {
      const f32x4 gam = *reinterpret_cast<const f32x4*>(sGam + 16 * T + 4 * g4);
      const float gi = sGam[16 * T + c16];
      float a[NJ];
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) a[jj] = sKh[(g4 + 4 * jj) * PS + 16 * T + c16] * (p.unbounded ? 1.f : gi);
#pragma unroll
      for (int C = 0; C < 2; ++C) {
        f32x4 acc = gam * st[T][C];
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[jj], bu[C][jj], acc, 0, 0, 0);
        st[T][C] = acc;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        __builtin_nontemporal_store((f32x2){st[T][0][e], st[T][1][e]},
                                    reinterpret_cast<f32x2*>(S + (16 * T + 4 * g4 + e) * D));
    }
    if (conv) {
      E* hs = static_cast<E*>(isk ? p.conv_k_state : p.conv_q_state);
      const size_t hb = ((size_t)n * 3 * H + h) * D + j;
      hs[hb] = from_f32<E>(x0);
      hs[hb + (size_t)H * D] = from_f32<E>(x1);
      hs[hb + (size_t)2 * H * D] = from_f32<E>(x2);
    }
  }
}

template <typename E, int LP, bool PRO, bool EPI>
hipError_t launch_replay_t(const ReplayArgs& a, hipStream_t stream) {
  const ReplayLayout lay(a.max_tokens, (int)sizeof(E), EPI, LP);
  auto fn = replay_kernel<E, LP, PRO, EPI>;
  if (lay.BYTES > 64u * 1024u) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lay.BYTES);
    if (e != hipSuccess) return e;
  }
  const int64_t units = (int64_t)a.num_seqs * a.num_heads;
  hipLaunchKernelGGL(fn, dim3((unsigned)units), dim3(kThreads), lay.BYTES, stream, a);
  return hipGetLastError();
}

template <typename E, int LP>
hipError_t launch_replay_lp(const ReplayArgs& a, hipStream_t stream) {
  const bool pro = a.conv_q_w || a.conv_k_w, epi = a.gate != nullptr;
  if (pro && epi) return launch_replay_t<E, LP, true, true>(a, stream);
  if (pro) return launch_replay_t<E, LP, true, false>(a, stream);
  if (epi) return launch_replay_t<E, LP, false, true>(a, stream);
  return launch_replay_t<E, LP, false, false>(a, stream);
}

template <typename E>
hipError_t launch_replay_e(const ReplayArgs& a, hipStream_t stream) {
  if (a.max_tokens <= 8) return launch_replay_lp<E, 8>(a, stream);
  return launch_replay_lp<E, 16>(a, stream);
}

}  // namespace

hipError_t launch_replay(const ReplayArgs& a, hipStream_t stream) {
  if (a.max_tokens < 1 || a.max_tokens > kReplayMaxTokens) return hipErrorInvalidValue;
  if (a.bf16) return launch_replay_e<__bf16>(a, stream);
  return launch_replay_e<float>(a, stream);
}

}  // namespace kda
