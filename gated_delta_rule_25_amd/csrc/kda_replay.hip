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
// Per (sequence n, head h) one 256-thread workgroup:
//   1. issues the 64 KiB state load (thread t owns columns 4(t%32)..+3 and
//      rows 16(t/32)..+15, as in the single-token decode) and every cached
//      input of the tokens it runs (16-byte pieces: q and k rows with their
//      three history rows when the convolution runs, v, log_alpha, gate),
//      all in flight together, the inputs staged in LDS;
//   2. forms per token the decay a = exp(log_alpha), the prologue
//      (ShortConv4 + SiLU, then L2 over the head's channels; "Kimi K3 架构…"
//      section 4.2.3) and the products a*q', a*k', k', q'.k';
//   3. runs the tokens one after another on the register-resident state:
//      x = sum_i a_i k_i S[i,:], y = sum_i a_i q_i S[i,:] (one LDS exchange
//      across the four waves), u = beta (v - x), S <- a S + k u^T,
//      o = y + (k.q) u, then RMSNorm x sigmoid(gate) (section 4.2.6);
//   4. writes the state and the three raw rows before the next token only
//      when a state output is given.
// The state is read once and written at most once however many tokens run,
// so the HBM bytes per token fall with the number of tokens.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kThreads = 256;

// Dynamic LDS of one workgroup for L cached tokens (byte offsets, all
// multiples of 16).
struct ReplayLayout {
  uint32_t RQ, RK, RV, RG, RLA, A, AQ, KP, AK, SC, PART, BYTES;
  __host__ __device__ ReplayLayout(int L, int es, bool gate) {
    const uint32_t rb = 128u * (uint32_t)es;
    RQ = 0;                                   // E [3 + L][128]: raw q, history rows then tokens
    RK = RQ + (3u + L) * rb;                  // E [3 + L][128]: raw k
    RV = RK + (3u + L) * rb;                  // E [L][128]
    RG = RV + (uint32_t)L * rb;               // E [L][128] gate logits
    RLA = RG + (gate ? (uint32_t)L * rb : 0u);  // f32 [L][128] log_alpha
    A = RLA + (uint32_t)L * 512u;             // f32 [L][128] a = exp(log_alpha)
    AQ = A + (uint32_t)L * 512u;              // f32 [L][128] q before L2, then a * q'
    KP = AQ + (uint32_t)L * 512u;             // f32 [L][128] k before L2, then k'
    AK = KP + (uint32_t)L * 512u;             // f32 [L][128] a * k'
    SC = AK + (uint32_t)L * 512u;             // f32 [L][4]  1/|q|, 1/|k|, q'.k', beta
    PART = SC + (uint32_t)L * 16u;            // f32 [2][4 waves][2][128] column-sum exchange
    BYTES = PART + 2u * 4u * 2u * 128u * 4u;
  }
};

template <typename E>
__device__ __forceinline__ float lds_elem(const unsigned char* base, int row, int j) {
  return to_f32(reinterpret_cast<const E*>(base)[row * D + j]);
}

template <typename E>
__device__ __forceinline__ void store4(E* dst, const f32x4& x);
template <>
__device__ __forceinline__ void store4<float>(float* dst, const f32x4& x) {
  *reinterpret_cast<f32x4*>(dst) = x;
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* dst, const f32x4& x) {
  const bf16x4 b = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
  *reinterpret_cast<bf16x4*>(dst) = b;
}

template <typename E, bool PRO, bool EPI>
__global__ __launch_bounds__(kThreads) void replay_kernel(const ReplayArgs p) {
  constexpr int ES = (int)sizeof(E);
  constexpr int RP = D * ES / 16;  // 16-byte pieces of one row in the I/O dtype
  constexpr int LP = D * 4 / 16;   // pieces of one log_alpha row
  extern __shared__ __align__(16) unsigned char smem[];

  const int L = p.max_tokens, H = p.num_heads;
  const ReplayLayout lay(L, ES, EPI);
  const int64_t u = blockIdx.x;  // n * H + h
  const int n = (int)(u / H), h = (int)(u % H);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int cg = tid & 31;  // columns 4cg .. 4cg+3
  const int rg = tid >> 5;  // rows 16rg .. 16rg+15
  int nt = p.num_tokens ? p.num_tokens[n] : L;
  nt = min(max(nt, 0), L);

  // ---- 1. state and token inputs in flight together ----
  f32x4 st[16];
  if (p.state_in) {
    const float* S = p.state_in + u * (D * D);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      st[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (16 * rg + i) * D + 4 * cg));
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  const bool cq = PRO && p.conv_q_w, ck = PRO && p.conv_k_w;
  const size_t rowb = (size_t)D * ES;
  // Staging: one guarded loop per input, each a fixed number of 16-byte
  // pieces per thread, every load issued before the first LDS store.
  // q / k: staged row r holds the history (rows 0..2, oldest first) or token
  // r - 3; without the convolution only rows 3 .. 3 + nt - 1 are loaded.
  constexpr int QKS = ((3 + kReplayMaxTokens) * RP + kThreads - 1) / kThreads;
  constexpr int VS = (kReplayMaxTokens * RP + kThreads - 1) / kThreads;
  constexpr int LS = (kReplayMaxTokens * LP + kThreads - 1) / kThreads;
  u32x4 rq[QKS], rk[QKS], rv[VS], rl[LS], rgt[EPI ? VS : 1];
  auto qk_src = [&](const void* tok, const void* hist, int r, int w) {
    const char* b = r < 3 ? static_cast<const char*>(hist) + ((size_t)(n * 3 + r) * H + h) * rowb
                          : static_cast<const char*>(tok) + ((size_t)(n * L + r - 3) * H + h) * rowb;
    return reinterpret_cast<const u32x4*>(b + w * 16);
  };
  auto tok_src = [&](const void* base, size_t rb, int t, int w) {
    return reinterpret_cast<const u32x4*>(static_cast<const char*>(base) + ((size_t)(n * L + t) * H + h) * rb +
                                          w * 16);
  };
  const int q0 = cq ? 0 : 3, k0 = ck ? 0 : 3;  // first staged row
  const int nq = (3 + nt - q0) * RP, nk = (3 + nt - k0) * RP, ntp = nt * RP, nlp = nt * LP;
#pragma unroll
  for (int i = 0; i < QKS; ++i) {
    const int pc = tid + kThreads * i;
    if (pc < nq) rq[i] = *qk_src(p.q, p.conv_q_state, q0 + pc / RP, pc % RP);
    if (pc < nk) rk[i] = *qk_src(p.k, p.conv_k_state, k0 + pc / RP, pc % RP);
  }
#pragma unroll
  for (int i = 0; i < VS; ++i) {
    const int pc = tid + kThreads * i;
    if (pc < ntp) rv[i] = *tok_src(p.v, rowb, pc / RP, pc % RP);
    if (EPI && pc < ntp) rgt[i] = *tok_src(p.gate, rowb, pc / RP, pc % RP);
  }
#pragma unroll
  for (int i = 0; i < LS; ++i) {
    const int pc = tid + kThreads * i;
    if (pc < nlp) rl[i] = *tok_src(p.log_alpha, D * 4, pc / LP, pc % LP);
  }
  float bt = 0.f;
  if (tid < nt) bt = p.beta[((size_t)n * L + tid) * H + h];
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
  auto put = [&](uint32_t off, const u32x4& x) { *reinterpret_cast<u32x4*>(smem + off) = x; };
#pragma unroll
  for (int i = 0; i < QKS; ++i) {
    const int pc = tid + kThreads * i;
    if (pc < nq) put(lay.RQ + (uint32_t)(q0 * RP + pc) * 16u, rq[i]);
    if (pc < nk) put(lay.RK + (uint32_t)(k0 * RP + pc) * 16u, rk[i]);
  }
#pragma unroll
  for (int i = 0; i < VS; ++i) {
    const int pc = tid + kThreads * i;
    if (pc < ntp) put(lay.RV + (uint32_t)pc * 16u, rv[i]);
    if (EPI && pc < ntp) put(lay.RG + (uint32_t)pc * 16u, rgt[i]);
  }
#pragma unroll
  for (int i = 0; i < LS; ++i) {
    const int pc = tid + kThreads * i;
    if (pc < nlp) put(lay.RLA + (uint32_t)pc * 16u, rl[i]);
  }
  float* sA = reinterpret_cast<float*>(smem + lay.A);
  float* sAQ = reinterpret_cast<float*>(smem + lay.AQ);
  float* sKP = reinterpret_cast<float*>(smem + lay.KP);
  float* sAK = reinterpret_cast<float*>(smem + lay.AK);
  float* sSC = reinterpret_cast<float*>(smem + lay.SC);
  if (tid < nt) sSC[4 * tid + 3] = bt;
  __syncthreads();

  // ---- 2. per-token operands ----
  {
    const unsigned char* rows = smem + (isk ? lay.RK : lay.RQ);
    float* pre = isk ? sKP : sAQ;  // before the L2 scale
    const float* sla = reinterpret_cast<const float*>(smem + lay.RLA);
    float x0 = 0.f, x1 = 0.f, x2 = 0.f;  // raw rows t-3, t-2, t-1 of channel j
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
        s = c / (1.f + __expf(-c));
        x0 = x1;
        x1 = x2;
        x2 = x3;
      }
      pre[t * D + j] = s;
      if (!isk) sA[t * D + j] = __expf(sla[t * D + j]);
    }
  }
  __syncthreads();
  // squared norms and q.k of every token (wave wv takes tokens wv, wv + 4, ...)
  for (int t = wv; t < nt; t += 4) {
    const float q0 = sAQ[t * D + lane], q1 = sAQ[t * D + 64 + lane];
    const float k0 = sKP[t * D + lane], k1 = sKP[t * D + 64 + lane];
    float sq = q0 * q0 + q1 * q1, sk = k0 * k0 + k1 * k1, qk = q0 * k0 + q1 * k1;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      sq += __shfl_xor(sq, m);
      sk += __shfl_xor(sk, m);
      qk += __shfl_xor(qk, m);
    }
    if (lane == 0) {
      const float iq = cq ? rsqrtf(sq + p.l2_eps) : 1.f;
      const float ik = ck ? rsqrtf(sk + p.l2_eps) : 1.f;
      sSC[4 * t] = iq;
      sSC[4 * t + 1] = ik;
      sSC[4 * t + 2] = qk * iq * ik;
    }
  }
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    const float a = sA[t * D + j];
    if (!isk) {
      sAQ[t * D + j] = a * (sAQ[t * D + j] * sSC[4 * t]);
    } else {
      const float kv = sKP[t * D + j] * sSC[4 * t + 1];
      sKP[t * D + j] = kv;
      sAK[t * D + j] = a * kv;
    }
  }
  __syncthreads();

  // ---- 3. the tokens, in order, on the register-resident state ----
  E* go = static_cast<E*>(p.o);
  const E* sV = reinterpret_cast<const E*>(smem + lay.RV);
  const E* sG = reinterpret_cast<const E*>(smem + lay.RG);
  float* part = reinterpret_cast<float*>(smem + lay.PART);
  f32x4 nw = {1.f, 1.f, 1.f, 1.f};
  if (EPI && p.norm_w) {
#pragma unroll
    for (int e = 0; e < 4; ++e) nw[e] = p.norm_w[4 * cg + e];
  }
  for (int t = 0; t < nt; ++t) {
    const f32x4* ak4 = reinterpret_cast<const f32x4*>(sAK + t * D + 16 * rg);
    const f32x4* aq4 = reinterpret_cast<const f32x4*>(sAQ + t * D + 16 * rg);
    f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 ka = ak4[i4], qa = aq4[i4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x += ka[e] * st[4 * i4 + e];
        y += qa[e] * st[4 * i4 + e];
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] += __shfl_xor(x[e], 32);
      y[e] += __shfl_xor(y[e], 32);
    }
    float* pp = part + (t & 1) * (4 * 2 * D);
    if ((tid & 32) == 0) {
      *reinterpret_cast<f32x4*>(pp + wv * 2 * D + 4 * cg) = x;
      *reinterpret_cast<f32x4*>(pp + wv * 2 * D + D + 4 * cg) = y;
    }
    __syncthreads();
    x = *reinterpret_cast<const f32x4*>(pp + 4 * cg);
    y = *reinterpret_cast<const f32x4*>(pp + D + 4 * cg);
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      x += *reinterpret_cast<const f32x4*>(pp + w * 2 * D + 4 * cg);
      y += *reinterpret_cast<const f32x4*>(pp + w * 2 * D + D + 4 * cg);
    }
    const f32x4 sc = *reinterpret_cast<const f32x4*>(sSC + 4 * t);  // 1/|q|, 1/|k|, q'.k', beta
    f32x4 vv;
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = to_f32(sV[t * D + 4 * cg + e]);
    const f32x4 uu = sc[3] * (vv - x);
    const f32x4* a4 = reinterpret_cast<const f32x4*>(sA + t * D + 16 * rg);
    const f32x4* k4 = reinterpret_cast<const f32x4*>(sKP + t * D + 16 * rg);
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 a = a4[i4], kk = k4[i4];
#pragma unroll
      for (int e = 0; e < 4; ++e) st[4 * i4 + e] = a[e] * st[4 * i4 + e] + kk[e] * uu;
    }
    if (wv == 0 && go) {
      // lanes 32..63 hold the same columns as lanes 0..31
      f32x4 oo = y + sc[2] * uu;
      if (EPI) {
        float ss = oo[0] * oo[0] + oo[1] * oo[1] + oo[2] * oo[2] + oo[3] * oo[3];
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
        const float inv = rsqrtf(ss * (1.f / D) + p.rms_eps);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gl = to_f32(sG[t * D + 4 * cg + e]);
          oo[e] = oo[e] * inv * nw[e] / (1.f + __expf(-gl));
        }
      }
      if (rg == 0) store4<E>(go + ((size_t)(n * L + t) * H + h) * D + 4 * cg, oo);
    }
  }

  // ---- 4. commit ----
  if (p.state_out) {
    float* S = p.state_out + u * (D * D);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      __builtin_nontemporal_store(st[i], reinterpret_cast<f32x4*>(S + (16 * rg + i) * D + 4 * cg));
    if (conv) {
      // raw rows nt-3 .. nt-1 are staged rows nt .. nt+2; only this thread read channel j of them
      E* hs = static_cast<E*>(isk ? p.conv_k_state : p.conv_q_state);
      const E* rows = reinterpret_cast<const E*>(smem + (isk ? lay.RK : lay.RQ));
#pragma unroll
      for (int m = 0; m < 3; ++m) hs[((size_t)(n * 3 + m) * H + h) * D + j] = rows[(nt + m) * D + j];
    }
  }
}

template <typename E, bool PRO, bool EPI>
hipError_t launch_replay_t(const ReplayArgs& a, hipStream_t stream) {
  const ReplayLayout lay(a.max_tokens, (int)sizeof(E), EPI);
  auto fn = replay_kernel<E, PRO, EPI>;
  if (lay.BYTES > 64u * 1024u) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lay.BYTES);
    if (e != hipSuccess) return e;
  }
  const int64_t units = (int64_t)a.num_seqs * a.num_heads;
  hipLaunchKernelGGL(fn, dim3((unsigned)units), dim3(kThreads), lay.BYTES, stream, a);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_replay_e(const ReplayArgs& a, hipStream_t stream) {
  const bool pro = a.conv_q_w || a.conv_k_w, epi = a.gate != nullptr;
  if (pro && epi) return launch_replay_t<E, true, true>(a, stream);
  if (pro) return launch_replay_t<E, true, false>(a, stream);
  if (epi) return launch_replay_t<E, false, true>(a, stream);
  return launch_replay_t<E, false, false>(a, stream);
}

}  // namespace

hipError_t launch_replay(const ReplayArgs& a, hipStream_t stream) {
  if (a.max_tokens < 1 || a.max_tokens > kReplayMaxTokens) return hipErrorInvalidValue;
  if (a.bf16) return launch_replay_e<__bf16>(a, stream);
  return launch_replay_e<float>(a, stream);
}

}  // namespace kda
