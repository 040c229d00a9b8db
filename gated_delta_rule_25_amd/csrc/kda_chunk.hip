// kda_chunk.hip — the two-kernel chunked prefill for gfx950.
//
// Method ("Kimi K3 架构、训练与系统全景解析", section 4.2.4 for the chunkwise
// form, section 4.2.5 for the bounded decay that keeps every exponent of the
// 16-token tiles in [-80, 0]).  For a chunk of n <= C tokens with incoming
// state S and per-channel cumulative log-decay g_r (within the chunk):
//   Kt = K (.) e^{g},  Qt = Q (.) e^{g},  Kh = K (.) e^{-g},  Kb = K (.) e^{g_n - g}
//   A  = strictly-lower( Diag(beta) Kt Kh^T ),   (I + A) [W | U'] = Diag(beta) [Kt | V]
//   U  = U' - W S,   O = Qt S + lower-incl( Qt Kh^T ) U,   S <- Diag(e^{g_n}) S + Kb^T U
// Everything up to W and U' depends on the inputs only.  Section 7.1 of the
// same page describes the state propagation as the serial part to keep
// short; so the work is split in two kernels:
//   prep_kernel   every (chunk, head) at once: decay prefix sums, scaled
//                 operand tiles, the Gram tiles on MFMA, the unit-triangular
//                 inverse, W and U' by blocked forward substitution; writes
//                 the factor block (-W, Qt, P, Kb^T, e^{g_n}, U') to the
//                 workspace (layout in kda_internal.h).
//   carry_kernel  one workgroup per (sequence, head, value-column block)
//                 walks the chunks in order with the fp32 state in MFMA
//                 accumulators: U = U' - W S, O = Qt S + P U, the optional
//                 RMSNorm x sigmoid-gate epilogue, and the state update.  The
//                 next chunk's factor block is loaded into registers while
//                 the current one is computed and lands in the other half of
//                 a double-buffered LDS area.
// Long inputs are processed in windows (every sequence advances by the same
// fraction of its chunks per window) so the factor store stays bounded; the
// state crosses windows through the final-state buffer.
#include "kda_chunk_util.h"

namespace kda {

// ---------------------------------------------------------------------------
// Window table: per sequence, its chunk range in window w and the first slot
// of that range in the factor store (exclusive prefix sum), clamped to `cap`
// slots so that inconsistent cu_seqlens cannot index past the store.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void window_table_kernel(const int32_t* __restrict__ cu, int N, int64_t T,
                                                             int C, int nw, int w, int cap,
                                                             int32_t* __restrict__ seq_first,
                                                             int32_t* __restrict__ seq_c0,
                                                             int32_t* __restrict__ seq_c1) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < N; base += 1024) {
    const int n = base + tid;
    int len = 0, c0 = 0;
    if (n < N) {
      const int64_t L = cu ? (int64_t)cu[n + 1] - (int64_t)cu[n] : T;
      const int64_t G = L > 0 ? (L + C - 1) / C : 0;
      const int64_t Q = (G + nw - 1) / nw;
      const int64_t a = min((int64_t)w * Q, G), b = min(a + Q, G);
      c0 = (int)a;
      len = (int)(b - a);
    }
    part[tid] = len;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int x = tid >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += x;
      __syncthreads();
    }
    if (n < N) {
      const int first = min(carry + part[tid] - len, cap);
      const int cnt = min(len, cap - first);
      seq_first[n] = first;
      seq_c0[n] = c0;
      seq_c1[n] = c0 + cnt;
    }
    carry = min(carry + part[1023], cap);
    __syncthreads();  // part[] is rewritten by the next round
  }
  if (tid == 0) seq_first[N] = carry;
}

hipError_t launch_window_table(const int32_t* cu, int num_seqs, int64_t total_tokens, int chunk, int nw, int w,
                               int cap, int32_t* seq_first, int32_t* seq_c0, int32_t* seq_c1, hipStream_t stream) {
  hipLaunchKernelGGL(window_table_kernel, dim3(1), dim3(1024), 0, stream, cu, num_seqs, total_tokens, chunk, nw, w,
                     cap, seq_first, seq_c0, seq_c1);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Carry kernel.
// ---------------------------------------------------------------------------
template <typename E, int C, int DV>
struct CarryLayout {
  using F = FactorBlock<(int)sizeof(E), C>;
  static constexpr int PAD = 16 / (int)sizeof(E);
  static constexpr int LDO = DV + PAD;
  // one buffer: the factor block's operand part [0, F::U) copied verbatim
  // (fragment order), rounded up to whole 4 KiB copy rounds
  static constexpr size_t BUF = ((size_t)F::U + 4095) & ~(size_t)4095;
  // two output staging tiles [C][LDO] (chunk i in tile i % 2)
  static constexpr size_t OST = al16((size_t)C * LDO * sizeof(E));
  static constexpr size_t O = 2 * BUF;
  static constexpr size_t SS = O + 2 * OST;              // f32 [4][C] row sums of squares
  static constexpr size_t BYTES = SS + (size_t)4 * C * 4;
};

template <typename E, int C, int DV, bool EPI>
__global__ __launch_bounds__(256) void carry_kernel(const CarryArgs p) {
  using L = CarryLayout<E, C, DV>;
  using F = FactorBlock<(int)sizeof(E), C>;
  constexpr int NT = C / 16;     // 16-token tiles per chunk
  constexpr int KT = C / 32;     // 32-deep token steps per chunk
  constexpr int NCW = DV / 4;    // value columns per wave
  constexpr int NCT = NCW / 16;  // 16-wide column tiles per wave
  constexpr int LDO = L::LDO;
  constexpr int ES = (int)sizeof(E);
  constexpr int PE = 16 / ES;                 // elements per 16-byte piece
  constexpr int RO = DV / PE;                 // pieces per output row of this block
  constexpr int NBP = (int)(L::BUF / 4096);   // 16-byte pieces per thread in one copy
  constexpr int NOP = C * RO / 256;
  static_assert(!EPI || DV == D, "the epilogue normalises whole heads");
  static_assert(NCT >= 1 && KT >= 1 && NT <= 4, "unsupported tile shape");
  static_assert((C * RO) % 256 == 0, "piece counts");
  static_assert(L::BYTES <= 160 * 1024, "LDS budget exceeded");

  extern __shared__ __align__(16) unsigned char smem[];
  float* sSS = reinterpret_cast<float*>(smem + L::SS);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, g = lane >> 4;
  // XCD-aware decode of the work item: blocks b and b + 8 run on the same XCD,
  // so the column blocks of one (sequence, head) share that XCD's L2.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int cb = slot % p.col_split;
  const int u = (slot / p.col_split) * 8 + xcd;
  if (u >= p.units) return;
  const int H = p.num_heads;
  const int rnk = u / H, h = u % H;
  const int n = p.order ? p.order[rnk] : rnk;
  const int64_t seq_bos = p.cu ? (int64_t)p.cu[n] : 0;
  const int64_t seq_eos = p.cu ? (int64_t)p.cu[n + 1] : p.total_tokens;
  const int c0 = p.seq_c0[n], nch = p.seq_c1[n] - c0, slot0 = p.seq_first[n];
  const int64_t rs = (int64_t)H * D;
  const int64_t hoff = (int64_t)h * D;
  const int col0 = cb * DV + wv * NCW;  // first value column owned by this wave
  E* go = static_cast<E*>(p.o);
  const char* fbase = static_cast<const char*>(p.factors);
  const uint32_t lane_fr = (uint32_t)lane * 8 * ES;

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
            p.state_in ? p.state_in[sbase + (size_t)(16 * rt8 + 4 * g + i) * D + col0 + 16 * ct + l16] : 0.f;

  // One chunk's factor block in flight: the operand part as 16-byte pieces
  // (piece tid + 256 j), and this wave's U' columns in accumulator order.
  const uint32_t p_off = (uint32_t)tid * 16;
  const uint32_t u_off = (uint32_t)(((col0 / 16) * 64 + lane) * 16);
  u32x4 rB[NBP];
  f32x4 rU[NT][NCT];
  auto load_block = [&](int ci) {
    const Rsrc rb = make_rsrc(fbase + ((size_t)(slot0 + ci) * H + h) * F::BYTES, F::BYTES);
#pragma unroll
    for (int j = 0; j < NBP; ++j) rB[j] = buf_ld16(rb, p_off, (uint32_t)(4096 * j));
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        rU[a][ct] = __builtin_bit_cast(f32x4, buf_ld16(rb, u_off, F::U + (uint32_t)(a * 8 + ct) * 1024));
  };
  // Output rows of chunk ci (staged in LDS tile ci % 2) to global memory.
  auto flush_o = [&](int ci) {
    const int64_t t0 = seq_bos + (int64_t)(c0 + ci) * C;
    const int nv = (int)min((int64_t)C, seq_eos - t0);
    const E* so = reinterpret_cast<const E*>(smem + L::O + (ci & 1) * L::OST);
#pragma unroll
    for (int j = 0; j < NOP; ++j) {
      const int pc = tid + 256 * j, r = pc / RO, c = (pc % RO) * PE;
      if (r < nv)
        *reinterpret_cast<u32x4*>(go + (t0 + r) * rs + hoff + cb * DV + c) =
            *reinterpret_cast<const u32x4*>(so + r * LDO + c);
    }
  };
  if (nch > 0) load_block(0);

  for (int ci = 0; ci < nch; ++ci) {
    const int64_t t0 = seq_bos + (int64_t)(c0 + ci) * C;
    const int nv = (int)min((int64_t)C, seq_eos - t0);
    unsigned char* buf = smem + (ci & 1) * L::BUF;
    const E* sW = reinterpret_cast<const E*>(buf + F::W + lane_fr);
    const E* sQt = reinterpret_cast<const E*>(buf + F::Q + lane_fr);
    const E* sP = reinterpret_cast<const E*>(buf + F::P + lane_fr);
    const E* sKbt = reinterpret_cast<const E*>(buf + F::K + lane_fr);
    const float* sGam = reinterpret_cast<const float*>(buf + F::G);
    constexpr int FRE = (int)F::FR / ES;  // elements per fragment
    E* sO = reinterpret_cast<E*>(smem + L::O + (ci & 1) * L::OST);

    // ---- factor block into this chunk's LDS half (the other half may still
    //      be read by waves finishing the previous chunk) ----
#pragma unroll
    for (int j = 0; j < NBP; ++j) *reinterpret_cast<u32x4*>(buf + p_off + 4096 * j) = rB[j];
    f32x4 accU[NT][NCT];
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) accU[a][ct] = rU[a][ct];
    __syncthreads();
    if (ci > 0) flush_o(ci - 1);
    if (ci + 1 < nch) load_block(ci + 1);

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
        ld_frag(fa, sW + (rt * 4 + ks) * FRE);   // W is stored negated
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
        ld_frag(fa, sQt + (rt * 4 + ks) * FRE);
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
          ld_frag(fa, sP + F::p_frag(rt, kt) * FRE);
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
          const int64_t row = (t0 + min(tok, nv - 1)) * rs + hoff;
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            const int col = col0 + 16 * ct + l16;
            const float w = p.norm_w ? p.norm_w[col] : 1.f;
            accO[rt][ct][i] *= inv * w * sigmoidf_fast(to_f32(gg[row + col]));
          }
        }
    }
    // outputs to this chunk's staging tile; written out after the next barrier
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          sO[(16 * rt + 4 * g + i) * LDO + wv * NCW + 16 * ct + l16] = from_f32<E>(accO[rt][ct][i]);

    // ---- S3: S <- Diag(e^{g_n}) S + Kb^T U ----
#pragma unroll
    for (int rt8 = 0; rt8 < 8; ++rt8) {
      const f32x4 gam = *reinterpret_cast<const f32x4*>(sGam + 16 * rt8 + 4 * g);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) accS[rt8][ct] *= gam;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        Frag<E> fa;
        ld_frag(fa, sKbt + (rt8 * KT + kt) * FRE);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) accS[rt8][ct] = mma(accS[rt8][ct], fa, uf[kt][ct]);
      }
    }
  }

  if (nch > 0) {
    __syncthreads();
    flush_o(nch - 1);
  }
  if (p.state_out) {
#pragma unroll
    for (int rt8 = 0; rt8 < 8; ++rt8)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          p.state_out[sbase + (size_t)(16 * rt8 + 4 * g + i) * D + col0 + 16 * ct + l16] = accS[rt8][ct][i];
  }
}

template <typename E, int C, int DV, bool EPI>
static hipError_t launch_carry_t(const CarryArgs& a, hipStream_t stream) {
  constexpr size_t lds = CarryLayout<E, C, DV>::BYTES;
  static_assert(lds <= 160 * 1024, "LDS budget exceeded");
  auto fn = carry_kernel<E, C, DV, EPI>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int groups = (a.units + 7) / 8;
  const unsigned grid = (unsigned)(8 * a.col_split * groups);
  if (a.units <= 0) return hipSuccess;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(256), lds, stream, a);
  return hipGetLastError();
}

template <typename E, int C>
static hipError_t launch_carry_dtype(const CarryArgs& a, hipStream_t stream) {
  if (a.gate) {
    if (a.col_split != 1) return hipErrorInvalidValue;
    return launch_carry_t<E, C, 128, true>(a, stream);
  }
  if (a.col_split == 2) return launch_carry_t<E, C, 64, false>(a, stream);
  if (a.col_split == 1) return launch_carry_t<E, C, 128, false>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_carry(const CarryArgs& a, hipStream_t stream) {
  if (a.bf16) return launch_carry_dtype<__bf16, 64>(a, stream);
  return launch_carry_dtype<float, 32>(a, stream);
}

}  // namespace kda
