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
  // One LDS slot holds the parts of a factor block every compute wave reads
  // in full: -W, Qt, Kb^T and gamma (P and U' go to registers).  Slot
  // offsets, with the block offset each 1 KiB piece is copied from:
  static constexpr uint32_t W = 0;                        // <- F::W
  static constexpr uint32_t Q = W + F::NT * 4 * F::FR;    // <- F::Q
  static constexpr uint32_t K = Q + F::NT * 4 * F::FR;    // <- F::K
  static constexpr uint32_t G = K + 8 * F::KT * F::FR;    // <- F::G (one piece)
  static constexpr uint32_t SLOT = G + 1024;
  static constexpr int PIECES = SLOT / 1024;
  static_assert(F::K % 1024 == 0 && F::G % 1024 == 0 && Q % 1024 == 0 && K % 1024 == 0, "1 KiB pieces");
  static constexpr int NBUF = 3;                          // chunks in flight
  static constexpr size_t SS = (size_t)NBUF * SLOT;       // f32 [DV / 16][C] row sums of squares
  static constexpr size_t BYTES = SS + (size_t)(DV / 16) * C * 4;
  // block offset of slot piece j

};

// Number of vector-memory operations allowed to stay outstanding in s_waitcnt.
__host__ __device__ constexpr int vmcnt_wait(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }

// Workgroup of DV / 16 compute waves plus one loader wave.  Compute wave w
// owns value columns 16 w .. 16 w + 15 of the block and keeps that slice of
// the fp32 state in MFMA accumulators.  The loader wave copies each chunk's
// factor block (its -W, Qt, Kb^T and gamma part) straight from global memory
// into LDS slot ci % 3, two chunks ahead, so the compute waves never wait
// behind the vector memory unit; they fetch P and U' one chunk ahead into
// registers and store their outputs directly.  One barrier per chunk hands
// the slots over: after barrier ci, slot ci % 3 holds chunk ci, and every
// wave is past chunk ci - 1, so the loader may refill slot (ci + 2) % 3.
template <typename E, int C, int DV, bool EPI>
__global__ __launch_bounds__(64 * (DV / 16 + 1)) void carry_kernel(const CarryArgs p) {
  using L = CarryLayout<E, C, DV>;
  using F = FactorBlock<(int)sizeof(E), C>;
  constexpr int NT = C / 16;     // 16-token tiles per chunk
  constexpr int KT = C / 32;     // 32-deep token steps per chunk
  constexpr int NWC = DV / 16;   // compute waves; wave NWC is the loader
  constexpr int ES = (int)sizeof(E);
  static_assert(!EPI || DV == D, "the epilogue normalises whole heads");
  static_assert(KT >= 1 && NT <= 4, "unsupported tile shape");
  static_assert(L::BYTES <= 160 * 1024, "LDS budget exceeded");
  static_assert(L::PIECES <= 63, "copy exceeds the outstanding-load counter");

  extern __shared__ __align__(16) unsigned char smem[];
  float* sSS = reinterpret_cast<float*>(smem + L::SS);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
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
  const char* fbase = static_cast<const char*>(p.factors);
  auto block_of = [&](int ci) { return fbase + ((size_t)(slot0 + ci) * H + h) * F::BYTES; };

  if (wv == NWC) {
    // ---- loader wave ----
    auto copy_block = [&](int ci) {
      const char* blk = block_of(ci);
      unsigned char* dst = smem + (ci % L::NBUF) * L::SLOT;
      constexpr uint32_t kSlotK = L::K, kBlockK = F::K;
#pragma unroll
      for (int j = 0; j < L::PIECES; ++j)
        __builtin_amdgcn_global_load_lds(blk + (j * 1024u < kSlotK ? j * 1024u : kBlockK + (j * 1024u - kSlotK)) + lane * 16,
                                         (__attribute__((address_space(3))) void*)(dst + j * 1024), 16, 0, 0);
    };
    if (nch > 0) copy_block(0);
    if (nch > 1) copy_block(1);
    for (int ci = 0; ci < nch; ++ci) {
      // chunk ci's copy has landed; the one of chunk ci + 1 may be in flight
      if (ci + 1 < nch) __builtin_amdgcn_s_waitcnt(vmcnt_wait(L::PIECES));
      else __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
      __syncthreads();
      if (ci + 2 < nch) copy_block(ci + 2);
      if (EPI) __syncthreads();  // the compute waves' row-sum exchange
    }
    return;
  }

  // ---- compute waves ----
  const int col0 = cb * DV + 16 * wv;  // first value column owned by this wave
  E* go = static_cast<E*>(p.o);
  const float norm_w = (EPI && p.norm_w) ? p.norm_w[col0 + (lane & 15)] : 1.f;

  // State slice: tile rt8 holds rows 16 rt8 + 4g + i, column col0 + l16.
  f32x4 accS[8];
  const size_t sbase = ((size_t)n * H + h) * (size_t)(D * D);
  {
    const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int rt8 = 0; rt8 < 8; ++rt8)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        accS[rt8][i] = p.state_in ? p.state_in[sbase + (size_t)(16 * rt8 + 4 * g + i) * D + col0 + l16] : 0.f;
  }

  // P fragments and this wave's U' columns (accumulator order) of the next
  // chunk, fetched into registers one chunk ahead (U' right after the
  // barrier, P once the current chunk's P has been used).
  Frag<E> rP[F::NP];
  f32x4 rU[NT];
  auto load_u = [&](int ci) {
    const Rsrc rb = make_rsrc(block_of(ci), F::BYTES);
    const uint32_t u_off = (uint32_t)((col0 / 16) * F::UT + lane * 4 * ES);
#pragma unroll
    for (int a = 0; a < NT; ++a) {
      if constexpr (ES == 2) {
        const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rb, (int)u_off, (int)(F::U + a * 8 * F::UT), 0);
        const bf16x4 b = __builtin_bit_cast(bf16x4, x);
        rU[a] = (f32x4){(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
      } else {
        rU[a] = __builtin_bit_cast(f32x4, buf_ld16(rb, u_off, F::U + a * 8 * F::UT));
      }
    }
  };
  auto load_p = [&](int ci) {
    const Rsrc rb = make_rsrc(block_of(ci), F::BYTES);
    const uint32_t lane_fr = (uint32_t)lane * 8 * ES;
#pragma unroll
    for (int f = 0; f < F::NP; ++f) {
      if constexpr (ES == 2) {
        rP[f].v = __builtin_bit_cast(bf16x8, buf_ld16(rb, lane_fr, F::P + f * F::FR));
      } else {
        rP[f].lo = __builtin_bit_cast(f32x4, buf_ld16(rb, lane_fr, F::P + f * F::FR));
        rP[f].hi = __builtin_bit_cast(f32x4, buf_ld16(rb, lane_fr + 16, F::P + f * F::FR));
      }
    }
  };
  // Whole-head blocks with the epilogue run nine waves, whose register budget
  // has no room for P in flight: they fetch P at the top of each chunk.
  constexpr bool PF_P = !EPI;
  if (nch > 0) {
    load_u(0);
    if (PF_P) load_p(0);
  }

  for (int ci = 0; ci < nch; ++ci) {
    // lane indices from an opaque copy of the thread id, so the per-lane
    // address arithmetic stays inside the loop rather than in registers
    int tidv = tid;
    asm volatile("" : "+v"(tidv));
    const int lane = tidv & 63, l16 = lane & 15, g = lane >> 4;
    const uint32_t lane_fr = (uint32_t)lane * 8 * ES;
    const int64_t t0 = seq_bos + (int64_t)(c0 + ci) * C;
    const int nv = (int)min((int64_t)C, seq_eos - t0);
    const unsigned char* buf = smem + (ci % L::NBUF) * L::SLOT;
    const E* sW = reinterpret_cast<const E*>(buf + L::W + lane_fr);
    const E* sQt = reinterpret_cast<const E*>(buf + L::Q + lane_fr);
    const E* sKbt = reinterpret_cast<const E*>(buf + L::K + lane_fr);
    const float* sGam = reinterpret_cast<const float*>(buf + L::G);
    constexpr int FRE = (int)F::FR / ES;  // elements per fragment

    f32x4 accU[NT];
#pragma unroll
    for (int a = 0; a < NT; ++a) accU[a] = rU[a];
    __syncthreads();
    if (!PF_P) load_p(ci);
    if (ci + 1 < nch) load_u(ci + 1);

    // Four-wave blocks: each stage first issues all of its LDS fragment
    // reads (the scheduling barrier keeps them ahead of the matrix-core work,
    // so they are in flight together instead of one at a time), then runs its
    // products with the independent accumulators interleaved.  The nine-wave
    // whole-head blocks lack the registers and stream one fragment at a time.
    constexpr bool BATCH = NWC == 4;
    Frag<E> sf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) frag_from_acc(sf[ks], accS[2 * ks], accS[2 * ks + 1]);
    f32x4 accO[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) accO[rt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if constexpr (BATCH) {
      // ---- S1: U = U' - W S ----
      Frag<E> fa[4 * NT];
#pragma unroll
      for (int i = 0; i < 4 * NT; ++i) ld_frag(fa[i], sW + i * FRE);   // W is stored negated
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) accU[rt] = mma(accU[rt], fa[rt * 4 + ks], sf[ks]);
      // ---- S2: O = Qt S (+ P U below) ----
#pragma unroll
      for (int i = 0; i < 4 * NT; ++i) ld_frag(fa[i], sQt + i * FRE);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) accO[rt] = mma(accO[rt], fa[rt * 4 + ks], sf[ks]);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
          Frag<E> fa;
          ld_frag(fa, sW + (rt * 4 + ks) * FRE);
          accU[rt] = mma(accU[rt], fa, sf[ks]);
        }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
          Frag<E> fa;
          ld_frag(fa, sQt + (rt * 4 + ks) * FRE);
          accO[rt] = mma(accO[rt], fa, sf[ks]);
        }
    }
    Frag<E> uf[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) frag_from_acc(uf[kt], accU[2 * kt], accU[2 * kt + 1]);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
        if (kt <= rt / 2) accO[rt] = mma(accO[rt], rP[F::p_frag(rt, kt)], uf[kt]);
    if (PF_P && ci + 1 < nch) load_p(ci + 1);

    if (EPI) {
      // head-wise RMSNorm over the 128 value channels, then the sigmoid gate;
      // the gate logits of this chunk are read through a buffer view with
      // 32-bit offsets (rows past the sequence end read its last row)
      const Rsrc gr = make_rsrc(static_cast<const E*>(p.gate) + t0 * rs, (uint32_t)(C * rs * ES));
      float gl[NT][4];
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = min(16 * rt + 4 * g + i, nv - 1);
          gl[rt][i] = buf_ld_elem(gr, (uint32_t)((tok * rs + hoff + col0 + l16) * ES), (E*)nullptr);
        }
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float ss = accO[rt][i] * accO[rt][i];
#pragma unroll
          for (int m = 1; m < 16; m <<= 1) ss += __shfl_xor(ss, m);
          if (l16 == 0) sSS[wv * C + 16 * rt + 4 * g + i] = ss;
        }
      __syncthreads();
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 16 * rt + 4 * g + i;
          float ms = 0.f;
#pragma unroll
          for (int q = 0; q < NWC; ++q) ms += sSS[q * C + tok];
          const float inv = rsqrtf(ms * (1.f / D) + p.rms_eps);
          accO[rt][i] *= inv * norm_w * sigmoidf_fast(gl[rt][i]);
        }
    }
    // outputs: each 16 x 16 tile transposed on the matrix cores to lane =
    // token, four consecutive columns, and stored straight to global memory
    {
      Frag16<E> id;
      {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (4 * g + e == l16) ? 1.f : 0.f;
        frag16_from_acc(id, x);
      }
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        Frag16<E> a;
        frag16_from_acc(a, accO[rt]);
        const f32x4 t = mma16((f32x4){0.f, 0.f, 0.f, 0.f}, a, id);
        const int tok = 16 * rt + l16;
        if (tok < nv) {
          E* dst = go + (t0 + tok) * rs + hoff + col0 + 4 * g;
          if constexpr (ES == 2)
            *reinterpret_cast<bf16x4*>(dst) = (bf16x4){(__bf16)t[0], (__bf16)t[1], (__bf16)t[2], (__bf16)t[3]};
          else
            *reinterpret_cast<f32x4*>(dst) = t;
        }
      }
    }

    // ---- S3: S <- Diag(e^{g_n}) S + Kb^T U ----
    if constexpr (BATCH) {
      Frag<E> fa[8 * KT];
#pragma unroll
      for (int i = 0; i < 8 * KT; ++i) ld_frag(fa[i], sKbt + i * FRE);
      f32x4 gam[8];
#pragma unroll
      for (int rt8 = 0; rt8 < 8; ++rt8) gam[rt8] = *reinterpret_cast<const f32x4*>(sGam + 16 * rt8 + 4 * g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rt8 = 0; rt8 < 8; ++rt8) accS[rt8] *= gam[rt8];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int rt8 = 0; rt8 < 8; ++rt8) accS[rt8] = mma(accS[rt8], fa[rt8 * KT + kt], uf[kt]);
    } else {
#pragma unroll
      for (int rt8 = 0; rt8 < 8; ++rt8) {
        accS[rt8] *= *reinterpret_cast<const f32x4*>(sGam + 16 * rt8 + 4 * g);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          Frag<E> fa;
          ld_frag(fa, sKbt + (rt8 * KT + kt) * FRE);
          accS[rt8] = mma(accS[rt8], fa, uf[kt]);
        }
      }
    }
  }

  if (p.state_out) {
    const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int rt8 = 0; rt8 < 8; ++rt8)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p.state_out[sbase + (size_t)(16 * rt8 + 4 * g + i) * D + col0 + l16] = accS[rt8][i];
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
  hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * (DV / 16 + 1)), lds, stream, a);
  return hipGetLastError();
}

template <typename E, int C>
static hipError_t launch_carry_dtype(const CarryArgs& a, hipStream_t stream) {
  // whole heads (the epilogue normalises over all 128 value columns), else
  // two 64-column blocks per head that share the factor reads through L2
  if (a.gate) return a.col_split == 1 ? launch_carry_t<E, C, 128, true>(a, stream) : hipErrorInvalidValue;
  return a.col_split == 2 ? launch_carry_t<E, C, 64, false>(a, stream) : hipErrorInvalidValue;
}

hipError_t launch_carry(const CarryArgs& a, hipStream_t stream) {
  if (a.bf16) return launch_carry_dtype<__bf16, 64>(a, stream);
  return launch_carry_dtype<float, 32>(a, stream);
}

}  // namespace kda
