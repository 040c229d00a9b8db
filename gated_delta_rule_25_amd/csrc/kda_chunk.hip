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
//                 RMSNorm x sigmoid-gate epilogue, and the state update.  A
//                 loader wave copies the factor blocks into a three-slot LDS
//                 ring two chunks ahead of the compute waves.
// Long inputs are processed in windows (every sequence advances by the same
// fraction of its chunks per window) so the factor store stays bounded; the
// state crosses windows through the final-state buffer.  With too few
// (sequence, head) chains to fill the GPU, the carry runs in two passes over
// segments of each window instead (section 7.1's in-device context
// parallelism): pass 1 traces each segment's affine pair from a zero state
// and from the identity, scan_kernel (kda_scan.hip) composes the pairs into
// incoming states, and pass 2 writes the outputs from them.
#include "kda_chunk_util.h"

namespace kda {

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
      int64_t bos, eos;
      seq_range(cu, n, T, bos, eos);
      const int64_t L = eos - bos;
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
// Segments of a window: sequence n's chunks [seq_c0[n], seq_c1[n]) cut into
// runs of seg_chunks; one workgroup, sequences 1024 at a time with a
// block-wide scan of the counts, entries clamped to cap.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void window_segments_kernel(const int32_t* __restrict__ seq_c0,
                                                                const int32_t* __restrict__ seq_c1, int N,
                                                                int seg_chunks, int cap,
                                                                int32_t* __restrict__ seg_first,
                                                                int32_t* __restrict__ seg_list,
                                                                int32_t* __restrict__ seg_count) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < N; base += 1024) {
    const int n = base + tid;
    int G = 0;
    if (n < N) {
      const int len = seq_c1[n] - seq_c0[n];
      G = len > 0 ? (len + seg_chunks - 1) / seg_chunks : 0;
    }
    part[tid] = G;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int x = tid >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += x;
      __syncthreads();
    }
    if (n < N) {
      const int first = min(carry + part[tid] - G, cap);
      const int cnt = min(G, cap - first);
      seg_first[n] = first;
      for (int j = 0; j < cnt; ++j) {
        seg_list[2 * (first + j)] = n;
        seg_list[2 * (first + j) + 1] = j;
      }
    }
    carry = min(carry + part[1023], cap);
    __syncthreads();  // part[] is rewritten by the next round
  }
  if (tid == 0) {
    seg_first[N] = carry;
    *seg_count = carry;
  }
}

hipError_t launch_window_segments(const int32_t* seq_c0, const int32_t* seq_c1, int num_seqs, int seg_chunks,
                                  int cap, int32_t* seg_first, int32_t* seg_list, int32_t* seg_count,
                                  hipStream_t stream) {
  hipLaunchKernelGGL(window_segments_kernel, dim3(1), dim3(1024), 0, stream, seq_c0, seq_c1, num_seqs, seg_chunks,
                     cap, seg_first, seg_list, seg_count);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Carry kernel.
// ---------------------------------------------------------------------------
template <typename E, int C, int NWC>
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
  static constexpr size_t SS = (size_t)NBUF * SLOT;       // f32 [NWC][C] per-wave row sums of squares
  static constexpr size_t BYTES = SS + (size_t)NWC * C * 4;
};

// Workgroup of NWC = DV / (16 CT) compute waves plus one loader wave.
// Compute wave w owns the CT 16-column tiles of value columns
// 16 CT w .. 16 CT (w + 1) - 1 of the block and keeps that slice of the fp32
// state in MFMA accumulators; every -W, Qt or Kb^T fragment it reads from LDS
// feeds CT products.  The loader wave copies each chunk's factor block (its
// -W, Qt, Kb^T and gamma part) straight from global memory into LDS slot
// ci % 3, two chunks ahead, so the compute waves never wait behind the
// vector memory unit; they fetch P and U' one chunk ahead into registers and
// store their outputs directly.  One barrier per chunk hands the slots over:
// after barrier ci, slot ci % 3 holds chunk ci, and every wave is past chunk
// ci - 1, so the loader may refill slot (ci + 2) % 3.
template <typename E, int C, int DV, bool EPI, int CT, int PASS>
__global__ __launch_bounds__(64 * (DV / (16 * CT) + 1)) void carry_kernel(const CarryArgs p) {
  constexpr int NWC = DV / (16 * CT);  // compute waves; wave NWC is the loader
  using L = CarryLayout<E, C, NWC>;
  using F = FactorBlock<(int)sizeof(E), C>;
  constexpr int NT = C / 16;     // 16-token tiles per chunk
  constexpr int KT = C / 32;     // 32-deep token steps per chunk
  constexpr int ES = (int)sizeof(E);
  static_assert(NWC * 16 * CT == DV, "column tiles must cover the block");
  static_assert(!EPI || DV == D, "the epilogue normalises whole heads");
  static_assert(!EPI || PASS != 1, "the pairs pass writes no outputs");
  static_assert(KT >= 1 && NT <= 4, "unsupported tile shape");
  static_assert(L::BYTES <= 160 * 1024, "LDS budget exceeded");
  static_assert(L::PIECES <= 63, "copy exceeds the outstanding-load counter");

  extern __shared__ __align__(16) unsigned char smem[];
  float* sSS = reinterpret_cast<float*>(smem + L::SS);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // XCD-aware decode of the work item: blocks b and b + 8 run on the same XCD,
  // so the column blocks of one (sequence, head) share that XCD's L2.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int cb_all = slot % p.col_split;
  const int u = (slot / p.col_split) * 8 + xcd;
  if (u >= p.units) return;
  const int H = p.num_heads;
  const int rnk = u / H, h = u % H;
  // work item: sequence n, chunks [c0, c0 + nch) of it, factor slots from slot0
  constexpr bool SEQ = PASS == 0 || PASS == 3 || PASS == 4;  // one work item per (sequence, head)
  int n, c0, nch, slot0;
  if constexpr (SEQ) {
    n = p.order ? p.order[rnk] : rnk;
    c0 = p.seq_c0[n];
    nch = p.seq_c1[n] - c0;
    slot0 = p.seq_first[n];
  } else {
    if (rnk >= *p.seg_count) return;
    n = p.seg_list[2 * rnk];
    const int first = p.seq_c0[n] + p.seg_list[2 * rnk + 1] * p.seg_chunks;
    c0 = first;
    nch = max(0, min(p.seq_c1[n], first + p.seg_chunks) - first);
    slot0 = p.seq_first[n] + (first - p.seq_c0[n]);
  }
  // pass 1: the second half of the blocks traces M (identity start, U' = 0)
  const bool mpart = PASS == 1 && cb_all >= p.col_split / 2;
  const int cb = PASS == 1 ? cb_all % (p.col_split / 2) : cb_all;
  constexpr bool write_o = PASS == 0 || PASS == 2 || PASS == 4;
  constexpr bool keep_su = PASS == 3 || PASS == 4;  // per-chunk S and U for the backward pass
  const size_t pair_base = ((size_t)rnk * H + h) * 2 * (size_t)(D * D);
  const float* s_in = SEQ ? (p.state_in ? p.state_in + ((size_t)n * H + h) * (size_t)(D * D) : nullptr)
                    : PASS == 2 ? p.pairs + pair_base : nullptr;
  float* s_out = SEQ ? (p.state_out ? p.state_out + ((size_t)n * H + h) * (size_t)(D * D) : nullptr)
               : PASS == 1 ? p.pairs + pair_base + (mpart ? (size_t)(D * D) : 0) : nullptr;
  int64_t seq_bos, seq_eos;
  seq_range(p.cu, n, p.total_tokens, seq_bos, seq_eos);
  const int64_t rs = (int64_t)H * D;
  const int64_t hoff = (int64_t)h * D;
  const char* fbase = static_cast<const char*>(p.factors);
  auto block_of = [&](int ci) { return fbase + ((size_t)(slot0 + ci) * H + h) * F::BYTES; };

  if (wv == NWC) {
    // ---- loader wave (the passes that form no outputs skip Qt) ----
    constexpr uint32_t kSlotQ = L::Q, kSlotK = L::K, kBlockK = F::K;
    constexpr int NPC = !write_o ? L::PIECES - (int)((kSlotK - kSlotQ) / 1024) : L::PIECES;  // pieces per chunk
    auto copy_block = [&](int ci) {
      const char* blk = block_of(ci);
      unsigned char* dst = smem + (ci % L::NBUF) * L::SLOT;
#pragma unroll
      for (int j = 0; j < L::PIECES; ++j) {
        if (!write_o && j * 1024u >= kSlotQ && j * 1024u < kSlotK) continue;
        __builtin_amdgcn_global_load_lds(blk + (j * 1024u < kSlotK ? j * 1024u : kBlockK + (j * 1024u - kSlotK)) + lane * 16,
                                         (__attribute__((address_space(3))) void*)(dst + j * 1024), 16, 0, 0);
      }
    };
    if (nch > 0) copy_block(0);
    if (nch > 1) copy_block(1);
    for (int ci = 0; ci < nch; ++ci) {
      // chunk ci's copy has landed; the one of chunk ci + 1 may be in flight
      if (ci + 1 < nch) __builtin_amdgcn_s_waitcnt(vmcnt_wait(NPC));
      else __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
      __syncthreads();
      if (ci + 2 < nch) copy_block(ci + 2);
      if (EPI) __syncthreads();  // the compute waves' row-sum exchange
    }
    return;
  }

  // ---- compute waves ----
  const int col0 = cb * DV + 16 * CT * wv;  // first value column owned by this wave
  E* go = static_cast<E*>(p.o);
  // RMSNorm weights of the columns this lane stores (col0 + 16 c + 4 g + e)
  f32x4 nw[CT];
  {
    const int g = lane >> 4;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) nw[c][e] = (EPI && p.norm_w) ? p.norm_w[col0 + 16 * c + 4 * g + e] : 1.f;
  }

  // State slice: tile (c, rt8) holds rows 16 rt8 + 4g + i, column col0 + 16 c + l16
  // (zero, the identity's columns for M, or the given state).
  f32x4 accS[CT][8];
  {
    const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int rt8 = 0; rt8 < 8; ++rt8)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * rt8 + 4 * g + i, col = col0 + 16 * c + l16;
          accS[c][rt8][i] = s_in ? s_in[(size_t)row * D + col] : (mpart && row == col) ? 1.f : 0.f;
        }
  }

  // P fragments and this wave's U' tiles (accumulator order, I/O dtype) of
  // the next chunk, fetched into registers one chunk ahead (U' right after
  // the barrier, P once the current chunk's P has been used).
  using Raw = std::conditional_t<ES == 2, u32x2, f32x4>;  // four I/O-dtype values
  auto raw_f32 = [](Raw x) -> f32x4 {
    if constexpr (ES == 2) {
      const bf16x4 b = __builtin_bit_cast(bf16x4, x);
      return (f32x4){(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
    } else {
      return x;
    }
  };
  auto buf_ld_raw = [](Rsrc rb, uint32_t voff, uint32_t soff) -> Raw {
    if constexpr (ES == 2)
      return __builtin_amdgcn_raw_buffer_load_b64(rb, (int)voff, (int)soff, 0);
    else
      return __builtin_bit_cast(f32x4, buf_ld16(rb, voff, soff));
  };
  Frag<E> rP[F::NP];
  Raw rU[CT][NT];
  auto load_u = [&](int ci) {
    if (mpart) {
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int a = 0; a < NT; ++a) rU[c][a] = Raw{};
      return;
    }
    const Rsrc rb = make_rsrc(block_of(ci), F::BYTES);
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const uint32_t u_off = (uint32_t)((col0 / 16 + c) * F::UT + lane * 4 * ES);
#pragma unroll
      for (int a = 0; a < NT; ++a) rU[c][a] = buf_ld_raw(rb, u_off, F::U + a * 8 * F::UT);
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
  // Epilogue gate logits of the current chunk in the output layout
  // (lane = token, four consecutive columns), through a buffer view with
  // 32-bit offsets whose rows past the sequence end read zero.
  Raw rG[EPI ? CT : 1][EPI ? NT : 1];
  auto load_gate = [&](int64_t t0, int nv) {
    const Rsrc gr = make_rsrc(static_cast<const E*>(p.gate) + t0 * rs, (uint32_t)((int64_t)nv * rs * ES));
    const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
        rG[c][rt] = buf_ld_raw(gr, (uint32_t)(((16 * rt + l16) * rs + hoff + col0 + 16 * c + 4 * g) * ES), 0);
  };
  if (nch > 0) {
    load_u(0);
    if (write_o) load_p(0);
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
    const E* sKbt = reinterpret_cast<const E*>(buf + L::K + lane * 4 * ES);  // fragments split in halves
    const float* sGam = reinterpret_cast<const float*>(buf + L::G);
    constexpr int FRE = (int)F::FR / ES;  // elements per fragment

    f32x4 accU[CT][NT];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int a = 0; a < NT; ++a) accU[c][a] = raw_f32(rU[c][a]);
    // states pass: the state entering this chunk (rows are key channels), in
    // the I/O dtype as 16 x 16 tiles, for the backward pass.  Each tile is
    // transposed on the matrix cores (a product with the identity, exact) so
    // that a lane holds four consecutive columns of one row and a store
    // instruction writes the whole 512-byte tile.
    Frag16<E> id16;
    if constexpr (keep_su) {
      {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (4 * g + e == l16) ? 1.f : 0.f;
        frag16_from_acc(id16, x);
      }
      const size_t blk = (size_t)(slot0 + ci) * H + h;
      E* cs_dst = static_cast<E*>(p.chunk_states) + blk * (size_t)(D * D);
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int rt8 = 0; rt8 < 8; ++rt8) {
          Frag16<E> a;
          frag16_from_acc(a, accS[c][rt8]);
          store_row4(cs_dst + tile16_index(16 * rt8 + l16, col0 + 16 * c + 4 * g),
                     mma16((f32x4){0.f, 0.f, 0.f, 0.f}, a, id16));
        }
    }
    __syncthreads();
    if (EPI) load_gate(t0, nv);
    // In the passes that write outputs, the next chunk's loads (on the last
    // chunk a repeat of this one's) and the output stores below are issued on
    // every path: with a load or store behind a branch the compiler cannot
    // count what is in flight after the P loads, and their wait drains every
    // outstanding access, the U' loads just issued included (measured: 269 ->
    // 257 us for the one-layer carry).  The passes without outputs keep the
    // conditional load, which measured faster there (242 against 276 us for
    // the states pass).
    if constexpr (write_o) load_u(ci + 1 < nch ? ci + 1 : ci);
    else if (ci + 1 < nch) load_u(ci + 1);

    // Four-wave single-tile blocks: each stage first issues all of its LDS
    // fragment reads (the scheduling barrier keeps them ahead of the
    // matrix-core work, so they are in flight together instead of one at a
    // time), then runs its products with the independent accumulators
    // interleaved.  Two-tile waves lack the registers for that and stream one
    // fragment at a time, each feeding both of their tiles.
    constexpr bool BATCH = NWC == 4 && CT == 1;
    Frag<E> sf[CT][4];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) frag_from_acc(sf[c][ks], accS[c][2 * ks], accS[c][2 * ks + 1]);
    f32x4 accO[CT][NT];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) accO[c][rt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if constexpr (BATCH) {
      // ---- S1: U = U' - W S ----
      Frag<E> fa[4 * NT];
#pragma unroll
      for (int i = 0; i < 4 * NT; ++i) ld_frag(fa[i], sW + i * FRE);   // W is stored negated
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) accU[0][rt] = mma(accU[0][rt], fa[rt * 4 + ks], sf[0][ks]);
      // ---- S2: O = Qt S (+ P U below) ----
      if constexpr (write_o) {
#pragma unroll
        for (int i = 0; i < 4 * NT; ++i) ld_frag(fa[i], sQt + i * FRE);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int rt = 0; rt < NT; ++rt) accO[0][rt] = mma(accO[0][rt], fa[rt * 4 + ks], sf[0][ks]);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
          Frag<E> fa;
          ld_frag(fa, sW + (rt * 4 + ks) * FRE);
#pragma unroll
          for (int c = 0; c < CT; ++c) accU[c][rt] = mma(accU[c][rt], fa, sf[c][ks]);
        }
      if constexpr (write_o)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int rt = 0; rt < NT; ++rt) {
            Frag<E> fa;
            ld_frag(fa, sQt + (rt * 4 + ks) * FRE);
#pragma unroll
            for (int c = 0; c < CT; ++c) accO[c][rt] = mma(accO[c][rt], fa, sf[c][ks]);
          }
    }
    if constexpr (keep_su) {
      // U = U' - W S of this chunk, [C x 128] 16 x 16 tiles in the I/O dtype
      // (rows past the sequence end are zero), transposed as the state
      E* u_dst = static_cast<E*>(p.chunk_u) + ((size_t)(slot0 + ci) * H + h) * (size_t)(C * D);
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int a = 0; a < NT; ++a) {
          Frag16<E> fr;
          frag16_from_acc(fr, accU[c][a]);
          store_row4(u_dst + tile16_index(16 * a + l16, col0 + 16 * c + 4 * g),
                     mma16((f32x4){0.f, 0.f, 0.f, 0.f}, fr, id16));
        }
    }
    Frag<E> uf[CT][KT];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) frag_from_acc(uf[c][kt], accU[c][2 * kt], accU[c][2 * kt + 1]);
    if constexpr (write_o)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
          if (kt <= rt / 2)
#pragma unroll
            for (int c = 0; c < CT; ++c) accO[c][rt] = mma(accO[c][rt], rP[F::p_frag(rt, kt)], uf[c][kt]);
    if (write_o) load_p(ci + 1 < nch ? ci + 1 : ci);

    // outputs: each 16 x 16 tile transposed on the matrix cores to lane =
    // token, four consecutive columns, then (with the epilogue) the head-wise
    // RMSNorm over the 128 value columns and the sigmoid gate, and stored
    // straight to global memory
    if constexpr (write_o) {
      Frag16<E> id;
      {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (4 * g + e == l16) ? 1.f : 0.f;
        frag16_from_acc(id, x);
      }
      // rows past the sequence end fall outside the buffer view and are dropped
      const Rsrc orb = make_rsrc(go + t0 * rs, (uint32_t)((int64_t)nv * rs * ES));
      auto store = [&](const f32x4& t, int c, int rt) {
        const uint32_t off = (uint32_t)(((16 * rt + l16) * rs + hoff + col0 + 16 * c + 4 * g) * ES);
        if constexpr (ES == 2) {
          const bf16x4 b = (bf16x4){(__bf16)t[0], (__bf16)t[1], (__bf16)t[2], (__bf16)t[3]};
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, b), orb, (int)off, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, t), orb, (int)off, 0, 0);
        }
      };
      if constexpr (EPI) {
        f32x4 ot[CT][NT];
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
          float ss = 0.f;
#pragma unroll
          for (int c = 0; c < CT; ++c) {
            Frag16<E> a;
            frag16_from_acc(a, accO[c][rt]);
            ot[c][rt] = mma16((f32x4){0.f, 0.f, 0.f, 0.f}, a, id);
#pragma unroll
            for (int e = 0; e < 4; ++e) ss += ot[c][rt][e] * ot[c][rt][e];
          }
          ss += __shfl_xor(ss, 16);
          ss += __shfl_xor(ss, 32);
          if (g == 0) sSS[wv * C + 16 * rt + l16] = ss;
        }
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
          const int tok = 16 * rt + l16;
          float ms = 0.f;
#pragma unroll
          for (int q = 0; q < NWC; ++q) ms += sSS[q * C + tok];
          const float inv = rsqrtf(ms * (1.f / D) + p.rms_eps);
#pragma unroll
          for (int c = 0; c < CT; ++c) {
            const f32x4 gl = raw_f32(rG[c][rt]);
            f32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = ot[c][rt][e] * (inv * nw[c][e] * sigmoidf_fast(gl[e]));
            store(y, c, rt);
          }
        }
      } else {
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
#pragma unroll
          for (int c = 0; c < CT; ++c) {
            Frag16<E> a;
            frag16_from_acc(a, accO[c][rt]);
            store(mma16((f32x4){0.f, 0.f, 0.f, 0.f}, a, id), c, rt);
          }
      }
    }

    // ---- S3: S <- Diag(e^{g_n}) S + Kb^T U ----
    if constexpr (BATCH) {
      Frag<E> fa[8 * KT];
#pragma unroll
      for (int i = 0; i < 8 * KT; ++i) ld_frag_pair(fa[i], sKbt + i * FRE, sKbt + i * FRE + FRE / 2);
      f32x4 gam[8];
#pragma unroll
      for (int rt8 = 0; rt8 < 8; ++rt8) gam[rt8] = *reinterpret_cast<const f32x4*>(sGam + 16 * rt8 + 4 * g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rt8 = 0; rt8 < 8; ++rt8) accS[0][rt8] *= gam[rt8];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int rt8 = 0; rt8 < 8; ++rt8) accS[0][rt8] = mma(accS[0][rt8], fa[rt8 * KT + kt], uf[0][kt]);
    } else {
#pragma unroll
      for (int rt8 = 0; rt8 < 8; ++rt8) {
        const f32x4 gam = *reinterpret_cast<const f32x4*>(sGam + 16 * rt8 + 4 * g);
#pragma unroll
        for (int c = 0; c < CT; ++c) accS[c][rt8] *= gam;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          Frag<E> fa;
          ld_frag_pair(fa, sKbt + (rt8 * KT + kt) * FRE, sKbt + (rt8 * KT + kt) * FRE + FRE / 2);
#pragma unroll
          for (int c = 0; c < CT; ++c) accS[c][rt8] = mma(accS[c][rt8], fa, uf[c][kt]);
        }
      }
    }
  }

  if (s_out) {
    const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int rt8 = 0; rt8 < 8; ++rt8)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_out[(size_t)(16 * rt8 + 4 * g + i) * D + col0 + 16 * c + l16] = accS[c][rt8][i];
  }
}

template <typename E, int C, int DV, bool EPI, int CT, int PASS>
static hipError_t launch_carry_t(const CarryArgs& a, hipStream_t stream) {
  constexpr int NWC = DV / (16 * CT);
  constexpr size_t lds = CarryLayout<E, C, NWC>::BYTES;
  static_assert(lds <= 160 * 1024, "LDS budget exceeded");
  auto fn = carry_kernel<E, C, DV, EPI, CT, PASS>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int groups = (a.units + 7) / 8;
  const unsigned grid = (unsigned)(8 * a.col_split * groups);
  if (a.units <= 0) return hipSuccess;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * (NWC + 1)), lds, stream, a);
  return hipGetLastError();
}

template <typename E, int C>
static hipError_t launch_carry_dtype(const CarryArgs& a, hipStream_t stream) {
  // whole heads on four two-tile waves (the epilogue normalises over all 128
  // value columns; the pass that traces B and M runs one block of each),
  // else 64-column blocks on four one-tile waves (two per work item), the
  // blocks sharing the factor reads through L2
  if (a.gate) {
    if (a.col_split != 1) return hipErrorInvalidValue;
    if (a.pass == 0) return launch_carry_t<E, C, 128, true, 2, 0>(a, stream);
    if (a.pass == 2) return launch_carry_t<E, C, 128, true, 2, 2>(a, stream);
    return hipErrorInvalidValue;
  }
  if (a.pass == 0 && a.col_split == 2) return launch_carry_t<E, C, 64, false, 1, 0>(a, stream);
  if (a.pass == 3 && a.col_split == 2 && a.chunk_states && a.chunk_u)
    return launch_carry_t<E, C, 64, false, 1, 3>(a, stream);
  if (a.pass == 4 && a.col_split == 2 && a.chunk_states && a.chunk_u)
    return launch_carry_t<E, C, 64, false, 1, 4>(a, stream);
  if (a.pass == 1 && a.col_split == 2) return launch_carry_t<E, C, 128, false, 2, 1>(a, stream);
  if (a.pass == 2 && a.col_split == 2) return launch_carry_t<E, C, 64, false, 1, 2>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_carry(const CarryArgs& a, hipStream_t stream) {
  if (a.bf16) return launch_carry_dtype<__bf16, 64>(a, stream);
  return launch_carry_dtype<float, 32>(a, stream);
}

}  // namespace kda
