// kda_prep.hip — token-parallel stage of the two-kernel chunked prefill (gfx950).
//
// Method ("Kimi K3 架构、训练与系统全景解析", section 4.2.4: the chunkwise form
// with the UT transform; section 4.2.5: the decay lower bound that keeps every
// exponent of a 16-token tile in [-80, 0]).  For a chunk of C tokens with
// per-channel cumulative log-decay g (within the chunk):
//   Kt = K (.) e^{g},  Qt = Q (.) e^{g},  Kh = K (.) e^{-g},  Kb = K (.) e^{g_n - g}
//   A  = strictly-lower( Diag(beta) Kt Kh^T ),   (I + A) [W | U'] = Diag(beta) [Kt | V]
//   P  = lower-incl( Qt Kh^T )
// None of it depends on the state, so every (chunk, head) is done at once here
// and written to the factor store; the carry kernel applies the state.
//
// Work split.  A workgroup of NT waves (NT = C / 16: four for bf16 I/O with
// 64-token chunks, two for fp32 with 32-token chunks) handles a run of chunks
// of one head.  Wave w owns token tile w.  Lane (r = l % 16, g = l / 16)
// holds token 16 w + r and the 32 channels
//     ch(s, e) = 32 s + 4 g + (e & 3) + 16 (e >> 2),    s = 0..3, e = 0..7,
// which is the operand fragment of a 32-deep matrix-core step over the
// channels (kda_device.h, d-permuted set).  So:
//   - the Gram products A_ab, P_ab (row tile a, column tile b <= a) take the
//     row tile's operands from registers; column tiles b < a come through LDS
//     once, pre-scaled by the producing wave;
//   - Qt leaves in exactly the carry kernel's fragment order;
//   - transposes (token-per-lane <-> channel-per-lane) run on the matrix cores
//     as products with 0/1 selection matrices, which are exact.
// Exponents: a tile's rows are referenced to the decay before the tile (rho_a)
// or after it (rho_{a+1}), so every factor formed is <= 1 except the diagonal
// tile's e^{rho_a - g} <= e^{80}, which is exactly the pages' bound.
// Unbounded decay (the negative-softplus gate the same section describes for
// Kimi Linear, where that factor can overflow): the UNB variant forms the
// diagonal tile's entries position by position instead,
//   A_ij = sum_c k_ic k_jc e^{g_ic - g_jc},  P_ij = sum_c q_ic k_jc e^{g_ic - g_jc},
// with e^{g_i - g_j} = alpha_i alpha_{i-1} ... alpha_{j+1} built up one DPP row
// shift at a time (every partial product is <= 1), and K_end from an in-tile
// suffix sum; every other factor is a sum of same-sign log-decays, so no
// exponent exceeds 0 and no difference of large sums is taken.
//
// Per chunk: loads and the in-tile decay scan (DPP row shifts); barrier;
// per-channel factors (e^{tot_a}, e^{rho_a}, e^{g_n - rho_{a+1}}, e^{g_n});
// barrier; operand fragments, Qt and Kb^T stores, scaled column-tile copies
// and the solve's right-hand sides to LDS; barrier; Gram products and the
// fp32 inverse of the diagonal block; P stores and the solve's blocks to LDS;
// barrier; blocked forward substitution on the matrix cores, -W and U' stores.
#include <type_traits>

#include "kda_chunk_util.h"

namespace kda {

namespace {

// 4 consecutive elements of one row: 8 bytes (bf16) or 16 bytes (fp32).
template <typename E>
struct Raw4;
template <>
struct Raw4<__bf16> {
  bf16x4 v;
};
template <>
struct Raw4<float> {
  f32x4 v;
};
__device__ __forceinline__ void ld_raw4(Raw4<float>& x, const float* p) { x.v = *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void cvt_raw4(float* y, const Raw4<__bf16>& x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = (float)x.v[i];
}
__device__ __forceinline__ void cvt_raw4(float* y, const Raw4<float>& x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = x.v[i];
}

// Inclusive prefix sum over the 16 lanes of a row (DPP row shifts, zero fill).
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xf, 0xf, true));
}
__device__ __forceinline__ float row_scan(float x) {
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  x += row_shr<8>(x);
  return x;
}
// Exclusive suffix sum over the 16 lanes of a row: lane r gets the sum over
// lanes r + 1 .. 15 (DPP row shifts left, zero fill).  Every term has the
// sign of the inputs, so nothing cancels.
template <int N>
__device__ __forceinline__ float row_shl(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x100 + N, 0xf, 0xf, true));
}
__device__ __forceinline__ float row_suffix_excl(float x) {
  x = row_shl<1>(x);
  x += row_shl<1>(x);
  x += row_shl<2>(x);
  x += row_shl<4>(x);
  x += row_shl<8>(x);
  return x;
}
// The same two sums within one 8-lane half of a row, for inputs that are zero
// in the other half: the prefix over lanes 8 .. r (for r >= 8) and the
// exclusive suffix over lanes r + 1 .. 7 (for r < 8).  Eight lanes need one
// doubling step less; the lanes the shorter span reaches beyond the half hold
// zeros.
__device__ __forceinline__ float row_scan_upper(float x) {
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  return x;
}
__device__ __forceinline__ float row_suffix_excl_lower(float x) {
  x = row_shl<1>(x);
  x += row_shl<1>(x);
  x += row_shl<2>(x);
  x += row_shl<4>(x);
  return x;
}

// Piece pc = 2 s + h of a lane's channels: channels 32 s + 16 h + 4 g + {0..3}.
__device__ __forceinline__ int piece_ch(int pc, int g) { return 32 * (pc >> 1) + 16 * (pc & 1) + 4 * g; }

// bf16 rows are read 16 bytes per lane: for 32-channel step st, lane group g
// loads channels wide_ch(st, g) .. + 7, so that the four groups of a token
// read its 64 contiguous bytes.  Group g then holds (in dwords 0-1 | 2-3)
//   g = 0: pieces (2 st, g 0) | (2 st, g 1)    g = 1: (2 st + 1, g 0) | (2 st + 1, g 1)
//   g = 2: pieces (2 st, g 2) | (2 st, g 3)    g = 3: (2 st + 1, g 2) | (2 st + 1, g 3)
// and one row swap (v_permlane16_swap: the odd rows of the first operand
// trade places with the even rows of the second, lane j with lane 16 + j)
// per dword leaves every group with its own pieces 2 st | 2 st + 1.
__device__ __forceinline__ int wide_ch(int st, int g) { return 32 * st + 16 * (g & 1) + 8 * (g >> 1); }
__device__ __forceinline__ u32x4 ld_wide(const __bf16* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void unpack_wide(Raw4<__bf16>& lo, Raw4<__bf16>& hi, u32x4 w) {
  const auto a = __builtin_amdgcn_permlane16_swap(w[0], w[2], false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(w[1], w[3], false, false);
  lo.v = __builtin_bit_cast(bf16x4, (u32x2){a[0], b[0]});
  hi.v = __builtin_bit_cast(bf16x4, (u32x2){a[1], b[1]});
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// 32-bit DPP moves within 16-lane rows: shift right by N (zero fill), rotate
// right by N, broadcast of lane N.  A rotate or broadcast reads a valid lane
// everywhere, so it needs no fallback value (no zeroed register to start from).
template <int N>
__device__ __forceinline__ uint32_t dpp_shr(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x110 + N, 0xf, 0xf, true);
}
template <int N>
__device__ __forceinline__ uint32_t dpp_ror(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x120 + N, 0xf, 0xf, true);
}
// Shift right by N; lanes with no source (the first N of a row) keep `old`.
template <int N>
__device__ __forceinline__ uint32_t dpp_shr_or(uint32_t old, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, 0x110 + N, 0xf, 0xf, false);
}
template <int N>
__device__ __forceinline__ float dpp_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N, 0xf, 0xf, true));
}

// Rows tok - 1 .. tok - 3 of a piece, for the lane at row position r: from
// lane r - s of the own rows when r >= s, else from lane r - s + 16 of the
// halo rows (row tok - 16 there).  x[s][0..3] receives row tok - s.  Both
// moves run in every lane (a DPP read from a lane switched off by a branch
// would return zero): the rotated halo is the shift's fallback value.
template <typename R>
__device__ __forceinline__ void shifted_rows(float (&x)[4][4], const R& own, const R& halo) {
  constexpr int NW = (int)sizeof(own.v) / 4;
  const auto ow = __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(NW))), own.v);
  const auto hw = __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(NW))), halo.v);
  static_for<1, 4>([&](auto sc) {
    constexpr int s = decltype(sc)::value;
    uint32_t __attribute__((ext_vector_type(NW))) y;
#pragma unroll
    for (int j = 0; j < NW; ++j) y[j] = dpp_shr_or<s>(dpp_ror<s>(hw[j]), ow[j]);
    R t;
    t.v = __builtin_bit_cast(decltype(own.v), y);
    cvt_raw4(x[s], t);
  });
}

// The four taps of channel piece_ch(pc, g) + i from lane 2 pc + i / 2 of the
// lane's row, which holds them at (i % 2) * 4 + m.
__device__ __forceinline__ void tap_bcast(float (&wt)[4], const float (&wl)[8], int pc, int i) {
  static_for<0, 16>([&](auto nc) {
    constexpr int n = decltype(nc)::value;
    if (n == 2 * pc + (i >> 1)) {
#pragma unroll
      for (int m = 0; m < 4; ++m) wt[m] = dpp_bcast<n>(wl[(i & 1) * 4 + m]);
    }
  });
}

// Fragment of step s from the lane's per-piece values x[8][4] (fp32 operands).
__device__ __forceinline__ void frag_step(Frag<float>& f, const float (&x)[8][4], int s) {
  f.lo = (f32x4){x[2 * s][0], x[2 * s][1], x[2 * s][2], x[2 * s][3]};
  f.hi = (f32x4){x[2 * s + 1][0], x[2 * s + 1][1], x[2 * s + 1][2], x[2 * s + 1][3]};
}
// hi + lo split of the same step (bf16); fp32 operands are exact, lo unused.
__device__ __forceinline__ void frag_step_split(Frag<__bf16>& hi, Frag<__bf16>& lo, const float (&x)[8][4], int s) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = x[2 * s + (e >> 2)][e & 3];
    const __bf16 b = (__bf16)v;
    hi.v[e] = b;
    lo.v[e] = (__bf16)(v - (float)b);
  }
}
__device__ __forceinline__ void frag_step_split(Frag<float>& hi, Frag<float>&, const float (&x)[8][4], int s) {
  frag_step(hi, x, s);
}

// B operand that picks channel 32 s + 16 h + (l % 16) out of an x32 step:
// lane (j, g) has a one at element 4 h + (j - 4 g) when 0 <= j - 4 g < 4.
template <typename E>
__device__ __forceinline__ Frag<E> select_frag(int h, int lane) {
  float x[8];
  const int j = lane & 15, g = lane >> 4;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = ((e >> 2) == h && 4 * g + (e & 3) == j) ? 1.f : 0.f;
  Frag<E> f;
  frag_from_f32(f, x);
  return f;
}
// 16 x 16 identity as the B operand of an x16 step.
template <typename E>
__device__ __forceinline__ Frag16<E> ident16(int lane) {
  const int j = lane & 15, g = lane >> 4;
  f32x4 x;
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = (4 * g + e == j) ? 1.f : 0.f;
  Frag16<E> f;
  frag16_from_acc(f, x);
  return f;
}

// Stores into the factor block (buffer view: out-of-range offsets are dropped).
__device__ __forceinline__ void st_frag_g(Rsrc rb, uint32_t off, const Frag<__bf16>& f) {
  buf_st16(__builtin_bit_cast(u32x4, f.v), rb, off, 0);
}
__device__ __forceinline__ void st_frag_g(Rsrc rb, uint32_t off, const Frag<float>& f) {
  buf_st16(__builtin_bit_cast(u32x4, f.lo), rb, off, 0);
  buf_st16(__builtin_bit_cast(u32x4, f.hi), rb, off + 16, 0);
}
// Four values as one half of a lane's fragment entry.
__device__ __forceinline__ void st_half_g(Rsrc rb, uint32_t off, f32x4 x, __bf16*) {
  const bf16x4 b = (bf16x4){(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
  buf_st8(__builtin_bit_cast(u32x2, b), rb, off, 0);
}
__device__ __forceinline__ void st_half_g(Rsrc rb, uint32_t off, f32x4 x, float*) {
  buf_st16(__builtin_bit_cast(u32x4, x), rb, off, 0);
}
// Both halves of a lane's fragment entry (first half lo, second half hi).
__device__ __forceinline__ void st_pair_g(Rsrc rb, uint32_t off, f32x4 lo, f32x4 hi, __bf16*) {
  const bf16x8 b = {(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                    (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
  buf_st16(__builtin_bit_cast(u32x4, b), rb, off, 0);
}
__device__ __forceinline__ void st_pair_g(Rsrc rb, uint32_t off, f32x4 lo, f32x4 hi, float*) {
  buf_st16(__builtin_bit_cast(u32x4, lo), rb, off, 0);
  buf_st16(__builtin_bit_cast(u32x4, hi), rb, off + 16, 0);
}

template <typename E, int C>
struct PrepLayout {
  static constexpr int NT = C / 16;
  static constexpr int NPAIR = NT * (NT - 1) / 2;
  static constexpr int ES = (int)sizeof(E);
  static constexpr int LDM = C + 16 / ES;                      // sM row stride (elements)
  static constexpr size_t TOT = 0;                             // f32 [NT][128] tile decay totals (log2)
  static constexpr size_t FE = TOT + (size_t)NT * 128 * 4;     // f32 [NT][128] e^{tot_a}
  static constexpr size_t FA = FE + (size_t)NT * 128 * 4;      // f32 [NT][128] e^{rho_a}
  static constexpr size_t FB = FA + (size_t)NT * 128 * 4;      // f32 [NT][128] e^{g_n - rho_{a+1}}
  static constexpr size_t BETA = FB + (size_t)NT * 128 * 4;    // f32 [C]
  static constexpr size_t KE = BETA + (size_t)C * 4;           // [NPAIR][4][64] fragments
  static constexpr size_t R = KE + (size_t)NPAIR * 4 * 64 * 8 * ES;  // [16][NT][64][4] right-hand sides
  static constexpr size_t AD = R + (size_t)16 * NT * 64 * 4 * ES;    // f32 [NT][16][16] diagonal blocks
  static constexpr size_t M = AD + (size_t)NT * 256 * 4;             // E [C][LDM] solve blocks
  static constexpr int MAXR = 16;                                    // chunks per workgroup, at most
  static constexpr size_t RNG = (M + (size_t)C * LDM * ES + 7) & ~(size_t)7;  // i64 [MAXR][3] t0, bos, nv
  static constexpr size_t BYTES = RNG + (size_t)MAXR * 3 * 8;
};

}  // namespace

// ---------------------------------------------------------------------------
// Workgroup (range, head h) handles the consecutive slots
// [range * chunks_per_block, ...) of head h.
// ---------------------------------------------------------------------------
template <typename E, int C, bool PRO, bool UNB>
__global__ __launch_bounds__(4 * C, 2) void prep_kernel(const PrepArgs p) {
  using L = PrepLayout<E, C>;
  using F = FactorBlock<(int)sizeof(E), C>;
  constexpr int NT = C / 16;          // token tiles = waves
  constexpr int NTH = 64 * NT;
  constexpr int CPW = 8 / NT;         // W (and U') column tiles per wave in the solve
  static_assert(CPW % 2 == 0, "a wave stores whole -W fragments");
  constexpr int NOWN = 2 * CPW;
  constexpr bool SPLIT = sizeof(E) == 2;
  constexpr int ES = (int)sizeof(E);
  constexpr float LOG2E = 1.4426950408889634f;
  static_assert(NT == 2 || NT == 4, "chunk of 32 or 64 tokens");
  static_assert(L::BYTES <= 80 * 1024, "two workgroups per compute unit");

  extern __shared__ __align__(16) unsigned char smem[];
  float* sTot = reinterpret_cast<float*>(smem + L::TOT);
  float* sFE = reinterpret_cast<float*>(smem + L::FE);
  float* sFA = reinterpret_cast<float*>(smem + L::FA);
  float* sFB = reinterpret_cast<float*>(smem + L::FB);
  float* sBeta = reinterpret_cast<float*>(smem + L::BETA);
  unsigned char* sKE = smem + L::KE;
  unsigned char* sR = smem + L::R;
  float* sAd = reinterpret_cast<float*>(smem + L::AD);
  E* sM = reinterpret_cast<E*>(smem + L::M);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, g = lane >> 4;
  const int H = p.num_heads, N = p.num_seqs;
  const int h = blockIdx.x % H;
  const int count = p.seq_first[N];
  // Ranges are handed out last-chunk-first: the carry kernel starts with the
  // first chunks, which the prep then has written most recently.
  const int nranges = (p.cap + p.chunks_per_block - 1) / p.chunks_per_block;
  const int s_begin = (nranges - 1 - (int)(blockIdx.x / H)) * p.chunks_per_block;
  if (s_begin >= count) return;
  const int s_end = min(count, s_begin + p.chunks_per_block);
  const int64_t rs = (int64_t)H * D;  // elements between consecutive tokens
  const int64_t hoff = (int64_t)h * D;
  const E* gq = static_cast<const E*>(p.q);
  const E* gk = static_cast<const E*>(p.k);
  const E* gv = static_cast<const E*>(p.v);
  const int tok = 16 * w + r;  // this lane's token within the chunk

  // Token range of every slot of this workgroup, found once up front and
  // kept in LDS: global loads in the chunk loop would make its waits drain
  // the factor stores in flight (loads and stores share one counter).
  int64_t* sRng = reinterpret_cast<int64_t*>(smem + L::RNG);
  if (tid < s_end - s_begin) {
    const int s = s_begin + tid;
    // sequence of slot s: the largest n with seq_first[n] <= s (seq_first[N] > s)
    int n = 0, hi = N;
    while (hi - n > 1) {
      const int mid = (n + hi) >> 1;
      if (p.seq_first[mid] <= s) n = mid;
      else hi = mid;
    }
    int64_t bos, eos;
    seq_range(p.cu, n, p.total_tokens, bos, eos);
    const int64_t t0 = bos + (int64_t)(p.seq_c0[n] + (s - p.seq_first[n])) * C;
    sRng[3 * tid] = t0;
    sRng[3 * tid + 1] = bos;
    sRng[3 * tid + 2] = min((int64_t)C, eos - t0);
  }
  __syncthreads();

  // Inputs of one chunk for this lane's token: q and k (after the prologue
  // when it runs; in the input dtype otherwise), v, log_alpha, beta.  For
  // bf16 inputs the next chunk's loads are issued as soon as the current
  // chunk's operands are formed, so they overlap its Gram products and solve:
  // all of them for plain inputs, log_alpha and beta with the prologue (its
  // raw rows would not fit the registers); fp32 inputs are loaded in place.
  constexpr bool PREFETCH = !PRO && sizeof(E) == 2;
  constexpr bool PREFETCH_LA = sizeof(E) == 2;
  using QK = std::conditional_t<PRO, Raw4<float>, Raw4<E>>;
  QK rq[8], rk[8];
  Raw4<E> rv[8];
  Raw4<float> rla[8];
  float rbt = 0.f;
  auto slot_range = [&](int s, int64_t& t0, int64_t& bos, int& nv) {
    const int j = s - s_begin;
    t0 = sRng[3 * j];
    bos = sRng[3 * j + 1];
    nv = (int)sRng[3 * j + 2];
  };
  constexpr bool WIDE = sizeof(E) == 2;  // bf16 rows: 16-byte loads, then a row swap
  u32x4 wq[WIDE ? 4 : 1], wk[WIDE ? 4 : 1], wv[WIDE ? 4 : 1];
  auto issue_la = [&](int64_t t0, int nv) {
    const int64_t row = t0 + min(tok, nv - 1);
    const int64_t base = row * rs + hoff;
#pragma unroll
    for (int pc = 0; pc < 8; ++pc) ld_raw4(rla[pc], p.log_alpha + base + piece_ch(pc, g));
    rbt = p.beta[row * H + h];
  };
  auto issue_rows = [&](int64_t t0, int nv) {
    const int64_t row = t0 + min(tok, nv - 1);
    const int64_t base = row * rs + hoff;
    if constexpr (WIDE) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        wv[st] = ld_wide(gv + base + wide_ch(st, g));
        if constexpr (!PRO) {
          wq[st] = ld_wide(gq + base + wide_ch(st, g));
          wk[st] = ld_wide(gk + base + wide_ch(st, g));
        }
      }
    } else {
#pragma unroll
      for (int pc = 0; pc < 8; ++pc) {
        ld_raw4(rv[pc], gv + base + piece_ch(pc, g));
        if constexpr (!PRO) {
          ld_raw4(rq[pc], gq + base + piece_ch(pc, g));
          ld_raw4(rk[pc], gk + base + piece_ch(pc, g));
        }
      }
    }
  };

  int64_t t0 = 0, seq_bos = 0;
  int nv = 0;
  slot_range(s_begin, t0, seq_bos, nv);
  if (PREFETCH_LA) issue_la(t0, nv);
  if (PREFETCH) issue_rows(t0, nv);
  // Prologue taps: lane (r, g) keeps those of channels piece_ch(r / 2, g)
  // + 2 (r % 2) + {0, 1} (four each), the lanes of a 16-lane row together
  // holding the taps of every channel that row uses.
  float wlq[8], wlk[8];
  if constexpr (PRO) {
    auto load_taps = [&](float (&wl)[8], const float* wc) {
      const int64_t ch = hoff + piece_ch(r >> 1, g) + 2 * (r & 1);
#pragma unroll
      for (int j = 0; j < 8; ++j) wl[j] = wc ? wc[ch * 4 + j] : 0.f;
    };
    load_taps(wlq, p.conv_q_w);
    load_taps(wlk, p.conv_k_w);
  }

  for (int s = s_begin; s < s_end; ++s) {
    // Lane indices re-derived from an opaque copy of the thread id in every
    // chunk: the address arithmetic of the unrolled stages then stays inside
    // the loop instead of occupying registers for the whole run.
    int tidv = tid;
    asm volatile("" : "+v"(tidv));
    const int lane = tidv & 63, w = tidv >> 6, r = lane & 15, g = lane >> 4;
    const int tok = 16 * w + r;
    const uint32_t lane_fr = (uint32_t)lane * 8 * ES;  // lane's entry in a fragment
    const bool valid = tok < nv;
    if (!PREFETCH_LA) issue_la(t0, nv);
    if (!PREFETCH) issue_rows(t0, nv);
    const Rsrc fb = make_rsrc(static_cast<char*>(p.factors) + ((size_t)s * H + h) * F::BYTES, F::BYTES);

    float dl[8][4];
    {
      if constexpr (PRO) {
        // causal depthwise conv over rows tok-3 .. tok (zero before the
        // sequence start), SiLU, then L2 over the head's 128 channels.  Each
        // lane loads its own row; rows tok-1 .. tok-3 come from the lanes
        // below it in the same 16-lane row (DPP row shifts), and for the
        // first three tokens of a tile from the halo row tok-16 that lanes
        // 13..15 load (DPP row rotates).  The taps come from the lanes that
        // hold them (row broadcasts).
        const int lo = (int)(seq_bos - t0);  // first row of the sequence, <= 0
        const int64_t own_row = t0 + min(tok, nv - 1);
        const bool has_halo = r >= 13 && tok - 16 >= lo;
        const int64_t halo_row = t0 + min(tok - 16, nv - 1);
        Raw4<E> oq[8], hq[8], ok[8], hk[8];
        if constexpr (WIDE) {
          u32x4 woq[4], whq[4], wok[4], whk[4];
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            woq[st] = ld_wide(gq + own_row * rs + hoff + wide_ch(st, g));
            wok[st] = ld_wide(gk + own_row * rs + hoff + wide_ch(st, g));
            whq[st] = (u32x4){0u, 0u, 0u, 0u};
            whk[st] = (u32x4){0u, 0u, 0u, 0u};
          }
          if (has_halo)
#pragma unroll
            for (int st = 0; st < 4; ++st) {
              whq[st] = ld_wide(gq + halo_row * rs + hoff + wide_ch(st, g));
              whk[st] = ld_wide(gk + halo_row * rs + hoff + wide_ch(st, g));
            }
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            unpack_wide(oq[2 * st], oq[2 * st + 1], woq[st]);
            unpack_wide(hq[2 * st], hq[2 * st + 1], whq[st]);
            unpack_wide(ok[2 * st], ok[2 * st + 1], wok[st]);
            unpack_wide(hk[2 * st], hk[2 * st + 1], whk[st]);
          }
        } else {
          auto load_rows = [&](Raw4<E> (&own)[8], Raw4<E> (&halo)[8], const E* src) {
#pragma unroll
            for (int pc = 0; pc < 8; ++pc) {
              ld_raw4(own[pc], src + own_row * rs + hoff + piece_ch(pc, g));
              halo[pc].v = 0;
            }
            if (has_halo)
#pragma unroll
              for (int pc = 0; pc < 8; ++pc) ld_raw4(halo[pc], src + halo_row * rs + hoff + piece_ch(pc, g));
          };
          load_rows(oq, hq, gq);
          load_rows(ok, hk, gk);
        }
        auto prologue = [&](QK (&y)[8], const Raw4<E> (&own)[8], const Raw4<E> (&halo)[8], const float (&wl)[8],
                            auto conv_c) {
          constexpr bool conv = decltype(conv_c)::value;
          float ss = 0.f;
#pragma unroll
          for (int pc = 0; pc < 8; ++pc) {
            float x[4][4];  // x[s] = row tok - s
            cvt_raw4(x[0], own[pc]);
            shifted_rows(x, own[pc], halo[pc]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float c = x[0][i];
              if constexpr (conv) {
                float wt[4];
                tap_bcast(wt, wl, pc, i);
                c = wt[0] * x[3][i] + wt[1] * x[2][i] + wt[2] * x[1][i] + wt[3] * x[0][i];
                c = c * sigmoidf_fast(c);
                ss += c * c;
              }
              y[pc].v[i] = c;
            }
          }
          if constexpr (conv) {
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
            const float inv = rsqrtf(ss + p.l2_eps);
#pragma unroll
            for (int pc = 0; pc < 8; ++pc) y[pc].v *= inv;
          }
        };
        // the convolution switch is taken once per tensor: inside the unrolled
        // element loop each element ended its own basic block, and the
        // exponentials and reciprocals of neighbouring elements could not overlap
        if (p.conv_q_w) prologue(rq, oq, hq, wlq, std::true_type{});
        else prologue(rq, oq, hq, wlq, std::false_type{});
        if (p.conv_k_w) prologue(rk, ok, hk, wlk, std::true_type{});
        else prologue(rk, ok, hk, wlk, std::false_type{});
      }
#pragma unroll
      for (int pc = 0; pc < 8; ++pc) cvt_raw4(dl[pc], rla[pc]);
    }
    const float bt = valid ? rbt : 0.f;
    if (!valid) {
      // (a 16-byte row piece is swapped only between lanes of the same token)
#pragma unroll
      for (int pc = 0; pc < 8; ++pc) {
        rq[pc].v = 0;
        rk[pc].v = 0;
        rv[pc].v = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) dl[pc][i] = 0.f;
      }
      if constexpr (WIDE)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          wq[st] = (u32x4){0u, 0u, 0u, 0u};
          wk[st] = (u32x4){0u, 0u, 0u, 0u};
          wv[st] = (u32x4){0u, 0u, 0u, 0u};
        }
    }

    // ---- unbounded decay: the diagonal tile position by position (lane r =
    //      token i of tile w; lane group g = a quarter of the channels) ----
    f32x4 gp_diag = (f32x4){0.f, 0.f, 0.f, 0.f};  // P_ww in the accumulator layout
    if constexpr (UNB) {
      // Pairs in the same 8-token half: running alpha products over DPP row
      // shifts (distances 1..7).  Pairs across the halves (rows 8..15,
      // columns 0..7): one 8 x 8 block on the matrix cores with both sides
      // referenced to the decay through token 7, e^{g_i - g_7} (a prefix sum
      // from token 8) and e^{g_7 - g_j} (a suffix sum up to token 7), both <= 1.
      float ga_d[8], gp_d[8];  // [delta]: A(i, i - delta), P(i, i - delta) over the lane's channels
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        ga_d[d] = 0.f;
        gp_d[d] = 0.f;
      }
      f32x4 ga_m = (f32x4){0.f, 0.f, 0.f, 0.f}, gp_m = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        float q8[8], k8[8];
        auto unpack = [&](float (&x)[8], const auto (&rp)[8], const u32x4 (&wp)[WIDE ? 4 : 1], bool wide) {
          if constexpr (WIDE) {
            if (wide) {
              Raw4<E> a, b;
              unpack_wide(a, b, wp[st]);
              cvt_raw4(x, a);
              cvt_raw4(x + 4, b);
              return;
            }
          }
          cvt_raw4(x, rp[2 * st]);
          cvt_raw4(x + 4, rp[2 * st + 1]);
        };
        unpack(q8, rq, wq, !PRO);
        unpack(k8, rk, wk, !PRO);
        float xr[8], xs_q[8][4], xs_c[8][4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float l2 = dl[2 * st + (e >> 2)][e & 3] * LOG2E;
          const float pre = row_scan_upper(r >= 8 ? l2 : 0.f);         // g_i - g_7, rows 8..15
          const float suf = row_suffix_excl_lower(r < 8 ? l2 : 0.f);  // g_7 - g_j, columns 0..7
          const float f = exp2_fast(r >= 8 ? pre : suf);               // a lane needs one of the two
          const float fr = r >= 8 ? f : 0.f;
          const float fc = r < 8 ? f : 0.f;
          xr[e] = k8[e] * fr;
          xs_q[2 * st + (e >> 2)][e & 3] = q8[e] * fr;
          xs_c[2 * st + (e >> 2)][e & 3] = k8[e] * fc;
          const float al = exp2_fast(l2);  // alpha_i
          gp_d[0] += q8[e] * k8[e];
          // u = k_{i-d} e^{g_i - g_{i-d}}, one distance further per step: the
          // lane below's value times alpha_i (zero where i - d < 0)
          float u = k8[e];
          static_for<1, 8>([&](auto D) {
            constexpr int d = decltype(D)::value;
            u = al * row_shr<1>(u);
            ga_d[d] += k8[e] * u;
            gp_d[d] += q8[e] * u;
          });
        }
        Frag<E> mk, mqh, mql, mch, mcl;
        frag_from_f32(mk, xr);
        frag_step_split(mqh, mql, xs_q, st);
        frag_step_split(mch, mcl, xs_c, st);
        ga_m = mma(ga_m, mk, mch);
        gp_m = mma(gp_m, mqh, mch);
        if constexpr (SPLIT) {
          gp_m = mma(gp_m, mql, mch);
          gp_m = mma(gp_m, mqh, mcl);
        }
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        ga_d[d] += __shfl_xor(ga_d[d], 16);
        ga_d[d] += __shfl_xor(ga_d[d], 32);
        gp_d[d] += __shfl_xor(gp_d[d], 16);
        gp_d[d] += __shfl_xor(gp_d[d], 32);
      }
      // P_ww rows (same-half entries; zero elsewhere) through this wave's
      // diagonal block into the accumulator layout (lane: column r, rows
      // 4 g .. 4 g + 3), plus the cross-half block; then Diag(beta) A_ww the
      // same way, into the block the inverse below reads
      float* ab = sAd + w * 256;
      const bool upper = r >= 8;
      auto same_half_rows = [&](const float (&v)[8], int d0, float scale) {
#pragma unroll
        for (int c = 0; c < 16; ++c) ab[r * 16 + c] = 0.f;
        static_for<0, 8>([&](auto D) {
          constexpr int d = decltype(D)::value;
          if (d >= d0 && d <= r && (!upper || r - d >= 8)) ab[r * 16 + r - d] = v[d] * scale;
        });
      };
      if (g == 0) same_half_rows(gp_d, 0, 1.f);
#pragma unroll
      for (int i = 0; i < 4; ++i) gp_diag[i] = ab[(4 * g + i) * 16 + r] + gp_m[i];
      if (g == 0) same_half_rows(ga_d, 1, bt);
#pragma unroll
      for (int i = 0; i < 4; ++i) ab[(4 * g + i) * 16 + r] += ga_m[i] * __shfl(bt, 4 * g + i);
    }

    // ---- decay, in log2 units, relative to the start of this lane's tile
    //      (unbounded decay: only the tile totals here; dl keeps the raw
    //      log-decays and each step below forms its prefix and suffix sums) ----
#pragma unroll
    for (int pc = 0; pc < 8; ++pc) {
      f32x4 tv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        tv[i] = row_scan(dl[pc][i] * LOG2E);
        if constexpr (!UNB) dl[pc][i] = tv[i];
      }
      if (r == 15) *reinterpret_cast<f32x4*>(sTot + w * 128 + piece_ch(pc, g)) = tv;
    }
    if (g == 0) sBeta[tok] = bt;
    __syncthreads();

    // ---- per-channel factors (rho_a: decay before tile a; rho_NT = g_n) ----
    for (int idx = tid; idx < 256; idx += NTH) {
      const int c = idx & 127, part = idx >> 7;
      float rho[NT + 1];
      rho[0] = 0.f;
#pragma unroll
      for (int a = 0; a < NT; ++a) rho[a + 1] = rho[a] + sTot[a * 128 + c];
      // (tile totals and their prefix and suffix sums: no differences)
      if (part == 0) {
#pragma unroll
        for (int a = 0; a < NT; ++a) sFE[a * 128 + c] = exp2_fast(sTot[a * 128 + c]);
        buf_st4(exp2_fast(rho[NT]), fb, F::G + 4 * c, 0);  // gamma = e^{g_n}
      } else {
        float after = 0.f;  // g_n - rho_{a+1}
#pragma unroll
        for (int a = NT - 1; a >= 0; --a) {
          sFA[a * 128 + c] = exp2_fast(rho[a]);
          sFB[a * 128 + c] = exp2_fast(after);
          after += sTot[a * 128 + c];
        }
      }
    }
    __syncthreads();

    // ---- per 32-channel step: operand fragments of the own tile, Qt, Kb^T,
    //      scaled column-tile copies, right-hand sides ----
    Frag<E> kr[4], qh[4], ql[4], kih[4], kil[4];
    {
      const Frag<E> sel0 = select_frag<E>(0, lane), sel1 = select_frag<E>(1, lane);
      // the step's 8 channels of a [128] factor table
      auto fac8 = [&](float (&y)[8], const float* v, int st) {
        const f32x4 t0v = *reinterpret_cast<const f32x4*>(v + piece_ch(2 * st, g));
        const f32x4 t1v = *reinterpret_cast<const f32x4*>(v + piece_ch(2 * st + 1, g));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y[i] = t0v[i];
          y[4 + i] = t1v[i];
        }
      };
      auto frag8 = [](Frag<E>& f, const float (&x)[8]) { frag_from_f32(f, x); };
      // channel-per-lane copy of 16 of the step's channels (half hh) via a
      // selection product: lane (channel 32 st + 16 hh + l % 16, tokens 4g..4g+3)
      auto select = [&](const Frag<E>& a, int hh) {
        return mma((f32x4){0.f, 0.f, 0.f, 0.f}, a, hh ? sel1 : sel0);
      };
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        float q8[8], k8[8], v8[8], ep[8], en[8], fac[8], x[8], y[8];
        // this step's pieces 2 st, 2 st + 1 (bf16 rows: row swap of the 16-byte loads)
        auto pieces = [&](float (&x)[8], const auto (&rp)[8], const u32x4 (&wp)[WIDE ? 4 : 1], bool wide) {
          if constexpr (WIDE) {
            if (wide) {
              Raw4<E> a, b;
              unpack_wide(a, b, wp[st]);
              cvt_raw4(x, a);
              cvt_raw4(x + 4, b);
              return;
            }
          }
          cvt_raw4(x, rp[2 * st]);
          cvt_raw4(x + 4, rp[2 * st + 1]);
        };
        pieces(q8, rq, wq, !PRO);
        pieces(k8, rk, wk, !PRO);
        pieces(v8, rv, wv, true);
        float sx[8];  // unbounded decay: rho_{w+1} - g, from the suffix sum
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float d = dl[2 * st + (e >> 2)][e & 3];
          if constexpr (UNB) {
            const float l2 = d * LOG2E;
            d = row_scan(l2);
            sx[e] = row_suffix_excl(l2);
          }
          ep[e] = exp2_fast(d);                       // e^{g - rho_w} <= 1
          if constexpr (!UNB) en[e] = exp2_fast(-d);  // e^{rho_w - g} <= e^{80}
        }
        // K_rel (A operand of the Gram products); beta Kt = beta K_rel e^{rho_w}
        // and beta V as channel-per-lane right-hand sides, sR[ct][w]
        fac8(fac, sFA + w * 128, st);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = k8[e] * ep[e];
        frag8(kr[st], x);
        Frag<E> a;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = x[e] * fac[e] * bt;
        frag8(a, y);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          Frag16<E> b;
          frag16_from_acc(b, select(a, hh));
          *reinterpret_cast<decltype(b.v)*>(sR + ((size_t)((2 * st + hh) * NT + w) * 64 + lane) * 4 * ES) = b.v;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = v8[e] * bt;
        frag8(a, y);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          Frag16<E> b;
          frag16_from_acc(b, select(a, hh));
          *reinterpret_cast<decltype(b.v)*>(sR + ((size_t)((8 + 2 * st + hh) * NT + w) * 64 + lane) * 4 * ES) = b.v;
        }
        // Q_rel (hi + lo) and Qt = Q_rel e^{rho_w}, already in the carry's order
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = q8[e] * ep[e];
        {
          float xs[8][4];
#pragma unroll
          for (int e = 0; e < 8; ++e) xs[2 * st + (e >> 2)][e & 3] = x[e];
          frag_step_split(qh[st], ql[st], xs, st);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = x[e] * fac[e];
        frag8(a, y);
        st_frag_g(fb, F::Q + (uint32_t)(w * 4 + st) * F::FR + lane_fr, a);
        if constexpr (!UNB) {
          // K_inv (hi + lo): B operand of the diagonal pair
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = k8[e] * en[e];
          {
            float xs[8][4];
#pragma unroll
            for (int e = 0; e < 8; ++e) xs[2 * st + (e >> 2)][e & 3] = x[e];
            frag_step_split(kih[st], kil[st], xs, st);
          }
        }
        // K_end = K e^{rho_{w+1} - g} <= 1 (K_inv e^{tot_w}, or from the
        // in-tile suffix sum when the decay is unbounded); Kb = K_end
        // e^{g_n - rho_{w+1}} as channel-per-lane halves of the Kb^T fragments
        // (rt8, kt = w / 2, half w % 2), each half a contiguous 64-lane block
        if constexpr (UNB) {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = k8[e] * exp2_fast(sx[e]);
        } else {
          fac8(fac, sFE + w * 128, st);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= fac[e];
        }
        fac8(fac, sFB + w * 128, st);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = x[e] * fac[e];
        frag8(a, y);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          st_half_g(fb, F::K + (uint32_t)((2 * st + hh) * F::KT + (w >> 1)) * F::FR + (uint32_t)(w & 1) * (F::FR / 2) +
                            (uint32_t)lane * 4 * ES,
                    select(a, hh), (E*)nullptr);
        // column-tile copies for the later row tiles a > w, scaled by
        // e^{rho_a - rho_{w+1}} = prod_{w < c < a} e^{tot_c}
        for (int at = w + 1; at < NT; ++at) {
          if (at > w + 1) {
            fac8(fac, sFE + (at - 1) * 128, st);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= fac[e];
          }
          frag8(a, x);
          const int q = at * (at - 1) / 2 + w;
          *reinterpret_cast<Frag<E>*>(sKE + ((size_t)(q * 4 + st) * 64 + lane) * 8 * ES) = a;
        }
      }
    }
    // the next chunk's inputs (they land while this chunk is finished)
    int64_t t0n = 0, bosn = 0;
    int nvn = 0;
    if (s + 1 < s_end) {
      slot_range(s + 1, t0n, bosn, nvn);
      if (PREFETCH_LA) issue_la(t0n, nvn);
      if (PREFETCH) issue_rows(t0n, nvn);
    }
    __syncthreads();

    // ---- Gram tiles of row tile a = w: (a, a) from registers, (a, b < a) with
    //      the scaled column tile from LDS.  P uses the hi + lo parts of Q_rel
    //      (and of K_inv on the diagonal) when the operands are bf16. ----
    f32x4 ga[NT], gp[NT];
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      ga[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
      gp[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (UNB) {
      gp[NT - 1] = gp_diag;  // (Diag(beta) A_ww is already in the wave's diagonal block)
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        ga[NT - 1] = mma(ga[NT - 1], kr[st], kih[st]);  // diagonal kept in slot NT-1
        gp[NT - 1] = mma(gp[NT - 1], qh[st], kih[st]);
        if constexpr (SPLIT) {
          gp[NT - 1] = mma(gp[NT - 1], ql[st], kih[st]);
          gp[NT - 1] = mma(gp[NT - 1], qh[st], kil[st]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < NT - 1; ++b) {
      if (b < w) {
        const int q = w * (w - 1) / 2 + b;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const Frag<E> kb = *reinterpret_cast<const Frag<E>*>(sKE + ((size_t)(q * 4 + st) * 64 + lane) * 8 * ES);
          ga[b] = mma(ga[b], kr[st], kb);
          gp[b] = mma(gp[b], qh[st], kb);
          if constexpr (SPLIT) gp[b] = mma(gp[b], ql[st], kb);
        }
      }
    }

    // ---- (I + Diag(beta) A_ww)^{-1} in fp32: lane j < 16 solves column j by
    //      forward substitution over this wave's own 16 x 16 block ----
    {
      float* ab = sAd + w * 256;
      if constexpr (!UNB)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 4 * g + i;
          ab[rr * 16 + r] = (r < rr) ? ga[NT - 1][i] * sBeta[16 * w + rr] : 0.f;
        }
      float xinv[16];
      if (lane < 16) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          float part[4] = {(rr == lane) ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q4 = 0; q4 < (rr + 3) / 4; ++q4) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(ab + rr * 16 + 4 * q4);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (4 * q4 + e < rr) part[e] -= av[e] * xinv[4 * q4 + e];
          }
          xinv[rr] = (part[0] + part[1]) + (part[2] + part[3]);
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) sM[(16 * w + rr) * L::LDM + 16 * w + lane] = from_f32<E>(xinv[rr]);
      }
    }
    // -(Diag(beta) A)_wb below the diagonal into the solve blocks
#pragma unroll
    for (int b = 0; b < NT - 1; ++b) {
      if (b < w) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 16 * w + 4 * g + i;
          sM[rr * L::LDM + 16 * b + r] = from_f32<E>(-ga[b][i] * sBeta[rr]);
        }
      }
    }
    // P tiles: transposed on the matrix cores into the carry's fragment order
    // (lane = token of tile w, four tokens of tile b); the diagonal tile keeps
    // its lower triangle; the tile right of an even diagonal is zero.  Tiles
    // 2 kt and 2 kt + 1 are the two halves of fragment (w, kt), stored together.
    {
      const Frag16<E> id = ident16<E>(lane);
      auto ptile = [&](int b) -> f32x4 {
        if (b > w) return (f32x4){0.f, 0.f, 0.f, 0.f};
        f32x4 pv = gp[b == w ? NT - 1 : b];
        if (b == w)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (r > 4 * g + i) pv[i] = 0.f;  // column r above row 4g+i
        Frag16<E> a;
        frag16_from_acc(a, pv);
        return mma16((f32x4){0.f, 0.f, 0.f, 0.f}, a, id);
      };
#pragma unroll
      for (int kt = 0; kt < NT / 2; ++kt)
        if (2 * kt <= w)
          st_pair_g(fb, F::P + (uint32_t)F::p_frag(w, kt) * F::FR + lane_fr, ptile(2 * kt), ptile(2 * kt + 1),
                    (E*)nullptr);
    }
    __syncthreads();

    // ---- blocked forward substitution on the matrix cores:
    //      Y_a = (I + A_aa)^{-1} (beta R_a - sum_{b<a} A_ab Y_b), tile row by
    //      tile row.  Wave w solves W column tiles CPW w .. and U' column tiles
    //      CPW w .., every Y_b it needs already in its registers. ----
    {
      const Frag16<E> id = ident16<E>(lane);
      Frag16<E> Yb[NOWN][NT];
#pragma unroll
      for (int a = 0; a < NT; ++a) {
        f32x4 z[NOWN];
        f32x4 w_even = (f32x4){0.f, 0.f, 0.f, 0.f};  // -W of the even channel tile, stored with the odd one
#pragma unroll
        for (int o = 0; o < NOWN; ++o) {
          const int ct = (o < CPW) ? CPW * w + o : 8 + CPW * w + (o - CPW);
          Frag16<E> rf;
          rf.v = *reinterpret_cast<const decltype(rf.v)*>(sR + ((size_t)(ct * NT + a) * 64 + lane) * 4 * ES);
          z[o] = frag16_to_f32(rf);
        }
#pragma unroll
        for (int b = 0; b < a; ++b) {
          Frag16<E> mf;
          ld_frag16(mf, sM + (16 * a + r) * L::LDM + 16 * b + 4 * g);
#pragma unroll
          for (int o = 0; o < NOWN; ++o) z[o] = mma16(z[o], mf, Yb[o][b]);
        }
        Frag16<E> md;
        ld_frag16(md, sM + (16 * a + r) * L::LDM + 16 * a + 4 * g);
#pragma unroll
        for (int o = 0; o < NOWN; ++o) {
          Frag16<E> zb;
          frag16_from_acc(zb, z[o]);
          const f32x4 y = mma16((f32x4){0.f, 0.f, 0.f, 0.f}, md, zb);
          frag16_from_acc(Yb[o][a], y);
          if (o < CPW) {
            // -W: the 16 x 16 tile transposed on the matrix cores to lane =
            // token, four channels; channel tile ct is half ct % 2 of key step
            // ct / 2, and this wave owns both tiles of its steps (CPW is even)
            Frag16<E> yn;
            frag16_from_acc(yn, -y);
            const f32x4 t = mma16((f32x4){0.f, 0.f, 0.f, 0.f}, yn, id);
            const int ct = CPW * w + o;
            if ((o & 1) == 0)
              w_even = t;
            else
              st_pair_g(fb, F::W + (uint32_t)(a * 4 + (ct >> 1)) * F::FR + lane_fr, w_even, t, (E*)nullptr);
          } else {
            // U' in accumulator order, in the I/O dtype
            const int ct = CPW * w + (o - CPW);
            st_half_g(fb, F::U + (uint32_t)(a * 8 + ct) * F::UT + (uint32_t)lane * 4 * ES, y, (E*)nullptr);
          }
        }
      }
    }
    // the next chunk rewrites sTot, sBeta and the factor tables only after the
    // next barrier; every LDS area written before that barrier is read-only here
    t0 = t0n;
    seq_bos = bosn;
    nv = nvn;
  }
}

namespace {

template <typename E, int C, bool PRO, bool UNB>
hipError_t launch_prep_t(const PrepArgs& a, hipStream_t stream) {
  constexpr size_t lds = PrepLayout<E, C>::BYTES;
  auto fn = prep_kernel<E, C, PRO, UNB>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (a.chunks_per_block < 1 || a.chunks_per_block > PrepLayout<E, C>::MAXR) return hipErrorInvalidValue;
  const int64_t ranges = ((int64_t)a.cap + a.chunks_per_block - 1) / a.chunks_per_block;
  const int64_t grid = ranges * a.num_heads;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(4 * C), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

template <typename E, int C, bool UNB>
hipError_t launch_prep_pro(const PrepArgs& a, hipStream_t stream) {
  const bool pro = a.conv_q_w != nullptr || a.conv_k_w != nullptr;
  return pro ? launch_prep_t<E, C, true, UNB>(a, stream) : launch_prep_t<E, C, false, UNB>(a, stream);
}

hipError_t launch_prep(const PrepArgs& a, hipStream_t stream) {
  if (a.bf16)
    return a.unbounded ? launch_prep_pro<__bf16, 64, true>(a, stream) : launch_prep_pro<__bf16, 64, false>(a, stream);
  return a.unbounded ? launch_prep_pro<float, 32, true>(a, stream) : launch_prep_pro<float, 32, false>(a, stream);
}

}  // namespace kda
