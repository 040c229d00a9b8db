// kda_bwd.hip — backward pass of the chunked KDA prefill for gfx950.
//
// "Kimi K3 架构、训练与系统全景解析", section 7.1 (FlashKDA): the chunked
// kernel serves training as well as prefill, so the recurrence needs its
// gradients.  The pages print no backward formulas; what follows is the exact
// derivative of the chunkwise form of section 4.2.4 (written out in
// kda_chunk.hip) for the loss  sum_t <dO_t, o_t> + <dS_T, S_T>.  Per chunk,
// with incoming state S, outgoing-state gradient dS' and U = U' - W S:
//
//   dU  = P^T dO + Kb dS'                      dS  = Diag(gamma) dS' + Qt^T dO - W^T dU
//   dQt = dO S^T          dW = -dU S^T          dKb = U dS'^T       dgamma = rowsum(dS' (.) S)
//   dP  = lower(dO U^T)   dT = dW Kt^T + dU V^T dKt = T^T dW        dV = T^T dU
//   T = M Diag(beta), M = (I + A)^{-1}:  dM = dT Diag(beta), dbeta_j += sum_r M_rj dT_rj,
//   dA = strictly-lower(-M^T dM M^T),  A = Diag(beta) B:  dB = Diag(beta) dA, dbeta_i += sum_j dA_ij B_ij
//
// and the Gram products B = Kt Kh^T, P = Qt Kh^T give the rest.  Every
// product that involves K e^{-g} is formed per 16-token tile against the
// tile's reference rho (the decay before the tile), exactly as the forward
// does, so no factor exceeds e^{80} under the decay bound [-5, 0]:
//   row tile a:    dK_t += e^{g_t - rho_a} (dB Kh_a)_t,  dQ_t += e^{g_t - rho_a} (dP Kh_a)_t
//   column tile b: dK_s += e^{rho_b - g_s} (dB^T K_b + dP^T Q_b)_s
// with Kh_a = K e^{rho_a - g} over tokens up to tile a and K_b, Q_b = (K, Q) e^{g - rho_b}
// over tokens from tile b on.  The log-decay gradient collects
//   dg_t = dQt (.) Qt + dKt (.) Kt - dKb (.) Kb + (tile terms) ,   dG = sum_t dKb (.) Kb + dgamma (.) gamma
// and dlog_alpha_t = sum_{t' >= t} dg_t' + dG  (g_t is the inclusive cumulative
// log-decay, G = g at the chunk's last token).
//
// Kernels, after the forward's prep kernel and its carry kernel in the states
// pass (which store S and U of every chunk):
//   bwd_prep_kernel   every (chunk, head): from the forward factor block and
//                     dO, the reverse carry's block (Kb and -W^T as operand
//                     fragments, P^T dO, Qt^T dO, gamma).
//   bwd_carry_kernel  one workgroup per (sequence, head, 64 value columns):
//                     walks the chunks backwards with dS in MFMA
//                     accumulators, storing dS' and dU of every chunk; the
//                     gradient reaching the first chunk is d_initial_state.
//   bwd_grad_kernel   every (chunk, head): all per-token gradients.
#include "kda_chunk_util.h"

namespace kda {
namespace {

// The sequence that owns slot s: the largest n with seq_first[n] <= s (empty
// sequences share their first slot with the next one and are skipped).
__device__ __forceinline__ int slot_seq(const int32_t* seq_first, int N, int s) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seq_first[mid] <= s)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Position of contraction index c (0..31 within a 32-deep step) in a lane's
// 8 fragment elements: lane group g = (c % 16) / 4, element (c % 4) + 4 (c / 16).
__device__ __forceinline__ int frag_elem(int c, int& grp) {
  grp = (c & 15) >> 2;
  return (c & 3) + ((c >> 4) << 2);
}

// Elements of forward factor-block fragments (layout in kda_internal.h).
// 16-token-row fragments (-W and Qt): fragment (t / 16) * 4 + i / 32, lane
// (group, t % 16), element frag_elem(i % 32).
template <typename E>
__device__ __forceinline__ float rowfrag_at(const E* f, int t, int i) {
  int grp;
  const int e = frag_elem(i & 31, grp);
  return to_f32(f[(((t >> 4) * 4 + (i >> 5)) * 64 + grp * 16 + (t & 15)) * 8 + e]);
}
// Kb[t][i] from the Kb^T fragments split in halves
template <typename E, int C>
__device__ __forceinline__ float kbt_at(const E* f, int t, int i) {
  constexpr int KT = C / 32;
  const int c = t & 31;
  return to_f32(f[(((i >> 4) * KT + (t >> 5)) * 2 + (c >> 4)) * 256 + (((c & 15) >> 2) * 16 + (i & 15)) * 4 + (c & 3)]);
}


// 4 consecutive elements (16-deep operand of one lane) as Frag16
__device__ __forceinline__ void ld4(Frag16<__bf16>& f, const __bf16* p) { f.v = *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ void ld4(Frag16<float>& f, const float* p) { f.v = *reinterpret_cast<const f32x4*>(p); }
// the same four values through a buffer view (byte offset; out of range reads zero)
__device__ __forceinline__ void buf_ld4(Frag16<__bf16>& f, Rsrc r, uint32_t off) {
  f.v = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ void buf_ld4(Frag16<float>& f, Rsrc r, uint32_t off) {
  f.v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// ---------------------------------------------------------------------------
// bwd_prep_kernel: one workgroup of four waves per (slot, head).  The factor
// block's Qt and P fragments and the chunk's dO rows are loaded into registers
// and scattered straight into row-major transposed LDS arrays (contraction
// index contiguous), so every 16-deep matrix-core step reads its four operand
// values per lane in one access.  The -W and Kb^T fragments are loaded at the
// start as well and staged raw in the same LDS bytes once the products are
// done, for the gathers into the reverse carry's operand order.  46 KiB of LDS
// lets three workgroups share a compute unit.  The products run in the I/O
// dtype: Qt, P and dO are values of that dtype already, so with fp32
// accumulation nothing is rounded.
// ---------------------------------------------------------------------------
template <typename E, int C>
struct PrepBwdLayout {
  using F = FactorBlock<(int)sizeof(E), C>;
  static constexpr int PT = C + 8;                                  // row pitch (elements) of the transposed arrays
  static constexpr size_t QT = 0;                                   // E [128][PT]  Qt^T
  static constexpr size_t PTR = QT + (size_t)D * PT * sizeof(E);    // E [C][PT]  P^T
  static constexpr size_t DOT = PTR + (size_t)C * PT * sizeof(E);   // E [128][PT] dO^T
  static constexpr size_t BYTES = DOT + (size_t)D * PT * sizeof(E);
  // second phase, over the same bytes: raw -W and Kb^T fragments
  static constexpr size_t RW = 0;
  static constexpr size_t RK = RW + (size_t)(C / 16) * 4 * F::FR;
  static_assert(RK + (size_t)8 * (C / 32) * F::FR <= BYTES, "raw fragments fit the transposed arrays");
  static_assert(PTR % 16 == 0 && DOT % 16 == 0 && RK % 16 == 0, "16-byte pieces");
};

template <typename E, int C>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdArgs p) {
  constexpr int ES = (int)sizeof(E);
  using F = FactorBlock<ES, C>;
  using DB = DCarryBlock<ES, C>;
  using L = PrepBwdLayout<E, C>;
  constexpr int NT = C / 16, KT = C / 32, PT = L::PT;
  constexpr int PER = 16 / ES;    // elements per 16-byte piece
  constexpr int LPC = 8 / PER;    // pieces per lane chunk (8 elements of one fragment lane)
  constexpr int NW = (int)(NT * 4 * F::FR / 16) / 256;  // -W pieces per thread
  constexpr int NK = (int)(8 * KT * F::FR / 16) / 256;  // Kb^T pieces per thread
  static_assert(NW * 256 * 16 == (int)(NT * 4 * F::FR) && NK * 256 * 16 == (int)(8 * KT * F::FR), "whole pieces");
  static_assert(L::BYTES <= 160 * 1024, "LDS budget exceeded");
  extern __shared__ __align__(16) unsigned char smem[];
  E* sQT = reinterpret_cast<E*>(smem + L::QT);
  E* sPT = reinterpret_cast<E*>(smem + L::PTR);
  E* sDOT = reinterpret_cast<E*>(smem + L::DOT);
  // dO^T[j][t] sits at column t ^ 4 ((j / 8) mod (C / 4)) of row j: the scatter
  // below writes rows 8 apart from neighbouring lanes, which this spreads over
  // the banks; groups of four tokens stay contiguous for the operand reads
  auto dot_at = [](int j, int t) { return j * PT + (t ^ (4 * ((j >> 3) & (C / 4 - 1)))); };
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int H = p.num_heads, h = blockIdx.x % H, slot = blockIdx.x / H;
  if (slot >= p.seq_first[p.num_seqs]) return;
  const int n = slot_seq(p.seq_first, p.num_seqs, slot);
  int64_t bos, eos;
  seq_range(p.cu, n, p.total_tokens, bos, eos);
  const int64_t t0 = bos + (int64_t)(slot - p.seq_first[n]) * C;
  const int nv = (int)max((int64_t)0, min((int64_t)C, eos - t0));
  const size_t blk = (size_t)slot * H + h;
  const char* fb = static_cast<const char*>(p.factors) + blk * F::BYTES;

  // -W and Kb^T pieces, held in registers until the second phase
  u32x4 rw[NW], rk[NK];
#pragma unroll
  for (int m = 0; m < NW; ++m) rw[m] = reinterpret_cast<const u32x4*>(fb + F::W)[tid + 256 * m];
#pragma unroll
  for (int m = 0; m < NK; ++m) rk[m] = reinterpret_cast<const u32x4*>(fb + F::K)[tid + 256 * m];
  // one lane chunk: fragment f, lane ln -> 8 elements (row t = 16 (f / 4) + ln % 16,
  // contraction index 32 (f % 4) + the fragment order)
  auto load_chunk = [&](uint32_t base, int f, int ln, E (&v)[8]) {
    u32x4 raw[LPC];
#pragma unroll
    for (int q = 0; q < LPC; ++q) raw[q] = reinterpret_cast<const u32x4*>(fb + base)[(f * 64 + ln) * LPC + q];
    __builtin_memcpy(v, raw, sizeof(raw));
  };
  auto frag_col = [](int ks, int grp, int e) { return 32 * ks + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4); };
  // Qt^T: chunk (f, ln) of the Qt fragments to sQT[key][t]
  for (int c = tid; c < NT * 4 * 64; c += 256) {
    const int f = c >> 6, ln = c & 63, rt = f >> 2, ks = f & 3, grp = ln >> 4, t = 16 * rt + (ln & 15);
    E v[8];
    load_chunk(F::Q, f, ln, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) sQT[frag_col(ks, grp, e) * PT + t] = v[e];
  }
  // P^T: fragments (rt, kt) with kt <= rt / 2 are stored (P is zero above the
  // diagonal); the rest of sPT is zero
  for (int c = tid; c < NT * KT * 64; c += 256) {
    const int pr = c >> 6, ln = c & 63, rt = pr / KT, kt = pr % KT, grp = ln >> 4, t = 16 * rt + (ln & 15);
    E v[8];
    if (kt <= rt / 2) {
      load_chunk(F::P, F::p_frag(rt, kt), ln, v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = from_f32<E>(0.f);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sPT[frag_col(kt, grp, e) * PT + t] = v[e];
  }
  // dO rows (16-byte pieces), transposed into dO^T[j][t]; zero past the end
  {
    const E* gdo = static_cast<const E*>(p.d_o);
    const int64_t rs = (int64_t)H * D;
    for (int i = tid; i < C * (D / PER); i += 256) {
      const int t = i / (D / PER), j0 = (i % (D / PER)) * PER;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (t < nv) raw = *reinterpret_cast<const u32x4*>(gdo + (t0 + t) * rs + (int64_t)h * D + j0);
      const E* x = reinterpret_cast<const E*>(&raw);
#pragma unroll
      for (int e = 0; e < PER; ++e) sDOT[dot_at(j0 + e, t)] = x[e];
    }
  }
  __syncthreads();
  char* dst = static_cast<char*>(p.dblocks) + blk * DB::BYTES;

  // X = P^T dO: tile (token tile sa, column tile jt); P[t][s] is zero for t < s
  E* dX = reinterpret_cast<E*>(dst + DB::X);
  for (int ti = wv; ti < NT * 8; ti += 4) {
    const int sa = ti / 8, jt = ti % 8;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kb = sa; kb < NT; ++kb) {
      Frag16<E> A, B;
      ld4(A, sPT + (16 * sa + l16) * PT + 16 * kb + 4 * g);
      ld4(B, sDOT + dot_at(16 * jt + l16, 16 * kb + 4 * g));
      acc = mma16(acc, A, B);
    }
    store_row4(dX + ((size_t)ti * 64 + lane) * 4, acc);
  }
  // Y = Qt^T dO: tile (key tile it, column tile jt)
  E* dY = reinterpret_cast<E*>(dst + DB::Y);
  for (int ti = wv; ti < 64; ti += 4) {
    const int it = ti / 8, jt = ti % 8;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NT; ++kb) {
      Frag16<E> A, B;
      ld4(A, sQT + (16 * it + l16) * PT + 16 * kb + 4 * g);
      ld4(B, sDOT + dot_at(16 * jt + l16, 16 * kb + 4 * g));
      acc = mma16(acc, A, B);
    }
    store_row4(dY + ((size_t)ti * 64 + lane) * 4, acc);
  }
  __syncthreads();  // the transposed arrays are no longer read
#pragma unroll
  for (int m = 0; m < NW; ++m) reinterpret_cast<u32x4*>(smem + L::RW)[tid + 256 * m] = rw[m];
#pragma unroll
  for (int m = 0; m < NK; ++m) reinterpret_cast<u32x4*>(smem + L::RK)[tid + 256 * m] = rk[m];
  __syncthreads();
  const E* sW = reinterpret_cast<const E*>(smem + L::RW);
  const E* sKbt = reinterpret_cast<const E*>(smem + L::RK);
  // Kb as A-operand fragments over the keys, -W^T as fragments over the tokens
  E* dKB = reinterpret_cast<E*>(dst + DB::KB);
  for (int i = tid; i < NT * 4 * 64; i += 256) {
    const int f = i / 64, ln = i % 64, rt = f / 4, ks = f % 4, r = ln & 15, gg = ln >> 4;
    E vals[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) vals[e] = from_f32<E>(kbt_at<E, C>(sKbt, 16 * rt + r, frag_col(ks, gg, e)));
#pragma unroll
    for (int e = 0; e < 8; ++e) dKB[((size_t)f * 64 + ln) * 8 + e] = vals[e];
  }
  E* dWT = reinterpret_cast<E*>(dst + DB::WT);
  for (int i = tid; i < 8 * KT * 64; i += 256) {
    const int f = i / 64, ln = i % 64, rt8 = f / KT, kt = f % KT, r = ln & 15, gg = ln >> 4;
    E vals[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) vals[e] = from_f32<E>(rowfrag_at(sW, frag_col(kt, gg, e), 16 * rt8 + r));
#pragma unroll
    for (int e = 0; e < 8; ++e) dWT[((size_t)f * 64 + ln) * 8 + e] = vals[e];
  }
  if (tid < D) reinterpret_cast<float*>(dst + DB::G)[tid] = reinterpret_cast<const float*>(fb + F::G)[tid];
}

// ---------------------------------------------------------------------------
// bwd_carry_kernel: four compute waves of 16 value columns plus one loader
// wave per (sequence, head, 64-column block), chunks in reverse order.  The
// loader copies each chunk's Kb, -W^T and gamma into a three-slot LDS ring
// two chunks ahead; one barrier per chunk hands the slots over (as in the
// forward carry).
// ---------------------------------------------------------------------------
template <typename E, int C>
struct CarryBwdLayout {
  using DB = DCarryBlock<(int)sizeof(E), C>;
  static constexpr uint32_t SLOT = DB::LDS_PART;
  static constexpr int PIECES = (int)(SLOT / 1024);
  static constexpr int NBUF = 3;
  static constexpr size_t BYTES = (size_t)NBUF * SLOT;
  static_assert(SLOT % 1024 == 0, "1 KiB pieces");
};

template <typename E, int C>
__global__ __launch_bounds__(320) void bwd_carry_kernel(const BwdArgs p) {
  constexpr int NWC = 4;
  constexpr int ES = (int)sizeof(E);
  using DB = DCarryBlock<ES, C>;
  using L = CarryBwdLayout<E, C>;
  constexpr int NT = C / 16, KT = C / 32;
  static_assert(L::BYTES <= 160 * 1024, "LDS budget exceeded");
  static_assert(L::PIECES <= 63, "copy exceeds the outstanding-load counter");
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // XCD-aware decode: blocks b and b + 8 (the two column blocks of one
  // (sequence, head)) run on the same XCD
  const int xcd = blockIdx.x & 7, sl = blockIdx.x >> 3;
  const int cb = sl % 2;
  const int u = (sl / 2) * 8 + xcd;
  const int H = p.num_heads;
  if (u >= p.num_seqs * H) return;
  const int rnk = u / H, h = u % H;
  const int n = p.order ? p.order[rnk] : rnk;
  const int slot0 = p.seq_first[n];
  const int nch = max(0, p.seq_first[n + 1] - slot0);
  const char* dbase = static_cast<const char*>(p.dblocks);
  auto block_of = [&](int ci) { return dbase + ((size_t)(slot0 + ci) * H + h) * DB::BYTES; };

  if (wv == NWC) {
    auto copy_block = [&](int k) {
      const char* blk = block_of(nch - 1 - k);
      unsigned char* dstl = smem + (k % L::NBUF) * L::SLOT;
#pragma unroll
      for (int j = 0; j < L::PIECES; ++j)
        __builtin_amdgcn_global_load_lds(blk + j * 1024u + lane * 16,
                                         (__attribute__((address_space(3))) void*)(dstl + j * 1024), 16, 0, 0);
    };
    if (nch > 0) copy_block(0);
    if (nch > 1) copy_block(1);
    for (int k = 0; k < nch; ++k) {
      if (k + 1 < nch)
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(L::PIECES));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
      __syncthreads();
      if (k + 2 < nch) copy_block(k + 2);
    }
    return;
  }

  const int l16 = lane & 15, g = lane >> 4;
  const int col0 = cb * 64 + 16 * wv, ct = col0 / 16;
  const size_t sbase = ((size_t)n * H + h) * (size_t)(D * D);
  // dS at the end of the sequence: d_final_state, or zero
  f32x4 accD[8];
#pragma unroll
  for (int rt8 = 0; rt8 < 8; ++rt8)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      accD[rt8][i] = p.d_final_state ? p.d_final_state[sbase + (size_t)(16 * rt8 + 4 * g + i) * D + col0 + l16] : 0.f;

  using Raw = std::conditional_t<ES == 2, u32x2, f32x4>;
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
  constexpr int FRE = 512;  // elements per fragment
  Frag16<E> id16;  // the 16 x 16 identity as a B operand
  {
    f32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (4 * g + e == l16) ? 1.f : 0.f;
    frag16_from_acc(id16, x);
  }

  for (int k = 0; k < nch; ++k) {
    const int ci = nch - 1 - k;
    const size_t blkid = (size_t)(slot0 + ci) * H + h;
    const Rsrc rb = make_rsrc(block_of(ci), DB::BYTES);
    Raw rX[NT], rY[8];
#pragma unroll
    for (int a = 0; a < NT; ++a) rX[a] = buf_ld_raw(rb, (uint32_t)(lane * 4 * ES), DB::X + (a * 8 + ct) * DB::TILE);
#pragma unroll
    for (int rt8 = 0; rt8 < 8; ++rt8)
      rY[rt8] = buf_ld_raw(rb, (uint32_t)(lane * 4 * ES), DB::Y + (rt8 * 8 + ct) * DB::TILE);
    // the gradient reaching this chunk's end (16 x 16 tiles, I/O dtype); each
    // tile is transposed on the matrix cores (a product with the identity,
    // exact) so that a lane stores four consecutive columns of one row and a
    // store instruction writes the whole 512-byte tile
    E* ds_dst = static_cast<E*>(p.chunk_ds) + blkid * (size_t)(D * D);
#pragma unroll
    for (int rt8 = 0; rt8 < 8; ++rt8) {
      Frag16<E> a;
      frag16_from_acc(a, accD[rt8]);
      store_row4(ds_dst + tile16_index(16 * rt8 + l16, col0 + 4 * g), mma16((f32x4){0.f, 0.f, 0.f, 0.f}, a, id16));
    }
    __syncthreads();  // slot k % 3 holds chunk ci
    const unsigned char* buf = smem + (k % L::NBUF) * L::SLOT;
    const E* sKB = reinterpret_cast<const E*>(buf + DB::KB + lane * 8 * ES);
    const E* sWT = reinterpret_cast<const E*>(buf + DB::WT + lane * 8 * ES);
    const float* sG = reinterpret_cast<const float*>(buf + DB::G);

    // dU = P^T dO + Kb dS'
    Frag<E> sf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) frag_from_acc(sf[ks], accD[2 * ks], accD[2 * ks + 1]);
    f32x4 accU[NT];
#pragma unroll
    for (int a = 0; a < NT; ++a) accU[a] = raw_f32(rX[a]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int a = 0; a < NT; ++a) {
        Frag<E> fa;
        ld_frag(fa, sKB + (a * 4 + ks) * FRE);
        accU[a] = mma(accU[a], fa, sf[ks]);
      }
    E* du_dst = static_cast<E*>(p.chunk_du) + blkid * (size_t)(C * D);
#pragma unroll
    for (int a = 0; a < NT; ++a) {
      Frag16<E> fr;
      frag16_from_acc(fr, accU[a]);
      store_row4(du_dst + tile16_index(16 * a + l16, col0 + 4 * g), mma16((f32x4){0.f, 0.f, 0.f, 0.f}, fr, id16));
    }
    // dS = Diag(gamma) dS' + Qt^T dO - W^T dU
    Frag<E> uf[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) frag_from_acc(uf[kt], accU[2 * kt], accU[2 * kt + 1]);
#pragma unroll
    for (int rt8 = 0; rt8 < 8; ++rt8) {
      const f32x4 gam = *reinterpret_cast<const f32x4*>(sG + 16 * rt8 + 4 * g);
      accD[rt8] = accD[rt8] * gam + raw_f32(rY[rt8]);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        Frag<E> fw;
        ld_frag(fw, sWT + (rt8 * KT + kt) * FRE);
        accD[rt8] = mma(accD[rt8], fw, uf[kt]);
      }
    }
  }
  if (p.d_initial_state) {
#pragma unroll
    for (int rt8 = 0; rt8 < 8; ++rt8)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p.d_initial_state[sbase + (size_t)(16 * rt8 + 4 * g + i) * D + col0 + l16] = accD[rt8][i];
  }
}

// ---------------------------------------------------------------------------
// bwd_grad_kernel: one workgroup of NW waves per (slot, head).  Wave w owns
// key tiles (8 / NW) w .. (8 / NW)(w + 1) - 1 of every per-token gradient;
// C x C quantities live in LDS.  The Gram tiles, the C x C chain and the
// tile-referenced products run in fp32 on the matrix cores (four
// v_mfma_f32_16x16x4_f32 per 16-deep step); the products with S, dS', U, dU,
// dO and V run in the I/O dtype, the precision those values are stored in.
// ---------------------------------------------------------------------------
template <typename E, int C>
struct GradLayout {
  static constexpr int PK = D + 8;   // pitch of [C][128] arrays (elements; 16-byte rows)
  static constexpr int PC = C + 4;   // pitch of [C][C] arrays
  static constexpr int JB = 32;      // value columns per staging block
  static constexpr int PJ = JB + 8;  // staging pitch (elements of E)
  static constexpr size_t K = 0;                                     // E   [C][PK] k
  static constexpr size_t Q = K + (size_t)C * PK * sizeof(E);        // E   [C][PK] q
  static constexpr size_t G = Q + (size_t)C * PK * sizeof(E);        // f32 [C][PK] g
  static constexpr size_t M = G + (size_t)C * PK * 4;                // f32 [C][PC] (I + A)^{-1}
  static constexpr size_t DP = M + (size_t)C * PC * 4;               // f32 [C][PC] dP
  static constexpr size_t UN = DP + (size_t)C * PC * 4;              // union area
  static constexpr size_t UN_STAGE = 4 * (size_t)C * PJ * sizeof(E); //   dO, U, dU, V column blocks (E)
  static constexpr size_t UN_DW = (size_t)C * PK * 4;                //   dW [C][PK]
  static constexpr size_t UN_CC = 2 * (size_t)C * PC * 4;            //   A, or dM / dB and X = dM M^T
  static constexpr size_t UN_BYTES = UN_STAGE > UN_DW ? (UN_STAGE > UN_CC ? UN_STAGE : UN_CC)
                                                     : (UN_DW > UN_CC ? UN_DW : UN_CC);
  static constexpr int NLT = (C / 16) * (C / 16 + 1) / 2;           // lower 16 x 16 tiles of a C x C matrix
  static constexpr size_t BETA = UN + UN_BYTES;                      // f32 [C]
  static constexpr size_t DBT = BETA + (size_t)C * 4;                // f32 [NLT][16] dbeta parts, T term (columns)
  static constexpr size_t DBB = DBT + (size_t)NLT * 16 * 4;          // f32 [NLT][16] dbeta parts, B term (rows)
  static constexpr size_t GRAM = DBB + (size_t)NLT * 16 * 4;         // f32 [C][PC] Gram B (lower tiles)
  static constexpr size_t BYTES = GRAM + (size_t)C * PC * 4;
};

template <typename E, int C, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_grad_kernel(const BwdArgs p) {
  using L = GradLayout<E, C>;
  constexpr int NTH = 64 * NW;      // threads
  constexpr int KPW = 8 / NW;       // 16-key tiles per wave
  static_assert(KPW * NW == 8, "the waves cover the 8 key tiles");
  constexpr int NT = C / 16, PK = L::PK, PC = L::PC, JB = L::JB, PJ = L::PJ;
  static_assert(L::BYTES <= 160 * 1024, "LDS budget exceeded");
  extern __shared__ __align__(16) unsigned char smem[];
  E* sK = reinterpret_cast<E*>(smem + L::K);
  E* sQ = reinterpret_cast<E*>(smem + L::Q);
  float* sG = reinterpret_cast<float*>(smem + L::G);
  float* sM = reinterpret_cast<float*>(smem + L::M);
  float* sDP = reinterpret_cast<float*>(smem + L::DP);
  float* sUN = reinterpret_cast<float*>(smem + L::UN);
  float* sBeta = reinterpret_cast<float*>(smem + L::BETA);
  // dbeta from per-tile parts summed in a fixed order at the end, so the
  // result does not depend on which wave finishes first
  float* sDbT = reinterpret_cast<float*>(smem + L::DBT);
  float* sDbB = reinterpret_cast<float*>(smem + L::DBB);
  float* sB = reinterpret_cast<float*>(smem + L::GRAM);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int H = p.num_heads, h = blockIdx.x % H, slot = blockIdx.x / H;
  if (slot >= p.seq_first[p.num_seqs]) return;
  const int n = slot_seq(p.seq_first, p.num_seqs, slot);
  int64_t bos, eos;
  seq_range(p.cu, n, p.total_tokens, bos, eos);
  const int64_t t0 = bos + (int64_t)(slot - p.seq_first[n]) * C;
  const int nv = (int)max((int64_t)0, min((int64_t)C, eos - t0));
  const size_t blk = (size_t)slot * H + h;
  const int64_t rs = (int64_t)H * D;
  const int64_t hoff = (int64_t)h * D;
  Frag16<E> id16;  // the 16 x 16 identity as a B operand
  {
    f32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (4 * g + e == l16) ? 1.f : 0.f;
    frag16_from_acc(id16, x);
  }

  // ---- inputs: k, q rows, the cumulative log-decay g (zeros past the end) ----
  // Every load is issued before the first one is used (rows past the end are
  // read from the last valid row and replaced by zeros), so the phase waits
  // for one memory round trip.
  if (nv <= 0) return;
  constexpr int PER = 16 / (int)sizeof(E);  // elements per 16-byte piece
  constexpr int KQ = C * (D / PER) / NTH;   // pieces of k (and of q) per thread
  static_assert(KQ * NTH == C * (D / PER), "whole pieces per thread");
  constexpr int QG = NTH / D;               // token groups of the cumulative sum
  constexpr int TG = C / QG;                // tokens per group
  static_assert(QG * D == NTH && TG * QG == C, "cumulative-sum groups");
  const E* gS = static_cast<const E*>(p.chunk_states) + blk * (size_t)(D * D);
  const E* gDS = static_cast<const E*>(p.chunk_ds) + blk * (size_t)(D * D);
  const E* gU = static_cast<const E*>(p.chunk_u) + blk * (size_t)(C * D);
  const E* gDU = static_cast<const E*>(p.chunk_du) + blk * (size_t)(C * D);
  const E* gdo = static_cast<const E*>(p.d_o);
  const E* gv = static_cast<const E*>(p.v);
  // Each 32-column block's dO, V, U and dU (16-byte pieces of E; U and dU
  // from their 16 x 16 tiles, where a piece never crosses a tile row) and the
  // wave's S and dS' operands are loaded into registers one block ahead, so
  // their latency overlaps the previous block's products.  The loads go
  // through buffer views and are issued for every block and lane: threads
  // without a piece, rows past the sequence end and the block after the last
  // read zero from outside the view.  With no load or store behind a branch,
  // the wait for a block's data counts only the accesses issued after it
  // instead of draining the dV stores too.
  constexpr int NSTG = C * (JB / PER);  // staging pieces per array and block
  static_assert(NSTG <= NTH, "one staging piece per thread");
  const int st_t = tid / (JB / PER), st_c = (tid % (JB / PER)) * PER;
  const bool st_ld = tid < NSTG && st_t < nv;
  constexpr uint32_t kOutside = 0x80000000u;  // past every view below
  constexpr int ES = (int)sizeof(E);
  const uint32_t rows_bytes = (uint32_t)((int64_t)nv * rs * ES);
  u32x4 nA, nB, nU, nDU;
  Frag16<E> nS[KPW][JB / 16], nD[KPW][JB / 16];
  auto fetch = [&](int j0, bool any) {
    const Rsrc rDO = make_rsrc(gdo + t0 * rs, any ? rows_bytes : 0u);
    const Rsrc rV = make_rsrc(gv + t0 * rs, any ? rows_bytes : 0u);
    const Rsrc rU = make_rsrc(gU, any ? (uint32_t)(C * D * ES) : 0u);
    const Rsrc rDU = make_rsrc(gDU, any ? (uint32_t)(C * D * ES) : 0u);
    const Rsrc rS = make_rsrc(gS, any ? (uint32_t)(D * D * ES) : 0u);
    const Rsrc rDS = make_rsrc(gDS, any ? (uint32_t)(D * D * ES) : 0u);
    const uint32_t orow = st_ld ? (uint32_t)((st_t * rs + hoff + j0 + st_c) * ES) : kOutside;
    const uint32_t otile = st_ld ? (uint32_t)(tile16_index(st_t, j0 + st_c) * ES) : kOutside;
    nA = buf_ld16(rDO, orow, 0);
    nB = buf_ld16(rV, orow, 0);
    nU = buf_ld16(rU, otile, 0);
    nDU = buf_ld16(rDU, otile, 0);
#pragma unroll
    for (int c = 0; c < KPW; ++c)
#pragma unroll
      for (int js = 0; js < JB / 16; ++js) {
        const int i = 16 * (KPW * wv + c) + l16;
        const uint32_t o = (uint32_t)(tile16_index(i, j0 + 16 * js + 4 * g) * ES);
        buf_ld4(nS[c][js], rS, o);
        buf_ld4(nD[c][js], rDS, o);
      }
  };
  {
    const E* gk = static_cast<const E*>(p.k);
    const E* gq = static_cast<const E*>(p.q);
    u32x4 ka[KQ], qa[KQ];
#pragma unroll
    for (int m = 0; m < KQ; ++m) {
      const int i = tid + NTH * m, t = i / (D / PER), c = (i % (D / PER)) * PER;
      const int64_t row = (t0 + min(t, nv - 1)) * rs + hoff + c;
      ka[m] = *reinterpret_cast<const u32x4*>(gk + row);
      qa[m] = *reinterpret_cast<const u32x4*>(gq + row);
    }
    const int gc = tid & (D - 1), grp = tid / D;
    float x[TG];
#pragma unroll
    for (int u = 0; u < TG; ++u) {
      const int t = grp * TG + u;
      x[u] = p.log_alpha[(t0 + min(t, nv - 1)) * rs + hoff + gc];
    }
    const float bt = p.beta[(t0 + min(tid, nv - 1)) * H + h];
    fetch(0, true);  // the first column block of the products with S and dS'
#pragma unroll
    for (int m = 0; m < KQ; ++m) {
      const int i = tid + NTH * m, t = i / (D / PER), c = (i % (D / PER)) * PER;
      const u32x4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(sK + t * PK + c) = t < nv ? ka[m] : z;
      *reinterpret_cast<u32x4*>(sQ + t * PK + c) = t < nv ? qa[m] : z;
    }
    // cumulative log-decay: each group sums its tokens, then adds the totals
    // of the groups before it (exchanged through the Gram array, unused yet)
    float run = 0.f;
#pragma unroll
    for (int u = 0; u < TG; ++u) {
      run += grp * TG + u < nv ? x[u] : 0.f;
      x[u] = run;
    }
    sB[grp * D + gc] = run;
    if (tid < C) sBeta[tid] = tid < nv ? bt : 0.f;
    for (int i = tid; i < C * PC; i += NTH) {
      sM[i] = 0.f;
      sDP[i] = 0.f;
      sUN[i] = 0.f;  // A (strictly lower part written below)
    }
    __syncthreads();
    float off = 0.f;
    for (int q = 0; q < grp; ++q) off += sB[q * D + gc];
#pragma unroll
    for (int u = 0; u < TG; ++u) sG[(grp * TG + u) * PK + gc] = off + x[u];
  }
  __syncthreads();
  auto kf = [&](int t, int i) { return to_f32(sK[t * PK + i]); };
  auto qf = [&](int t, int i) { return to_f32(sQ[t * PK + i]); };
  auto gf = [&](int t, int i) { return sG[t * PK + i]; };
  // decay before token tile a (its reference), per key channel
  auto rho = [&](int a, int i) { return a == 0 ? 0.f : sG[(16 * a - 1) * PK + i]; };
  auto Gc = [&](int i) { return sG[(C - 1) * PK + i]; };

  // Gram tile B[t][s] = sum_i K_t e^{g_t - rho_a} K_s e^{rho_a - g_s} (a = t's tile)
  auto gram_tile = [&](int a, int b) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < 8; ++kb) {
      Frag16<float> A, B;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * kb + 4 * g + e;
        const float r = rho(a, i);
        const int t = 16 * a + l16, s = 16 * b + l16;
        A.v[e] = kf(t, i) * __expf(gf(t, i) - r);
        B.v[e] = kf(s, i) * __expf(r - gf(s, i));
      }
      acc = mma16(acc, A, B);
    }
    return acc;  // rows t = 16a + 4g + e, column s = 16b + l16
  };
  // lower tiles (a, b), b <= a, enumerated row by row
  constexpr int NLT = NT * (NT + 1) / 2;
  auto lower_tile = [](int idx, int& a, int& b) {
    a = 0;
    while ((a + 1) * (a + 2) / 2 <= idx) ++a;
    b = idx - a * (a + 1) / 2;
  };

  // ---- A = strictly-lower(Diag(beta) B) into the union area; B kept for dbeta ----
  float* sA = sUN;
  for (int idx = wv; idx < NLT; idx += NW) {
    int a, b;
    lower_tile(idx, a, b);
    const f32x4 acc = gram_tile(a, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * a + 4 * g + e, s = 16 * b + l16;
      sB[t * PC + s] = acc[e];
      if (s < t) sA[t * PC + s] = sBeta[t] * acc[e];
    }
  }
  __syncthreads();
  // ---- M = (I + A)^{-1}: diagonal 16 x 16 blocks by forward substitution ----
  if (wv < NT && g == 0) {
    const int a = wv, j = l16;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = (r == j) ? 1.f : 0.f;
#pragma unroll
      for (int c = 0; c < r; ++c) v -= sA[(16 * a + r) * PC + 16 * a + c] * x[c];
      x[r] = v;
      sM[(16 * a + r) * PC + 16 * a + j] = v;
    }
  }
  __syncthreads();
  // ... then the blocks below the diagonal, one block row at a time:
  // M_ab = -M_aa sum_{c=b}^{a-1} A_ac M_cb
  for (int a = 1; a < NT; ++a) {
    if (wv < a) {
      const int b = wv;
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
      for (int c = b; c < a; ++c) {
        Frag16<float> A, B;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          A.v[e] = sA[(16 * a + l16) * PC + 16 * c + 4 * g + e];
          B.v[e] = sM[(16 * c + 4 * g + e) * PC + 16 * b + l16];
        }
        z = mma16(z, A, B);
      }
      Frag16<float> A, B;
#pragma unroll
      for (int e = 0; e < 4; ++e) A.v[e] = sM[(16 * a + l16) * PC + 16 * a + 4 * g + e];
      B.v = z;
      const f32x4 m = mma16((f32x4){0.f, 0.f, 0.f, 0.f}, A, B);
#pragma unroll
      for (int e = 0; e < 4; ++e) sM[(16 * a + 4 * g + e) * PC + 16 * b + l16] = -m[e];
    }
    __syncthreads();
  }

  // ---- products with S and dS' over the value columns, 32 at a time ----
  E* sDO = reinterpret_cast<E*>(sUN);
  E* sU = sDO + C * PJ;
  E* sDU = sDO + 2 * C * PJ;
  E* sV = sDO + 3 * C * PJ;
  f32x4 rQs[NT][KPW], rW[NT][KPW], rKb[NT][KPW];
  float gpart[KPW];
#pragma unroll
  for (int c = 0; c < KPW; ++c) gpart[c] = 0.f;
#pragma unroll
  for (int rt = 0; rt < NT; ++rt)
#pragma unroll
    for (int c = 0; c < KPW; ++c) rQs[rt][c] = rW[rt][c] = rKb[rt][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  constexpr int MAXLT = (NLT + NW - 1) / NW;  // lower tiles per wave
  f32x4 rdP[MAXLT], rdT[MAXLT];
#pragma unroll
  for (int x = 0; x < MAXLT; ++x) rdP[x] = rdT[x] = (f32x4){0.f, 0.f, 0.f, 0.f};
  E* gdv = static_cast<E*>(p.dv);
  __syncthreads();  // A (in the union area) is no longer read
  for (int j0 = 0; j0 < D; j0 += JB) {
    if (tid < NSTG) {
      *reinterpret_cast<u32x4*>(sDO + st_t * PJ + st_c) = nA;
      *reinterpret_cast<u32x4*>(sV + st_t * PJ + st_c) = nB;
      *reinterpret_cast<u32x4*>(sU + st_t * PJ + st_c) = nU;
      *reinterpret_cast<u32x4*>(sDU + st_t * PJ + st_c) = nDU;
    }
    Frag16<E> cS[KPW][JB / 16], cD[KPW][JB / 16];
#pragma unroll
    for (int c = 0; c < KPW; ++c)
#pragma unroll
      for (int js = 0; js < JB / 16; ++js) {
        cS[c][js] = nS[c][js];
        cD[c][js] = nD[c][js];
      }
    __syncthreads();
    fetch(j0 + JB < D ? j0 + JB : j0, j0 + JB < D);
    // dQt += dO S^T, (dU S^T), dKb += U dS'^T, dgamma partials: own key tiles
#pragma unroll
    for (int c = 0; c < KPW; ++c) {
#pragma unroll
      for (int js = 0; js < JB / 16; ++js) {
        const Frag16<E> BS = cS[c][js], BD = cD[c][js];
#pragma unroll
        for (int e = 0; e < 4; ++e) gpart[c] += (float)BS.v[e] * (float)BD.v[e];
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
          const int off = (16 * rt + l16) * PJ + 16 * js + 4 * g;
          Frag16<E> A;
          ld4(A, sDO + off);
          rQs[rt][c] = mma16(rQs[rt][c], A, BS);
          ld4(A, sDU + off);
          rW[rt][c] = mma16(rW[rt][c], A, BS);
          ld4(A, sU + off);
          rKb[rt][c] = mma16(rKb[rt][c], A, BD);
        }
      }
    }
    // dP += dO U^T and dT += dU V^T on this wave's lower tiles
#pragma unroll
    for (int x = 0; x < MAXLT; ++x) {
      const int idx = wv + NW * x;
      if (idx < NLT) {
        int a, b;
        lower_tile(idx, a, b);
#pragma unroll
        for (int js = 0; js < JB / 16; ++js) {
          const int offa = (16 * a + l16) * PJ + 16 * js + 4 * g;
          const int offb = (16 * b + l16) * PJ + 16 * js + 4 * g;
          Frag16<E> A, B;
          ld4(A, sDO + offa);
          ld4(B, sU + offb);
          rdP[x] = mma16(rdP[x], A, B);
          ld4(A, sDU + offa);
          ld4(B, sV + offb);
          rdT[x] = mma16(rdT[x], A, B);
        }
      }
    }
    // dV = T^T dU for these columns: tile (token tile st, column tile jt);
    // T[t][s] = M[t][s] beta_s is zero for t < s.  One tile per wave, stored
    // through a view of the chunk's rows (rows past the end are dropped).
    constexpr int NDV = NT * (JB / 16);
    static_assert(NDV <= NW, "at most one dV tile per wave");
    if (NDV == NW || wv < NDV) {
      const int ti = wv;
      const int st = ti / (JB / 16), jt = ti % (JB / 16);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int kb = st; kb < NT; ++kb) {
        Frag16<float> A, B;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * kb + 4 * g + e;
          A.v[e] = sM[t * PC + 16 * st + l16];
          B.v[e] = to_f32(sDU[t * PJ + 16 * jt + l16]);
        }
        acc = mma16(acc, A, B);
      }
      // scaled by beta per token, then transposed on the matrix cores (exact)
      // so that a lane stores four consecutive columns of one token
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] *= sBeta[16 * st + 4 * g + e];
      Frag16<E> fr;
      frag16_from_acc(fr, acc);
      const f32x4 tr = mma16((f32x4){0.f, 0.f, 0.f, 0.f}, fr, id16);
      const Rsrc rdv = make_rsrc(gdv + t0 * rs, rows_bytes);
      const uint32_t off = (uint32_t)(((16 * st + l16) * rs + hoff + j0 + 16 * jt + 4 * g) * ES);
      if constexpr (ES == 2) {
        const bf16x4 b = (bf16x4){(__bf16)tr[0], (__bf16)tr[1], (__bf16)tr[2], (__bf16)tr[3]};
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, b), rdv, (int)off, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, tr), rdv, (int)off, 0, 0);
      }
    }
    __syncthreads();
  }
  // dgamma for this wave's keys (lane l16 of each key tile)
  float dgam[KPW];
#pragma unroll
  for (int c = 0; c < KPW; ++c) {
    float v = gpart[c];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    dgam[c] = v;
  }

  // ---- dW = -dU S^T to LDS, dP (lower) to LDS ----
  float* sDW = sUN;
#pragma unroll
  for (int rt = 0; rt < NT; ++rt)
#pragma unroll
    for (int c = 0; c < KPW; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) sDW[(16 * rt + 4 * g + e) * PK + 16 * (KPW * wv + c) + l16] = -rW[rt][c][e];
#pragma unroll
  for (int x = 0; x < MAXLT; ++x) {
    const int idx = wv + NW * x;
    if (idx < NLT) {
      int a, b;
      lower_tile(idx, a, b);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * a + 4 * g + e, s = 16 * b + l16;
        sDP[t * PC + s] = s <= t ? rdP[x][e] : 0.f;
      }
    }
  }
  __syncthreads();
  // dT += dW Kt^T (Kt = K e^{g}); dbeta_j += sum_r M_rj dT_rj
#pragma unroll
  for (int x = 0; x < MAXLT; ++x) {
    const int idx = wv + NW * x;
    if (idx < NLT) {
      int a, b;
      lower_tile(idx, a, b);
      for (int kb = 0; kb < 8; ++kb) {
        Frag16<float> A, B;
        A.v = *reinterpret_cast<const f32x4*>(sDW + (16 * a + l16) * PK + 16 * kb + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = 16 * b + l16, i = 16 * kb + 4 * g + e;
          B.v[e] = kf(s, i) * __expf(gf(s, i));
        }
        rdT[x] = mma16(rdT[x], A, B);
      }
      float col = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) col += sM[(16 * a + 4 * g + e) * PC + 16 * b + l16] * rdT[x][e];
      col += __shfl_xor(col, 16);
      col += __shfl_xor(col, 32);
      if (g == 0) sDbT[idx * 16 + l16] = col;
    }
  }
  // dKt = T^T dW on this wave's keys: rows s, dW from registers (rows t)
  f32x4 rKt[NT][KPW];
#pragma unroll
  for (int st = 0; st < NT; ++st)
#pragma unroll
    for (int c = 0; c < KPW; ++c) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NT; ++kb) {
        if (kb < st) continue;
        Frag16<float> A, B;
#pragma unroll
        for (int e = 0; e < 4; ++e) A.v[e] = sM[(16 * kb + 4 * g + e) * PC + 16 * st + l16];
        B.v = -rW[kb][c];
        acc = mma16(acc, A, B);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] *= sBeta[16 * st + 4 * g + e];
      rKt[st][c] = acc;
    }
  __syncthreads();  // dW is no longer read
  // ---- dA = strictly-lower(-M^T dM M^T), dM = dT Diag(beta) ----
  float* sDM = sUN;            // dM, later dB
  float* sX = sUN + C * PC;    // X = dM M^T
  for (int i = tid; i < C * PC; i += NTH) sDM[i] = 0.f;
  __syncthreads();
#pragma unroll
  for (int x = 0; x < MAXLT; ++x) {
    const int idx = wv + NW * x;
    if (idx < NLT) {
      int a, b;
      lower_tile(idx, a, b);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * a + 4 * g + e, s = 16 * b + l16;
        sDM[t * PC + s] = s < t ? rdT[x][e] * sBeta[s] : 0.f;
      }
    }
  }
  __syncthreads();
  // X[m][c] = sum_j dM[m][j] M[c][j], j <= c (lower tiles suffice)
  for (int idx = wv; idx < NLT; idx += NW) {
    int a, b;
    lower_tile(idx, a, b);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int jb = 0; jb <= b; ++jb) {
      Frag16<float> A, B;
      A.v = *reinterpret_cast<const f32x4*>(sDM + (16 * a + l16) * PC + 16 * jb + 4 * g);
      B.v = *reinterpret_cast<const f32x4*>(sM + (16 * b + l16) * PC + 16 * jb + 4 * g);
      acc = mma16(acc, A, B);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) sX[(16 * a + 4 * g + e) * PC + 16 * b + l16] = acc[e];
  }
  __syncthreads();
  // dA[r][c] = -sum_{m >= r} M[m][r] X[m][c]; dB = Diag(beta) dA into sDM;
  // dbeta_r += sum_c dA[r][c] B[r][c]
  f32x4 rdB[MAXLT];
#pragma unroll
  for (int x = 0; x < MAXLT; ++x) {
    const int idx = wv + NW * x;
    rdB[x] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (idx < NLT) {
      int a, b;
      lower_tile(idx, a, b);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int mb = a; mb < NT; ++mb) {
        Frag16<float> A, B;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 16 * mb + 4 * g + e;
          A.v[e] = sM[m * PC + 16 * a + l16];
          B.v[e] = sX[m * PC + 16 * b + l16];
        }
        acc = mma16(acc, A, B);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * a + 4 * g + e, c = 16 * b + l16;
        const float da = c < r ? -acc[e] : 0.f;
        rdB[x][e] = sBeta[r] * da;
        float v = da * sB[r * PC + c];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        if (l16 == 0) sDbB[idx * 16 + 4 * g + e] = v;
      }
    }
  }
  __syncthreads();  // every wave is past reading dM and X
#pragma unroll
  for (int x = 0; x < MAXLT; ++x) {
    const int idx = wv + NW * x;
    if (idx < NLT) {
      int a, b;
      lower_tile(idx, a, b);
#pragma unroll
      for (int e = 0; e < 4; ++e) sDM[(16 * a + 4 * g + e) * PC + 16 * b + l16] = rdB[x][e];
    }
  }
  __syncthreads();
  const float* sDB = sDM;

  // ---- per-token gradients of this wave's keys, one token tile rt at a time:
  // row side YB = dB Kh_rt, YP = dP Kh_rt over tokens s <= tile rt; column side
  // Z = dB^T K_rt + dP^T Q_rt over tokens t >= tile rt (both referenced to rho_rt)
  f32x4 odq[NT][KPW], odk[NT][KPW], odg[NT][KPW];
  float dGp[KPW];
#pragma unroll
  for (int c = 0; c < KPW; ++c) dGp[c] = 0.f;
#pragma unroll
  for (int rt = 0; rt < NT; ++rt)
#pragma unroll
    for (int c = 0; c < KPW; ++c) {
      const int i = 16 * (KPW * wv + c) + l16;
      const float Gi = Gc(i), r = rho(rt, i);
      f32x4 yb = {0.f, 0.f, 0.f, 0.f}, yp = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sb = 0; sb < NT; ++sb) {
        if (sb > rt) continue;
        Frag16<float> AB, AP, B;
        AB.v = *reinterpret_cast<const f32x4*>(sDB + (16 * rt + l16) * PC + 16 * sb + 4 * g);
        AP.v = *reinterpret_cast<const f32x4*>(sDP + (16 * rt + l16) * PC + 16 * sb + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = 16 * sb + 4 * g + e;
          B.v[e] = kf(s, i) * __expf(r - gf(s, i));
        }
        yb = mma16(yb, AB, B);
        yp = mma16(yp, AP, B);
      }
#pragma unroll
      for (int tb = 0; tb < NT; ++tb) {
        if (tb < rt) continue;
        Frag16<float> AB, AP, BK, BQ;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * tb + 4 * g + e;
          AB.v[e] = sDB[t * PC + 16 * rt + l16];
          AP.v[e] = sDP[t * PC + 16 * rt + l16];
          const float f = __expf(gf(t, i) - r);
          BK.v[e] = kf(t, i) * f;
          BQ.v[e] = qf(t, i) * f;
        }
        z = mma16(z, AB, BK);
        z = mma16(z, AP, BQ);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * rt + 4 * g + e;
        const float gi = gf(t, i), kv = kf(t, i), qv = qf(t, i);
        const float eg = __expf(gi), eb = __expf(Gi - gi), ra = __expf(gi - r), rb = __expf(r - gi);
        const float dQs = rQs[rt][c][e], dKt = rKt[rt][c][e], dKb = rKb[rt][c][e];
        odq[rt][c][e] = dQs * eg + yp[e] * ra;
        odk[rt][c][e] = dKt * eg + dKb * eb + yb[e] * ra + z[e] * rb;
        odg[rt][c][e] = dQs * (qv * eg) + dKt * (kv * eg) - dKb * (kv * eb) + (kv * ra) * yb[e] +
                        (qv * ra) * yp[e] - (kv * rb) * z[e];
        dGp[c] += dKb * (kv * eb);
      }
    }
  // dlog_alpha_t = sum_{t' >= t} dg_t' + dG, in registers: a lane holds the
  // tokens 16 rt + 4 g + e of its channel; the sums of its four-token groups
  // are exchanged across the lane groups g, then each token adds the groups
  // after it and its own group's tail.  Tokens past the end carry dg = 0
  // (their k and q are zero).  Stored straight from registers: 16 lanes
  // write one token's 16 channels (64 bytes).
#pragma unroll
  for (int c = 0; c < KPW; ++c) {
    float v = dGp[c];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    const int i = 16 * (KPW * wv + c) + l16;
    const float dGi = v + dgam[c] * __expf(Gc(i));
    float after[NT], tot[NT];  // groups g' > g of tile rt; all four groups of tile rt
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      const float bs = (odg[rt][c][0] + odg[rt][c][1]) + (odg[rt][c][2] + odg[rt][c][3]);
      after[rt] = 0.f;
      tot[rt] = 0.f;
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const float bg = __shfl(bs, l16 + 16 * gg);
        tot[rt] += bg;
        if (gg > g) after[rt] += bg;
      }
    }
    float later = dGi;  // dG plus every tile after rt
#pragma unroll
    for (int rt = NT - 1; rt >= 0; --rt) {
      float run = later + after[rt];
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        run += odg[rt][c][e];
        const int t = 16 * rt + 4 * g + e;
        if (t < nv) p.dlog_alpha[(t0 + t) * rs + hoff + i] = run;
      }
      later += tot[rt];
    }
  }
  __syncthreads();  // k and q are no longer read: their LDS takes dq and dk
  E* oQ = sK;
  E* oK = sQ;
#pragma unroll
  for (int rt = 0; rt < NT; ++rt)
#pragma unroll
    for (int c = 0; c < KPW; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * rt + 4 * g + e, i = 16 * (KPW * wv + c) + l16;
        oQ[t * PK + i] = from_f32<E>(odq[rt][c][e]);
        oK[t * PK + i] = from_f32<E>(odk[rt][c][e]);
      }
  __syncthreads();
  E* gdq = static_cast<E*>(p.dq);
  E* gdk = static_cast<E*>(p.dk);
  for (int i = tid; i < nv * (D / PER); i += NTH) {
    const int t = i / (D / PER), c = (i % (D / PER)) * PER;
    *reinterpret_cast<u32x4*>(gdq + (t0 + t) * rs + hoff + c) = *reinterpret_cast<const u32x4*>(oQ + t * PK + c);
    *reinterpret_cast<u32x4*>(gdk + (t0 + t) * rs + hoff + c) = *reinterpret_cast<const u32x4*>(oK + t * PK + c);
  }
  // dbeta_s: the T-term parts of the tiles in column tile s / 16 (row tiles
  // s / 16 .. NT - 1), then the B-term parts of the tiles in row tile s / 16
  if (tid < nv) {
    const int st = tid >> 4, sl = tid & 15;
    float db = 0.f;
    for (int a = st; a < NT; ++a) db += sDbT[(a * (a + 1) / 2 + st) * 16 + sl];
    for (int b = 0; b <= st; ++b) db += sDbB[(st * (st + 1) / 2 + b) * 16 + sl];
    p.dbeta[(t0 + tid) * H + h] = db;
  }
}

template <typename Kern>
hipError_t launch_lds(Kern fn, unsigned grid, unsigned block, size_t lds, const BwdArgs& a, hipStream_t stream) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(block), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)((size_t)a.slots * a.num_heads);
  if (a.bf16)
    return launch_lds(bwd_prep_kernel<__bf16, 64>, grid, 256, PrepBwdLayout<__bf16, 64>::BYTES, a, stream);
  return launch_lds(bwd_prep_kernel<float, 32>, grid, 256, PrepBwdLayout<float, 32>::BYTES, a, stream);
}

hipError_t launch_bwd_carry(const BwdArgs& a, hipStream_t stream) {
  const int units = a.num_seqs * a.num_heads;
  const unsigned grid = (unsigned)(8 * 2 * ((units + 7) / 8));
  if (a.bf16)
    return launch_lds(bwd_carry_kernel<__bf16, 64>, grid, 320, CarryBwdLayout<__bf16, 64>::BYTES, a, stream);
  return launch_lds(bwd_carry_kernel<float, 32>, grid, 320, CarryBwdLayout<float, 32>::BYTES, a, stream);
}

hipError_t launch_bwd_grad(const BwdArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)((size_t)a.slots * a.num_heads);
  constexpr int NW = 8;  // one 16-key tile per wave
  if (a.bf16)
    return launch_lds(bwd_grad_kernel<__bf16, 64, NW>, grid, 64 * NW, GradLayout<__bf16, 64>::BYTES, a, stream);
  return launch_lds(bwd_grad_kernel<float, 32, NW>, grid, 64 * NW, GradLayout<float, 32>::BYTES, a, stream);
}

}  // namespace kda
