// kda_chunk_util.h — LDS layout and per-thread helpers shared by the chunked
// prefill kernels (the token-parallel prep kernel and the state-carry kernel).
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Raw buffer views: out-of-range offsets read zero and drop writes.
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// `bytes` bytes at p (word 3: the raw 32-bit access format).
__device__ __forceinline__ Rsrc make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ void buf_st16(u32x4 v, Rsrc r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void buf_st8(u32x2 v, Rsrc r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void buf_st4(float v, Rsrc r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)voff, (int)soff, 0);
}

// One element of the I/O dtype at byte offset off, as fp32.
__device__ __forceinline__ float buf_ld_elem(Rsrc r, uint32_t off, __bf16*) {
  const unsigned short v = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
  return (float)__builtin_bit_cast(__bf16, v);
}
__device__ __forceinline__ float buf_ld_elem(Rsrc r, uint32_t off, float*) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

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
  // channel-major [D][C] / [DV][C] tiles and the [C][C] tiles; rows stay
  // 16-byte aligned for the 16-byte operand reads
  static constexpr int LDT = C + PAD;
  static constexpr size_t TOK = (size_t)C * LDK * sizeof(E);
  static constexpr size_t CHM = (size_t)D * LDT * sizeof(E);
  static constexpr size_t VTB = (size_t)DV * LDT * sizeof(E);
  static constexpr size_t CCE = (size_t)C * LDT * sizeof(E);
  // Region R, during the Gram products: K_rel | K_inv (hi) | [K_inv lo] | Q_rel (hi) | [Q_rel lo].
  static constexpr size_t S_KR = 0;
  static constexpr size_t S_KIH = TOK;
  static constexpr size_t S_KIL = 2 * TOK;
  static constexpr size_t S_QRH = (SPLIT ? 3 : 2) * TOK;
  static constexpr size_t S_QRL = 4 * TOK;
  static constexpr size_t R_BYTES = (SPLIT ? 5 : 3) * TOK;
  // After them, [0, S_QRH) holds P | M | W, and the Q_rel slot is
  // turned into Qt = Q (.) e^{g} in place.  M holds the blocks of the
  // triangular solve: -A_ab below the diagonal, (I + A_aa)^{-1} on it.
  static constexpr size_t R_P = 0;
  static constexpr size_t R_M = al16(CCE);
  static constexpr size_t R_W = R_M + al16(CCE);
  static_assert(R_W + TOK <= S_QRH, "post-Gram tiles overflow their region");
  static constexpr size_t O_KTT = R_BYTES;
  static constexpr size_t O_KBT = O_KTT + CHM;
  static constexpr size_t O_VT = O_KBT + CHM;
  static constexpr size_t O_TOT = al16(O_VT + VTB);                 // f32 [4][D] per-wave decay totals
  static constexpr size_t O_EF = O_TOT + (size_t)4 * D * 4;          // f32 [NOFF][D]
  static constexpr size_t O_ERA = O_EF + (size_t)(NOFF > 0 ? NOFF : 1) * D * 4;  // f32 [NT][D]
  static constexpr size_t O_GAM = O_ERA + (size_t)NT * D * 4;        // f32 [D]
  static constexpr size_t O_BETA = O_GAM + (size_t)D * 4;            // f32 [C]
  static constexpr size_t O_SS = O_BETA + (size_t)C * 4;             // f32 [4][C]
  // fp32 diagonal 16x16 blocks of A (outside region R, so each wave can solve
  // its own block before the others finish reading the Gram operands)
  static constexpr int AST = 16;
  static constexpr size_t O_AD = O_SS + (size_t)4 * C * 4;           // f32 [NT][16][AST]
  static constexpr size_t BASE_BYTES = O_AD + (size_t)NT * 16 * AST * 4;
  // Qt gets its own tile (written straight from fp32 in the operand stage)
  // when it fits; otherwise it is formed in place over Q_rel after the Gram.
  static constexpr bool QT_OWN = BASE_BYTES + TOK <= 160 * 1024;
  static constexpr size_t O_QT = BASE_BYTES;
  static constexpr size_t BYTES = BASE_BYTES + (QT_OWN ? TOK : 0);
};

// Strictly-lower pairs (a, b < a) in the order (1,0) (2,0) (2,1) (3,0) ...
__device__ __forceinline__ int off_a(int q) { return q < 1 ? 1 : q < 3 ? 2 : 3; }
__device__ __forceinline__ int off_b(int q) { const int a = off_a(q); return q - a * (a - 1) / 2; }
__device__ __forceinline__ int off_idx(int a, int b) { return a * (a - 1) / 2 + b; }

// Element offset of (row, token) in a channel-major [rows][C] tile.  Tokens
// are grouped in 8-token units whose order within a row is XOR-permuted by
// row / 8: the operand stage stores 16 lanes on rows 8 apart at once, which
// would otherwise all land on the same LDS banks.  Every access of up to 4
// aligned tokens stays inside one unit.
template <int C, int LDT>
__device__ __forceinline__ int cm_off(int row, int tok) {
  constexpr int NU = C / 8;
  return row * LDT + ((((tok >> 3) ^ (row >> 3)) & (NU - 1)) << 3) + (tok & 7);
}

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

// 8 consecutive channels of one row as fp32 (16-byte aligned for bf16, 32 for fp32).
__device__ __forceinline__ void ld8(float* x, const __bf16* p) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)v[j];
}
__device__ __forceinline__ void ld8(float* x, const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = a[j];
    x[j + 4] = b[j];
  }
}
__device__ __forceinline__ void st8(__bf16* p, const float* x) {
  Frag<__bf16> f;
  frag_from_f32(f, x);
  st_frag(p, f);
}
__device__ __forceinline__ void st8(float* p, const float* x) {
  Frag<float> f;
  frag_from_f32(f, x);
  st_frag(p, f);
}
// 8 values and their bf16 residuals (x - hi); plain copy for fp32 operands.
__device__ __forceinline__ void st8_split(__bf16* phi, __bf16* plo, const float* x) {
  Frag<__bf16> hi, lo;
  frag_split(hi, lo, x);
  st_frag(phi, hi);
  st_frag(plo, lo);
}
__device__ __forceinline__ void st8_split(float* phi, float*, const float* x) { st8(phi, x); }
// N consecutive elements (N = 1, 2 or 4) of a channel-major row.
template <int N>
__device__ __forceinline__ void stN(__bf16* p, const float* x) {
  if constexpr (N == 1) {
    p[0] = (__bf16)x[0];
  } else if constexpr (N == 2) {
    *reinterpret_cast<uint32_t*>(p) = __builtin_bit_cast(uint32_t, (bf16x2){(__bf16)x[0], (__bf16)x[1]});
  } else {
    *reinterpret_cast<bf16x4*>(p) = (bf16x4){(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
  }
}
template <int N>
__device__ __forceinline__ void stN(float* p, const float* x) {
  if constexpr (N == 1) {
    p[0] = x[0];
  } else if constexpr (N == 2) {
    *reinterpret_cast<f32x2*>(p) = (f32x2){x[0], x[1]};
  } else {
    *reinterpret_cast<f32x4*>(p) = (f32x4){x[0], x[1], x[2], x[3]};
  }
}

// Raw 8-element row pieces as loaded from global memory.  A chunk's inputs are
// loaded into these while the previous chunk is still in its carried stage,
// and only converted (and masked past the sequence end) when the chunk starts.
template <typename T>
struct Raw8;
template <>
struct Raw8<__bf16> {
  bf16x8 v;
};
template <>
struct Raw8<float> {
  f32x4 a, b;
};
__device__ __forceinline__ void ld_raw8(Raw8<__bf16>& r, const __bf16* p) {
  r.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void ld_raw8(Raw8<float>& r, const float* p) {
  r.a = *reinterpret_cast<const f32x4*>(p);
  r.b = *reinterpret_cast<const f32x4*>(p + 4);
}
__device__ __forceinline__ void cvt_raw8(float* x, const Raw8<__bf16>& r) {
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)r.v[j];
}
__device__ __forceinline__ void cvt_raw8(float* x, const Raw8<float>& r) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = r.a[j];
    x[j + 4] = r.b[j];
  }
}

// Rows r0 .. r0+N-1 as fp32, zero at or past nv (the raw loads read row nv-1 there).
template <typename T, int N>
__device__ __forceinline__ void rows_from_raw(float (*dst)[8], const Raw8<T>* raw, int r0, int nv, bool full) {
#pragma unroll
  for (int i = 0; i < N; ++i) cvt_raw8(dst[i], raw[i]);
  if (!full) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (r0 + i >= nv)
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[i][j] = 0.f;
  }
}

// Prologue for rows r0 .. r0+N-1, 8 channels, from raw rows r0-3 .. r0+N-1:
// causal depthwise conv (4 taps; zero history before the sequence start,
// chunk row `lo`), SiLU, then L2 normalisation over the 128 channels of the
// head, which are spread over the 16 lanes of this lane's group.
template <typename T, int N>
__device__ __forceinline__ void prologue_from_raw(float (*dst)[8], const Raw8<T>* raw, int r0, int nv, int lo,
                                                  const float (*w)[4], float eps) {
  float x[N + 3][8];
#pragma unroll
  for (int i = 0; i < N + 3; ++i) {
    const int row = r0 - 3 + i;
    cvt_raw8(x[i], raw[i]);
    if (row < lo || row >= nv)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[i][j] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float c = w[j][0] * x[i][j] + w[j][1] * x[i + 1][j] + w[j][2] * x[i + 2][j] + w[j][3] * x[i + 3][j];
      const float sv = c * sigmoidf_fast(c);
      dst[i][j] = sv;
      ss += sv * sv;
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) ss += __shfl_xor(ss, m);
    const float inv = rsqrtf(ss + eps);
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[i][j] *= inv;
  }
}

}  // namespace kda
