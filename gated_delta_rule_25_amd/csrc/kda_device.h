// kda_device.h — device-side building blocks for the gfx950 KDA kernels.
//
// Matrix-core fragments.  Every contraction uses the 16x16 output tile of the
// CDNA4 MFMA unit with fp32 accumulation:
//   bf16 operands:  v_mfma_f32_16x16x32_bf16   (one instruction per 32-deep step)
//   fp32 operands:  v_mfma_f32_16x16x4_f32     (eight instructions per 32-deep step)
// For both, lane l of a 64-wide wave supplies 8 operand values of row (A) or
// column (B) l % 16 for the lane group g = l / 16, and receives the output
// rows 4g..4g+3 of column l % 16.  Which 8 contraction indices a lane group
// carries is free as long as the A and B operands agree; two index sets are
// used:
//   contiguous:  k0 + 8g + {0..7}
//   d-permuted:  k0 + 4g + {0..3}  and  k0 + 16 + 4g + {0..3}
// The d-permuted set is exactly what a lane holds of two vertically stacked
// output tiles, so an fp32 result tile pair can feed the next contraction as
// a B operand straight from registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;  // d_k = d_v

template <typename E>
struct Frag;

template <>
struct Frag<__bf16> {
  bf16x8 v;
};

template <>
struct Frag<float> {
  f32x4 lo, hi;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename E>
__device__ __forceinline__ E from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// 8 consecutive operand values (contiguous index set); p must be 16-byte aligned.
__device__ __forceinline__ void ld_frag(Frag<__bf16>& f, const __bf16* p) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void ld_frag(Frag<float>& f, const float* p) {
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 4);
}

// d-permuted index set from two separate 4-element pieces (k0 + 4g and k0 + 16 + 4g).
__device__ __forceinline__ void ld_frag_pair(Frag<__bf16>& f, const __bf16* lo, const __bf16* hi) {
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(lo);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(hi);
  f.v = (bf16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void ld_frag_pair(Frag<float>& f, const float* lo, const float* hi) {
  f.lo = *reinterpret_cast<const f32x4*>(lo);
  f.hi = *reinterpret_cast<const f32x4*>(hi);
}

// B operand from two stacked fp32 output tiles held by this lane.
__device__ __forceinline__ void frag_from_acc(Frag<__bf16>& f, f32x4 x0, f32x4 x1) {
  f.v = (bf16x8){(__bf16)x0[0], (__bf16)x0[1], (__bf16)x0[2], (__bf16)x0[3],
                 (__bf16)x1[0], (__bf16)x1[1], (__bf16)x1[2], (__bf16)x1[3]};
}
__device__ __forceinline__ void frag_from_acc(Frag<float>& f, f32x4 x0, f32x4 x1) {
  f.lo = x0;
  f.hi = x1;
}

// Operand from 8 fp32 values.
__device__ __forceinline__ void frag_from_f32(Frag<__bf16>& f, const float* x) {
  f.v = (bf16x8){(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3],
                 (__bf16)x[4], (__bf16)x[5], (__bf16)x[6], (__bf16)x[7]};
}
__device__ __forceinline__ void frag_from_f32(Frag<float>& f, const float* x) {
  f.lo = (f32x4){x[0], x[1], x[2], x[3]};
  f.hi = (f32x4){x[4], x[5], x[6], x[7]};
}

// acc += A * B over one 32-deep contraction step.
__device__ __forceinline__ f32x4 mma(f32x4 acc, const Frag<__bf16>& a, const Frag<__bf16>& b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x4 acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[j], b.lo[j], acc, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[j], b.hi[j], acc, 0, 0, 0);
  return acc;
}

// 1 / (1 + e^-x) with the hardware reciprocal (1 ulp) instead of the IEEE
// division's scale / refine / fix-up sequence, about ten instructions
__device__ __forceinline__ float sigmoidf_fast(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// s_waitcnt operand that lets n vector-memory operations stay outstanding.
__host__ __device__ constexpr int vmcnt_wait(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }

// 2^x with the hardware exp unit (inputs here lie in [-128, 128]; results
// below the normal range flush toward zero, which is the intended limit).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace kda

namespace kda {

// 16-deep contraction steps (v_mfma_f32_16x16x16_bf16 / four v_mfma_f32_16x16x4_f32):
// lane (row or column l % 16, group g) carries contraction indices 4g .. 4g+3,
// which is exactly the row set of one output tile held by that lane.
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <typename E>
struct Frag16;
template <>
struct Frag16<__bf16> {
  bf16x4 v;
};
template <>
struct Frag16<float> {
  f32x4 v;
};

__device__ __forceinline__ void ld_frag16(Frag16<__bf16>& f, const __bf16* p) {
  f.v = *reinterpret_cast<const bf16x4*>(p);
}
__device__ __forceinline__ void ld_frag16(Frag16<float>& f, const float* p) {
  f.v = *reinterpret_cast<const f32x4*>(p);
}
__device__ __forceinline__ void frag16_from_acc(Frag16<__bf16>& f, f32x4 x) {
  f.v = (bf16x4){(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
}
__device__ __forceinline__ void frag16_from_acc(Frag16<float>& f, f32x4 x) { f.v = x; }
__device__ __forceinline__ f32x4 frag16_to_f32(const Frag16<__bf16>& f) {
  return (f32x4){(float)f.v[0], (float)f.v[1], (float)f.v[2], (float)f.v[3]};
}
__device__ __forceinline__ f32x4 frag16_to_f32(const Frag16<float>& f) { return f.v; }

__device__ __forceinline__ f32x4 mma16(f32x4 acc, const Frag16<__bf16>& a, const Frag16<__bf16>& b) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a.v), __builtin_bit_cast(s16x4, b.v),
                                                    acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f32x4 acc, const Frag16<float>& a, const Frag16<float>& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
  return acc;
}

}  // namespace kda
