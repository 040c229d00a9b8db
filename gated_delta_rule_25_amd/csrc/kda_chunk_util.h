// kda_chunk_util.h — raw buffer loads and stores shared by the chunked
// prefill kernels (the token-parallel prep kernel and the state-carry kernel).
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Raw buffer views: out-of-range offsets read zero and drop writes.  The
// stores are the prep kernel's factor-block writes: each block is read once,
// by the carry kernel, long after it is written, so they use the streaming
// (non-temporal) cache policy (measured: 1.5 % off a one-layer prefill, where
// the same policy on the input loads or the output stores costs 5-7 %).
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kStreamStore = 2;  // cache-policy operand: non-temporal
// `bytes` bytes at p (word 3: the raw 32-bit access format).
__device__ __forceinline__ Rsrc make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ void buf_st16(u32x4 v, Rsrc r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, (int)soff, kStreamStore);
}
__device__ __forceinline__ void buf_st8(u32x2 v, Rsrc r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)voff, (int)soff, kStreamStore);
}
__device__ __forceinline__ void buf_st4(float v, Rsrc r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)voff, (int)soff, kStreamStore);
}

// Four consecutive values of E at dst (one 8- or 16-byte store), from fp32.
template <typename E>
__device__ __forceinline__ void store_row4(E* dst, f32x4 x) {
  if constexpr (sizeof(E) == 2)
    *reinterpret_cast<bf16x4*>(dst) = (bf16x4){(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
  else
    *reinterpret_cast<f32x4*>(dst) = x;
}

}  // namespace kda
