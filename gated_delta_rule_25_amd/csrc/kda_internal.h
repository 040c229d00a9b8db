// kda_internal.h — launch descriptors shared by the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
  float* state;
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;
  const float* beta;
  void* o;
  int num_seqs;
  int num_heads;
  bool bf16;
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;
  const float* beta;
  const float* init;        // [N,H,128,128] or null
  const int32_t* cu;        // [N+1] or null (one sequence of total_tokens)
  int32_t* order;           // workspace: N sequence indices, longest first (null if N == 1)
  void* o;
  float* fin;               // [N,H,128,128] or null
  const float* conv_q_w;    // [H*128,4] or null
  const float* conv_k_w;    // [H*128,4] or null
  const void* gate;         // [T,H,128] or null
  const float* norm_w;      // [128] or null
  float l2_eps;
  float rms_eps;
  int num_seqs;
  int num_heads;
  int64_t total_tokens;
  int units;                // num_seqs * num_heads
  int col_split;            // value-column blocks per (n, h): 1 or 2
  bool bf16;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// Longest-first ordering of the packed sequences (device-side, no host sync).
hipError_t launch_worklist(const int32_t* cu, int num_seqs, int32_t* order, hipStream_t stream);

}  // namespace kda
