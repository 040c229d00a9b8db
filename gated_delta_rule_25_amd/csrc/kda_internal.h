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
  int units;                // work items: num_seqs * num_heads, or segments * num_heads
  int col_split;            // column blocks per work item (see mode)
  bool bf16;
  // Segmented form (in-device context parallelism).  mode 0: plain.  mode 1:
  // per segment, column blocks [0, col_split/2) run the value columns from a
  // zero state (B) and the rest run the identity with V = 0 (M); the final
  // states go to `pairs` [seg][H][2][128][128] (B first, then M) and no
  // outputs are written.  mode 2: per segment, start from `pairs` slot B
  // (the scan overwrites B_j with the segment's incoming state) and write
  // the outputs only.  mode 1 and 2 list their work in seg_list.
  int mode;
  int seg_len;              // tokens per segment (multiple of the chunk)
  const int32_t* seg_list;  // [2 * max segments]: sequence, segment index
  const int32_t* seg_count; // device: number of segments
  float* pairs;
};

struct ScanArgs {
  float* pairs;             // [seg][H][2][128][128]: B_j (overwritten by S_in(j)), then M_j
  const int32_t* seq_first; // [N+1]: first segment of each sequence (exclusive prefix sum)
  const float* init;        // [N,H,128,128] or null
  float* fin;               // [N,H,128,128] or null
  int num_seqs;
  int num_heads;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// Longest-first ordering of the packed sequences (device-side, no host sync).
hipError_t launch_worklist(const int32_t* cu, int num_seqs, int32_t* order, hipStream_t stream);
// Segment table: per-sequence segment counts, their exclusive prefix sum
// (seq_first, [N+1]), the (sequence, segment) list and the total count.
// At most `cap` segments are listed.
hipError_t launch_segment_table(const int32_t* cu, int num_seqs, int64_t total_tokens, int seg_len, int cap,
                                int32_t* seq_first, int32_t* seg_list, int32_t* seg_count, hipStream_t stream);
hipError_t launch_scan(const ScanArgs& a, hipStream_t stream);

}  // namespace kda
