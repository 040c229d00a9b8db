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

// Multi-token decode from cached token inputs (speculative-decoding replay).
struct ReplayArgs {
  const float* state_in;     // [N,H,128,128] or null (zeros)
  float* state_out;          // [N,H,128,128] or null (not written); may equal state_in
  const void* q;             // [N,L,H,128] (raw rows when the q convolution runs)
  const void* k;
  const void* v;
  const float* log_alpha;    // [N,L,H,128]
  const float* beta;         // [N,L,H]
  const int32_t* num_tokens; // [N] tokens to run, clamped to [0, L]; null = L
  const float* conv_q_w;     // [H*128,4] or null
  const float* conv_k_w;
  void* conv_q_state;        // [N,3,H,128] raw rows before token 0; advanced when state_out is set
  void* conv_k_state;
  const void* gate;          // [N,L,H,128] or null
  const float* norm_w;       // [128] or null
  float l2_eps, rms_eps;
  void* o;                   // [N,L,H,128] or null
  int num_seqs;
  int num_heads;
  int max_tokens;            // L
  bool bf16;
  bool unbounded;            // log_alpha not bounded below: pairwise decay products, no 1 / D
};

// Inputs of the optional precondition checks (kda_debug.hip).
struct CheckArgs {
  int64_t rows;              // (token, head) rows of log_alpha / beta / q / k
  int heads;                 // H
  int tokens_per_seq;        // L for [N, L, H] inputs with counts, else 1
  const int32_t* counts;     // [N] rows t >= counts[n] are not checked, or null
  const float* log_alpha;    // [rows, 128]
  const float* beta;         // [rows]
  const void* q;             // [rows, 128] or null (not checked)
  const void* k;
  const int32_t* cu;         // [N+1] or null
  int num_seqs;
  int64_t total_tokens;
  bool bf16;
  float la_min;              // log_alpha must lie in [la_min, 0] (-inf: any value <= 0)
};

struct ScanArgs {
  float* pairs;             // [seg][H][2][128][128]: B_j (overwritten by S_in(j)), then M_j
  const int32_t* seq_first; // [N+1]: first segment of each sequence (exclusive prefix sum)
  const float* init;        // [N,H,128,128] or null
  float* fin;               // [N,H,128,128] or null
  int num_seqs;
  int num_heads;
};

// ---------------------------------------------------------------------------
// Two-kernel chunked prefill.  The prep kernel turns every (chunk, head) of
// the inputs into a factor block, independently of the state; the carry
// kernel walks each (sequence, head) through its chunks with the state.
// Chunk length C: 64 tokens for bf16 I/O, 32 for fp32 (NT = C / 16 token tiles).
//
// Factor block of one (chunk, head).  Every matrix operand is stored in the
// order in which the carry kernel's matrix-core steps consume it: a fragment
// is 64 lanes x 8 elements of the I/O dtype, lane-linear (FR bytes).  Lane l
// (row l % 16 of a 16-row tile, group g = l / 16) of a fragment over the
// 32-deep contraction step k0 holds the contraction indices
// k0 + 4g + {0..3} (elements 0..3) and k0 + 16 + 4g + {0..3} (elements 4..7).
//   W  [NT][4]    -W (W = T Kt): row tile rt = tokens 16 rt + l % 16,
//                 step ks over the key channels
//   Q  [NT][4]    Qt = Q (.) e^{g}, same order
//   P  [NP]       lower-incl(Qt Kh^T): (rt, kt) for kt <= rt / 2 in that
//                 order; rows tokens of tile rt, step kt over the tokens
//                 (entries above the diagonal are zero)
//   K  [8][C/32]  Kb^T: row tile rt8 = key channels 16 rt8 + l % 16, step kt
//                 over the tokens; each fragment split in halves, [2][64][4]
//                 (elements 0..3 of every lane, then elements 4..7), as the
//                 two token tiles of a step come from different prep waves
//   G  [128]      e^{g_n} per key channel (fp32)
//   U  [NT][8][64][4]  U' = T V in accumulator order: token tile a, column
//                 tile ct, lane, element i = (token 16 a + 4 (lane / 16) + i,
//                 column 16 ct + lane % 16), in the I/O dtype (the carry
//                 rounds U = U' - W S to it for its products anyway)
template <int ES, int C>
struct FactorBlock {
  static constexpr int NT = C / 16;
  static constexpr int KT = C / 32;
  static constexpr uint32_t FR = 512u * ES;
  __host__ __device__ static constexpr int p_before(int rt) {
    int n = 0;
    for (int r = 0; r < rt; ++r) n += (r / 2 + 1 < KT) ? (r / 2 + 1) : KT;
    return n;
  }
  static constexpr int NP = p_before(NT);
  // fragment index of P (rt, kt), kt <= rt / 2
  __host__ __device__ static constexpr int p_frag(int rt, int kt) { return p_before(rt) + kt; }
  static constexpr uint32_t W = 0;
  static constexpr uint32_t Q = W + NT * 4 * FR;
  static constexpr uint32_t P = Q + NT * 4 * FR;
  static constexpr uint32_t K = P + NP * FR;
  static constexpr uint32_t G = K + 8 * KT * FR;
  static constexpr uint32_t U = G + 128 * 4;
  static constexpr uint32_t UT = 256u * ES;  // one U' tile: 64 lanes x 4 elements
  static constexpr uint32_t BYTES = (U + NT * 8 * UT + 255) & ~255u;
};
constexpr int chunk_len(bool bf16) { return bf16 ? 64 : 32; }

// Token range [bos, eos) of sequence n (all T tokens without cu_seqlens),
// clamped into [0, T] with eos >= bos: cu_seqlens outside its preconditions
// then gives wrong results but never addresses a token outside the inputs.
__device__ __forceinline__ void seq_range(const int32_t* cu, int n, int64_t T, int64_t& bos, int64_t& eos) {
  if (!cu) {
    bos = 0;
    eos = T;
    return;
  }
  const int64_t a = cu[n], b = cu[n + 1];
  bos = a < 0 ? 0 : (a > T ? T : a);
  eos = b < bos ? bos : (b > T ? T : b);
}
constexpr size_t factor_block_bytes(bool bf16) {
  return bf16 ? FactorBlock<2, 64>::BYTES : FactorBlock<4, 32>::BYTES;
}

// Factor store of one window: slot s of head h at ((s * H) + h) * block bytes.
// A window holds, for every sequence n, chunks [c0_n, c1_n) in slots
// [seq_first[n], seq_first[n] + c1_n - c0_n); seq_first[N] is the slot count.
struct PrepArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;
  const float* beta;
  const int32_t* cu;
  const float* conv_q_w;
  const float* conv_k_w;
  float l2_eps;
  int num_seqs;
  int num_heads;
  int64_t total_tokens;
  bool bf16;
  const int32_t* seq_first;  // [N+1]
  const int32_t* seq_c0;     // [N]
  int cap;                   // slots the store can hold
  int chunks_per_block;      // consecutive slots per workgroup
  void* factors;
  bool unbounded;            // log_alpha not bounded below: per-position diagonal tiles
};

struct CarryArgs {
  const void* factors;
  const int32_t* cu;
  const int32_t* order;      // sequences longest first, or null (identity)
  const int32_t* seq_first;
  const int32_t* seq_c0;
  const int32_t* seq_c1;
  const float* state_in;     // [N,H,128,128] or null (zero)
  float* state_out;          // [N,H,128,128] or null (not written)
  const void* gate;          // [T,H,128] or null
  const float* norm_w;
  float rms_eps;
  void* o;
  int num_seqs;
  int num_heads;
  int64_t total_tokens;
  int units;                 // num_seqs * num_heads, or (segments bound) * num_heads
  int col_split;             // value-column blocks per work item (pass 1: B blocks then M blocks)
  bool bf16;
  // Segmented form (in-device context parallelism) over the window's chunks.
  // pass 0: one work item per (sequence, head), state_in -> state_out.
  // pass 1: one per (segment, head): blocks [0, col_split/2) run the value
  //   columns from a zero state (B), the others the identity with U' = 0 (M);
  //   the end states go to pairs[seg][h][0 or 1], no outputs are written.
  // pass 2: one per (segment, head): from pairs[seg][h][0] (which the scan
  //   has overwritten with the segment's incoming state), outputs only.
  // pass 3 (states pass of the backward): as pass 0 without outputs; every
  //   chunk's incoming state goes to chunk_states [slot][H][128 x 128] and its
  //   U = U' - W S to chunk_u [slot][H][C x 128], both in the I/O dtype as
  //   16 x 16 tiles (tile16_index).
  // pass 4 (forward for training): pass 0 and pass 3 in one walk, the outputs
  //   and the final state as pass 0, the per-chunk S and U as pass 3.
  int pass;
  void* chunk_states;
  void* chunk_u;
  const int32_t* seg_list;   // [2 * segments]: sequence, segment index within the window's range
  const int32_t* seg_count;  // device: number of segments
  int seg_chunks;            // chunks per segment
  float* pairs;              // [segments][H][2][128][128] fp32
};

// ---------------------------------------------------------------------------
// Backward pass (kda_bwd.hip).  One factor-store window covers every chunk, so
// a slot index is a global chunk index (sequence n owns slots
// [seq_first[n], seq_first[n + 1])).  Per slot and head the workspace holds
// the forward factor block, the chunk's incoming state S and U = U' - W S
// (the carry's states pass), the reverse carry's block below, and the
// gradient dS reaching the chunk's end plus dU = P^T dO + Kb dS (the reverse
// carry); S, U, dS and dU in the I/O dtype as 16 x 16 tiles (tile16_index).
//
// Reverse-carry block of one (chunk, head), in the fragment order of the
// reverse carry's matrix-core steps (fragments as in FactorBlock):
//   KB [NT][4]    Kb = K (.) e^{g_n - g}: row tile = 16 tokens, step over keys
//   WT [8][KT]    -W^T: row tile = 16 key channels, step over tokens
//   G  [128]      e^{g_n} (fp32, in a 1 KiB piece)
//   X  [NT][8][64][4]  P^T dO in accumulator order (token tile, column tile)
//   Y  [8][8][64][4]   Qt^T dO in accumulator order (key tile, column tile)
// X and Y in the I/O dtype.  KB, WT and G are contiguous, so one copy moves
// them into LDS.
template <int ES, int C>
struct DCarryBlock {
  static constexpr int NT = C / 16;
  static constexpr int KT = C / 32;
  static constexpr uint32_t FR = 512u * ES;
  static constexpr uint32_t TILE = 256u * ES;  // one accumulator-order tile
  static constexpr uint32_t KB = 0;
  static constexpr uint32_t WT = KB + NT * 4 * FR;
  static constexpr uint32_t G = WT + 8 * KT * FR;
  static constexpr uint32_t X = G + 1024;
  static constexpr uint32_t Y = X + NT * 8 * TILE;
  static constexpr uint32_t BYTES = (Y + 64 * TILE + 255) & ~255u;
  static constexpr uint32_t LDS_PART = X;  // the part the loader copies
};
constexpr size_t dcarry_block_bytes(bool bf16) {
  return bf16 ? DCarryBlock<2, 64>::BYTES : DCarryBlock<4, 32>::BYTES;
}

// Storage of an [R][128] matrix as row-major 16 x 16 tiles, tiles in row-major
// order: element (r, j) sits at ((r / 16) * 8 + j / 16) * 256 + (r % 16) * 16 + j % 16,
// so the 16 values of a tile row are contiguous and a tile is 256 elements.
__host__ __device__ constexpr size_t tile16_index(int r, int j) {
  return ((size_t)((r >> 4) * 8 + (j >> 4)) << 8) + (size_t)((r & 15) * 16 + (j & 15));
}

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* log_alpha;
  const float* beta;
  const void* d_o;               // [T,H,128] dtype
  const float* d_final_state;    // [N,H,128,128] or null (zero)
  const int32_t* cu;
  const int32_t* order;          // longest-first sequences or null
  const int32_t* seq_first;      // [N+1] first slot of each sequence
  int num_seqs;
  int num_heads;
  int64_t total_tokens;
  int slots;                     // slot capacity (grid bound of the per-chunk kernels)
  bool bf16;
  const void* factors;           // forward factor blocks [slot][H]
  void* dblocks;                 // reverse-carry blocks [slot][H]
  // per-chunk matrices in the I/O dtype, 16 x 16 tiles (tile16_index)
  const void* chunk_states;      // [slot][H][128 x 128]: S entering the chunk
  const void* chunk_u;           // [slot][H][C x 128]: U = U' - W S
  void* chunk_ds;                // [slot][H][128 x 128]: dS at the chunk's end
  void* chunk_du;                // [slot][H][C x 128]
  void* dq;                      // [T,H,128] dtype
  void* dk;
  void* dv;
  float* dlog_alpha;             // [T,H,128]
  float* dbeta;                  // [T,H]
  float* d_initial_state;        // [N,H,128,128] or null (not written)
};
hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_carry(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_grad(const BwdArgs& a, hipStream_t stream);

// Window w of nw: sequence n of G_n chunks gets chunks
// [min(w Q_n, G_n), min((w + 1) Q_n, G_n)) with Q_n = ceil(G_n / nw).
hipError_t launch_window_table(const int32_t* cu, int num_seqs, int64_t total_tokens, int chunk, int nw, int w,
                               int cap, int32_t* seq_first, int32_t* seq_c0, int32_t* seq_c1, hipStream_t stream);
// Segments of the window: sequence n's chunks [seq_c0[n], seq_c1[n]) in runs
// of seg_chunks; seg_first [N+1] is the exclusive prefix sum of the counts and
// seg_list lists (n, j); at most cap entries.
hipError_t launch_window_segments(const int32_t* seq_c0, const int32_t* seq_c1, int num_seqs, int seg_chunks,
                                  int cap, int32_t* seg_first, int32_t* seg_list, int32_t* seg_count,
                                  hipStream_t stream);
hipError_t launch_prep(const PrepArgs& a, hipStream_t stream);
hipError_t launch_carry(const CarryArgs& a, hipStream_t stream);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
constexpr int kReplayMaxTokens = 16;
hipError_t launch_replay(const ReplayArgs& a, hipStream_t stream);
// Runs the checks on `stream`, waits, and returns the KDA_CHECK_* bits that failed.
hipError_t run_checks(const CheckArgs& a, hipStream_t stream, uint32_t* flags);
// Longest-first ordering of the packed sequences (device-side, no host sync).
hipError_t launch_worklist(const int32_t* cu, int num_seqs, int32_t* order, hipStream_t stream);
// Segment table: per-sequence segment counts, their exclusive prefix sum
// (seq_first, [N+1]), the (sequence, segment) list and the total count.
// At most `cap` segments are listed.
hipError_t launch_scan(const ScanArgs& a, hipStream_t stream);

}  // namespace kda
