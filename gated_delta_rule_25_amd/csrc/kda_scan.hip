// kda_scan.hip — the segmented form of the chunked prefill.
//
// The recurrence is affine in the state: over a segment j of a sequence,
//   S_out = M_j S_in + B_j,
// where B_j is what the segment produces from a zero state and M_j (128 x 128
// over the key dimension) is what it produces from the identity with V = 0
// (each state column evolves on its own, so the identity's columns trace M_j).
// "Kimi K3 架构、训练与系统全景解析", section 7.1 (in-device context
// parallelism), splits long sequences this way so that segments run in
// parallel; the incoming states then follow from a sequential composition of
// the pairs, and a last pass writes the outputs from them.
//
// This file holds the two small kernels of that form:
//   segment_table_kernel  per-sequence segment counts, their exclusive prefix
//                         sum and the (sequence, segment) work list;
//   scan_kernel           one workgroup per (sequence, head) composes the
//                         pairs in order: S_in(j) overwrites B_j in place and
//                         the state after the last segment is the final state.
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// One workgroup of 1024 threads; sequences are taken 1024 at a time with a
// block-wide inclusive scan of the segment counts.  Writes are clamped to
// `cap` entries so that inconsistent cu_seqlens cannot write out of bounds.
__global__ __launch_bounds__(1024) void segment_table_kernel(const int32_t* __restrict__ cu, int N,
                                                              int64_t total_tokens, int seg_len, int cap,
                                                              int32_t* __restrict__ seq_first,
                                                              int32_t* __restrict__ seg_list,
                                                              int32_t* __restrict__ seg_count) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  int carry = 0;
  for (int base = 0; base < N; base += 1024) {
    const int n = base + tid;
    int G = 0;
    if (n < N) {
      const int64_t L = cu ? (int64_t)cu[n + 1] - (int64_t)cu[n] : total_tokens;
      G = L > 0 ? (int)((L + seg_len - 1) / seg_len) : 0;
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
      seq_first[n] = first;
      for (int s = 0; s < cnt; ++s) {
        seg_list[2 * (first + s)] = n;
        seg_list[2 * (first + s) + 1] = s;
      }
    }
    carry = min(carry + part[1023], cap);
    __syncthreads();  // part[] is rewritten by the next round
  }
  if (tid == 0) {
    seq_first[N] = carry;
    *seg_count = carry;
  }
}

hipError_t launch_segment_table(const int32_t* cu, int num_seqs, int64_t total_tokens, int seg_len, int cap,
                                int32_t* seq_first, int32_t* seg_list, int32_t* seg_count, hipStream_t stream) {
  hipLaunchKernelGGL(segment_table_kernel, dim3(1), dim3(1024), 0, stream, cu, num_seqs, total_tokens, seg_len,
                     cap, seq_first, seg_list, seg_count);
  return hipGetLastError();
}

// One workgroup (4 waves) per (sequence, head).  Wave w keeps state columns
// 32w .. 32w+31 in the accumulator layout of the 16x16 fp32 MFMA tile (lane
// holds rows 4g..4g+3 of column l % 16 of each tile), which is also the B
// operand layout of a 16-deep fp32 step, so M_j S runs straight from registers
// with M_j read from memory as the A operand.  Each lane reads B_j and writes
// S_in(j) at the same addresses, so the in-place overwrite needs no barrier.
__global__ __launch_bounds__(256) void scan_kernel(const ScanArgs a) {
  const int H = a.num_heads;
  const int n = blockIdx.x / H, h = blockIdx.x % H;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int c0 = 32 * wv;
  const size_t sbase = ((size_t)n * H + h) * (size_t)(D * D);

  f32x4 S[8][2];
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const size_t idx = (size_t)(16 * rt + 4 * g + i) * D + c0 + 16 * ct + l16;
        S[rt][ct][i] = a.init ? a.init[sbase + idx] : 0.f;
      }

  const int j0 = a.seq_first[n], j1 = a.seq_first[n + 1];
  for (int j = j0; j < j1; ++j) {
    float* Bj = a.pairs + ((size_t)j * H + h) * (size_t)(2 * D * D);
    const float* Mj = Bj + D * D;
    f32x4 acc[8][2];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const size_t idx = (size_t)(16 * rt + 4 * g + i) * D + c0 + 16 * ct + l16;
          acc[rt][ct][i] = Bj[idx];
          Bj[idx] = S[rt][ct][i];
        }
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      Frag16<float> mf[8];
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) ld_frag16(mf[kt], Mj + (size_t)(16 * rt + l16) * D + 16 * kt + 4 * g);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
          Frag16<float> sf;
          sf.v = S[kt][ct];
          acc[rt][ct] = mma16(acc[rt][ct], mf[kt], sf);
        }
    }
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) S[rt][ct] = acc[rt][ct];
  }

  if (a.fin) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const size_t idx = (size_t)(16 * rt + 4 * g + i) * D + c0 + 16 * ct + l16;
          a.fin[sbase + idx] = S[rt][ct][i];
        }
  }
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.num_seqs * a.num_heads;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(scan_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kda
