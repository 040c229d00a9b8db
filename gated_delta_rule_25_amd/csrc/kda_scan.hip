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
// the pairs, and a last pass writes the outputs from them.  The pairs and the
// outputs come from the carry kernel (passes 1 and 2, kda_chunk.hip); this
// file holds the composition:
//   scan_kernel  one workgroup per (sequence, head) composes the pairs in
//                order: S_in(j) overwrites B_j in place and the state after
//                the last segment is the final state.
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

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
