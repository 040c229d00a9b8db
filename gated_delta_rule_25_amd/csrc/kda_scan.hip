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
//   scan_kernel  one workgroup per (sequence, head, 16-column tile)
//                composes the pairs in order: S_in(j) overwrites B_j in place
//                and the state after the last segment is the final state.
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// One workgroup (4 waves) per (sequence n, head h, 16-column tile ct): the
// state's columns evolve independently, so the eight column tiles of a head
// run side by side.  Wave w owns row tiles 2w and 2w + 1 of the tile, in the
// accumulator layout of the 16x16 fp32 MFMA tile (lane holds rows 4g..4g+3
// of column l % 16), which is also the B operand layout of a 16-deep fp32
// step; the whole 128 x 16 tile, the B operand of every wave's M_j S, is
// exchanged through LDS after each step.  The next segment's M_j rows and
// B_j entries are fetched while the current step runs.  Each lane reads B_j
// and writes S_in(j) at the same addresses, so the in-place overwrite needs
// no barrier.
__global__ __launch_bounds__(256) void scan_kernel(const ScanArgs a) {
  const int H = a.num_heads;
  const int ct = blockIdx.x & 7;
  const int nh = blockIdx.x >> 3;
  const int n = nh / H, h = nh % H;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int col = 16 * ct + l16;
  const size_t sbase = ((size_t)n * H + h) * (size_t)(D * D);
  __shared__ f32x4 sS[8][64];  // the state tile: [row tile][lane]

  auto row_of = [&](int q, int i) { return 16 * (2 * wv + q) + 4 * g + i; };
  f32x4 mine[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) mine[q][i] = a.init ? a.init[sbase + (size_t)row_of(q, i) * D + col] : 0.f;
#pragma unroll
  for (int q = 0; q < 2; ++q) sS[2 * wv + q][lane] = mine[q];
  __syncthreads();

  const int j0 = a.seq_first[n], j1 = a.seq_first[n + 1];
  // this wave's M_j rows (row tiles 2w, 2w+1 x 8 steps) and B_j entries
  Frag16<float> mf[2][8];
  f32x4 bj[2];
  auto fetch = [&](int j) {
    const float* Bj = a.pairs + ((size_t)j * H + h) * (size_t)(2 * D * D);
    const float* Mj = Bj + D * D;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) ld_frag16(mf[q][kt], Mj + (size_t)(16 * (2 * wv + q) + l16) * D + 16 * kt + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) bj[q][i] = Bj[(size_t)row_of(q, i) * D + col];
    }
  };
  if (j0 < j1) fetch(j0);
  for (int j = j0; j < j1; ++j) {
    float* Bj = a.pairs + ((size_t)j * H + h) * (size_t)(2 * D * D);
    f32x4 acc[2];
    Frag16<float> mcur[2][8];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      acc[q] = bj[q];
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) mcur[q][kt] = mf[q][kt];
#pragma unroll
      for (int i = 0; i < 4; ++i) Bj[(size_t)row_of(q, i) * D + col] = mine[q][i];  // S_in(j)
    }
    if (j + 1 < j1) fetch(j + 1);
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      Frag16<float> sf;
      sf.v = sS[kt][lane];
#pragma unroll
      for (int q = 0; q < 2; ++q) acc[q] = mma16(acc[q], mcur[q][kt], sf);
    }
    __syncthreads();  // every wave has read the tile of step j
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      mine[q] = acc[q];
      sS[2 * wv + q][lane] = acc[q];
    }
    __syncthreads();
  }

  if (a.fin) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.fin[sbase + (size_t)row_of(q, i) * D + col] = mine[q][i];
  }
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.num_seqs * a.num_heads * 8;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(scan_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kda
