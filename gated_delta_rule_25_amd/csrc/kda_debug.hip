// kda_debug.hip — optional precondition checks (environment variable
// KDA_DEBUG_CHECKS).
//
// The entry points document preconditions that the fast path does not check:
// log_alpha in [-5, 0] (the lower-bounded decay with bound -5 of
// "Kimi K3 架构、训练与系统全景解析", sections 2.1 and 4.2.5, which the chunked
// kernels' exponent ranges rely on), or only <= 0 where a call accepts
// unbounded decay, beta in [0, 1], q and k of unit norm per
// (token, head) when no prologue normalises them (the L2-normalised inputs of
// section 4.2.3), and cu_seqlens non-decreasing from 0 to total_tokens.  With
// the checks switched on, a call first runs them on its stream, waits for
// them, and returns KDA_ERR_PRECONDITION instead of launching anything when
// one fails.  The result is a bit mask kept in one device word of this
// module.
#include <algorithm>

#include "kda.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

__device__ unsigned int g_check_flags;

constexpr float kNormTol = 0.02f;  // |(||x||) - 1| allowed for "unit norm" (bf16 rounding is ~0.002)

// One wave per (token, head) row, grid-stride over rows.  Row index
// ((n * L + t) * H + h); with counts, rows t >= count[n] are not checked
// (the kernels do not read them).
template <typename E>
__global__ __launch_bounds__(256) void check_rows_kernel(const CheckArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * 4;
  unsigned int bad = 0;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < a.rows; row += waves) {
    if (a.counts) {
      const int64_t t = (row / a.heads) % a.tokens_per_seq;
      const int64_t n = row / ((int64_t)a.heads * a.tokens_per_seq);
      if (t >= a.counts[n]) continue;
    }
    const float* la = a.log_alpha + row * D;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float x = la[lane + 64 * i];
      if (!(x >= a.la_min && x <= 0.f)) bad |= KDA_CHECK_LOG_ALPHA;
    }
    if (lane == 0) {
      const float b = a.beta[row];
      if (!(b >= 0.f && b <= 1.f)) bad |= KDA_CHECK_BETA;
    }
    const E* vecs[2] = {static_cast<const E*>(a.q), static_cast<const E*>(a.k)};
    const unsigned int bits[2] = {KDA_CHECK_Q_NORM, KDA_CHECK_K_NORM};
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      if (!vecs[v]) continue;
      const E* x = vecs[v] + row * D;
      const float x0 = to_f32(x[lane]), x1 = to_f32(x[lane + 64]);
      float ss = x0 * x0 + x1 * x1;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
      if (lane == 0 && !(fabsf(sqrtf(ss) - 1.f) <= kNormTol)) bad |= bits[v];
    }
  }
  if (bad) atomicOr(&g_check_flags, bad);
}

__global__ __launch_bounds__(256) void check_cu_kernel(const int32_t* cu, int num_seqs, int64_t total_tokens) {
  unsigned int bad = 0;
  for (int n = blockIdx.x * blockDim.x + threadIdx.x; n < num_seqs; n += gridDim.x * blockDim.x) {
    if (cu[n + 1] < cu[n]) bad = KDA_CHECK_CU_SEQLENS;
    if (n == 0 && (cu[0] != 0 || (int64_t)cu[num_seqs] != total_tokens)) bad = KDA_CHECK_CU_SEQLENS;
  }
  if (bad) atomicOr(&g_check_flags, bad);
}

}  // namespace

hipError_t run_checks(const CheckArgs& a, hipStream_t stream, uint32_t* flags) {
  *flags = 0;
  void* dflag = nullptr;
  hipError_t e = hipGetSymbolAddress(&dflag, HIP_SYMBOL(g_check_flags));
  if (e != hipSuccess) return e;
  // (the checks wait on the stream, so they can never be part of a captured graph)
  e = hipMemsetAsync(dflag, 0, sizeof(unsigned int), stream);
  if (e != hipSuccess) return e;
  if (a.rows > 0) {
    const int64_t blocks = std::min<int64_t>((a.rows + 3) / 4, 65536);
    if (a.bf16)
      hipLaunchKernelGGL(check_rows_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(check_rows_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.cu) {
    const int blocks = std::max(1, std::min((a.num_seqs + 255) / 256, 1024));
    hipLaunchKernelGGL(check_cu_kernel, dim3(blocks), dim3(256), 0, stream, a.cu, a.num_seqs, a.total_tokens);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  unsigned int host = 0;
  e = hipMemcpyAsync(&host, dflag, sizeof(host), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  *flags = host;
  return hipSuccess;
}

}  // namespace kda
