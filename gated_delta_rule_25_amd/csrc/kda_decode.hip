// kda_decode.hip — single-token KDA step for many independent sequences.
//
// Per (sequence n, head h) the 128x128 fp32 state S is advanced in place by
// one token ("Kimi K3 架构、训练与系统全景解析", section 4.2.2 update, 4.2.7
// in-place decode).  Expanding the update with a = exp(log_alpha):
//     x_j = sum_i a_i k_i S[i][j]          (old prediction at key k)
//     u_j = beta (v_j - x_j)
//     S[i][j] <- a_i S[i][j] + k_i u_j
//     o_j = sum_i q_i S_new[i][j] = sum_i a_i q_i S[i][j] + (k . q) u_j
// so one pass reads S once (both column sums x and y = sum_i a_i q_i S[i][j]
// come from the same registers) and writes it once.  The kernel is bound by
// HBM: 2 x 64 KiB of state per (n, h) against ~7 x 128^2 flops.
//
// Launch: one 256-thread workgroup per (n, h).  Thread t owns columns
// 4*(t % 32) .. +3 and rows 16*(t / 32) .. +15 of the state, loaded with
// 16-byte non-temporal loads (each 32-lane half-wave streams whole 512-byte
// rows).  Column sums are reduced across the 8 row groups with one
// cross-lane swap and one LDS exchange.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <typename E>
__global__ __launch_bounds__(256) void decode_kernel(float* __restrict__ state, const E* __restrict__ q,
                                                     const E* __restrict__ k, const E* __restrict__ v,
                                                     const float* __restrict__ log_alpha,
                                                     const float* __restrict__ beta, E* __restrict__ o) {
  const int64_t u = blockIdx.x;  // (n, h) pair, n * H + h
  const int t = threadIdx.x;
  const int cg = t & 31;   // column group: columns 4cg .. 4cg+3
  const int rg = t >> 5;   // row group: rows 16rg .. 16rg+15
  const int wv = t >> 6;

  __shared__ float s_a[D], s_ak[D], s_aq[D], s_k[D];
  __shared__ float s_part[4][2][D];
  __shared__ float s_kq[2];

  float* S = state + u * (D * D);
  f32x4 st[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    st[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (16 * rg + i) * D + 4 * cg));

  const f32x4 vv = (f32x4){to_f32(v[u * D + 4 * cg + 0]), to_f32(v[u * D + 4 * cg + 1]),
                           to_f32(v[u * D + 4 * cg + 2]), to_f32(v[u * D + 4 * cg + 3])};
  const float b = beta[u];

  if (t < D) {
    const float a = __expf(log_alpha[u * D + t]);
    const float kk = to_f32(k[u * D + t]);
    const float qq = to_f32(q[u * D + t]);
    s_a[t] = a;
    s_ak[t] = a * kk;
    s_aq[t] = a * qq;
    s_k[t] = kk;
    float p = kk * qq;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) p += __shfl_xor(p, m);
    if ((t & 63) == 0) s_kq[t >> 6] = p;
  }
  __syncthreads();

  f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 16 * rg + i;
    x += s_ak[r] * st[i];
    y += s_aq[r] * st[i];
  }
  // combine the two row groups of this wave (lanes t and t ^ 32)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] += __shfl_xor(x[j], 32);
    y[j] += __shfl_xor(y[j], 32);
  }
  if ((t & 32) == 0) {
    *reinterpret_cast<f32x4*>(&s_part[wv][0][4 * cg]) = x;
    *reinterpret_cast<f32x4*>(&s_part[wv][1][4 * cg]) = y;
  }
  __syncthreads();
  x = *reinterpret_cast<const f32x4*>(&s_part[0][0][4 * cg]);
  y = *reinterpret_cast<const f32x4*>(&s_part[0][1][4 * cg]);
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    x += *reinterpret_cast<const f32x4*>(&s_part[w][0][4 * cg]);
    y += *reinterpret_cast<const f32x4*>(&s_part[w][1][4 * cg]);
  }
  const float kq = s_kq[0] + s_kq[1];
  const f32x4 uu = b * (vv - x);

#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 16 * rg + i;
    const f32x4 ns = s_a[r] * st[i] + s_k[r] * uu;
    __builtin_nontemporal_store(ns, reinterpret_cast<f32x4*>(S + r * D + 4 * cg));
  }
  if (rg == 0) {
    const f32x4 oo = y + kq * uu;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[u * D + 4 * cg + j] = from_f32<E>(oo[j]);
  }
}

template <typename E>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const int64_t units = (int64_t)a.num_seqs * a.num_heads;
  hipLaunchKernelGGL(decode_kernel<E>, dim3((unsigned)units), dim3(256), 0, stream, a.state,
                     static_cast<const E*>(a.q), static_cast<const E*>(a.k), static_cast<const E*>(a.v),
                     a.log_alpha, a.beta, static_cast<E*>(a.o));
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.bf16) return launch_decode_t<__bf16>(a, stream);
  return launch_decode_t<float>(a, stream);
}

}  // namespace kda
