// pa_combine.hip -- merge the KV-partition states of each (sequence, query head).
//
// For a sequence with n > 1 partitions, partition p left (m_p, l_p, acc_p) with
// m_p in base-2 units. The merged result is
//
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p acc_p / sum_p w_p l_p,
//
// the max-rescaling combine of page "Paged Attention Kernel Architecture for
// BI-V100", section 2 (the compound attention_partial op), folded over all
// partitions at once; only p < n is read. Sequences with one partition were
// already written by the partition kernel and are skipped here.
//
// Grid (D / 64, H_q, B), 256 threads: lane = one of 64 dims, wave = a stripe of
// the partitions (p = wave, wave + 4, ...); the four stripes meet in LDS.
#include "pa_kernels.h"

namespace pa {
namespace {

__global__ void __launch_bounds__(256) combine_kernel(Params p) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int d = blockIdx.x * 64 + lane;
  const int L = clamped_len(p, b, false);
  const int n = (L + p.part - 1) / p.part;
  if (n <= 1) return;

  const int64_t row = ((int64_t)b * p.Hq + h) * p.pmax;
  const float* mrow = p.ws_m + row;
  const float* lrow = p.ws_l + row;

  float M = -INFINITY;
  for (int i = lane; i < n; i += 64) M = fmaxf(M, mrow[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float mu = M == -INFINITY ? 0.f : M;

  float a = 0.f, ls = 0.f;
  for (int i = w; i < n; i += 4) {
    const float wgt = exp2_fast(mrow[i] - mu);
    ls += wgt * lrow[i];
    a += wgt * p.ws_acc[(row + i) * p.D + d];
  }

  __shared__ float s_a[4][64], s_l[4];
  s_a[w][lane] = a;
  if (lane == 0) s_l[w] = ls;
  __syncthreads();
  if (w == 0) {
    const float tot = s_l[0] + s_l[1] + s_l[2] + s_l[3];
    const float num = s_a[0][lane] + s_a[1][lane] + s_a[2][lane] + s_a[3][lane];
    p.out[((int64_t)b * p.Hq + h) * p.D + d] = tot > 0.f ? num / tot : 0.f;
  }
}

}  // namespace

hipError_t launch_combine(const Params& p, hipStream_t s) {
  dim3 grid(p.D / 64, p.Hq, p.B);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pa
