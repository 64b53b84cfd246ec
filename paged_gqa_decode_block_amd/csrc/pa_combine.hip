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
// Grid (D / 64, H_q, B), 256 threads: thread (stripe s, quad u) owns dims
// 4u .. 4u+3 of a 64-dim slice (float4 loads) and partitions p = s, s + 16, ...;
// the 16 stripes meet in LDS.
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kStripes = 16;

__global__ void __launch_bounds__(256) combine_kernel(Params p) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int u = tid & 15, s = tid >> 4;
  const int d = blockIdx.x * 64 + 4 * u;
  const int L = clamped_len(p, b, false);
  const int n = (L + p.part - 1) / p.part;
  if (n <= 1) return;

  const int64_t row = ((int64_t)b * p.Hq + h) * p.pmax;
  const float* mrow = p.ws_m + row;
  const float* lrow = p.ws_l + row;

  // M = max over all n partitions (every wave computes it)
  float M = -INFINITY;
  for (int i = lane; i < n; i += 64) M = fmaxf(M, mrow[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float mu = M == -INFINITY ? 0.f : M;

  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  float ls = 0.f;
  const float* arow = p.ws_acc + row * p.D + d;
  int i = s;
  for (; i + 3 * kStripes < n; i += 4 * kStripes) {  // four partitions in flight
    float4 x[4];
    float w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = *(const float4*)(arow + (int64_t)(i + k * kStripes) * p.D);
      w[k] = exp2_fast(mrow[i + k * kStripes] - mu);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ls += w[k] * lrow[i + k * kStripes];
      a.x += w[k] * x[k].x;
      a.y += w[k] * x[k].y;
      a.z += w[k] * x[k].z;
      a.w += w[k] * x[k].w;
    }
  }
  for (; i < n; i += kStripes) {
    const float4 x = *(const float4*)(arow + (int64_t)i * p.D);
    const float w = exp2_fast(mrow[i] - mu);
    ls += w * lrow[i];
    a.x += w * x.x;
    a.y += w * x.y;
    a.z += w * x.z;
    a.w += w * x.w;
  }

  __shared__ float4 s_a[kStripes][16];
  __shared__ float s_l[kStripes];
  s_a[s][u] = a;
  if (u == 0) s_l[s] = ls;
  __syncthreads();
  if (tid < 16) {
    float tot = 0.f;
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < kStripes; ++k) {
      tot += s_l[k];
      num.x += s_a[k][tid].x;
      num.y += s_a[k][tid].y;
      num.z += s_a[k][tid].z;
      num.w += s_a[k][tid].w;
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    *(float4*)(p.out + ((int64_t)b * p.Hq + h) * p.D + d) =
        make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
  }
}

}  // namespace

hipError_t launch_combine(const Params& p, hipStream_t s) {
  dim3 grid(p.D / 64, p.Hq, p.B);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pa
