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
// 4u .. 4u+3 of a 64-dim slice (float4 loads) and partitions p = s, s + 16, ....
// Each thread folds its partitions with the same max-rescaling op, eight
// partitions' loads in flight per round, so no pass over all maxima has to
// finish first; the 16 stripes' states then meet in LDS.
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kStripes = 16;

// kBatch: partitions per thread per round (1, 4 or 8, from the partition count).
template <int kBatch>
__global__ void __launch_bounds__(256) combine_kernel(Params p) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int tid = threadIdx.x;
  const int u = tid & 15, s = tid >> 4;
  const int d = blockIdx.x * 64 + 4 * u;
  const int L = clamped_len(p, b, false);
  const int n = (L + p.part - 1) / p.part;
  if (n <= 1) return;

  const int64_t row = ((int64_t)b * p.Hq + h) * p.pmax;
  const float* mrow = p.ws_m + row;
  const float* lrow = p.ws_l + row;
  const float* arow = p.ws_acc + row * p.D + d;

  float Ms = -INFINITY, Ls = 0.f;
  float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = s; i0 < n; i0 += kStripes * kBatch) {
    float mv[kBatch], lv[kBatch];
    float4 av[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = i0 + k * kStripes;
      mv[k] = -INFINITY;
      lv[k] = 0.f;
      av[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < n) {
        mv[k] = mrow[i];
        lv[k] = lrow[i];
        av[k] = *(const float4*)(arow + (int64_t)i * p.D);
      }
    }
    float bm = Ms;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) bm = fmaxf(bm, mv[k]);
    const float bu = bm == -INFINITY ? 0.f : bm;
    const float sc = exp2_fast(Ms - bu);
    Ls *= sc;
    A.x *= sc;
    A.y *= sc;
    A.z *= sc;
    A.w *= sc;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float w = exp2_fast(mv[k] - bu);
      Ls += w * lv[k];
      A.x += w * av[k].x;
      A.y += w * av[k].y;
      A.z += w * av[k].z;
      A.w += w * av[k].w;
    }
    Ms = bm;
  }

  __shared__ float4 s_a[kStripes][16];
  __shared__ float s_m[kStripes], s_l[kStripes];
  s_a[s][u] = A;
  if (u == 0) {
    s_m[s] = Ms;
    s_l[s] = Ls;
  }
  __syncthreads();
  if (tid < 16) {
    float M = s_m[0];
#pragma unroll
    for (int k = 1; k < kStripes; ++k) M = fmaxf(M, s_m[k]);
    const float mu = M == -INFINITY ? 0.f : M;
    float tot = 0.f;
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < kStripes; ++k) {
      const float w = exp2_fast(s_m[k] - mu);
      tot += w * s_l[k];
      num.x += w * s_a[k][tid].x;
      num.y += w * s_a[k][tid].y;
      num.z += w * s_a[k][tid].z;
      num.w += w * s_a[k][tid].w;
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    *(float4*)(p.out + ((int64_t)b * p.Hq + h) * p.D + d) =
        make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
  }
}

}  // namespace

hipError_t launch_combine(const Params& p, hipStream_t s) {
  dim3 grid(p.D / 64, p.Hq, p.B);
  if (p.pmax <= kStripes)
    hipLaunchKernelGGL(combine_kernel<1>, grid, dim3(256), 0, s, p);
  else if (p.pmax <= 4 * kStripes)
    hipLaunchKernelGGL(combine_kernel<4>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(combine_kernel<8>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pa
