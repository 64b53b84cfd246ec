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
// After the streaming kernel the states to merge are not partitions but the
// waves' states of each (sequence, KV head) stream: the stream's record names
// the slot of its first wave's state and the number n of consecutive waves
// whose states make up the stream (0 when its output was written directly);
// wave w_a + i, i >= 1, left its state in its slot 0. A record is trusted only
// for a non-empty stream (every non-empty stream's record is rewritten by
// each call); an empty sequence gets zeros. With prefix folding a sequence has
// two such runs: its group's folded prefix (the states' column for this
// member and head) and its own stream past the prefix, if not empty.
//
// Grid (D / 64, H_q, B), 16 x S threads: thread (stripe s, quad u) owns dims
// 4u .. 4u+3 of a 64-dim slice (float4 loads) and states i = s, s + S, ....
// Each thread folds its states with the same max-rescaling op, a batch of
// states' loads in flight per round, so no pass over all maxima has to finish
// first; the S stripes' states then meet, four per wave by cross-lane
// exchanges and the waves' through LDS. S is 4 or 8 when there are at most
// that many states per (sequence, head), 16 up to 64, and 64 (32 beyond 256)
// above (the host's bound or estimate of that count), so one round usually
// covers them all. A grid of many (sequence, head, slice) items instead runs
// one wave per item up to 64 states (S = 4, a batch of up to 4 states per
// thread and round), eight items (heads) per workgroup: there the launch's
// waves outnumber what the compute units hold at once, and the fewer waves and
// workgroups the sooner the last one ends.
#include "pa_kernels.h"

namespace pa {
namespace {

// kStripes: partition stripes (4, 8, 16, 32 or 64); kBatch: partitions per
// thread per round (1, 2, 4 or 8); both chosen from the grid and the partition
// count. kItems: heads per workgroup, one wave each (with kStripes = 4 only).
// kFold: after the streaming kernel with prefix folding (its own rows and the
// prefix states).
template <int kStripes, int kBatch, bool kFold, int kItems = 1>
__global__ void __launch_bounds__(16 * kStripes * kItems) combine_kernel(Params p) {
  static_assert(kStripes % 4 == 0, "whole waves of four stripes");
  static_assert(kItems == 1 || kStripes == 4, "one wave per item");
  const int b = blockIdx.z;
  const int h = kItems > 1 ? (int)blockIdx.y * kItems + (int)(threadIdx.x >> 6) : (int)blockIdx.y;
  if (kItems > 1 && h >= p.Hq) return;  // (a whole wave)
  const int tid = kItems > 1 ? (int)(threadIdx.x & 63) : (int)threadIdx.x;
  const int u = tid & 15, s = tid >> 4;
  const int d = blockIdx.x * 64 + 4 * u;
  const bool waves = p.ws_link != nullptr;  // states of the streaming kernel's waves
  const int hk = h / p.G, g = h - hk * p.G;
  const int gi = p.fold > 0 ? b / p.fold : 0;
  const bool folded = kFold;  // (the host launches kFold only with folding)
  // the loads issued before any is used
  const int2 rec = waves ? *(const int2*)(p.ws_link + 2 * ((int64_t)b * p.Hkv + hk)) : make_int2(0, 0);
  const int2 recf =
      folded ? *(const int2*)(p.ws_link + 2 * ((int64_t)(p.B + gi) * p.Hkv + hk)) : make_int2(0, 0);
  const int pre = folded ? p.ws_vlen[gi * (p.fold + 1)] : 0;
  const int L = clamped_len(p, b, false);
  int n, nf = 0;
  // a record is always in range when this call's partition kernel wrote it;
  // anything else reads nothing (zeros) rather than outside the slots. x = -1:
  // one state in the stream's own rows (folding only)
  auto in_range = [&](int2 r, int c) {
    if (kFold && r.x == -1) return c == 1;
    return r.x >= 0 && r.x < 2 * p.nwaves && c >= 0 && (r.x >> 1) + c <= p.nwaves;
  };
  if (waves) {
    const bool own = L > pre;  // the sequence's own stream has tokens
    if (own && pre == 0 && rec.y == 0) return;  // written out by the partition kernel
    n = own ? rec.y : 0;
    if (!in_range(rec, n)) n = 0;
    nf = pre > 0 ? recf.y : 0;
    if (!in_range(recf, nf)) nf = 0;
  } else {
    n = (L + p.part - 1) / p.part;
    if (n <= 1) return;
  }

  // state i of the (sequence, head): its max, sum and unnormalised output;
  // after the own stream's n states come the folded prefix's nf
  const int64_t row = ((int64_t)b * p.Hq + h) * p.pmax;
  const int colf = (b - gi * p.fold) * p.G + g;  // this head's column in the prefix states
  const int nown = n;
  // the state's row, in the wave slots or (x = -1) in the stream's own rows
  // (negative: own row -1 - row)
  auto state_row = [&](int i) -> int64_t {
    if (!waves) return -1;
    if (!kFold || i < nown) {
      if (kFold && rec.x == -1) return -1 - (((int64_t)b * p.Hkv + hk) * p.rps + g);
      const int slot = i == 0 ? rec.x : 2 * ((rec.x >> 1) + i);
      return (int64_t)slot * p.rps + g;
    }
    const int k = i - nown;
    if (recf.x == -1) return -1 - (((int64_t)(p.B + gi) * p.Hkv + hk) * p.rps + colf);
    const int slot = k == 0 ? recf.x : 2 * ((recf.x >> 1) + k);
    return (int64_t)slot * p.rps + colf;
  };
  n += nf;

  // (m, l, a) <- (m, l, a) merged with (cm, cl, ca)
  auto merge = [](float& m, float& l, float4& a, float cm, float cl, float4 ca) {
    const float M = fmaxf(m, cm);
    const float mu = M == -INFINITY ? 0.f : M;
    const float w0 = exp2_fast(m - mu), w1 = exp2_fast(cm - mu);
    l = w0 * l + w1 * cl;
    a.x = w0 * a.x + w1 * ca.x;
    a.y = w0 * a.y + w1 * ca.y;
    a.z = w0 * a.z + w1 * ca.z;
    a.w = w0 * a.w + w1 * ca.w;
    m = M;
  };
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
        if (waves && kFold) {
          // one load of each, from the slots or the own rows (selected addresses)
          const int64_t sr = state_row(i);
          const bool o = sr < 0;
          const int64_t rr = o ? -1 - sr : sr;
          mv[k] = (o ? p.ws_om : p.ws_cm)[rr];
          lv[k] = (o ? p.ws_ol : p.ws_cl)[rr];
          av[k] = *(const float4*)((o ? p.ws_oacc : p.ws_cacc) + rr * p.D + d);
        } else if (waves) {
          const int64_t sr = state_row(i);
          mv[k] = p.ws_cm[sr];
          lv[k] = p.ws_cl[sr];
          av[k] = *(const float4*)(p.ws_cacc + sr * p.D + d);
        } else {
          mv[k] = p.ws_m[row + i];
          lv[k] = p.ws_l[row + i];
          av[k] = *(const float4*)(p.ws_acc + (row + i) * p.D + d);
        }
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

  // Merge the stripes: the four stripes of a wave (lanes 16 apart, same dims)
  // by two cross-lane exchanges, then the waves' states through LDS.
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    const float om = __shfl_xor(Ms, off), ol = __shfl_xor(Ls, off);
    float4 oa;
    oa.x = __shfl_xor(A.x, off);
    oa.y = __shfl_xor(A.y, off);
    oa.z = __shfl_xor(A.z, off);
    oa.w = __shfl_xor(A.w, off);
    merge(Ms, Ls, A, om, ol, oa);
  }
  if constexpr (kStripes == 4) {
    // one wave: every lane holds the merged state of its dims
    if (tid < 16) {
      const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
      store_out4(p, ((int64_t)b * p.Hq + h) * p.D + d, A.x * inv, A.y * inv, A.z * inv,
                 A.w * inv);
    }
    return;
  }
  constexpr int kWaves = kStripes / 4;
  __shared__ float4 s_a[kWaves][16];
  __shared__ float s_m[kWaves], s_l[kWaves];
  const int wv = tid >> 6;
  if ((tid & 63) < 16) {
    s_a[wv][u] = A;
    if (u == 0) {
      s_m[wv] = Ms;
      s_l[wv] = Ls;
    }
  }
  __syncthreads();
  if (tid < 16) {
    float M = s_m[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) M = fmaxf(M, s_m[k]);
    const float mu = M == -INFINITY ? 0.f : M;
    float tot = 0.f;
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      const float w = exp2_fast(s_m[k] - mu);
      tot += w * s_l[k];
      num.x += w * s_a[k][tid].x;
      num.y += w * s_a[k][tid].y;
      num.z += w * s_a[k][tid].z;
      num.w += w * s_a[k][tid].w;
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    store_out4(p, ((int64_t)b * p.Hq + h) * p.D + d, num.x * inv, num.y * inv, num.z * inv,
               num.w * inv);
  }
}

template <bool kFold>
hipError_t launch_combine_t(const Params& p, hipStream_t s) {
  dim3 grid(p.D / 64, p.Hq, p.B);
  // one wave per item when the grid alone fills the GPU (about one wave per
  // SIMD of 256 compute units), eight heads per workgroup; a batch of 2 or 4
  // states per thread per round
  const int64_t items = (int64_t)grid.x * grid.y * grid.z;
  if (items >= 1024 && p.pmax <= 64) {
    const dim3 g8(grid.x, (grid.y + 7) / 8, grid.z);
    if (p.pmax <= 8)
      hipLaunchKernelGGL((combine_kernel<4, 2, kFold, 8>), g8, dim3(512), 0, s, p);
    else
      hipLaunchKernelGGL((combine_kernel<4, 4, kFold, 8>), g8, dim3(512), 0, s, p);
    return hipGetLastError();
  }
  // stripes sized to the partition count: with few partitions per sequence
  // (long partitions over a large batch) small workgroups leave no thread idle
  if (p.pmax <= 4)
    hipLaunchKernelGGL((combine_kernel<4, 1, kFold>), grid, dim3(64), 0, s, p);
  else if (p.pmax <= 8)
    hipLaunchKernelGGL((combine_kernel<8, 1, kFold>), grid, dim3(128), 0, s, p);
  else if (p.pmax <= 16)
    hipLaunchKernelGGL((combine_kernel<16, 1, kFold>), grid, dim3(256), 0, s, p);
  else if (p.pmax <= 64)
    hipLaunchKernelGGL((combine_kernel<16, 4, kFold>), grid, dim3(256), 0, s, p);
  else if (p.pmax <= 256)
    hipLaunchKernelGGL((combine_kernel<64, 4, kFold>), grid, dim3(1024), 0, s, p);
  else  // 512 threads: a batch of 8 needs more than the 128 registers of 1024-thread blocks
    hipLaunchKernelGGL((combine_kernel<32, 8, kFold>), grid, dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const Params& p, hipStream_t s) {
  return p.fold > 0 && p.ws_link && p.ws_om ? launch_combine_t<true>(p, s)
                                            : launch_combine_t<false>(p, s);
}

}  // namespace pa
