// pa_partition_valu.hip -- split-KV partition kernel on the vector ALUs.
//
// One workgroup of four waves per (KV partition p, KV head, sequence b). A token
// row of d elements is spread over C = d / E lanes, each holding one 16-byte
// chunk (E = 4 fp32 or 8 fp16/bf16 values), so a wave covers 64 / C token rows
// per load and the row slots of the four waves walk the partition's tokens in
// an interleaved order. Per token a lane forms the partial dot products of its
// chunk with the G query heads of the group and the C lanes of the row sum them
// with DPP / ds_swizzle butterflies (page "Paged Attention Kernel Architecture
// for BI-V100", section 2 level 1, written for 64-lane waves); the K and V
// chunks in registers are shared by all G heads (same page, section 4).
//
// Each row slot keeps a running (max, sum, output) state per head, updated every
// U tokens (page "v10_triton_paged_gqa", core principle). At the end the row
// slots of a wave merge across lanes and the four waves merge through LDS with
// the max-rescaling combine (same BI-V100 page, section 2 levels 1-2), and the
// result is written as a partition state or, for a one-partition sequence, as
// the normalised output. Scores are kept in base-2 units.
#include "pa_kernels.h"

namespace pa {
namespace {

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                         CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of C lanes; every lane of a group gets the group sum.
template <int C>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (C >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (C >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (C >= 8) x += dpp<0x141>(x);  // row_half_mirror: the other quad of 8
  if constexpr (C >= 16) x += dpp<0x140>(x); // row_mirror: the other half of 16
  if constexpr (C >= 32)
    x += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
  if constexpr (C >= 64) x += __shfl_xor(x, 32);
  return x;
}

template <typename T>
__device__ __forceinline__ void widen(const uint4& raw, float* f);

template <>
__device__ __forceinline__ void widen<float>(const uint4& raw, float* f) {
  f[0] = __builtin_bit_cast(float, raw.x);
  f[1] = __builtin_bit_cast(float, raw.y);
  f[2] = __builtin_bit_cast(float, raw.z);
  f[3] = __builtin_bit_cast(float, raw.w);
}

template <>
__device__ __forceinline__ void widen<_Float16>(const uint4& raw, float* f) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
    f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
  }
}

template <>
__device__ __forceinline__ void widen<__bf16>(const uint4& raw, float* f) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
  }
}

template <typename T, int D, int G>
__global__ void __launch_bounds__(256) partition_valu_kernel(Params p) {
  constexpr int E = 16 / (int)sizeof(T);  // elements per lane chunk
  constexpr int C = D / E;                // lanes per token row
  constexpr int R = 64 / C;               // token rows per wave
  constexpr int NW = 4;
  constexpr int S = NW * R;               // row slots per workgroup
  constexpr int U = 2;                    // tokens per row slot per update

  __shared__ int s_ids[kTableCap];
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ float s_acc[NW][G][D];

  // partition-major grid: x = b * H_kv + hk, y = partition
  const int b = blockIdx.x / p.Hkv, hk = blockIdx.x - (blockIdx.x / p.Hkv) * p.Hkv;
  const int part = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = lane / C, cl = lane % C;
  const int slot = w * R + row;

  const int L = clamped_len(p, b, part == 0 && hk == 0 && tid == 0);
  if (L == 0) {
    if (part == 0) {
      for (int i = tid; i < G * D; i += 256)
        store_out1(p, ((int64_t)b * p.Hq + hk * G + i / D) * D + i % D, 0.f);
    }
    return;
  }
  const int npart = (L + p.part - 1) / p.part;
  if (part >= npart) return;
  const int t0 = part * p.part;
  const int t1 = min(L, t0 + p.part);
  const int bsm = (1 << p.bs_log2) - 1;
  const int j0 = t0 >> p.bs_log2;
  stage_block_ids(p, b, j0, (t1 - 1) >> p.bs_log2, s_ids, tid, 256);
  __syncthreads();

  float qv[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t qrow = ((int64_t)b * p.Hq + hk * G + g) * D + cl * E;
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const float4 x = load_q4(p, qrow + e);
      qv[g][e] = x.x * p.qscale;
      qv[g][e + 1] = x.y * p.qscale;
      qv[g][e + 2] = x.z * p.qscale;
      qv[g][e + 3] = x.w * p.qscale;
    }
  }

  float m[G], l[G], acc[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
  }

  const T* kbase = (const T*)p.k + (int64_t)hk * p.ksh + cl * E;
  const T* vbase = (const T*)p.v + (int64_t)hk * p.vsh + cl * E;

  for (int c = t0; c < t1; c += S * U) {
    float kf[U][E], vf[U][E];
    bool val[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = c + slot + S * u;
      const int id = t < t1 ? s_ids[(t >> p.bs_log2) - j0] : -1;
      val[u] = id >= 0;
      uint4 kr = make_uint4(0, 0, 0, 0), vr = make_uint4(0, 0, 0, 0);
      if (id >= 0) {
        kr = *(const uint4*)(kbase + (int64_t)id * p.ksb + (int64_t)(t & bsm) * p.kst);
        vr = *(const uint4*)(vbase + (int64_t)id * p.vsb + (int64_t)(t & bsm) * p.vst);
      }
      widen<T>(kr, kf[u]);
      widen<T>(vr, vf[u]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) x = fmaf(qv[g][e], kf[u][e], x);
        x = group_sum<C>(x);
        s[u] = val[u] ? x : -INFINITY;
      }
      float mt = s[0];
#pragma unroll
      for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[u]);
      const float mn = fmaxf(m[g], mt);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = exp2_fast(m[g] - mu);
      float pu[U], ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        pu[u] = exp2_fast(s[u] - mu);
        ps += pu[u];
      }
      l[g] = l[g] * alpha + ps;
      m[g] = mn;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float a = acc[g][e] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) a = fmaf(pu[u], vf[u][e], a);
        acc[g][e] = a;
      }
    }
  }

  // merge the R row slots of the wave (lanes that differ in the row bits)
#pragma unroll
  for (int off = C; off < 64; off *= 2) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float a = exp2_fast(m[g] - mu), ao = exp2_fast(mo - mu);
      l[g] = a * l[g] + ao * lo;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] = a * acc[g][e] + ao * __shfl_xor(acc[g][e], off);
      m[g] = mn;
    }
  }
  if (row == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < E; ++e) s_acc[w][g][cl * E + e] = acc[g][e];
      if (cl == 0) {
        s_m[w][g] = m[g];
        s_l[w][g] = l[g];
      }
    }
  }
  __syncthreads();

  for (int i = tid; i < G * D; i += 256) {
    const int g = i / D, d = i % D;
    float M = s_m[0][g];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, s_m[ww][g]);
    const float mu = M == -INFINITY ? 0.f : M;
    float ls = 0.f, as = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float wgt = exp2_fast(s_m[ww][g] - mu);
      ls += wgt * s_l[ww][g];
      as += wgt * s_acc[ww][g][d];
    }
    const int h = hk * G + g;
    if (npart == 1) {
      store_out1(p, ((int64_t)b * p.Hq + h) * D + d, ls > 0.f ? as / ls : 0.f);
    } else {
      const int64_t rw = ((int64_t)b * p.Hq + h) * p.pmax + part;
      p.ws_acc[rw * D + d] = as;
      if (d == 0) {
        p.ws_m[rw] = M;
        p.ws_l[rw] = ls;
      }
    }
  }
}

template <typename T, int D, int G>
hipError_t launch_t(const Params& p, hipStream_t s) {
  dim3 grid(p.B * p.Hkv, p.pmax);
  hipLaunchKernelGGL((partition_valu_kernel<T, D, G>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_g(const Params& p, hipStream_t s) {
  switch (p.G) {
    case 1: return launch_t<T, D, 1>(p, s);
    case 2: return launch_t<T, D, 2>(p, s);
    case 3: return launch_t<T, D, 3>(p, s);
    case 4: return launch_t<T, D, 4>(p, s);
    case 5: return launch_t<T, D, 5>(p, s);
    case 6: return launch_t<T, D, 6>(p, s);
    case 7: return launch_t<T, D, 7>(p, s);
    case 8: return launch_t<T, D, 8>(p, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_d(const Params& p, hipStream_t s) {
  switch (p.D) {
    case 64: return launch_g<T, 64>(p, s);
    case 128: return launch_g<T, 128>(p, s);
    case 256: return launch_g<T, 256>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool valu_supports(int dtype, int D, int G) {
  return (dtype >= 0 && dtype <= 2) && (D == 64 || D == 128 || D == 256) && G >= 1 && G <= 8;
}

hipError_t launch_partition_valu(const Params& p, int dtype, hipStream_t s) {
  if (dtype == 0) return launch_d<float>(p, s);
  if (dtype == 1) return launch_d<_Float16>(p, s);
  if (dtype == 2) return launch_d<__bf16>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
