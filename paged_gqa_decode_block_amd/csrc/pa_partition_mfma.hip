// pa_partition_mfma.hip -- split-KV partition kernel on the gfx950 matrix cores.
//
// One wave (64 lanes) per (KV partition p, KV head, sequence b). The partition's
// tokens are visited in chunks of 32; per chunk:
//
//   scores  S^T[token, head] = K[token, :] . Q'[head, :]   two 16x16x32 MFMA tiles
//           (tokens in M, the G query heads of the group in N, padded to 16),
//           K fed to the A operand straight from a 16-byte global load per lane;
//   update  the running max m, sum l and output acc of each head, in base 2
//           (page "v10_triton_paged_gqa", core principle: m_new = max(m, max s),
//           alpha = exp(m - m_new), p = exp(s - m_new), l = alpha l + sum p,
//           acc = alpha acc + p V);
//   output  O^T[dim, head] += V^T[dim, token] . P^T[token, head]   one 16x16x32
//           MFMA per 16 dims, V staged through LDS to put tokens in K.
//
// K and V of the KV head are loaded once per chunk and shared by all G query
// heads of the group (page "Paged Attention Kernel Architecture for BI-V100",
// section 4). Q and P are split into a high and a low 16-bit part (two MFMAs
// each), so the products carry ~16 mantissa bits instead of 8 and the fp32
// accumulation stays within the fp16/bf16-KV tolerance for any score spread.
//
// Partition states go to the workspace (max, sum, unnormalised output; page
// "Paged Attention Kernel Architecture for BI-V100", section 2, level 3), or,
// when the sequence has one partition, the normalised output goes straight to
// out. Tokens at or past L_b and tokens whose table entry is invalid are never
// loaded; their scores are -inf.
#include "pa_kernels.h"

namespace pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mma<_Float16> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x4 mma(vec a, vec b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// Split x into hi + lo, both rounded to T (round to nearest even).
template <typename T>
__device__ __forceinline__ void split2(float x, T& hi, T& lo) {
  hi = (T)x;
  lo = (T)(x - (float)hi);
}

// LDS layout of the V chunk: 32 token rows of D elements; the 16-byte column
// chunks of row R are XOR-permuted by f(R) = 2*((R>>2)&3) + (R&1) so that the
// transposing 2-byte reads of the P.V operand and the 16-byte writes both spread
// over the banks.
__device__ __forceinline__ int vswz(int R) { return (((R >> 2) & 3) << 1) | (R & 1); }

// Waves per SIMD the register allocation is held to: 2 for d <= 128, 1 for d = 256.
template <int D>
struct Occ {
  static constexpr int waves = D <= 128 ? 2 : 1;
};

template <typename T, int D>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(Occ<D>::waves)))
partition_mfma_kernel(Params p) {
  typedef typename Mma<T>::vec V8;
  constexpr int KS = D / 32;  // k-steps of a 16-token score tile
  constexpr int MB = D / 16;  // 16-dim output tiles

  __shared__ int s_ids[kTableCap];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[32 * D];
  __shared__ __attribute__((aligned(16))) V8 s_q[2][KS][64];  // Q' fragments, hi / lo

  const int part = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int r = lane & 15, q = lane >> 4;
  const int G = p.G;

  const int L = clamped_len(p, b, part == 0 && hk == 0 && lane == 0);
  if (L == 0) {
    if (part == 0) {  // empty context: zeros
      for (int i = lane; i < G * D / 4; i += 64) {
        const int g = i / (D / 4), c4 = i % (D / 4);
        *(float4*)(p.out + ((int64_t)b * p.Hq + hk * G + g) * D + 4 * c4) = make_float4(0, 0, 0, 0);
      }
    }
    return;
  }
  const int npart = (L + p.part - 1) / p.part;
  if (part >= npart) return;
  const int t0 = part * p.part;
  const int t1 = min(L, t0 + p.part);
  const int bsm = (1 << p.bs_log2) - 1;
  const int j0 = t0 >> p.bs_log2;
  stage_block_ids(p, b, j0, (t1 - 1) >> p.bs_log2, s_ids, lane, 64);

  // Q' = q * scale * log2(e) of head r of the group (zero for padded heads),
  // dims 32*ks + 8*q .. +7: the B-operand fragments of the score MFMAs, split
  // into hi / lo parts and parked in LDS (one 16-byte slot per lane).
  {
    const bool hv = r < G;
    const float* qp = p.q + ((int64_t)b * p.Hq + hk * G + (hv ? r : 0)) * D + 8 * q;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float4 a = hv ? *(const float4*)(qp + 32 * ks) : make_float4(0, 0, 0, 0);
      float4 c = hv ? *(const float4*)(qp + 32 * ks + 4) : make_float4(0, 0, 0, 0);
      const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
      V8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        T h, l2;
        split2<T>(x[e] * p.qscale, h, l2);
        hi[e] = h;
        lo[e] = l2;
      }
      s_q[0][ks][lane] = hi;
      s_q[1][ks][lane] = lo;
    }
  }
  __syncthreads();

  const T* kbase = (const T*)p.k + (int64_t)hk * p.ksh + 8 * q;
  const T* vbase = (const T*)p.v + (int64_t)hk * p.vsh + 8 * q;
  // V rows are loaded with a 4x4 transpose of r so each 8-lane group writes
  // 8 different bank groups.
  const int sig = ((r & 3) << 2) | (r >> 2);

  f32x4 acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  // K of chunk c for the A operand: lane (q, r) takes token c + 16*tau + r,
  // dims 32*ks + 8*q .. +7. Returns whether each of its two tokens was loaded.
  auto load_k = [&](int c, uint4 (&kr)[2][KS], bool (&kv)[2]) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int tk = c + 16 * tau + r;
      const int id = tk < t1 ? s_ids[(tk >> p.bs_log2) - j0] : -1;
      kv[tau] = id >= 0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kr[tau][ks] = make_uint4(0, 0, 0, 0);
      if (id >= 0) {
        const T* kp = kbase + (int64_t)id * p.ksb + (int64_t)(tk & bsm) * p.kst;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kr[tau][ks] = *(const uint4*)(kp + 32 * ks);
      }
    }
  };
  auto load_v = [&](int c, uint4 (&vr)[2][KS]) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int tv = c + 16 * tau + sig;
      const int id = tv < t1 ? s_ids[(tv >> p.bs_log2) - j0] : -1;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) vr[tau][ks] = make_uint4(0, 0, 0, 0);
      if (id >= 0) {
        const T* vp = vbase + (int64_t)id * p.vsb + (int64_t)(tv & bsm) * p.vst;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) vr[tau][ks] = *(const uint4*)(vp + 32 * ks);
      }
    }
  };

  // One chunk: kcur holds its K; knext receives the next chunk's K; vr holds
  // this chunk's V and then receives the next chunk's V.
  auto step = [&](int c, uint4 (&kcur)[2][KS], bool (&kval)[2], uint4 (&knext)[2][KS],
                  bool (&knv)[2], uint4 (&vr)[2][KS]) {
    const bool more = c + 32 < t1;
    if (more) load_k(c + 32, knext, knv);

    // ---- stage V of this chunk in LDS (row-major, swizzled), then refill vr
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int R = 16 * tau + sig;
      const int f = vswz(R);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int pc = (4 * ks + q) ^ f;
        *(uint4*)(s_v + R * D + 8 * pc) = vr[tau][ks];
      }
    }
    if (more) load_v(c + 32, vr);

    // ---- scores: two 16-token tiles, K . Q'hi + K . Q'lo
    f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const V8 qh = s_q[0][ks][lane];
      const V8 ql = s_q[1][ks][lane];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const V8 a = __builtin_bit_cast(V8, kcur[tau][ks]);
        st[tau] = Mma<T>::mma(a, qh, st[tau]);
        st[tau] = Mma<T>::mma(a, ql, st[tau]);
      }
    }
    // token 16*tau + x was loaded iff lane x (quad 0) had a valid id for it
    const uint64_t bal0 = __ballot(kval[0]);
    const uint64_t bal1 = __ballot(kval[1]);
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = ((bal0 >> (4 * q + i)) & 1) ? st[0][i] : -INFINITY;
      sv[4 + i] = ((bal1 >> (4 * q + i)) & 1) ? st[1][i] : -INFINITY;
    }

    // ---- running softmax state of head r (same in all four quads)
    float mt = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sv[i]);
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m, mt);
    const float mu = mn == -INFINITY ? 0.f : mn;
    const float alpha = exp2_fast(m - mu);
    float pv[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = exp2_fast(sv[i] - mu);
      ps += pv[i];
    }
    l = l * alpha + ps;
    m = mn;
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[i] *= alpha;

    // P^T fragment: k-slot j holds token 16*(j>>2) + 4*q + (j&3)
    V8 phi, plo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      T h, lo;
      split2<T>(pv[j], h, lo);
      phi[j] = h;
      plo[j] = lo;
    }

    // ---- O^T += V^T P^T, one MFMA (x2 for hi/lo P) per 16 dims
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int col = 16 * mb + r;
      u16x8 a;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int R = 16 * (j >> 2) + 4 * q + (j & 3);
        const int pc = (col >> 3) ^ vswz(R);
        a[j] = s_v[R * D + 8 * pc + (col & 7)];
      }
      const V8 av = __builtin_bit_cast(V8, a);
      acc[mb] = Mma<T>::mma(av, phi, acc[mb]);
      acc[mb] = Mma<T>::mma(av, plo, acc[mb]);
    }
  };

  uint4 kA[2][KS], kB[2][KS], vr[2][KS];
  bool vA[2], vB[2] = {false, false};
  load_k(t0, kA, vA);
  load_v(t0, vr);
  for (int c = t0; c < t1; c += 64) {
    step(c, kA, vA, kB, vB, vr);
    if (c + 32 >= t1) break;
    step(c + 32, kB, vB, kA, vA, vr);
  }

  // l summed over the four quads (each holds its own tokens' share)
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);

  if (r >= G) return;
  const int h = hk * G + r;
  if (npart == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* op = p.out + ((int64_t)b * p.Hq + h) * D + 4 * q;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const f32x4 o = acc[mb] * inv;
      *(float4*)(op + 16 * mb) = make_float4(o[0], o[1], o[2], o[3]);
    }
  } else {
    const int64_t row = ((int64_t)b * p.Hq + h) * p.pmax + part;
    float* ap = p.ws_acc + row * D + 4 * q;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      *(float4*)(ap + 16 * mb) = make_float4(acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]);
    if (q == 0) {
      p.ws_m[row] = m;
      p.ws_l[row] = l;
    }
  }
}

template <typename T, int D>
hipError_t launch_t(const Params& p, hipStream_t s) {
  dim3 grid(p.pmax, p.Hkv, p.B);
  hipLaunchKernelGGL((partition_mfma_kernel<T, D>), grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_d(const Params& p, hipStream_t s) {
  switch (p.D) {
    case 64: return launch_t<T, 64>(p, s);
    case 128: return launch_t<T, 128>(p, s);
    case 256: return launch_t<T, 256>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool mfma_supports(int dtype, int D, int G) {
  return (dtype == 1 || dtype == 2) && (D == 64 || D == 128 || D == 256) && G >= 1 && G <= 16;
}

hipError_t launch_partition_mfma(const Params& p, int dtype, hipStream_t s) {
  if (dtype == 1) return launch_d<_Float16>(p, s);
  if (dtype == 2) return launch_d<__bf16>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
