// pa_prefill.hip -- paged varlen prefill on the matrix cores (gfx950).
//
// Sequence b has q_len_b query rows, rows cu_q[b] .. cu_q[b+1]-1 of the packed
// q ([total_q, H_q, d], the varlen indexing of the paged-attention docs page),
// and L_b keys in the paged pool (the new tokens already written there). With
// the causal rule, its query i sits at position L_b - q_len_b + i and attends
// tokens [0, L_b - q_len_b + i]; a query with no token to attend gets zeros.
// Otherwise every query attends all L_b tokens.
//
// One wave per (tile of 16 query rows of one sequence, query head). The 16
// rows are the 16 columns of the score and output tiles, so the chunk loop is
// the decode kernel's with positions in place of heads:
//
//   scores  S^T[token, row] = K[token, :] . Q'[row, :]       16x16x32 MFMAs
//   update  running max m, sum l, output per row (base 2, lazily rescaled)
//   output  O^T[dim, row] += V^T[dim, token] . P^T[token, row]  16x16x16
//
// with Q' and P split into hi + lo 16-bit parts. The wave walks the tokens up
// to the tile's last row's key end in 16-token chunks through a ring of NBUF
// chunks in registers (raw buffer loads, descriptors cut to the attended rows
// of the chunk, an invalid table entry never dereferenced), each chunk staged
// in LDS; a token is masked per column, so rows of the tile end at their own
// causal bound. No partial state leaves the wave: the tile is normalised and
// written at the end.
//
// Requires 16-bit K/V and block_size >= 16.
#include "pa_mfma_util.h"

namespace pa {
namespace {

template <typename T, int D, int NBUF, int OCC, bool QL, int QO>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
prefill_kernel(Params p, const int32_t* __restrict__ cu_q, int causal) {
  typedef Mx<T> M;
  typedef typename M::v8 V8;
  typedef typename M::v4 V4;
  typedef Cfg<D> C;
  constexpr int LPC = C::LPC, KS = C::KS, MB = C::MB;
  static_assert((NBUF - 1) * 2 * LPC <= 63, "ring deeper than the vector-memory counter");
  __shared__ __attribute__((aligned(16))) uint16_t s_k[16 * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[16 * D];
  __shared__ __attribute__((aligned(16))) V8 s_q[QL ? 2 : 1][QL ? KS : 1][64];

  const int lane = threadIdx.x;
  const int r = lane & 15, q = lane >> 4;
  const int b = blockIdx.z, h = blockIdx.y, p0 = 16 * (int)blockIdx.x;
  const int r0 = cu_q[b];
  const int ql = cu_q[b + 1] - r0;
  // rows beyond the grid would be left unwritten: report
  if (blockIdx.x == 0 && h == 0 && lane == 0 && p.status && (ql < 0 || ql > 16 * (int)gridDim.x))
    atomicOr(p.status, kStatusBadSeqlen);
  if (p0 >= ql) return;
  const int L = clamped_len(p, b, blockIdx.x == 0 && h == 0 && lane == 0);
  const int hk = h / p.G;

  // column r: query position p0 + r of the sequence; its keys are [0, kend_r)
  const bool col_ok = p0 + r < ql;
  const int kend_r =
      !col_ok ? 0 : causal ? min(L, max(0, L - ql + p0 + r + 1)) : L;
  const int plast = min(p0 + 15, ql - 1);
  const int kend = causal ? min(L, max(0, L - ql + plast + 1)) : L;  // the tile's
  const int nch = (kend + 15) >> 4;

  // Q' fragments of row p0 + r (zero for rows past the sequence)
  const int64_t qrow = ((int64_t)(r0 + (col_ok ? p0 + r : 0)) * p.Hq + h) * D + 8 * q;
  V8 qhi[QL ? 1 : KS], qlo[QL ? 1 : KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const float4 a = load_q4<QO>(p, qrow + 32 * ks);
    const float4 c = load_q4<QO>(p, qrow + 32 * ks + 4);
    const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    V8 hi, lo;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float y = col_ok ? x[k] * p.qscale : 0.f;
      const T hh = (T)y;
      hi[k] = hh;
      lo[k] = (T)(y - (float)hh);
    }
    if constexpr (QL) {
      s_q[0][ks][lane] = hi;
      s_q[1][ks][lane] = lo;
    } else {
      qhi[ks] = hi;
      qlo[ks] = lo;
    }
  }

  const int bsm = (1 << p.bs_log2) - 1;
  const int rowL = lane / C::CPR;
  const int cc = lane % C::CPR;
  const int tj = r >> 2, tk = r & 3;
  const int kst_bytes = (int)(p.kst * (int)sizeof(T)), vst_bytes = (int)(p.vst * (int)sizeof(T));
  int koffs[LPC], voffs[LPC];
#pragma unroll
  for (int s = 0; s < LPC; ++s) {
    koffs[s] = (s * C::RPI + rowL) * kst_bytes + 16 * cc;
    voffs[s] = (s * C::RPI + rowL) * vst_bytes + 16 * cc;
  }

  const int32_t* trow = p.table + (int64_t)b * p.MBS;
  const char* kbase = (const char*)p.k + (int64_t)hk * p.ksh * (int)sizeof(T);
  const char* vbase = (const char*)p.v + (int64_t)hk * p.vsh * (int)sizeof(T);
  const int nblk = (kend + bsm) >> p.bs_log2;
  const __amdgpu_buffer_rsrc_t rst = uniform_rsrc((const char*)trow, nblk * 4);
  auto fetch_id = [&](int cn) -> int {
    return (int)__builtin_amdgcn_raw_buffer_load_b32(rst, ((16 * cn) >> p.bs_log2) * 4, 0, 0);
  };
  int idr[NBUF];
  static_for<0, NBUF>([&](auto S) { idr[decltype(S)::value] = fetch_id(decltype(S)::value); });

  int bad_block = 0;
  // (both lambdas are forced inline: called out of line, their ring arguments
  // would live in scratch memory)
  auto issue = [&](int cn, uint4 (&rk)[LPC], uint4 (&rv)[LPC], int& ids)
      __attribute__((always_inline)) -> int {
    int id = __builtin_amdgcn_readfirstlane(ids);
    if (cn >= nch) {
      id = -1;
    } else if (id < 0 || id >= p.NB) {
      bad_block = 1;
      id = -1;
    }
    const int tok0 = 16 * cn;
    const int rows = id >= 0 ? min(16, kend - tok0) : 0;
    const int64_t row0 = id >= 0 ? (int64_t)(tok0 & bsm) : 0;
    const int64_t idc = id >= 0 ? (int64_t)id : 0;
    const __amdgpu_buffer_rsrc_t rsk =
        uniform_rsrc(kbase + (idc * p.ksb + row0 * p.kst) * (int)sizeof(T), rows * kst_bytes);
    const __amdgpu_buffer_rsrc_t rsv =
        uniform_rsrc(vbase + (idc * p.vsb + row0 * p.vst) * (int)sizeof(T), rows * vst_bytes);
#pragma unroll
    for (int s = 0; s < LPC; ++s) {
      rk[s] = buf_load<2>(rsk, koffs[s]);
      rv[s] = buf_load<2>(rsv, voffs[s]);
    }
    ids = fetch_id(cn + NBUF);
    return rows;
  };

  f32x4 acc[MB];
#pragma unroll
  for (int k = 0; k < MB; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  auto consume = [&](int cn, const uint4 (&rk)[LPC], const uint4 (&rv)[LPC])
      __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < LPC; ++s) {
      const int R = s * C::RPI + rowL;
      *(uint4*)(s_k + R * D + 8 * (cc ^ (R & 7))) = rk[s];
      *(uint4*)(s_v + R * D + 8 * (cc ^ vswz(R))) = rv[s];
    }
    // scores: lane (q, r) gets tokens 4q..4q+3 of the chunk for row r
    f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const V8 a = *(const V8*)(s_k + r * D + 8 * ((4 * ks + q) ^ (r & 7)));
      if constexpr (QL) {
        st = M::mma32(a, s_q[0][ks][lane], st);
        st = M::mma32(a, s_q[1][ks][lane], st);
      } else {
        st = M::mma32(a, qhi[ks], st);
        st = M::mma32(a, qlo[ks], st);
      }
    }
    // the row's own key bound (causal) also covers the chunk's attended rows
    float sv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) sv[k] = (16 * cn + 4 * q + k < kend_r) ? st[k] : -INFINITY;
    const float mt = quad_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    const bool raise = mt > m + 8.f;
    if (__ballot(raise)) {
      const float mn = raise ? mt : m;
      const float alpha = exp2_fast(m - (mn == -INFINITY ? 0.f : mn));
      l *= alpha;
#pragma unroll
      for (int k = 0; k < MB; ++k) acc[k] *= alpha;
      m = mn;
    }
    const float mu = m == -INFINITY ? 0.f : m;
    float pv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) pv[k] = exp2_fast(sv[k] - mu);
    l += (pv[0] + pv[1]) + (pv[2] + pv[3]);
    typename M::e4 ph, pl2;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const T hh = (T)pv[k];
      ph[k] = hh;
      pl2[k] = (T)(pv[k] - (float)hh);
    }
    const V4 phi = M::pack(ph), plo = M::pack(pl2);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int pc = 2 * (mb ^ tj) + ((tk >> 1) ^ (q & 1));
      const s16x4 a4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(s_v + (4 * q + tj) * D + 8 * pc + 4 * (tk & 1)));
      const V4 av = __builtin_bit_cast(V4, a4);
      acc[mb] = M::mma16(av, phi, acc[mb]);
      acc[mb] = M::mma16(av, plo, acc[mb]);
    }
  };

  // the ring: chunk c + NBUF - 1 is issued just before chunk c is consumed
  // (unconditionally: past the end the descriptors are empty)
  uint4 rk[NBUF][LPC], rv[NBUF][LPC];
  static_for<0, NBUF - 1>([&](auto S) {
    constexpr int s = decltype(S)::value;
    issue(s, rk[s], rv[s], idr[s]);
  });
  for (int cb = 0; cb < nch; cb += NBUF) {
    static_for<0, NBUF>([&](auto S) {
      constexpr int s = decltype(S)::value;
      constexpr int sn = (s + NBUF - 1) % NBUF;
      const int c = cb + s;
      issue(c + NBUF - 1, rk[sn], rv[sn], idr[sn]);
      __builtin_amdgcn_sched_barrier(0);
      if (c < nch) consume(c, rk[s], rv[s]);
    });
  }

  const float lt = quad_sum(l);
  if (col_ok) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t orow = ((int64_t)(r0 + p0 + r) * p.Hq + h) * D + 4 * q;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const f32x4 o = acc[mb] * inv;
      store_out4<QO>(p, orow + 16 * mb, o[0], o[1], o[2], o[3]);
    }
  }
  if (bad_block && lane == 0 && p.status) atomicOr(p.status, kStatusBadBlock);
}

// {ring slots, waves per SIMD, Q' in LDS} per head_dim (as the decode kernel's)
constexpr int kPrefillCfg[3][3] = {{6, 2, 0}, {3, 2, 0}, {3, 1, 1}};
constexpr int pdim(int D) { return D == 64 ? 0 : D == 128 ? 1 : 2; }

template <typename T, int D, int QO>
hipError_t launch_p(const Params& p, const int32_t* cu_q, int max_q, int causal, hipStream_t s) {
  constexpr int NB_ = kPrefillCfg[pdim(D)][0], OCC = kPrefillCfg[pdim(D)][1];
  constexpr bool QL = kPrefillCfg[pdim(D)][2] != 0;
  dim3 grid((max_q + 15) / 16, p.Hq, p.B);
  hipLaunchKernelGGL((prefill_kernel<T, D, NB_, OCC, QL, QO>), grid, dim3(64), 0, s, p, cu_q,
                     causal);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_pd(const Params& p, const int32_t* cu_q, int max_q, int causal, hipStream_t s) {
  const bool bf = p.qo_bf16 != 0;
  switch (p.D) {
    case 64: return bf ? launch_p<T, 64, 1>(p, cu_q, max_q, causal, s)
                       : launch_p<T, 64, 0>(p, cu_q, max_q, causal, s);
    case 128: return bf ? launch_p<T, 128, 1>(p, cu_q, max_q, causal, s)
                        : launch_p<T, 128, 0>(p, cu_q, max_q, causal, s);
    case 256: return bf ? launch_p<T, 256, 1>(p, cu_q, max_q, causal, s)
                        : launch_p<T, 256, 0>(p, cu_q, max_q, causal, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const Params& p, int dtype, const int32_t* cu_q, int max_q, int causal,
                          hipStream_t s) {
  if (max_q <= 0 || p.B <= 0) return hipSuccess;
  if (dtype == 1) return launch_pd<_Float16>(p, cu_q, max_q, causal, s);
  if (dtype == 2) return launch_pd<__bf16>(p, cu_q, max_q, causal, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
